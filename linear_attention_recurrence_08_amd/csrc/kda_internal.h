// Internal declarations shared by the KDA HIP sources (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// Arguments of one prefill call after validation.  Token t of sequence n lives at packed index
// bos(n) + t, where bos(n) = cu[n] when cu != nullptr and n * T otherwise.
struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const void* beta;
    const float* h0;      // [N, H, dk, dv] or nullptr (zeros)
    const int32_t* cu;    // [N+1] or nullptr
    void* o;              // [Ttot, H, dv]
    float* hT;            // [N, H, dk, dv] or nullptr
    float* snaps = nullptr;              // [Nsnap, H, dk, dv] or nullptr (no snapshots)
    const int32_t* snap_cu = nullptr;    // first snapshot index per sequence, or nullptr
    int64_t snap_tiles = 0;              // snapshot stride in 16-token tiles (0: none)
    int64_t snap_per_seq = 0;            // snapshots per sequence when snap_cu == nullptr
    int64_t N;            // sequences
    int64_t T;            // per-sequence length when cu == nullptr
    int64_t H, dk, dv;
    int dtype;            // 0 = bf16, 1 = f32
    // token-range split (split > 1; bf16, dk = dv = 128): every sequence is cut into segments of
    // seg_len tokens (a multiple of 64), at most `split` of them, the last one running to the
    // sequence end.  Segment 0 runs from h0 into o;
    // each later segment runs as a part B (zero entering state, into o) and a part M (v = 0,
    // identity entering state, its outputs M_t^T q_t into oM); every run's final state goes to
    // seg_states.  launch_split_finish composes the entering states, writes hT and adds
    // S_in^T (M_t^T q_t) to the outputs of the later segments.
    int64_t split = 1;
    int64_t seg_len = 0;
    void* oM = nullptr;             // [Ttot, H, dk] bf16
    float* seg_states = nullptr;    // [split, 2, N * H, dk, dv]
    // fused output stage (gate != nullptr; bf16, dk = dv = 128, the one-workgroup-per-head
    // kernel): y = RMSNorm(o) * weight * sigmoid(gate) per (token, head) row; o may then be
    // nullptr (not written)
    const void* gate = nullptr;          // [Ttot, H, dv]
    const float* weight = nullptr;       // [dv] or nullptr (ones)
    float eps = 0.f;
    void* y = nullptr;                   // [Ttot, H, dv]
};

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const void* beta;
    float* S;             // [N, H, dk, dv], updated in place
    void* o;              // [N, H, dv]
    int64_t N, H, dk, dv;
    int dtype;
    // fused output stage (nullptr gate: none): y = RMSNorm(o) * weight * sigmoid(gate)
    const void* gate = nullptr;          // [N, H, dv]
    const float* weight = nullptr;       // [dv] or nullptr (ones)
    float eps = 0.f;
    void* y = nullptr;                   // [N, H, dv]
    // fused input stage (xq != nullptr; with the output stage, dk = dv = 128): q, k, v, g and
    // beta come from the token's pre-activations and the convolution state, which is updated in
    // place; q, k, v, g and beta above are then unused, and o may be nullptr (not written)
    const void* xq = nullptr;            // [N, H, dk] pre-activations (dtype)
    const void* xk = nullptr;
    const void* xv = nullptr;            // [N, H, dv]
    const void* xz = nullptr;            // [N, H, dk] decay logits before the bias
    const void* xb = nullptr;            // [N, H] write-strength logits
    const float* wq = nullptr;           // [H * dk, 4] convolution taps (tap 3 = current token)
    const float* wk = nullptr;
    const float* wv = nullptr;           // [H * dv, 4]
    const float* zbias = nullptr;        // [H * dk]
    const float* A = nullptr;            // [H]
    float g_min = 0.f, norm_eps = 0.f;
    void* conv = nullptr;                // [N, 3, H * (2 dk + dv)] (dtype), read and overwritten
};

// Output stage over rows of dv values: y = o / sqrt(mean(o^2) + eps) * weight * sigmoid(gate).
struct GateArgs {
    const void* o;
    const void* gate;
    const float* weight;  // [dv] or nullptr (ones)
    float eps;
    void* y;
    int64_t rows;         // Ttot * H
    int64_t dv;
    int dtype;
};

// Input stage (short convolution, Swish, L2 norm, sigmoid beta, bounded log-decay).
struct FrontArgs {
    const void* xq;       // [Ttot, H, dk] pre-activations (dtype)
    const void* xk;       // [Ttot, H, dk]
    const void* xv;       // [Ttot, H, dv]
    const void* xz;       // [Ttot, H, dk] decay logits before the bias
    const void* xb;       // [Ttot, H] write-strength logits
    const float* wq;      // [H * dk, 4] convolution taps (tap 3 = current token)
    const float* wk;      // [H * dk, 4]
    const float* wv;      // [H * dv, 4]
    const float* zbias;   // [H * dk]
    const float* A;       // [H]
    float g_min, eps;
    const int32_t* cu;    // [N + 1] or nullptr (N sequences of length T)
    const void* conv_in;  // [N, 3, H * (2 dk + dv)] (dtype) or nullptr (zeros)
    void* conv_out;       // [N, 3, H * (2 dk + dv)] or nullptr; may alias conv_in
    void* q;              // [Ttot, H, dk] outputs (dtype)
    void* k;
    void* v;              // [Ttot, H, dv]
    void* g;              // [Ttot, H, dk]
    void* beta;           // [Ttot, H]
    int64_t N, T, Ttot, H, dk, dv;
    int dtype;
};

// Each launcher returns hipSuccess or the launch error.
hipError_t launch_prefill_general(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t s);   // bf16, dk = dv = 128
hipError_t launch_prefill_c64(const PrefillArgs& a, hipStream_t s);    // 64-token chunks
hipError_t launch_split_finish(const PrefillArgs& a, hipStream_t s);   // after a split prefill
hipError_t launch_decode_d128(const DecodeArgs& a, hipStream_t s);     // dk = dv = 128
hipError_t launch_output_gate(const GateArgs& a, hipStream_t s);      // 16-byte aligned rows
hipError_t launch_frontend(const FrontArgs& a, hipStream_t s);        // 16-byte aligned rows

// ---------------------------------------------------------------------------------------------
// Number-format helpers (device)
// ---------------------------------------------------------------------------------------------
typedef uint16_t bf16_t;  // raw bfloat16 bits

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Two float32 values to packed bfloat16 (low half = lo), rounding to nearest even, NaN kept a
// NaN: one v_cvt_pk_bf16_f32.
typedef float kda_fpair __attribute__((ext_vector_type(2)));
typedef __bf16 kda_bfpair __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const kda_fpair v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, kda_bfpair));
}
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    return static_cast<bf16_t>(pack_bf16x2(f, 0.f) & 0xffffu);
}

// Sum over each aligned group of 16 lanes, left in every lane of the group: a butterfly of DPP
// moves within the 16-lane row (mirror, half-mirror, then swaps of neighbours and of pairs in
// each quad), no LDS traffic.
template <int CTRL> __device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float sum16(float x) {
    x += dpp_mov<0x140>(x);   // row_mirror: lane i <- lane 15 - i
    x += dpp_mov<0x141>(x);   // row_half_mirror: lane i <- lane 7 - i within each half
    x += dpp_mov<0xB1>(x);    // quad_perm [1, 0, 3, 2]
    x += dpp_mov<0x4E>(x);    // quad_perm [2, 3, 0, 1]
    return x;
}

template <typename T> struct io;
template <> struct io<float> {
    __device__ static __forceinline__ float load(const float* p) { return *p; }
    __device__ static __forceinline__ void store(float* p, float x) { *p = x; }
};
template <> struct io<bf16_t> {
    __device__ static __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(*p); }
    __device__ static __forceinline__ void store(bf16_t* p, float x) { *p = f32_to_bf16(x); }
};

// Eight consecutive elements as float32, one 16-byte access for bf16 and two for float32
// (non-temporal: the streaming stages touch each element once).  Addresses must be 16-byte
// aligned.
typedef float f32v4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32v4 __attribute__((ext_vector_type(4)));
template <typename T> struct Row8;
template <> struct Row8<bf16_t> {
    static __device__ __forceinline__ void load(const bf16_t* p, float x[8]) {
        const u32v4 u = __builtin_nontemporal_load(reinterpret_cast<const u32v4*>(p));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(u[i] << 16);
            x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void store(bf16_t* p, const float x[8]) {
        u32v4 u;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            u[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
        __builtin_nontemporal_store(u, reinterpret_cast<u32v4*>(p));
    }
};
// The same eight elements kept in their stored form (fewer registers while loads are in flight).
template <typename T> struct Raw8;
template <> struct Raw8<bf16_t> {
    u32v4 u;
    __device__ __forceinline__ void load(const bf16_t* p) {
        u = __builtin_nontemporal_load(reinterpret_cast<const u32v4*>(p));
    }
    __device__ __forceinline__ void zero() { u = (u32v4){0u, 0u, 0u, 0u}; }
    __device__ __forceinline__ void unpack(float x[8]) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(u[i] << 16);
            x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    }
};
template <> struct Raw8<float> {
    f32v4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = __builtin_nontemporal_load(reinterpret_cast<const f32v4*>(p));
        b = __builtin_nontemporal_load(reinterpret_cast<const f32v4*>(p) + 1);
    }
    __device__ __forceinline__ void zero() { a = (f32v4){0.f, 0.f, 0.f, 0.f}; b = a; }
    __device__ __forceinline__ void unpack(float x[8]) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
    }
};
template <> struct Row8<float> {
    static __device__ __forceinline__ void load(const float* p, float x[8]) {
        const f32v4 a = __builtin_nontemporal_load(reinterpret_cast<const f32v4*>(p));
        const f32v4 b = __builtin_nontemporal_load(reinterpret_cast<const f32v4*>(p) + 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
    }
    static __device__ __forceinline__ void store(float* p, const float x[8]) {
        __builtin_nontemporal_store((f32v4){x[0], x[1], x[2], x[3]},
                                    reinterpret_cast<f32v4*>(p));
        __builtin_nontemporal_store((f32v4){x[4], x[5], x[6], x[7]},
                                    reinterpret_cast<f32v4*>(p) + 1);
    }
};

}  // namespace kda
