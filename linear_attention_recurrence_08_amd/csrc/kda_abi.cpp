// C ABI of the KDA library: argument validation, optional content checks, and dispatch to the
// HIP launchers.  Declared in include/kda.h, which states the operation, layouts, ownership and
// error behaviour.
#include "kda.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "kda_internal.h"

namespace kda {
// the 64-token-chunk matrix-core path (bf16, dk = dv = 128)
size_t c64_mfma_workspace_bytes(int64_t nchunks, int64_t N, int64_t H);
hipError_t launch_prefill_c64_mfma(const PrefillArgs& a, void* workspace, int64_t nchunks,
                                   hipStream_t s);
}  // namespace kda

namespace {

bool supported_dim(int d) { return d >= 16 && d <= 128 && d % 16 == 0; }

bool force_general() { return std::getenv("KDA_FORCE_GENERAL") != nullptr; }

// chunks the 64-token-chunk matrix-core path provisions for (an upper bound on the sum over
// sequences of ceil(len / 64)); -1 when the float32 path applies
int64_t c64_mfma_chunks(bool varlen, int64_t N, int64_t B, int64_t T, int dk, int dv, int dtype) {
    if (dtype != KDA_BF16 || dk != 128 || dv != 128 || force_general()) return -1;
    return varlen ? T / 64 + N : B * ((T + 63) / 64);
}

// One token's row of a tensor (H * d elements) is at most 2^20 elements: the streaming kernels
// address a few dozen consecutive rows with 32-bit byte offsets.
bool rows_ok(int H, int dk, int dv) {
    return static_cast<int64_t>(H) * (dk > dv ? dk : dv) <= (int64_t{1} << 20);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool validate_enabled() {
    const char* e = std::getenv("KDA_VALIDATE");
    return e && std::strcmp(e, "1") == 0;
}

float host_bf16(uint16_t b) {
    uint32_t u = static_cast<uint32_t>(b) << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

// Copy a device buffer to the host on the caller's stream and wait (validation mode only).
int fetch(void* dst, const void* src, size_t bytes, hipStream_t s) {
    if (bytes == 0) return KDA_OK;
    if (hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToHost, s) != hipSuccess) return KDA_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return KDA_ERR_HIP;
    return KDA_OK;
}

int check_gate_range(const void* g, int64_t count, int dtype, hipStream_t s) {
    if (count == 0) return KDA_OK;
    if (dtype == KDA_BF16) {
        std::vector<uint16_t> h(static_cast<size_t>(count));
        int st = fetch(h.data(), g, h.size() * 2, s);
        if (st) return st;
        for (uint16_t b : h) {
            const float x = host_bf16(b);
            if (!(x >= -5.0f && x <= 0.0f)) return KDA_ERR_RANGE;
        }
    } else {
        std::vector<float> h(static_cast<size_t>(count));
        int st = fetch(h.data(), g, h.size() * 4, s);
        if (st) return st;
        for (float x : h)
            if (!(x >= -5.0f && x <= 0.0f)) return KDA_ERR_RANGE;
    }
    return KDA_OK;
}

// Token-range split: every sequence is cut into segments of seg_len tokens, at most P of them,
// the last running to the sequence end (P = 1: none).  It applies to bf16 with dk = dv = 128.
// The plan is made for sequences of L tokens (T, or the caller's max_seqlen bound with
// cu_seqlens): requested = 0 picks the largest P whose 2 (2 P - 1) N H workgroups hold one CU each
// (256 CUs), with at least 256 tokens per segment; a requested count is capped at kMaxSplit.
// seg_len is a multiple of 64 so that the output correction's 64-token blocks never straddle two
// segments.
constexpr int64_t kMaxSplit = 16;
struct SplitPlan {
    int64_t P = 1;
    int64_t seg_len = 0;
};
SplitPlan split_plan(bool varlen, int num_seqs, int max_seqlen, int B, int T, int H, int dk,
                     int dv, int dtype, int requested) {
    SplitPlan sp;
    const int64_t N = varlen ? num_seqs : B;
    const int64_t L = varlen ? max_seqlen : T;
    if (dtype != KDA_BF16 || dk != 128 || dv != 128 || force_general() || N <= 0 || L <= 0 ||
        H <= 0 || requested < 0 || (varlen && B != 1))
        return sp;
    const int64_t pairs = N * H;
    if (pairs > 65535) return sp;          // the completion kernels put pairs on the grid's y
    int64_t P = requested;
    if (P == 0) {
        if (2 * pairs >= 128) return sp;
        P = std::min<int64_t>((128 / pairs + 1) / 2, L / 256);
    }
    P = std::min(P, kMaxSplit);
    if (P <= 1) return sp;
    const int64_t len = ((L + P - 1) / P + 63) / 64 * 64;
    const int64_t used = (L + len - 1) / len;
    if (used <= 1) return sp;
    sp.P = used;
    sp.seg_len = len;
    return sp;
}
// workspace of a split: M_t^T q_t of every token [Ttot, H, 128] bf16, then the final states of
// both parts of every segment [P, 2, N H, 128, 128] float32
size_t split_om_bytes(int64_t Ttot, int H) {
    return (static_cast<size_t>(Ttot) * H * 128 * 2 + 255) / 256 * 256;
}
size_t split_workspace_bytes(const SplitPlan& sp, int64_t N, int64_t Ttot, int H) {
    if (sp.P <= 1) return 0;
    return split_om_bytes(Ttot, H) + static_cast<size_t>(sp.P) * 2 * N * H * 128 * 128 * 4;
}

// The output stage after a prefill, y = RMSNorm(o) * weight * sigmoid(gate) per (token, head).
struct GateSpec {
    const void* gate;
    const float* weight;
    float eps;
    void* y;
};

// The fused output stage runs inside the one-workgroup-per-head prefill kernel.
bool gate_fuses(int64_t N, int H, int dk, int dv, int dtype) {
    return dtype == KDA_BF16 && dk == 128 && dv == 128 && !force_general() && N * H >= 256;
}

// Prefill with optional snapshots (snap_stride 0: none); chunk64 selects the 64-token-chunk
// kernel (no snapshots); split (P > 1) the token-range split of the matrix-core kernel; gs the
// output stage (no snapshots, chunk64 or split; o may then be NULL).
int chunk_fwd_impl(const void* q, const void* k, const void* v, const void* g, const void* beta,
                   const float* h0, const int32_t* cu_seqlens, int num_seqs, void* o, float* hT,
                   float* snaps, const int32_t* snap_offsets, int snap_stride, int B, int T,
                   int H, int dk, int dv, int dtype, void* stream, bool chunk64 = false,
                   void* workspace = nullptr, size_t workspace_bytes = 0,
                   const SplitPlan* split = nullptr, const GateSpec* gs = nullptr) {
    if (dtype != KDA_BF16 && dtype != KDA_F32) return KDA_ERR_DTYPE;
    if (B < 0 || T < 0 || H <= 0 || num_seqs < 0) return KDA_ERR_SHAPE;
    if (!supported_dim(dk) || !supported_dim(dv)) return KDA_ERR_UNSUPPORTED;
    if (!rows_ok(H, dk, dv)) return KDA_ERR_SHAPE;
    if (gs && (!(gs->eps >= 0.f) || !std::isfinite(gs->eps))) return KDA_ERR_RANGE;
    if (snap_stride < 0 || snap_stride % 16 != 0) return KDA_ERR_STRIDE;
    const bool want_snaps = snap_stride > 0;
    int64_t N, Ttot;
    if (cu_seqlens) {
        if (B != 1) return KDA_ERR_SEQLENS;
        N = num_seqs;
        Ttot = T;
        if (want_snaps && !snap_offsets) return KDA_ERR_NULL;
    } else {
        N = B;
        Ttot = static_cast<int64_t>(B) * T;
    }
    if (Ttot > 0 && (!q || !k || !v || !g || !beta || (!o && !gs))) return KDA_ERR_NULL;
    if (gs && Ttot > 0 && (!gs->gate || !gs->y)) return KDA_ERR_NULL;
    if (gs && Ttot > 0 &&
        (!aligned(gs->gate, 16) || !aligned(gs->y, 16) || (o && !aligned(o, 16))))
        return KDA_ERR_ALIGN;
    // with equal lengths, snapshots exist iff T >= stride; with cu_seqlens the offsets say so
    if (want_snaps && !snaps && !cu_seqlens && N > 0 && T >= snap_stride) return KDA_ERR_NULL;
    if (N == 0 || (Ttot == 0 && !hT)) return KDA_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int64_t c64_chunks = -1;   // >= 0: the 64-token-chunk matrix-core path, with this many chunks
    const bool splitting = split && split->P > 1 && !want_snaps && !chunk64;
    if (splitting && (!workspace || workspace_bytes < split_workspace_bytes(*split, N, Ttot, H) ||
                      (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0))
        return KDA_ERR_WORKSPACE;
    if (chunk64) {
        c64_chunks = c64_mfma_chunks(cu_seqlens != nullptr, N, B, T, dk, dv, dtype);
        if (c64_chunks >= 0 &&
            (!workspace || workspace_bytes < kda::c64_mfma_workspace_bytes(c64_chunks, N, H) ||
             (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0))
            return KDA_ERR_WORKSPACE;
    }

    if (validate_enabled()) {
        std::vector<int32_t> cu;
        if (cu_seqlens) {
            cu.resize(static_cast<size_t>(N + 1));
            int st = fetch(cu.data(), cu_seqlens, cu.size() * 4, s);
            if (st) return st;
            if (cu[0] != 0 || cu[N] != Ttot) return KDA_ERR_SEQLENS;
            for (int64_t i = 0; i < N; ++i)
                if (cu[i + 1] < cu[i]) return KDA_ERR_SEQLENS;
        }
        if (want_snaps && cu_seqlens) {
            std::vector<int32_t> so(static_cast<size_t>(N + 1));
            int st = fetch(so.data(), snap_offsets, so.size() * 4, s);
            if (st) return st;
            if (so[0] != 0) return KDA_ERR_STRIDE;
            for (int64_t i = 0; i < N; ++i)
                if (so[i + 1] - so[i] != (cu[i + 1] - cu[i]) / snap_stride) return KDA_ERR_STRIDE;
            if (so[N] > 0 && !snaps) return KDA_ERR_NULL;
        }
        int st = check_gate_range(g, Ttot * H * dk, dtype, s);
        if (st) return st;
    }

    // the output stage: inside the prefill kernel, or after it on the outputs (written into y
    // when the caller wants no o, so that the stage then runs in place)
    const bool fused = gs && gate_fuses(N, H, dk, dv, dtype);
    if (gs && !fused && !o) o = gs->y;

    kda::PrefillArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.h0 = h0; a.cu = cu_seqlens; a.o = o; a.hT = hT;
    if (fused) {
        a.gate = gs->gate; a.weight = gs->weight; a.eps = gs->eps; a.y = gs->y;
    }
    a.N = N; a.T = cu_seqlens ? 0 : T; a.H = H; a.dk = dk; a.dv = dv; a.dtype = dtype;
    if (want_snaps && snaps) {
        a.snaps = snaps;
        a.snap_cu = cu_seqlens ? snap_offsets : nullptr;
        a.snap_tiles = snap_stride / 16;
        a.snap_per_seq = cu_seqlens ? 0 : T / snap_stride;
    }

    hipError_t e;
    if (splitting) {
        a.split = split->P;
        a.seg_len = split->seg_len;
        a.oM = workspace;
        a.seg_states = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                split_om_bytes(Ttot, H));
        e = kda::launch_prefill_mfma(a, s);
        if (e == hipSuccess) e = kda::launch_split_finish(a, s);
    } else if (chunk64)
        e = c64_chunks >= 0 ? kda::launch_prefill_c64_mfma(a, workspace, c64_chunks, s)
                            : kda::launch_prefill_c64(a, s);
    else if (dtype == KDA_BF16 && dk == 128 && dv == 128 && !force_general())
        e = kda::launch_prefill_mfma(a, s);
    else
        e = kda::launch_prefill_general(a, s);
    if (e == hipSuccess && gs && !fused && Ttot > 0) {
        kda::GateArgs ga;
        ga.o = o; ga.gate = gs->gate; ga.weight = gs->weight; ga.eps = gs->eps; ga.y = gs->y;
        ga.rows = Ttot * H; ga.dv = dv; ga.dtype = dtype;
        e = kda::launch_output_gate(ga, s);
    }
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

extern "C" {

int kda_version(void) { return 100; }  // 0.1.0

const char* kda_status_string(int status) {
    switch (status) {
        case KDA_OK: return "ok";
        case KDA_ERR_NULL: return "a required pointer is NULL";
        case KDA_ERR_SHAPE: return "negative or inconsistent sizes, or H * max(dk, dv) > 2^20";
        case KDA_ERR_DTYPE: return "dtype must be KDA_BF16 or KDA_F32";
        case KDA_ERR_UNSUPPORTED: return "dk and dv must be multiples of 16 in [16, 128]";
        case KDA_ERR_SEQLENS: return "bad cu_seqlens (needs B == 1; non-decreasing from 0 to T)";
        case KDA_ERR_RANGE: return "g (log alpha) outside [-5, 0], or eps < 0";
        case KDA_ERR_HIP: return "HIP runtime error";
        case KDA_ERR_STRIDE:
            return "snapshot stride must be a positive multiple of 16, with matching snap_offsets";
        case KDA_ERR_ALIGN: return "output-stage buffers must be 16-byte aligned";
        case KDA_ERR_WORKSPACE:
            return "workspace missing, smaller than the size its query returns "
                   "(kda_chunk_fwd_chunk64_workspace_bytes, kda_chunk_fwd_split_workspace_bytes), "
                   "or not 256-byte aligned";
        case KDA_ERR_SCRATCH:
            return "the call needs more workspace than the library's static device array holds "
                   "(kda_chunk_fwd_split_noalloc: 32 MiB per device)";
        default: return "unknown status";
    }
}

int kda_chunk_fwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
                  const float* h0, const int32_t* cu_seqlens, int num_seqs, void* o, float* hT,
                  int B, int T, int H, int dk, int dv, int dtype, void* stream) {
    return chunk_fwd_impl(q, k, v, g, beta, h0, cu_seqlens, num_seqs, o, hT, nullptr, nullptr, 0,
                          B, T, H, dk, dv, dtype, stream);
}

int kda_chunk_fwd_gated(const void* q, const void* k, const void* v, const void* g,
                        const void* beta, const float* h0, const int32_t* cu_seqlens,
                        int num_seqs, const void* gate, const float* weight, float eps, void* o,
                        void* y, float* hT, int B, int T, int H, int dk, int dv, int dtype,
                        void* stream) {
    const GateSpec gs{gate, weight, eps, y};
    return chunk_fwd_impl(q, k, v, g, beta, h0, cu_seqlens, num_seqs, o, hT, nullptr, nullptr, 0,
                          B, T, H, dk, dv, dtype, stream, false, nullptr, 0, nullptr, &gs);
}

int kda_chunk_fwd_gated_fuses(int num_seqs, int B, int H, int dk, int dv, int dtype,
                              int varlen) {
    if (B < 0 || num_seqs < 0 || H <= 0) return 0;
    return gate_fuses(varlen ? num_seqs : B, H, dk, dv, dtype) ? 1 : 0;
}

int kda_chunk_fwd_chunk64(const void* q, const void* k, const void* v, const void* g,
                          const void* beta, const float* h0, const int32_t* cu_seqlens,
                          int num_seqs, void* o, float* hT,
                          int B, int T, int H, int dk, int dv, int dtype,
                          void* workspace, size_t workspace_bytes, void* stream) {
    return chunk_fwd_impl(q, k, v, g, beta, h0, cu_seqlens, num_seqs, o, hT, nullptr, nullptr, 0,
                          B, T, H, dk, dv, dtype, stream, true, workspace, workspace_bytes);
}

size_t kda_chunk_fwd_chunk64_workspace_bytes(const int32_t* cu_seqlens, int num_seqs, int B,
                                             int T, int H, int dk, int dv, int dtype) {
    if ((dtype != KDA_BF16 && dtype != KDA_F32) || B < 0 || T < 0 || H <= 0 || num_seqs < 0 ||
        !supported_dim(dk) || !supported_dim(dv) || !rows_ok(H, dk, dv) ||
        (cu_seqlens && B != 1))
        return 0;
    const int64_t N = cu_seqlens ? num_seqs : B;
    const int64_t chunks = c64_mfma_chunks(cu_seqlens != nullptr, N, B, T, dk, dv, dtype);
    return chunks < 0 || N == 0 ? 0 : kda::c64_mfma_workspace_bytes(chunks, N, H);
}

int kda_chunk_fwd_split(const void* q, const void* k, const void* v, const void* g,
                        const void* beta, const float* h0, const int32_t* cu_seqlens,
                        int num_seqs, int max_seqlen, void* o, float* hT,
                        int B, int T, int H, int dk, int dv, int dtype, int segments,
                        void* workspace, size_t workspace_bytes, void* stream) {
    if (segments < 0 || (cu_seqlens && max_seqlen < 0)) return KDA_ERR_SHAPE;
    const SplitPlan sp = split_plan(cu_seqlens != nullptr, num_seqs, max_seqlen, B, T, H, dk, dv,
                                    dtype, segments);
    return chunk_fwd_impl(q, k, v, g, beta, h0, cu_seqlens, num_seqs, o, hT, nullptr, nullptr, 0,
                          B, T, H, dk, dv, dtype, stream, false, workspace, workspace_bytes, &sp);
}

int kda_chunk_fwd_split_segments(const int32_t* cu_seqlens, int num_seqs, int max_seqlen, int B,
                                 int T, int H, int dk, int dv, int dtype, int segments) {
    return static_cast<int>(split_plan(cu_seqlens != nullptr, num_seqs, max_seqlen, B, T, H, dk,
                                       dv, dtype, segments).P);
}

size_t kda_chunk_fwd_split_workspace_bytes(const int32_t* cu_seqlens, int num_seqs,
                                           int max_seqlen, int B, int T, int H, int dk, int dv,
                                           int dtype, int segments) {
    if (B < 0 || T < 0 || H <= 0 || num_seqs < 0 || !rows_ok(H, dk, dv)) return 0;
    const bool varlen = cu_seqlens != nullptr;
    const int64_t N = varlen ? num_seqs : B;
    const int64_t Ttot = varlen ? T : static_cast<int64_t>(B) * T;
    return split_workspace_bytes(split_plan(varlen, num_seqs, max_seqlen, B, T, H, dk, dv, dtype,
                                            segments), N, Ttot, H);
}

int kda_chunk_fwd_snapshots(const void* q, const void* k, const void* v, const void* g,
                            const void* beta, const float* h0, const int32_t* cu_seqlens,
                            int num_seqs, void* o, float* hT, float* snaps,
                            const int32_t* snap_offsets, int snap_stride,
                            int B, int T, int H, int dk, int dv, int dtype, void* stream) {
    if (snap_stride <= 0) return KDA_ERR_STRIDE;
    return chunk_fwd_impl(q, k, v, g, beta, h0, cu_seqlens, num_seqs, o, hT, snaps, snap_offsets,
                          snap_stride, B, T, H, dk, dv, dtype, stream);
}

int kda_output_gate(const void* o, const void* gate, const float* weight, float eps, void* y,
                    int Ttot, int H, int dv, int dtype, void* stream) {
    if (dtype != KDA_BF16 && dtype != KDA_F32) return KDA_ERR_DTYPE;
    if (Ttot < 0 || H <= 0) return KDA_ERR_SHAPE;
    if (!supported_dim(dv)) return KDA_ERR_UNSUPPORTED;
    if (!rows_ok(H, dv, dv)) return KDA_ERR_SHAPE;
    if (!(eps >= 0.f) || !std::isfinite(eps)) return KDA_ERR_RANGE;
    if (Ttot == 0) return KDA_OK;
    if (!o || !gate || !y) return KDA_ERR_NULL;
    if (!aligned(o, 16) || !aligned(gate, 16) || !aligned(y, 16)) return KDA_ERR_ALIGN;
    kda::GateArgs a;
    a.o = o; a.gate = gate; a.weight = weight; a.eps = eps; a.y = y;
    a.rows = static_cast<int64_t>(Ttot) * H; a.dv = dv; a.dtype = dtype;
    const hipError_t e = kda::launch_output_gate(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

namespace {
// Decode with an optional fused output stage (gate == nullptr: none).
int decode_impl(const void* q, const void* k, const void* v, const void* g, const void* beta,
                float* S, const void* gate, const float* weight, float eps, void* o, void* y,
                int N, int H, int dk, int dv, int dtype, void* stream) {
    if (dtype != KDA_BF16 && dtype != KDA_F32) return KDA_ERR_DTYPE;
    if (N < 0 || H <= 0) return KDA_ERR_SHAPE;
    if (!supported_dim(dk) || !supported_dim(dv)) return KDA_ERR_UNSUPPORTED;
    if (!rows_ok(H, dk, dv)) return KDA_ERR_SHAPE;
    if (N == 0) return KDA_OK;
    if (!q || !k || !v || !g || !beta || !S || !o) return KDA_ERR_NULL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (validate_enabled()) {
        int st = check_gate_range(g, static_cast<int64_t>(N) * H * dk, dtype, s);
        if (st) return st;
    }
    hipError_t e;
    // the 128 x 128 kernel uses 16-byte state accesses and 4-element input/output accesses
    const uintptr_t va = dtype == KDA_BF16 ? 8 : 16;
    if (dk == 128 && dv == 128 && aligned(S, 16) && aligned(v, va) && aligned(o, va) &&
        (!gate || (aligned(gate, va) && aligned(y, va)))) {
        kda::DecodeArgs a;
        a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.S = S; a.o = o;
        a.N = N; a.H = H; a.dk = dk; a.dv = dv; a.dtype = dtype;
        a.gate = gate; a.weight = weight; a.eps = eps; a.y = y;
        return kda::launch_decode_d128(a, s) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
    } else {
        // other head sizes: the general tile path over N one-token sequences, state in place
        kda::PrefillArgs a;
        a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
        a.h0 = S; a.cu = nullptr; a.o = o; a.hT = S;
        a.N = N; a.T = 1; a.H = H; a.dk = dk; a.dv = dv; a.dtype = dtype;
        e = kda::launch_prefill_general(a, s);
    }
    if (e != hipSuccess) return KDA_ERR_HIP;
    if (gate) return kda_output_gate(o, gate, weight, eps, y, N, H, dv, dtype, stream);
    return KDA_OK;
}
}  // namespace

int kda_decode_step(const void* q, const void* k, const void* v, const void* g, const void* beta,
                    float* S, void* o, int N, int H, int dk, int dv, int dtype, void* stream) {
    return decode_impl(q, k, v, g, beta, S, nullptr, nullptr, 0.f, o, nullptr, N, H, dk, dv,
                       dtype, stream);
}

int kda_decode_step_gated(const void* q, const void* k, const void* v, const void* g,
                          const void* beta, float* S, const void* gate, const float* weight,
                          float eps, void* o, void* y, int N, int H, int dk, int dv, int dtype,
                          void* stream) {
    if (dtype != KDA_BF16 && dtype != KDA_F32) return KDA_ERR_DTYPE;
    if (N < 0 || H <= 0) return KDA_ERR_SHAPE;
    if (!supported_dim(dk) || !supported_dim(dv)) return KDA_ERR_UNSUPPORTED;
    if (!rows_ok(H, dk, dv)) return KDA_ERR_SHAPE;
    if (!(eps >= 0.f) || !std::isfinite(eps)) return KDA_ERR_RANGE;
    if (N == 0) return KDA_OK;
    if (!gate || !y) return KDA_ERR_NULL;
    // decided before anything runs: the fused kernel (same test as in decode_impl), else the
    // decode followed by the output-stage kernel, which needs 16-byte aligned rows
    const uintptr_t va = dtype == KDA_BF16 ? 8 : 16;
    const bool fused = dk == 128 && dv == 128 && aligned(S, 16) && aligned(v, va) &&
                       aligned(o, va) && aligned(gate, va) && aligned(y, va);
    if (!fused && (!aligned(o, 16) || !aligned(gate, 16) || !aligned(y, 16))) return KDA_ERR_ALIGN;
    return decode_impl(q, k, v, g, beta, S, gate, weight, eps, o, y, N, H, dk, dv, dtype, stream);
}

int kda_frontend(const void* x_q, const void* x_k, const void* x_v, const void* x_z,
                 const void* x_b, const float* w_q, const float* w_k, const float* w_v,
                 const float* z_bias, const float* A, float g_min, float eps,
                 const int32_t* cu_seqlens, int num_seqs, const void* conv_in, void* conv_out,
                 void* q, void* k, void* v, void* g, void* beta,
                 int B, int T, int H, int dk, int dv, int dtype, void* stream) {
    if (dtype != KDA_BF16 && dtype != KDA_F32) return KDA_ERR_DTYPE;
    if (B < 0 || T < 0 || H <= 0 || num_seqs < 0) return KDA_ERR_SHAPE;
    if (!supported_dim(dk) || !supported_dim(dv)) return KDA_ERR_UNSUPPORTED;
    if (!rows_ok(H, dk, dv)) return KDA_ERR_SHAPE;
    if (!(g_min < 0.f) || !std::isfinite(g_min) || !(eps >= 0.f) || !std::isfinite(eps))
        return KDA_ERR_RANGE;
    int64_t N, Ttot;
    if (cu_seqlens) {
        if (B != 1) return KDA_ERR_SEQLENS;
        N = num_seqs;
        Ttot = T;
    } else {
        N = B;
        Ttot = static_cast<int64_t>(B) * T;
    }
    if (N == 0 || (Ttot == 0 && !conv_out)) return KDA_OK;
    if (Ttot > 0 && (!x_q || !x_k || !x_v || !x_z || !x_b || !w_q || !w_k || !w_v || !z_bias ||
                     !A || !q || !k || !v || !g || !beta))
        return KDA_ERR_NULL;
    for (const void* p : {x_q, x_k, x_v, x_z, conv_in, static_cast<const void*>(conv_out),
                          static_cast<const void*>(q), static_cast<const void*>(k),
                          static_cast<const void*>(v), static_cast<const void*>(g)})
        if (p && !aligned(p, 16)) return KDA_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (validate_enabled() && cu_seqlens) {
        std::vector<int32_t> cu(static_cast<size_t>(N + 1));
        int st = fetch(cu.data(), cu_seqlens, cu.size() * 4, s);
        if (st) return st;
        if (cu[0] != 0 || cu[N] != Ttot) return KDA_ERR_SEQLENS;
        for (int64_t i = 0; i < N; ++i)
            if (cu[i + 1] < cu[i]) return KDA_ERR_SEQLENS;
    }
    kda::FrontArgs a;
    a.xq = x_q; a.xk = x_k; a.xv = x_v; a.xz = x_z; a.xb = x_b;
    a.wq = w_q; a.wk = w_k; a.wv = w_v; a.zbias = z_bias; a.A = A; a.g_min = g_min; a.eps = eps;
    a.cu = cu_seqlens; a.conv_in = conv_in; a.conv_out = conv_out;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.N = N; a.T = cu_seqlens ? 0 : T; a.Ttot = Ttot; a.H = H; a.dk = dk; a.dv = dv;
    a.dtype = dtype;
    return kda::launch_frontend(a, s) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

int kda_decode_step_layer(const void* x_q, const void* x_k, const void* x_v, const void* x_z,
                          const void* x_b, const float* w_q, const float* w_k, const float* w_v,
                          const float* z_bias, const float* A, float g_min, float norm_eps,
                          void* conv_state, float* S, const void* gate, const float* weight,
                          float eps, void* o, void* y, int N, int H, int dk, int dv, int dtype,
                          void* stream) {
    if (dtype != KDA_BF16 && dtype != KDA_F32) return KDA_ERR_DTYPE;
    if (N < 0 || H <= 0) return KDA_ERR_SHAPE;
    if (dk != 128 || dv != 128) return KDA_ERR_UNSUPPORTED;   // the fused kernel's head size
    if (!rows_ok(H, dk, dv)) return KDA_ERR_SHAPE;
    if (!(g_min < 0.f) || !std::isfinite(g_min) || !(norm_eps >= 0.f) ||
        !std::isfinite(norm_eps) || !(eps >= 0.f) || !std::isfinite(eps))
        return KDA_ERR_RANGE;
    if (N == 0) return KDA_OK;
    if (!x_q || !x_k || !x_v || !x_z || !x_b || !w_q || !w_k || !w_v || !z_bias || !A ||
        !conv_state || !S || !gate || !y)
        return KDA_ERR_NULL;
    // 16-byte state accesses, 4-element gate/o/y accesses (the inputs are read per element)
    const uintptr_t va = dtype == KDA_BF16 ? 8 : 16;
    if (!aligned(S, 16) || !aligned(gate, va) || !aligned(y, va) || (o && !aligned(o, va)))
        return KDA_ERR_ALIGN;
    kda::DecodeArgs a;
    a.q = a.k = a.v = a.g = a.beta = nullptr;
    a.S = S; a.o = o; a.N = N; a.H = H; a.dk = dk; a.dv = dv; a.dtype = dtype;
    a.gate = gate; a.weight = weight; a.eps = eps; a.y = y;
    a.xq = x_q; a.xk = x_k; a.xv = x_v; a.xz = x_z; a.xb = x_b;
    a.wq = w_q; a.wk = w_k; a.wv = w_v; a.zbias = z_bias; a.A = A;
    a.g_min = g_min; a.norm_eps = norm_eps; a.conv = conv_state;
    return kda::launch_decode_d128(a, static_cast<hipStream_t>(stream)) == hipSuccess
               ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
