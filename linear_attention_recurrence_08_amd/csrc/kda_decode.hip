// KDA single-token decode step for dk = dv = 128, in place on the float32 state.
//
// One token per sequence: S' = Diag(alpha) S, u = beta (v - S'^T k), S <- S' + k u^T,
// o = S^T q = S'^T q + (k.q) u.  ("Kimi K3, explained", section "Kimi Delta Attention: making the
// radical option work": k and v update S(t-1), q reads the updated S(t); "Kimi K3's hybrid block,
// from first principles", paragraph "What the state costs": a fixed 128 x 128 state per head.)
//
// The step is bound by HBM: each (sequence, head) reads and writes its 64 KiB state once and
// does ~7 flops per state element.  A workgroup of 256 threads owns two (sequence, head) pairs
// (one when N * H is odd) and requests both states before reducing the first, so one head's
// loads overlap the other's reduction and stores.  Per head:
// thread (rg, cg) holds rows rg, rg+8, ..., rg+120 (16 rows) x columns 4cg..4cg+3 of S in
// registers as 16 float4, so the state is loaded once with full 16-byte accesses, reduced over
// the key axis (two column partial sums S'^T k and S'^T q, plus k.q) with one cross-lane step
// and one LDS step, then written back once with non-temporal stores.  Variants fuse the output
// stage after the step and the input stage before it (the whole token mixer in one launch).
#include "kda_internal.h"

namespace kda {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

template <typename Tin>
__device__ __forceinline__ void load4(const Tin* p, float out[4]);
template <>
__device__ __forceinline__ void load4<float>(const float* p, float out[4]) {
    const f4 x = *reinterpret_cast<const f4*>(p);
    out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
}
template <>
__device__ __forceinline__ void load4<bf16_t>(const bf16_t* p, float out[4]) {
    const uint2 x = *reinterpret_cast<const uint2*>(p);
    out[0] = __uint_as_float(x.x << 16);
    out[1] = __uint_as_float(x.x & 0xffff0000u);
    out[2] = __uint_as_float(x.y << 16);
    out[3] = __uint_as_float(x.y & 0xffff0000u);
}

template <typename Tin>
__device__ __forceinline__ void store4(Tin* p, const float x[4]);
template <>
__device__ __forceinline__ void store4<float>(float* p, const float x[4]) {
    f4 y = {x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f4*>(p) = y;
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, const float x[4]) {
    uint2 y;
    y.x = pack_bf16x2(x[0], x[1]);
    y.y = pack_bf16x2(x[2], x[3]);
    *reinterpret_cast<uint2*>(p) = y;
}

constexpr int D = 128;
constexpr int NRED = 9;  // per column group: S'^T k (4), S'^T q (4), k.q

__device__ __forceinline__ float sigm(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

// HPW heads per workgroup: every head's 64 KiB state is requested before the first one is
// reduced, so the second head's loads are in flight while the first head is reduced and stored.
// GATED adds the output stage y = o / sqrt(mean(o^2) + eps) * w * sigmoid(gate) over the head's
// 128 outputs ("Kimi K3's hybrid block, from first principles", section "From linear attention to
// the delta rule": the output is RMS-normalised per head and multiplied by a sigmoid gate of the
// token): every 32-lane half-wave holds the whole row (4 columns per lane), so the sum of squares
// is five xor shuffles.
// FRONT adds the input stage in front (same section: q and k get a four-tap causal convolution,
// Swish and unit-length normalisation, v the convolution and Swish, beta a sigmoid of the token's
// logit, and the log-decay g = g_min sigmoid(A_h (z + bias_c)), the reading kda_frontend takes).
// Thread (head hp, channel c) convolves its channel of q, k and v over the three saved inputs and
// the current one, shifts the saved inputs by one token in place, and forms g and beta; the two
// L2 norms of a head span its two waves and meet in LDS.  q, k, v, g and beta stay in float32 and
// never reach HBM, while the state loads issued before them are in flight.
// The one-launch layer step (FRONT) asks for three waves per SIMD: 168 registers with 20 spilled,
// 3.4% faster than two waves per SIMD at 186 registers.  The other forms keep two (three made
// the plain step 2.2% slower and the gated one 0.4%).
template <typename Tin, int HPW, bool GATED, bool FRONT>
__global__ __launch_bounds__(256, FRONT ? 3 : 1) void kda_decode_d128_kernel(DecodeArgs a) {
    static_assert(!FRONT || GATED, "the fused input stage comes with the output stage");
    __shared__ float sk[HPW][D], sq[HPW][D], sa[HPW][D];
    __shared__ float red[HPW][4][32][NRED + 1];
    __shared__ float sv[FRONT ? HPW : 1][D], sb[HPW], snorm[HPW][2][2];

    const int tid = threadIdx.x;
    const int cg = tid & 31;          // columns 4cg .. 4cg+3
    const int rg = tid >> 5;          // rows rg + 8 i
    const int w = tid >> 6, lane = tid & 63;
    const int64_t unit0 = (int64_t)blockIdx.x * HPW;   // (n * H + h) of the first head

    f4 s[HPW][16];
    float vv[HPW][4], b[HPW];
#pragma unroll
    for (int hp = 0; hp < HPW; ++hp) {
        const int64_t unit = unit0 + hp;
        const float* S = a.S + unit * (int64_t)(D * D);
#pragma unroll
        for (int i = 0; i < 16; ++i)
            s[hp][i] = __builtin_nontemporal_load(
                reinterpret_cast<const f4*>(S + (rg + 8 * i) * D + 4 * cg));
    }
    if constexpr (FRONT) {
        const int hp = tid >> 7, c = tid & (D - 1);   // this thread's head and channel
        float yq = 0.f, yk = 0.f, yv = 0.f, al = 0.f, bt = 0.f;
        if (hp < HPW) {
            const int64_t unit = unit0 + hp, n = unit / a.H, h = unit % a.H;
            const int64_t C = a.H * 3 * D;            // columns of the convolution state
            Tin* cs = static_cast<Tin*>(a.conv) + n * 3 * C;
            const int64_t col[3] = {h * D + c, (a.H + h) * D + c, (2 * a.H + h) * D + c};
            const Tin* xs[3] = {static_cast<const Tin*>(a.xq), static_cast<const Tin*>(a.xk),
                                static_cast<const Tin*>(a.xv)};
            const float* ws[3] = {a.wq, a.wk, a.wv};
            float y3[3];
#pragma unroll
            for (int t = 0; t < 3; ++t) {
                const float x = io<Tin>::load(xs[t] + unit * D + c);
                const float s0 = io<Tin>::load(cs + col[t]);
                const float s1 = io<Tin>::load(cs + C + col[t]);
                const float s2 = io<Tin>::load(cs + 2 * C + col[t]);
                const float* w = ws[t] + (h * D + c) * 4;
                const float u = w[0] * s0 + w[1] * s1 + w[2] * s2 + w[3] * x;
                y3[t] = u * sigm(u);
                // the saved inputs move on by one token (this thread alone reads this column)
                io<Tin>::store(cs + col[t], s1);
                io<Tin>::store(cs + C + col[t], s2);
                io<Tin>::store(cs + 2 * C + col[t], x);
            }
            yq = y3[0];
            yk = y3[1];
            yv = y3[2];
            const float z = io<Tin>::load(static_cast<const Tin*>(a.xz) + unit * D + c);
            al = __expf(a.g_min * sigm(a.A[h] * (z + a.zbias[h * D + c])));
            if (c == 0) bt = sigm(io<Tin>::load(static_cast<const Tin*>(a.xb) + unit));
        }
        // the sums of squares of q and k over the head's 128 channels (two waves)
        float ssq = yq * yq, ssk = yk * yk;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            ssq += __shfl_xor(ssq, m, 64);
            ssk += __shfl_xor(ssk, m, 64);
        }
        if (hp < HPW && lane == 0) {
            snorm[hp][w & 1][0] = ssq;
            snorm[hp][w & 1][1] = ssk;
        }
        __syncthreads();
        if (hp < HPW) {
            const float rq = __builtin_amdgcn_rsqf(snorm[hp][0][0] + snorm[hp][1][0] + a.norm_eps);
            const float rk = __builtin_amdgcn_rsqf(snorm[hp][0][1] + snorm[hp][1][1] + a.norm_eps);
            sq[hp][c] = yq * rq;
            sk[hp][c] = yk * rk;
            sa[hp][c] = al;
            sv[hp][c] = yv;
            if (c == 0) sb[hp] = bt;
        }
        __syncthreads();
#pragma unroll
        for (int hp2 = 0; hp2 < HPW; ++hp2) {
#pragma unroll
            for (int j = 0; j < 4; ++j) vv[hp2][j] = sv[hp2][4 * cg + j];
            b[hp2] = sb[hp2];
        }
    } else {
#pragma unroll
        for (int hp = 0; hp < HPW; ++hp) {
            const int64_t unit = unit0 + hp;
            const Tin* q = static_cast<const Tin*>(a.q) + unit * D;
            const Tin* k = static_cast<const Tin*>(a.k) + unit * D;
            const Tin* g = static_cast<const Tin*>(a.g) + unit * D;
            if (tid < D) {
                sk[hp][tid] = io<Tin>::load(k + tid);
                sq[hp][tid] = io<Tin>::load(q + tid);
                sa[hp][tid] = __expf(io<Tin>::load(g + tid));
            }
            load4<Tin>(static_cast<const Tin*>(a.v) + unit * D + 4 * cg, vv[hp]);
            b[hp] = io<Tin>::load(static_cast<const Tin*>(a.beta) + unit);
        }
        __syncthreads();
    }

#pragma unroll
    for (int hp = 0; hp < HPW; ++hp) {
        const int64_t unit = unit0 + hp;
        // fade and partial reductions over this thread's 16 rows
        float part[NRED] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = rg + 8 * i;
            const float al = sa[hp][r], kr = sk[hp][r], qr = sq[hp][r];
            s[hp][i] *= al;
            part[0] += s[hp][i].x * kr; part[1] += s[hp][i].y * kr;
            part[2] += s[hp][i].z * kr; part[3] += s[hp][i].w * kr;
            part[4] += s[hp][i].x * qr; part[5] += s[hp][i].y * qr;
            part[6] += s[hp][i].z * qr; part[7] += s[hp][i].w * qr;
            part[8] += kr * qr;
        }
        // lanes l and l^32 of a wave hold row groups 2w and 2w+1 of the same columns
#pragma unroll
        for (int j = 0; j < NRED; ++j) part[j] += __shfl_xor(part[j], 32, 64);
        if (lane < 32) {
#pragma unroll
            for (int j = 0; j < NRED; ++j) red[hp][w][lane][j] = part[j];
        }
        __syncthreads();
        float tot[NRED];
#pragma unroll
        for (int j = 0; j < NRED; ++j)
            tot[j] = red[hp][0][cg][j] + red[hp][1][cg][j] + red[hp][2][cg][j] + red[hp][3][cg][j];

        float u[4], out[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u[j] = b[hp] * (vv[hp][j] - tot[j]);
            out[j] = tot[4 + j] + tot[8] * u[j];
        }
        if (rg == 0 && (!FRONT || a.o)) store4<Tin>(static_cast<Tin*>(a.o) + unit * D + 4 * cg, out);
        if (GATED) {
            float gz[4];
            load4<Tin>(static_cast<const Tin*>(a.gate) + unit * D + 4 * cg, gz);
            float ss = out[0] * out[0] + out[1] * out[1] + out[2] * out[2] + out[3] * out[3];
#pragma unroll
            for (int m = 16; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 32);
            const float r = rsqrtf(ss * (1.f / D) + a.eps);
            float yv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float w = a.weight ? a.weight[4 * cg + j] : 1.f;
                yv[j] = out[j] * r * w * __builtin_amdgcn_rcpf(1.f + __expf(-gz[j]));
            }
            if (rg == 0) store4<Tin>(static_cast<Tin*>(a.y) + unit * D + 4 * cg, yv);
        }

        float* S = a.S + unit * (int64_t)(D * D);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float kr = sk[hp][rg + 8 * i];
            f4 y = s[hp][i];
            y.x += kr * u[0]; y.y += kr * u[1]; y.z += kr * u[2]; y.w += kr * u[3];
            __builtin_nontemporal_store(y, reinterpret_cast<f4*>(S + (rg + 8 * i) * D + 4 * cg));
        }
    }
}

}  // namespace

namespace {
template <bool GATED, bool FRONT>
void launch_d128(const DecodeArgs& a, hipStream_t s, int64_t units) {
    const bool pair = (units % 2) == 0;
    const dim3 grid((unsigned)(pair ? units / 2 : units));
    const dim3 block(256);
    if (a.dtype == 0) {
        if (pair)
            hipLaunchKernelGGL((kda_decode_d128_kernel<bf16_t, 2, GATED, FRONT>), grid, block, 0,
                               s, a);
        else
            hipLaunchKernelGGL((kda_decode_d128_kernel<bf16_t, 1, GATED, FRONT>), grid, block, 0,
                               s, a);
    } else {
        if (pair)
            hipLaunchKernelGGL((kda_decode_d128_kernel<float, 2, GATED, FRONT>), grid, block, 0,
                               s, a);
        else
            hipLaunchKernelGGL((kda_decode_d128_kernel<float, 1, GATED, FRONT>), grid, block, 0,
                               s, a);
    }
}
}  // namespace

hipError_t launch_decode_d128(const DecodeArgs& a, hipStream_t s) {
    const int64_t units = a.N * a.H;
    if (units <= 0) return hipSuccess;
    if (a.xq) {
        if (!a.gate) return hipErrorInvalidValue;   // the input stage comes with the output stage
        launch_d128<true, true>(a, s, units);
    } else if (a.gate) {
        launch_d128<true, false>(a, s, units);
    } else {
        launch_d128<false, false>(a, s, units);
    }
    return hipGetLastError();
}

}  // namespace kda
