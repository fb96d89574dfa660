// Completion of a token-range split prefill: the entering state of every segment and the
// correction of its outputs.
//
// The recurrence S_t = (I - b k k^T) Diag(e^g) S_{t-1} + b k v^T is affine in the state ("Kimi
// K3's hybrid block, from first principles", section "From linear attention to the delta rule":
// a 16-token tile maps its entering state S to M S + B, and so does any run of tiles).  A segment
// that starts from the unknown state S_in therefore has S_t = M_t S_in + B_t, where B_t is the run
// from a zero state with the segment's values and M_t the run from the identity with v = 0; its
// outputs are o_t = S_t^T q_t = B_t^T q_t + S_in^T (M_t^T q_t).  The prefill kernel leaves B_t^T q_t
// in o, M_t^T q_t in oM and the final B and M of every segment in seg_states; here
//   S_in(1) = final state of segment 0,   S_in(s + 1) = M_s S_in(s) + B_s,   hT = S_in(split),
// then o_t += S_in(s)^T (M_t^T q_t) for every token of segment s >= 1.  Both steps run in float32
// on the vector ALUs (the products are small: 128 x 128 per segment and head, and 128 x 128 per
// token of the later segments).
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int D = 128;

// One workgroup per (16-column block, pair): the columns of the state evolve independently under
// the row maps M_s.  Thread (row r, columns c8 .. c8 + 7 of the block).  S_in(s) replaces B_s in
// seg_states once B_s has been used (each thread overwrites only the entries it read).
__global__ __launch_bounds__(256) void kda_split_compose_kernel(PrefillArgs a) {
    __shared__ float sc[D][16];            // the column block of the current entering state
    const int tid = threadIdx.x;
    const int r = tid >> 1, c8 = (tid & 1) * 8;
    const int64_t cbase = 16 * (int64_t)blockIdx.x + c8;
    const int64_t p = blockIdx.y, pairs = a.N * a.H;
    auto slot = [&](int64_t seg, int part) {
        return a.seg_states + ((2 * seg + part) * pairs + p) * (int64_t)(D * D);
    };
    {
        const float* src = slot(0, 0) + r * D + cbase;      // S_in(1)
#pragma unroll
        for (int c = 0; c < 8; ++c) sc[r][c8 + c] = src[c];
    }
    __syncthreads();
    for (int64_t sg = 1; sg < a.split; ++sg) {
        float* bs = slot(sg, 0) + r * D + cbase;            // B_s, row r
        const float* ms = slot(sg, 1) + r * D;              // M_s, row r
        float acc[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] = bs[c];
        for (int kk = 0; kk < D; kk += 4) {
            const float4 m4 = *reinterpret_cast<const float4*>(ms + kk);
            const float mv[4] = {m4.x, m4.y, m4.z, m4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[c] += mv[i] * sc[kk + i][c8 + c];
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) bs[c] = sc[r][c8 + c];  // S_in(s) in B_s's place
        __syncthreads();
#pragma unroll
        for (int c = 0; c < 8; ++c) sc[r][c8 + c] = acc[c];
        __syncthreads();
    }
    if (a.hT) {
        float* dst = a.hT + p * (int64_t)(D * D) + r * D + cbase;
#pragma unroll
        for (int c = 0; c < 8; ++c) dst[c] = sc[r][c8 + c];
    }
}

// One workgroup per (64-token block of the later segments, pair); a block lies in one segment
// because seg_len is a multiple of 64.  The block's M_t^T q_t rows are staged transposed in LDS as
// float32; thread (column j, 32 tokens) accumulates sum_c S_in[c][j] (M_t^T q_t)[c] and adds it to
// the bf16 output B_t^T q_t already in o.
constexpr int TB = 64;
__global__ __launch_bounds__(256) void kda_split_fixup_kernel(PrefillArgs a) {
    __shared__ float mt[D][TB];
    const int tid = threadIdx.x;
    const int64_t p = blockIdx.y, H = a.H, n = p / H, h = p % H;
    const int64_t trel = a.seg_len + (int64_t)blockIdx.x * TB;   // within the sequence
    if (trel >= a.T) return;
    const int nt = (int)min<int64_t>(TB, a.T - trel);
    const int64_t seg = trel / a.seg_len;
    const float* S = a.seg_states + (2 * seg * a.N * H + p) * (int64_t)(D * D);   // S_in(seg)
    const int64_t t0 = n * a.T + trel;                           // packed token index
    const bf16_t* om = static_cast<const bf16_t*>(a.oM);
    bf16_t* o = static_cast<bf16_t*>(a.o);
    for (int i = tid; i < TB * D; i += 256) {
        const int tk = i / D, c = i % D;
        mt[c][tk] = tk < nt ? bf16_to_f32(om[((t0 + tk) * H + h) * D + c]) : 0.f;
    }
    __syncthreads();
    const int j = tid & (D - 1), tq = (tid >> 7) * 32;
    float acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = 0.f;
    for (int c = 0; c < D; ++c) {
        const float sv = S[c * D + j];
#pragma unroll
        for (int i = 0; i < 32; i += 4) {
            const float4 m4 = *reinterpret_cast<const float4*>(&mt[c][tq + i]);
            acc[i] += sv * m4.x;
            acc[i + 1] += sv * m4.y;
            acc[i + 2] += sv * m4.z;
            acc[i + 3] += sv * m4.w;
        }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        const int tk = tq + i;
        if (tk < nt) {
            bf16_t* dst = o + ((t0 + tk) * H + h) * D + j;
            *dst = f32_to_bf16(bf16_to_f32(*dst) + acc[i]);
        }
    }
}

}  // namespace

hipError_t launch_split_finish(const PrefillArgs& a, hipStream_t s) {
    const int64_t pairs = a.N * a.H;
    if (a.split <= 1 || pairs <= 0 || a.T <= 0) return hipSuccess;
    hipLaunchKernelGGL(kda_split_compose_kernel, dim3(D / 16, (unsigned)pairs), dim3(256), 0, s,
                       a);
    const int64_t later = a.T - a.seg_len;
    if (later > 0)
        hipLaunchKernelGGL(kda_split_fixup_kernel, dim3((unsigned)((later + TB - 1) / TB),
                                                        (unsigned)pairs),
                           dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace kda
