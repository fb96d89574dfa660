// Completion of a token-range split prefill: the entering state of every segment and the
// correction of its outputs.
//
// The recurrence S_t = (I - b k k^T) Diag(e^g) S_{t-1} + b k v^T ("Kimi K3's hybrid block, from
// first principles", section "From linear attention to the delta rule") is affine in the state,
// so any run of tokens maps its entering state S to M S + B.  A segment
// that starts from the unknown state S_in therefore has S_t = M_t S_in + B_t, where B_t is the run
// from a zero state with the segment's values and M_t the run from the identity with v = 0; its
// outputs are o_t = S_t^T q_t = B_t^T q_t + S_in^T (M_t^T q_t).  The prefill kernel leaves
// B_t^T q_t in o, M_t^T q_t in oM and the final B and M of every segment in seg_states; here
//   S_in(1) = final state of segment 0,   S_in(s + 1) = M_s S_in(s) + B_s,   hT = S_in(split),
// then o_t += S_in(s)^T (M_t^T q_t) for every token of segment s >= 1.  Both are matrix-core
// products whose float32 operands enter as hi + lo bf16 pairs (float32-accurate): one 128 x 128
// product per segment and head on the serial chain of the composition, and one 128 x 128 product
// per token of the later segments for the correction.
#include "kda_internal.h"
#include "kda_mfma.h"

namespace kda {
namespace {

using namespace mfma;

constexpr int D = 128;

// first token and length of sequence n in the packed token axis
__device__ __forceinline__ void seq_bounds(const PrefillArgs& a, int64_t n, int64_t& start,
                                           int64_t& len) {
    if (a.cu) {
        start = a.cu[n];
        len = a.cu[n + 1] - start;
    } else {
        start = n * a.T;
        len = a.T;
    }
}
// segments sequence n is cut into: seg_len tokens each, at most a.split, the last one running to
// the sequence end (an empty sequence keeps its segment 0, which passes h0 through)
__device__ __forceinline__ int64_t seq_segments(const PrefillArgs& a, int64_t len) {
    return len <= 0 ? 1 : min((len + a.seg_len - 1) / a.seg_len, a.split);
}

__device__ __forceinline__ float hi_of(uint32_t u, int half) {   // one bf16 of a pair, as float
    return __uint_as_float(half ? (u & 0xffff0000u) : (u << 16));
}
// eight float32 values as hi and lo bf16 operands
__device__ __forceinline__ void split8(const float x[8], bf16x8& hi, bf16x8& lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[i] = pk2(x[2 * i], x[2 * i + 1]);
        l[i] = pk2(x[2 * i] - hi_of(h[i], 0), x[2 * i + 1] - hi_of(h[i], 1));
    }
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    hi = __builtin_bit_cast(bf16x8, (u32x4){h[0], h[1], h[2], h[3]});
    lo = __builtin_bit_cast(bf16x8, (u32x4){l[0], l[1], l[2], l[3]});
}
// K = 32 operand slot j of lane group lg stands for index 16 (j / 4) + 4 lg + (j % 4)
__device__ __forceinline__ int kslot(int j, int lg) { return 16 * (j >> 2) + 4 * lg + (j & 3); }

// One workgroup per (16-column block, pair): the columns of the state evolve independently under
// the row maps M_s.  The block of the current entering state sits in LDS; wave w forms rows
// [32 w, 32 w + 32) of M_s S_in(s) + B_s as two 16 x 16 matrix-core blocks, with both float32
// operands split into hi + lo bf16 parts (hi hi + hi lo + lo hi: float32-accurate products).
// S_in(s) replaces B_s in seg_states once B_s has been read (each lane overwrites only the
// entries it read).
__global__ __launch_bounds__(256) void kda_split_compose_kernel(PrefillArgs a) {
    __shared__ float sc[D][16];            // the column block of the current entering state
    const int tid = threadIdx.x, lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const int w = tid >> 6;
    const int64_t c0 = 16 * (int64_t)blockIdx.x;
    const int64_t p = blockIdx.y, pairs = a.N * a.H;
    int64_t start, len;
    seq_bounds(a, p / a.H, start, len);
    const int64_t nseg = seq_segments(a, len);
    auto slot = [&](int64_t seg, int part) {
        return a.seg_states + ((2 * seg + part) * pairs + p) * (int64_t)(D * D);
    };
    for (int i = tid; i < D * 16; i += 256)
        sc[i >> 4][i & 15] = slot(0, 0)[(i >> 4) * D + c0 + (i & 15)];
    lds_barrier();
    // this wave's rows of M_s (A operands: row r0 + ln over the channels of step ks) and of B_s
    // (the accumulator's start), loaded one step ahead so that the chain waits only on LDS and
    // the matrix cores
    float4 mr[2][4][2];
    f32x4 br[2];
    auto load_step = [&](int64_t sg) {
        const float* ms = slot(sg, 1);
        const float* bs = slot(sg, 0);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int r0 = 32 * w + 16 * b;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const float* mrow = ms + (r0 + ln) * D + 32 * ks + 4 * lg;
                mr[b][ks][0] = *reinterpret_cast<const float4*>(mrow);
                mr[b][ks][1] = *reinterpret_cast<const float4*>(mrow + 16);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) br[b][r] = bs[(r0 + 4 * lg + r) * D + c0 + ln];
        }
    };
    if (nseg > 1) load_step(1);
    for (int64_t sg = 1; sg < nseg; ++sg) {
        float* bs = slot(sg, 0);
        // B operands: the entering state's block over channel steps ks (column ln)
        bf16x8 bh[4], bl[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            float x[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = sc[32 * ks + kslot(j, lg)][ln];
            split8(x, bh[ks], bl[ks]);
        }
        bf16x8 mh[2][4], ml[2][4];
        f32x4 acc[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            acc[b] = br[b];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const float4 m0 = mr[b][ks][0], m1 = mr[b][ks][1];
                const float x[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
                split8(x, mh[b][ks], ml[b][ks]);
            }
        }
        if (sg + 1 < nseg) load_step(sg + 1);
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                acc[b] = mma32(mh[b][ks], bh[ks], acc[b]);
                acc[b] = mma32(mh[b][ks], bl[ks], acc[b]);
                acc[b] = mma32(ml[b][ks], bh[ks], acc[b]);
            }
        // S_in(s) in B_s's place (the entries this lane read), then the new block into LDS
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 32 * w + 16 * b + 4 * lg + r;
                bs[row * D + c0 + ln] = sc[row][ln];
            }
        lds_barrier();
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r) sc[32 * w + 16 * b + 4 * lg + r][ln] = acc[b][r];
        lds_barrier();
    }
    if (a.hT) {
        float* dst = a.hT + p * (int64_t)(D * D);
        for (int i = tid; i < D * 16; i += 256)
            dst[(i >> 4) * D + c0 + (i & 15)] = sc[i >> 4][i & 15];
    }
}

// One wave per (64-token block of the later segments, pair); a block lies in one segment because
// seg_len is a multiple of 64.  The correction out^T = S_in^T (M_t^T q_t)^T is a matrix-core
// product per 16 x 16 block (column block of S_in, 16 tokens): S_in's float32 values enter as a
// hi + lo pair of bf16 operands (x = hi + lo to 2^-17 relative), M_t^T q_t as the bf16 values the
// prefill stored; the transposed form leaves each lane 4 consecutive columns of one token, added
// to the bf16 output B_t^T q_t already in o.
constexpr int TB = 64;
__global__ __launch_bounds__(256) void kda_split_fixup_kernel(PrefillArgs a) {
    const int lane = threadIdx.x & 63, ln = lane & 15, lg = lane >> 4;
    const int64_t p = blockIdx.y, H = a.H, n = p / H, h = p % H;
    int64_t start, len;
    seq_bounds(a, n, start, len);
    const bf16_t* om = static_cast<const bf16_t*>(a.oM);
    bf16_t* o = static_cast<bf16_t*>(a.o);
    // the sequence's 64-token blocks after segment 0, strided over the grid's waves
    const int64_t stride = (int64_t)gridDim.x * 4;
    for (int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);; blk += stride) {
        const int64_t trel = a.seg_len + blk * TB;                   // within the sequence
        if (trel >= len) break;                                      // the whole wave leaves
        const int nt = (int)min<int64_t>(TB, len - trel);
        const int64_t seg = min(trel / a.seg_len, a.split - 1);
        const float* S = a.seg_states + (2 * seg * a.N * H + p) * (int64_t)(D * D);   // S_in(seg)
        const int64_t t0 = start + trel;                             // packed token index
        // B operands: (M_t^T q_t)^T over channel steps ks, token ln of each 16-token sub-block tb
        bf16x8 bm[4][4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            const int tok = 16 * tb + ln;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                uint2 u0 = make_uint2(0u, 0u), u1 = make_uint2(0u, 0u);
                if (tok < nt) {
                    const bf16_t* row = om + ((t0 + tok) * H + h) * D + 32 * ks + 4 * lg;
                    u0 = *reinterpret_cast<const uint2*>(row);
                    u1 = *reinterpret_cast<const uint2*>(row + 16);
                }
                typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
                bm[tb][ks] = __builtin_bit_cast(bf16x8, (u32x4){u0.x, u0.y, u1.x, u1.y});
            }
        }
        // S_in^T rows (S_in columns 16 cb + ln) over the channels of step ks, for the A operands;
        // the next column block's values are loaded while the current one is multiplied
        float xs[4][8];
        auto load_s = [&](int cb) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    xs[ks][j] = S[(32 * ks + kslot(j, lg)) * D + 16 * cb + ln];
        };
        load_s(0);
        // this lane's 4 columns 16 cb + 4 lg .. + 3 of token 16 tb + ln (B_t^T q_t, bf16), for
        // every column block, all in flight from the start
        uint2 ob[D / 16][4];
#pragma unroll
        for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const int tok = 16 * tb + ln;
                ob[cb][tb] = tok < nt ? *reinterpret_cast<const uint2*>(
                                            o + ((t0 + tok) * H + h) * D + 16 * cb + 4 * lg)
                                      : make_uint2(0u, 0u);
            }
#pragma unroll
        for (int cb = 0; cb < D / 16; ++cb) {
            bf16x8 ah[4], al[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) split8(xs[ks], ah[ks], al[ks]);
            if (cb + 1 < D / 16) load_s(cb + 1);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    acc = mma32(ah[ks], bm[tb][ks], acc);
                    acc = mma32(al[ks], bm[tb][ks], acc);
                }
                // acc register r: column 16 cb + 4 lg + r of token 16 tb + ln
                const int tok = 16 * tb + ln;
                if (tok < nt) {
                    const uint2 u = ob[cb][tb];
                    *reinterpret_cast<uint2*>(o + ((t0 + tok) * H + h) * D + 16 * cb + 4 * lg) =
                        make_uint2(pk2(hi_of(u.x, 0) + acc[0], hi_of(u.x, 1) + acc[1]),
                                   pk2(hi_of(u.y, 0) + acc[2], hi_of(u.y, 1) + acc[3]));
                }
            }
        }

    }
}

}  // namespace

hipError_t launch_split_finish(const PrefillArgs& a, hipStream_t s) {
    const int64_t pairs = a.N * a.H;
    if (a.split <= 1 || pairs <= 0) return hipSuccess;
    hipLaunchKernelGGL(kda_split_compose_kernel, dim3(D / 16, (unsigned)pairs), dim3(256), 0, s,
                       a);
    // one wave per 64-token block after segment 0 of the longest sequence the plan assumed
    // (a.split segments), at most 256 workgroups per pair; blocks past them, if a sequence is
    // longer, are taken in the kernel's strided loop
    const int64_t later = (a.split - 1) * a.seg_len;
    const int64_t blocks = (later + TB - 1) / TB;
    const int64_t gx = min((blocks + 3) / 4, (int64_t)256);
    hipLaunchKernelGGL(kda_split_fixup_kernel, dim3((unsigned)gx, (unsigned)pairs), dim3(256), 0,
                       s, a);
    return hipGetLastError();
}

}  // namespace kda
