// KDA chunkwise prefill on the CDNA4 matrix cores: bf16 inputs, dk = dv = 128, float32 state.
//
// Method ("Kimi K3's hybrid block, from first principles", section "From linear attention to the
// delta rule": the tokens of a chunk together, the state passed between chunks; the summed
// log-decay of a 16-token tile lies in (-80, 0), so the rescaling factors stay finite and every
// tile runs as dense matrix products).  Per 16-token tile with entering state S (dk x dv), write
//     Gp_i = Gam_i - Gam_C = -sum_{j>i} g_j >= 0        (log-decay to the tile end, per channel)
//     E = e^{Gp} >= 1,  D = e^{-Gp} <= 1,  eC = e^{Gam_C}  (per channel)
//     Kp = K.E,  Qp = Q.E,  Kd = K.D,  St = Diag(eC) S       (St: the state decayed to the tile end)
//     A = strict_lower(Kp Kd^T),  P = lower(Qp Kd^T)          (A_ij = sum_c k_ic k_jc e^{Gam_ic-Gam_jc})
//     T = (I + Diag(beta) A)^-1,  Tb = T Diag(beta)
//     W = Tb Kp,  Ut = Tb V,  Qpp = Qp - P W,  PUt = P Ut     (independent of the state)
//     U = Ut - W St,   O = Qpp St + PUt,   S <- St + Kd^T U   (the serial carry)
// which is the token loop S_t = (I - b k k^T) Diag(e^g) S_{t-1} + b k v^T, o_t = S_t^T q_t unrolled
// over the tile (the reference point of the cumulative decay sits at the tile end here, which
// only regroups per-channel factors).  T is the unit-lower-triangular inverse, evaluated exactly
// as the finite product (I - N)(I + N^2)(I + N^4)(I + N^8) with N = Diag(beta) A (N^16 = 0).
//
// Mapping to gfx950.  One workgroup of 12 waves owns one (sequence, head, 64-column slice of dv);
// when the (sequence, head) pairs alone fill the chip, one workgroup owns a whole head (a
// 128-column slice: each stage-S wave carries two strips, and stages A and B1 run once per head).
// The two slices of a head are dispatched to the same XCD so their shared q/k/g reads meet in
// that XCD's L2, and in a variable-length batch (up to 65,536 sequences) the longest sequences
// are dispatched first (the short ones fill the tail).  With a token-range split (small batches;
// the completion kernels are in kda_prefill_split.hip) a workgroup runs one segment of a sequence:
// segment 0 from h0, or a later segment from a zero state (its part B) or from the identity with
// v = 0 (its part M), and leaves the segment's final state for the composition.  Each wave keeps
// one role for the whole sequence, and the work of a tile runs as a software pipeline with a
// single workgroup barrier per period; period q holds
//   stage A (waves 4-7) for tile q: wave s loads key channels [32s, 32s+32) of q, k, g (eight
//      consecutive channels per lane, one 16-byte load per tensor) and value columns of the slice
//      through buffer resources (wave 0 also beta), runs the cumulative log-decay as a product
//      with a triangular 0/1 matrix, and forms the decayed operands Kp, Qp, Kd (the exponentials
//      are the only transcendental work);
//   stage B1 (waves 8-11) for tiles q-1 and q-2: A, A^T, P^T over all 128 channels and T, split
//      into two halves that run in consecutive periods; waves 8-9 take even tiles and waves
//      10-11 odd ones, so each SIMD carries half an inverse per period;
//   stage B2 (waves 8-11, beside B1) for tile q-3: W and Qpp for key channels [32s, 32s+32), Ut
//      and PUt for columns [16s, 16s+16), and the channel-major Kd blocks the carry consumes
//      (its inputs from stage A are read at the end of the period before);
//   stage S (waves 0-3) for tile q-4: wave s carries its 128 x 16 strip of S (two strips in the
//      128-column slice), which lives in registers as eight 16x16 float32 accumulator blocks per
//      strip for the whole sequence, and writes o.
// (The wave numbers are those of the 64-column kernel.  The plain 128-column kernel rotates the
// roles by one group of four: stage A on waves 0-3, B on 4-7, S on 8-11.  Both 128-column
// kernels run B1 on one wave of each pair only, and in the one with the output stage the
// stage-B waves also carry the gate.)
// Three waves share each SIMD.  Loads run two tiles ahead of their use.  All products use
// v_mfma_f32_16x16x{16,32}_bf16.  Token-major -> channel-major changes of layout are LDS transpose
// reads where the data already sits in LDS, and a product with a 0/1 selector matrix on the
// matrix cores for g (both exact for bf16 data).  The output and P Ut are formed as transposed
// products (operands swapped), which leaves them token-major as o is stored.
//
// Fragment conventions for a 16x16 block, lane l = ln + 16 lg (ln = l % 16, lg = l / 16):
//   accumulator  acc(X): register r holds X[4 lg + r][ln]
//   A operand of Z = X Y is acc(X^T) (as bf16); B operand is acc(Y).
// For the K = 32 products over key channels, slot j of lane group lg stands for channel 8 lg + j of
// the 32-channel group, as stage A loads it; A and B operands always use this order.  Split into
// 16-channel halves hh = j / 4 (the 16x16 blocks of the transposes, the scan and the state's rows),
// internal channel (hh, 4 lg + r) is key channel 8 lg + 4 hh + r of the group.
#include "kda_internal.h"
#include "kda_mfma.h"

#include <type_traits>

namespace kda {
namespace {

using namespace mfma;

constexpr int C = 16;      // tile tokens
constexpr int D = 128;     // dk = dv
constexpr int NT = 768;    // threads per workgroup (12 waves: 4 per stage)
constexpr int kLptMaxSeqs = 65536;   // varlen batches up to this many sequences run longest first

// (workgroup index) -> (pair index p = n * H + head, slice) with both slices of a pair on one XCD
// (workgroups are dealt to the 8 XCDs round-robin by index); one slice per pair: p = b.
__device__ __forceinline__ void map_workgroup(int64_t b, int64_t pairs, int nslice, int64_t& p,
                                              int& slice) {
    if (nslice == 1) {
        p = b;
        slice = 0;
        return;
    }
    const int64_t full = (pairs / 8) * 16;
    if (b < full) {
        const int64_t xcd = b % 8, j = b / 8;
        slice = (int)(j % 2);
        p = (j / 2) * 8 + xcd;
    } else {
        const int64_t t = b - full;
        slice = (int)(t % 2);
        p = (pairs / 8) * 8 + t / 2;
    }
}

// The sequence of rank r (0 <= r < N <= 65536) in the order of decreasing length, ties by
// increasing index, for the whole workgroup: a radix select over the unique 48-bit keys
// (length << 16) | (0xFFFF - index), eight bits per pass from the highest digit in which the keys
// differ; batches whose lengths lie within a sixteenth of the shortest keep index order.  Each
// pass counts the keys that still match the digits chosen so far into 256 bins (LDS), and one
// wave picks the bin that holds the rank.  scratch: 264 + NT / 16 words of LDS, free until the
// barrier at the end.
constexpr int kSelectHeld = 4;     // keys a thread keeps in registers (N <= 4 NT: one load)
__device__ __forceinline__ uint64_t length_key(const int32_t* cu, int i) {
    return ((uint64_t)(uint32_t)(cu[i + 1] - cu[i]) << 16) | (uint64_t)(0xFFFF - i);
}
__device__ int select_by_length(const int32_t* cu, int N, int r, int tid, uint32_t* scratch) {
    uint32_t* hist = scratch;
    uint32_t* sel = scratch + 256;    // the chosen bin, and the keys counted above it
    uint64_t prefix = 0, mask = 0;
    uint32_t rem = (uint32_t)r;       // the rank among the keys that match the prefix
    const bool held = N <= kSelectHeld * NT;
    uint64_t kh[kSelectHeld];
    uint64_t kmin = ~uint64_t{0}, kmax = 0;
#pragma unroll
    for (int c = 0; c < kSelectHeld; ++c) {
        const int i = tid + c * NT;
        kh[c] = (held && i < N) ? length_key(cu, i) : 0;
        if (held && i < N) {
            kmin = min(kmin, kh[c]);
            kmax = max(kmax, kh[c]);
        }
    }
    if (!held) {
        for (int i = tid; i < N; i += NT) {
            const uint64_t key = length_key(cu, i);
            kmin = min(kmin, key);
            kmax = max(kmax, key);
        }
    }
    // the digits above the highest one in which the smallest and largest keys differ are common
    // to all keys: the passes start there (equal lengths leave only the index digits, which
    // spread over the bins instead of piling onto one)
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        kmin = min(kmin, (uint64_t)__shfl_xor((unsigned long long)kmin, d));
        kmax = max(kmax, (uint64_t)__shfl_xor((unsigned long long)kmax, d));
    }
    uint64_t* wmm = reinterpret_cast<uint64_t*>(scratch + 264);   // [NT / 64][2]
    if ((tid & 63) == 0) {
        wmm[2 * (tid >> 6)] = kmin;
        wmm[2 * (tid >> 6) + 1] = kmax;
    }
    __syncthreads();
    for (int w = 0; w < NT / 64; ++w) {
        kmin = min(kmin, wmm[2 * w]);
        kmax = max(kmax, wmm[2 * w + 1]);
    }
    // lengths within a sixteenth of the shortest: little to gain from reordering, so the batch
    // keeps index order (the order the ranks already are in when all lengths are equal)
    const uint64_t lmin = kmin >> 16, lmax = kmax >> 16;
    if (lmax - lmin <= lmin / 16) {
        __syncthreads();   // every thread has read wmm before the scratch is reused
        return r;
    }
    const uint64_t diff = kmin ^ kmax;    // nonzero: N >= 2 distinct keys
    const int top = (63 - __builtin_clzll(diff)) & ~7;
    mask = ~((uint64_t{1} << (top + 8)) - 1);
    prefix = kmax & mask;
    for (int shift = top; shift >= 0; shift -= 8) {
        for (int b = tid; b < 256; b += NT) hist[b] = 0u;
        __syncthreads();
        if (held) {
#pragma unroll
            for (int c = 0; c < kSelectHeld; ++c)
                if (tid + c * NT < N && (kh[c] & mask) == prefix)
                    atomicAdd(&hist[(kh[c] >> shift) & 255u], 1u);
        } else {
            for (int i = tid; i < N; i += NT) {
                const uint64_t key = length_key(cu, i);
                if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
            }
        }
        __syncthreads();
        if (tid < 64) {
            // lane j holds bins 255 - 4 j .. 252 - 4 j (the largest digits first)
            uint32_t c[4], tot = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                c[e] = hist[255 - 4 * tid - e];
                tot += c[e];
            }
            uint32_t incl = tot;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const uint32_t u = __shfl_up(incl, d);
                if (tid >= d) incl += u;
            }
            const uint32_t excl = incl - tot;
            if (excl <= rem && rem < incl) {   // exactly one lane
                uint32_t before = excl;
                int bin = 255 - 4 * tid;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (rem < before + c[e]) {
                        bin = 255 - 4 * tid - e;
                        break;
                    }
                    before += c[e];
                }
                sel[0] = (uint32_t)bin;
                sel[1] = before;
            }
        }
        __syncthreads();
        prefix |= (uint64_t)sel[0] << shift;
        mask |= (uint64_t)0xFF << shift;
        rem -= sel[1];
    }
    __syncthreads();   // every thread has read sel before the scratch is reused
    return 0xFFFF - (int)(prefix & 0xFFFFu);
}

// Raw inputs of one tile for one stage-A lane: token ln, key channels 32s + 8lg .. 32s + 8lg + 7
// (one 16-byte load per tensor), value columns 32s + 8lg .. + 7 with the output stage (16 bytes,
// as v[0], v[1]) or 64m + 16s + 4lg .. + 3 (8 bytes each, v[m]), and on stage-A wave 0 beta of
// token ln.  They are read through buffer resources whose record count ends at the sequence's
// last token, so a token past the end (and every token of a tile past the end) reads as zero:
// with beta = 0 and k = v = 0 it neither writes the state nor reaches a stored output, and with
// g = 0 it does not decay the state.
struct Raw {
    uint4 q, k, g;
    uint2 v[2];
    uint32_t b;   // raw bf16 bits of beta in the low half
};

// Stage-to-stage buffers, grouped by hand-off so that one dynamic base address reaches every
// member of a group.  NS = slice width / 64 strips of 16 columns per stage-S wave; with two, P Ut
// travels as bf16 so that LDS still holds the pipeline (it is added to o, which is bf16 anyway).
template <int NS> struct PutOf { typedef f32x4 T; };
template <> struct PutOf<2> { typedef uint2 T; };
template <int NS>
struct FromA {                 // stage A -> stages B1 and B2 (indexed by tile % 4)
    bf16x8 kp[4][64];          // token-major Kp per 32-channel k-step (operand fragments)
    bf16x8 kd[4][64];          // token-major Kd
    bf16x8 qp[4][64];          // token-major Qp
    f32x4 qpf[8][64];          // Qp in float32 as acc(Qp^T) per 16-channel block (C input)
    uint2 vraw[4 * NS][64];    // token-major V per 16-column strip (A operand of the transpose)
    float beta[C];
};
struct FromB1 {                // stage B1 -> stage B2 (indexed by tile % 2)
    uint2 tbt[64];             // acc((T Diag(beta))^T) as bf16
    uint2 y3[64];              // acc((P T Diag(beta))^T) as bf16
};
template <int NS>
struct FromB {                 // stage B2 -> stage S (indexed by tile % 2)
    uint4 kdc[4][64];          // channel-major Kd, blocks 2j (.xy) and 2j + 1 (.zw)
    bf16x8 w[4][64];           // A operands of W per 32-channel k-step
    bf16x8 qpp[4][64];         // A operands of Qpp per 32-channel k-step
    f32x4 ut[4 * NS][64];      // Ut per strip (accumulator fragments)
    typename PutOf<NS>::T put[4 * NS][64];   // (P Ut)^T per strip (token-major like o)
};
template <int NS>
struct Shared {
    FromA<NS> a[4];
    FromB<NS> b[2];
    FromB1 b1[2];
    float ec[8][D];            // e^{Gam_C} (stage A -> stage S, tile % 8)
};

// The fused output stage (GATED, one workgroup per head).  y = o / sqrt(mean(o^2) + eps) * w *
// sigmoid(gate) per (token, head) row ("Kimi K3's hybrid block, from first principles", section
// "From linear attention to the delta rule": each head's output row is normalised by its root
// mean square and, ahead of the output projection, scaled by a sigmoid gate computed from the
// token).  Stage-B wave s loads the gate of tile j in period j + 2 and, in period j + 4, leaves
// w * sigmoid(gate) (bf16) for stage-S wave s, lane by lane, at the columns of o that lane holds.
// The row's sum of squares spans the four stage-S waves: in the period that forms tile j's o
// (period j + 4) each adds its 32 columns and leaves the sum in ssq; in the next period, after the
// barrier that orders those writes, each reads the four sums and finishes tile j's y from the o
// it kept in registers.  No wave waits for another outside the pipeline's own barrier.  (Stage A
// carrying the gate instead measured 1.7-3.3% slower: it paces the period when most CUs are
// busy.)
struct GateLds {
    uint4 gw[2][4][64];     // by tile % 2, stage-S wave, lane: bf16 w * sigmoid(gate) of token ln,
                            // columns 16 s + 4 lg + r (.xy) and 64 + 16 s + 4 lg + r (.zw)
    float ssq[2][C][4];     // by tile % 2, token of the tile: the stage-S waves' sums of o^2
    float w[D];             // the gain per column (ones without one)
};

// PRIO_ROLE: the role whose waves win issue ties on their SIMD (1: stage A, 2: stage B).
template <int PRIO_ROLE, int BVT, bool GATED>
__global__ __launch_bounds__(NT) void kda_prefill_mfma_kernel(PrefillArgs a) {
    constexpr int NS = BVT / 64;       // 16-column strips per stage-S wave
    static_assert(!GATED || NS == 2, "the fused output stage needs a whole head per workgroup");
    __shared__ Shared<NS> sh;
    __shared__ typename std::conditional<GATED, GateLds, char>::type gsh;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
    const int lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    // 0: stage S, 1: stage A, 2: stage B.  Wave slots 0-3 hold stage S, except in the plain
    // 128-column kernel, where they hold stage A and stage S takes slots 8-11.  The same code
    // in a different wave order measured: 64 columns at H = 96, 1% faster with S first; plain
    // 128 columns on the 16-sequence batch, 2.5% faster with A first (neutral at 4 x 4096
    // tokens); 128 columns with the output stage, 0.4% faster with S first.
    constexpr int kRoleShift = (BVT == 128 && !GATED) ? 1 : 0;
    const int role = ((wave >> 2) + kRoleShift) % 3;
    const int s = wave & 3;            // channel group / strip index of this wave
    const int64_t H = a.H;

    int64_t p;
    int slice;
    // with a token-range split, unit u of pair p is segment 0 (u = 0), the part B of segment u
    // (0 < u < split) or the part M of segment u - split + 1; units of one pair share nothing
    const int64_t units = a.split > 1 ? 2 * a.split - 1 : 1;
    map_workgroup(blockIdx.x, a.N * H * units, D / BVT, p, slice);
    const int64_t unit = p / (a.N * H);
    p %= a.N * H;
    const int seg = (int)(unit < a.split ? unit : unit - a.split + 1);
    const bool part_m = unit >= a.split;   // the transition part: v = 0, identity entering state
    const int64_t h = p % H;
    int64_t n = p / H;
    if (a.cu && a.N > 1 && a.N <= kLptMaxSeqs) {
        // longest first: pair index p / H is a rank in the order of decreasing length (ties by
        // index), so the longest sequences are dispatched first and the short ones fill the tail
        // (the pipeline's LDS serves as scratch; its first use comes after the barrier inside)
        // (the same in every lane: readfirstlane keeps what derives from it in scalar registers)
        n = __builtin_amdgcn_readfirstlane(
            select_by_length(a.cu, (int)a.N, (int)n, tid, reinterpret_cast<uint32_t*>(&sh)));
        p = n * H + h;                                   // the state's (sequence, head) index
    }
    int64_t bos, eos;
    if (a.cu) { bos = a.cu[n]; eos = a.cu[n + 1]; }
    else { bos = n * a.T; eos = bos + a.T; }
    if (a.split > 1) {
        // the segment's tokens: seg_len from its start (a multiple of 64), the last segment up to
        // the sequence end; segments past the end of a shorter sequence are empty
        const int64_t send = eos;
        bos = min(bos + seg * a.seg_len, send);
        if (seg + 1 < a.split) eos = min(send, bos + a.seg_len);
    }
    const int64_t ntiles = (eos - bos + C - 1) / C;

    const bf16_t* __restrict__ q = static_cast<const bf16_t*>(a.q);
    const bf16_t* __restrict__ k = static_cast<const bf16_t*>(a.k);
    const bf16_t* __restrict__ v = static_cast<const bf16_t*>(a.v);
    const bf16_t* __restrict__ g = static_cast<const bf16_t*>(a.g);
    const bf16_t* __restrict__ beta = static_cast<const bf16_t*>(a.beta);
    bf16_t* __restrict__ o = static_cast<bf16_t*>(part_m ? a.oM : a.o);
    const bf16_t* __restrict__ gate = static_cast<const bf16_t*>(a.gate);
    bf16_t* __restrict__ y = static_cast<bf16_t*>(a.y);
    if constexpr (GATED) {
        // read before the first barrier of every role; the first use comes three periods later
        if (tid < D) gsh.w[tid] = a.weight ? a.weight[tid] : 1.f;
    }

    // ---- constant fragments ----
    // selector (B, K = 32): column n of g's product with it is internal channel (hh, n), element
    // 8 (n / 4) + 4 hh + n % 4 of the wave's 32 channels; the product is the channel-major
    // transpose of that half
    bf16x8 sel[2];
    for (int hh = 0; hh < 2; ++hh)
        for (int j = 0; j < 8; ++j)
            sel[hh][j] = (__bf16)((lg == (ln >> 2) && j == 4 * hh + (ln & 3)) ? 1.f : 0.f);
    // M^T scaled by log2(e) as a two-term bf16 split (hi + lo = log2(e) to 5e-6 relative), with
    // M[i][j] = -1 for j > i: row i of M g gives -log2(e) sum_{j>i} g_j, the exponent in base 2
    bf16x4 scanHi, scanLo;
    for (int j = 0; j < 4; ++j) {
        const bool up = 4 * lg + j > ln;
        scanHi[j] = (__bf16)(up ? -L2E_HI : 0.f);
        scanLo[j] = (__bf16)(up ? -L2E_LO : 0.f);
    }
    const bf16x8 scanHL = cat8(scanHi, scanLo);   // both terms in one K = 32 product
    bf16x4 onesA;    // all ones (A operand): column c of the product is Gam_C of channel c
    for (int j = 0; j < 4; ++j) onesA[j] = (__bf16)1.f;

    // ---- stage S state: strip m holds column col + 64 m of this workgroup's slice, in the rows
    //      of the pipeline's internal key-channel order: register r of block mb in lane group lg
    //      is internal row 16 mb + 4 lg + r, key channel real_row(mb, r).  Stage A loads eight
    //      consecutive channels per lane, and its fragments keep them in place, so the order that
    //      every stage shares is this one; only the state's entry and exit translate it. ----
    const int64_t col = (int64_t)slice * BVT + 16 * s + ln;
    auto real_row = [&](int mb, int r) { return 32 * (mb >> 1) + 8 * lg + 4 * (mb & 1) + r; };
    const int64_t sbase = p * (int64_t)(D * D);
    // (declared here, set and used by the stage-S waves only, so that it occupies registers in
    // their branch alone)
    f32x4 S[NS][8];
    // the state strips to or from a [dk, dv] float32 matrix (src == nullptr: zeros, or the
    // identity for the transition part of a split segment)
    auto state_in = [&](const float* src, bool ident) {
#pragma unroll
        for (int m = 0; m < NS; ++m)
#pragma unroll
            for (int mb = 0; mb < 8; ++mb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    S[m][mb][r] = src ? src[(int64_t)real_row(mb, r) * D + col + 64 * m] : 0.f;
        if (ident) {
            // the diagonal entry of column cc = col + 64 m is key channel cc: blocks with
            // mb / 2 = cc / 32 (the same for the whole wave), then mb % 2 = (cc / 4) % 2, lane
            // group (cc / 8) % 4 and register cc % 4
#pragma unroll
            for (int m = 0; m < NS; ++m) {
                const int cc = (int)(col + 64 * m);
                const int hi = (int)((col - ln + 64 * m) >> 5);
#pragma unroll
                for (int mb = 0; mb < 8; ++mb)
                    if ((mb >> 1) == hi) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if ((mb & 1) == ((cc >> 2) & 1) && lg == ((cc >> 3) & 3) &&
                                r == (cc & 3))
                                S[m][mb][r] = 1.f;
                    }
            }
        }
    };
    auto state_out = [&](float* dst) {
#pragma unroll
        for (int m = 0; m < NS; ++m)
#pragma unroll
            for (int mb = 0; mb < 8; ++mb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dst[(int64_t)real_row(mb, r) * D + col + 64 * m] = S[m][mb][r];
    };
    // entering state and final-state destination of this run: with a split, segment 0 starts
    // from h0, later segments from zero (part B) or the identity (part M), and every final state
    // goes to the segment-state buffer [split, 2, N * H, dk, dv]
    const float* h_in = a.h0 ? a.h0 + sbase : nullptr;
    float* h_out = a.hT ? a.hT + sbase : nullptr;
    if (a.split > 1) {
        if (seg > 0) h_in = nullptr;
        h_out = a.seg_states + ((2 * seg + (part_m ? 1 : 0)) * a.N * H + p) * (int64_t)(D * D);
    }
    if (ntiles == 0) {
        if (role == 0 && h_out) {
            state_in(h_in, part_m);
            state_out(h_out);
        }
        return;
    }

    // ---- stage A: loads.  Tile j of the sequence starts at token bos + 16 j; its buffer
    //      resources start at that token's head row (scalar base) and end after the last token
    //      of the sequence that the tile holds; lanes add a fixed byte offset ----
    const int64_t chan0 = 32 * s + 8 * lg;
    const int64_t vcol0 = (int64_t)slice * BVT + 16 * s + 4 * lg;
    const int64_t len = eos - bos;
    const int64_t row_bytes = H * D * 2;                       // one token, all heads
    const uint32_t vo_qkg = (uint32_t)(ln * row_bytes + chan0 * 2);
    // v: with the output stage (128 columns), 16 bytes per lane (columns 32 s + 8 lg .. + 7),
    // which stage A scatters to the stage-S strips in LDS; otherwise 8 bytes per lane (columns
    // 16 s + 4 lg .. + 3 of each strip, the lane's own strip entries).  Against 8-byte loads
    // (outputs bit-identical), the 16-byte form was 3.4-5.6% faster with the output stage on the
    // 16-sequence batch, within +-0.6% without it, and 6-10% slower with 64 columns, where only
    // two stage-A waves would carry v.
    constexpr bool kV16 = GATED;
    const uint32_t vo_v = kV16 ? (uint32_t)(ln * row_bytes + (32 * s + 8 * lg) * 2)
                               : (uint32_t)(ln * row_bytes + vcol0 * 2);
    const uint32_t vo_b = (uint32_t)(ln * H * 2);
    int ld_tile = 0;                                           // next tile to load (uniform)
    const int len32 = (int)len;                                // token counts fit int32 (ABI)
    const int rb32 = (int)row_bytes, hb32 = (int)(H * 2);
    auto load_tile = [&](Raw& R) {
        const int64_t t0 = bos + (int64_t)ld_tile * C;
        // tokens of the sequence held by this tile, 0..16; the record counts end after the last
        // of them (row_bytes >= 256 and H >= 1 make both counts 0 for an empty tile)
        const int nv = min(max(len32 - ld_tile * C, 0), C);
        const int nrec = max((nv - 1) * rb32 + D * 2, 0);
        const int nrec_b = max((nv - 1) * hb32 + 2, 0);
        const int64_t e0 = (t0 * H + h) * D;                   // element offset of the head row
        const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(q + e0), (short)0, nrec, kBufferFlags);
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(k + e0), (short)0, nrec, kBufferFlags);
        const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(g + e0), (short)0, nrec, kBufferFlags);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(v + e0), (short)0, part_m ? 0 : nrec, kBufferFlags);   // part M: v = 0
        const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(beta + (t0 * H + h)), (short)0, nrec_b, kBufferFlags);
        R.q = ld16(rq, vo_qkg);
        R.k = ld16(rk, vo_qkg);
        R.g = ld16(rg, vo_qkg);
        if constexpr (kV16) {
            const uint4 t = ld16(rv, vo_v);
            R.v[0] = make_uint2(t.x, t.y);
            R.v[1] = make_uint2(t.z, t.w);
        } else {
#pragma unroll
            for (int m = 0; m < NS; ++m) R.v[m] = ld8(rv, vo_v + 128 * m);
        }
        // beta: stage-A wave 0 alone (the tile's 16 values reach every stage through LDS)
        if (s == 0) R.b = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rb, vo_b, 0, 0);
        ++ld_tile;
    };

    // Buffer indices of a tile: FromA by tile % 4, FromB and FromB1 by tile % 2, ec by tile % 8.
    auto fa = [&](int64_t tile) -> FromA<NS>& { return sh.a[(uint32_t)tile & 3u]; };
    auto fb = [&](int64_t tile) -> FromB<NS>& { return sh.b[(uint32_t)tile & 1u]; };
    auto fb1 = [&](int64_t tile) -> FromB1& { return sh.b1[(uint32_t)tile & 1u]; };
    auto ecb = [&](int64_t tile) -> float* { return sh.ec[(uint32_t)tile & 7u]; };

    // stage A for tile `tile`
    auto stage_a = [&](int64_t tile, const Raw& R) {
        FromA<NS>& A = fa(tile);
        float* ec = ecb(tile);
        // internal channel (hh, 4 lg + r) of this lane is key channel 32 s + 8 lg + 4 hh + r, which
        // half hh of its 16-byte loads holds; the selector below picks g's channels in that order
        const bf16x8 ga = __builtin_bit_cast(bf16x8, R.g);
        const f32x4 kf[2] = {unpack4(make_uint2(R.k.x, R.k.y)), unpack4(make_uint2(R.k.z, R.k.w))};
        const f32x4 qf[2] = {unpack4(make_uint2(R.q.x, R.q.y)), unpack4(make_uint2(R.q.z, R.q.w))};
        f32x4 X[2];    // log2(e) * Gp, token-major
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const bf16x4 gc = bf4(mma32(ga, sel[hh], zero4()));   // channel-major g (exact)
            X[hh] = mma32(cat8(gc, gc), scanHL, zero4());
            // Gam_C of internal channel (hh, ln), in every register and lane group, stored at its
            // internal row 32s + 16hh + ln; all four lane groups store the same value
            const f32x4 gsum = mma16(onesA, gc, zero4());
            ec[32 * s + 16 * hh + ln] = __builtin_amdgcn_exp2f(gsum[0] * LOG2E);
        }
        bf16x4 Kpb[2], Qpb[2], Kdb[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            f32x4 kp, kd, qp;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float e = __builtin_amdgcn_exp2f(X[hh][r]);
                const float dd = __builtin_amdgcn_exp2f(-X[hh][r]);
                kp[r] = kf[hh][r] * e;
                qp[r] = qf[hh][r] * e;
                kd[r] = kf[hh][r] * dd;
            }
            Kpb[hh] = bf4(kp);
            Qpb[hh] = bf4(qp);
            Kdb[hh] = bf4(kd);
            A.qpf[2 * s + hh][lane] = qp;
        }
        if (s == 0) A.beta[ln] = __uint_as_float(R.b << 16);   // every lane group writes the same
        A.kp[s][lane] = cat8(Kpb[0], Kpb[1]);
        A.qp[s][lane] = cat8(Qpb[0], Qpb[1]);
        A.kd[s][lane] = cat8(Kdb[0], Kdb[1]);
        if constexpr (kV16) {
            // columns c .. c + 3 of token ln go to strip (c % 64) / 16 + 4 (c / 64), at the lane
            // of the stage-S layout that holds them, ln + 16 ((c % 16) / 4)
            const int c0 = 32 * s + 8 * lg;
            uint2* dst = A.vraw[((c0 & 63) >> 4) + 4 * (c0 >> 6)];
            const int l0 = ln + 16 * ((c0 & 15) >> 2);
            dst[l0] = R.v[0];
            dst[l0 + 16] = R.v[1];
        } else {
#pragma unroll
            for (int m = 0; m < NS; ++m) A.vraw[s + 4 * m][lane] = R.v[m];
        }
    };

    // fused output stage, stage B's part.  In period t + 2 stage-B wave s loads the gate of tile
    // t, 16 bytes per lane: token ln, columns 32 s + 8 lg .. + 7 (zeros past the sequence end).
    // In period t + 4 it leaves w * sigmoid(gate) for those columns in the buffer of tile t % 2,
    // at the lanes of the stage-S waves that hold them (columns c .. c + 3 of token ln go to wave
    // (c % 64) / 16, lane ln + 16 ((c % 16) / 4), half c / 64).  Measured against 8-byte loads of
    // each stage-S wave's own columns (two per wave and tile, 32 bytes of a token row per load):
    // 3.5% faster on the 16-sequence batch and 5.8% at 4 x 4096 tokens, bit-identical outputs.
    struct GateRaw { uint4 z; };
    const uint32_t vo_gz =
        (uint32_t)(ln * row_bytes + ((int64_t)slice * BVT + 32 * s + 8 * lg) * 2);
    auto gate_load = [&](int64_t tile, GateRaw& G) {
        const int nvg = min(max(len32 - (int)tile * C, 0), C);
        const int nrecg = max((nvg - 1) * rb32 + D * 2, 0);
        const int64_t tg0 = bos + min(tile * C, len);
        const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(gate + (tg0 * H + h) * D), (short)0, nrecg, kBufferFlags);
        G.z = ld16(rz, vo_gz);
    };
    auto gate_step = [&](int64_t tile, const GateRaw& G) {
        if constexpr (GATED) {
            const int c0 = 32 * s + 8 * lg;
            const f32x4 z[2] = {unpack4(make_uint2(G.z.x, G.z.y)),
                                unpack4(make_uint2(G.z.z, G.z.w))};
            const int sd = (c0 & 63) >> 4, lgd = (c0 & 15) >> 2, half = c0 >> 6;
            uint4* dst = gsh.gw[(uint32_t)tile & 1u][sd];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const f32x4 w = *reinterpret_cast<const f32x4*>(&gsh.w[c0 + 4 * u]);
                f32x4 gw;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    gw[r] = w[r] * __builtin_amdgcn_rcpf(1.f + __expf(-z[u][r]));
                reinterpret_cast<uint2*>(&dst[ln + 16 * (lgd + u)])[half] =
                    make_uint2(pk2(gw[0], gw[1]), pk2(gw[2], gw[3]));
            }
        }
    };

    // stage B1 for tile `tile`: A, A^T, P^T over all 128 channels and the inverse T, in two
    // halves that run in consecutive periods (the registers in B1Carry cross the barrier).  Waves
    // 8 and 9 take the even tiles and waves 10 and 11 the odd ones.  In the 64-column kernel both
    // waves of a pair compute it (identical results), so every SIMD runs one half per period; the
    // 128-column kernels run it on the first wave of each pair only.
    struct B1Carry { f32x4 N4, N4t, Gt, Pt, brow; float bcol; };
    auto stage_b1a = [&](int64_t tile) -> B1Carry {
        const FromA<NS>& A = fa(tile);
        f32x4 Am = zero4(), At = zero4(), Pt = zero4();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 kp8 = A.kp[ks][lane], kd8 = A.kd[ks][lane], qp8 = A.qp[ks][lane];
            Am = mma32(kp8, kd8, Am);    // A  = Kp Kd^T
            At = mma32(kd8, kp8, At);    // A^T
            Pt = mma32(kd8, qp8, Pt);    // P^T = Kd Qp^T
        }
        B1Carry c;
        c.bcol = A.beta[ln];
        c.brow = *reinterpret_cast<const f32x4*>(&A.beta[4 * lg]);
        f32x4 N, Nt, F1t;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 4 * lg + r;
            N[r] = (ln < i) ? c.brow[r] * Am[r] : 0.f;    // N[i][ln]
            Nt[r] = (i < ln) ? c.bcol * At[r] : 0.f;      // N^T[i][ln]
            c.Pt[r] = (i <= ln) ? Pt[r] : 0.f;            // P^T[i][ln]
            F1t[r] = ((i == ln) ? 1.f : 0.f) - Nt[r];     // (I - N)^T
        }
        // T = (I - N)(I + N^2)(I + N^4)(I + N^8); only the transposes that are consumed as A
        // operands are formed; the identity of each factor enters as the product's C input
        const bf16x4 Nb = bf4(N), Ntb = bf4(Nt);
        const f32x4 N2 = mma16(Ntb, Nb, zero4()), N2t = mma16(Nb, Ntb, zero4());
        const bf16x4 N2b = bf4(N2), N2tb = bf4(N2t);
        c.N4 = mma16(N2tb, N2b, zero4());
        c.N4t = mma16(N2b, N2tb, zero4());
        c.Gt = mma16(N2b, bf4(F1t), F1t);             // ((I - N)(I + N^2))^T
        return c;
    };
    auto stage_b1b = [&](int64_t tile, const B1Carry& c) {
        FromB1& B = fb1(tile);
        f32x4 id;
#pragma unroll
        for (int r = 0; r < 4; ++r) id[r] = (4 * lg + r == ln) ? 1.f : 0.f;
        const f32x4 F8 = mma16(bf4(c.N4t), bf4(c.N4), id);          // I + N^8
        const f32x4 Ht = mma16(bf4(c.N4), bf4(c.Gt), c.Gt);   // ((I-N)(I+N^2)(I+N^4))^T
        const bf16x4 Htb = bf4(Ht), F8b = bf4(F8);
        const f32x4 Tm = mma16(Htb, F8b, zero4());     // T
        const f32x4 Tt = mma16(F8b, Htb, zero4());     // T^T
        f32x4 TbT, Tb;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            TbT[r] = c.brow[r] * Tt[r];   // (T Diag(beta))^T
            Tb[r] = c.bcol * Tm[r];       // T Diag(beta)
        }
        B.tbt[lane] = as_u2(bf4(TbT));
        B.y3[lane] = as_u2(bf4(mma16(bf4(Tb), bf4(c.Pt), zero4())));   // (P Tb)^T
    };

    // stage B2 for tile `tile`, wave 8 + s: W and Qpp for channels [32s, 32s+32), Ut and PUt for
    // columns [16s, 16s+16), and the channel-major Kd blocks of those channels
    // stage B2's inputs from stage A, read at the end of the period before (stage A wrote them two
    // periods before that), so that only stage B1's hand-off is read after the barrier
    struct B2In { bf16x4 kpc[2]; uint2 kdh[2]; f32x4 qpf[2]; bf16x4 vcs[NS]; };
    auto b2_in = [&](int64_t tile) -> B2In {
        const FromA<NS>& A = fa(tile);
        const int src = 4 * lg + (ln >> 2) + 16 * (ln & 3);
        B2In x;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            x.kpc[hh] = lds_tr16(reinterpret_cast<const char*>(&A.kp[s][src]) + 8 * hh);
            x.kdh[hh] = as_u2(lds_tr16(reinterpret_cast<const char*>(&A.kd[s][src]) + 8 * hh));
            x.qpf[hh] = A.qpf[2 * s + hh][lane];
        }
#pragma unroll
        for (int m = 0; m < NS; ++m) x.vcs[m] = lds_tr16(&A.vraw[s + 4 * m][src]);
        return x;
    };
    auto stage_b2 = [&](int64_t tile, const B2In& x) {
        FromB<NS>& B = fb(tile);
        const uint2 tbu = fb1(tile).tbt[lane], y3u = fb1(tile).y3[lane];
        const bf16x4 TbTb = as_bf4(tbu), Y3b = as_bf4(y3u);
        const bf16x4 nY3b = as_bf4(make_uint2(y3u.x ^ 0x80008000u, y3u.y ^ 0x80008000u));
        // channel-major blocks by transpose reads of the token-major fragments: this lane
        // addresses token 4lg + ln / 4, channels 4 (ln % 4) .. +3 of each 16-channel half,
        // which stage-A lane (token) + 16 (ln % 4) stored
        bf16x4 Wf[2], Qf[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            Wf[hh] = bf4(mma16(x.kpc[hh], TbTb, zero4()));                   // W^T
            Qf[hh] = bf4(mma16(x.kpc[hh], nY3b, x.qpf[hh]));                 // Qpp^T
        }
        B.kdc[s][lane] = make_uint4(x.kdh[0].x, x.kdh[0].y, x.kdh[1].x, x.kdh[1].y);
        B.w[s][lane] = cat8(Wf[0], Wf[1]);
        B.qpp[s][lane] = cat8(Qf[0], Qf[1]);
#pragma unroll
        for (int m = 0; m < NS; ++m) {
            const bf16x4 vcs = x.vcs[m];                           // column-major V
            B.ut[s + 4 * m][lane] = mma16(TbTb, vcs, zero4());     // Tb V
            const f32x4 pu = mma16(vcs, Y3b, zero4());             // (P Tb V)^T
            if constexpr (NS == 1) B.put[s][lane] = pu;
            else B.put[s + 4 * m][lane] = as_u2(bf4(pu));
        }
    };

    // stage S for tile `tile`: strips s + 4 m; leaves the token-major o fragments in Ot
    // With one strip per wave, the decay of the state to the next tile's end and its bf16 copy
    // run at the end of the previous period (after the update), so that a period opens with
    // matrix-core products while stage A issues its vector work.
    constexpr bool kPre = NS == 1;
    bf16x8 Sb[4];       // one strip (kPre)
    auto decay = [&](int64_t tile) {
        const float* ec = ecb(tile);
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
            const f32x4 e = *reinterpret_cast<const f32x4*>(&ec[16 * mb + 4 * lg]);
#pragma unroll
            for (int m = 0; m < NS; ++m) S[m][mb] *= e;                         // St
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) Sb[ks] = cat8(bf4(S[0][2 * ks]), bf4(S[0][2 * ks + 1]));
    };
    auto stage_s = [&](int64_t tile, bf16x4 (&Ot)[NS]) {
        const FromB<NS>& B = fb(tile);
        if constexpr (!kPre) {
            const float* ec = ecb(tile);
#pragma unroll
            for (int mb = 0; mb < 8; ++mb) {
                const f32x4 e = *reinterpret_cast<const f32x4*>(&ec[16 * mb + 4 * lg]);
#pragma unroll
                for (int m = 0; m < NS; ++m) S[m][mb] *= e;                     // St
            }
        }
        // In the plain two-strip kernel the period's W / Qpp, Ut, PUt and Kd fragments are all
        // requested as the period opens, ahead of the products.  Against reads next to their
        // products (outputs bit-identical): 7.8% faster on the 16-sequence batch and 11.1% at
        // 4 x 4096 tokens, although the registers they hold make the compiler spill 36 values
        // (reading Kd only after the W / Qpp products kept fewer and gained 2-3%).  With one
        // strip (3.5% slower at H = 96) and with the output stage (2% slower) the reads stay next
        // to their products.
        constexpr bool kEarly = NS == 2 && !GATED;
        bf16x8 wfa[4], qfa[4];
        f32x4 uta[NS];
        typename PutOf<NS>::T puta[NS];
        uint4 kda[4];
        if constexpr (kEarly) {
#pragma unroll
            for (int j = 0; j < 4; ++j) kda[j] = B.kdc[j][lane];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                wfa[ks] = B.w[ks][lane];
                qfa[ks] = B.qpp[ks][lane];
            }
#pragma unroll
            for (int m = 0; m < NS; ++m) {
                uta[m] = B.ut[s + 4 * m][lane];
                puta[m] = B.put[s + 4 * m][lane];
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // k-steps outside, strips inside
        f32x4 XW[NS], XQ[NS];
#pragma unroll
        for (int m = 0; m < NS; ++m) XW[m] = XQ[m] = zero4();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 wf = kEarly ? wfa[ks] : B.w[ks][lane];
            const bf16x8 qf = kEarly ? qfa[ks] : B.qpp[ks][lane];
#pragma unroll
            for (int m = 0; m < NS; ++m) {
                bf16x8 sb;
                if constexpr (kPre) sb = Sb[ks];
                else sb = cat8(bf4(S[m][2 * ks]), bf4(S[m][2 * ks + 1]));
                XW[m] = mma32(wf, sb, XW[m]);
                XQ[m] = mma32(sb, qf, XQ[m]);   // (Qpp St)^T: o already token-major
            }
        }
        bf16x4 Ub[NS];
#pragma unroll
        for (int m = 0; m < NS; ++m) {
            Ub[m] = bf4((kEarly ? uta[m] : B.ut[s + 4 * m][lane]) - XW[m]);     // U
            f32x4 O;
            if constexpr (NS == 1) O = XQ[m] + B.put[s][lane];
            else O = XQ[m] + unpack4(kEarly ? puta[m] : B.put[s + 4 * m][lane]);
            Ot[m] = bf4(O);
        }
        // S <- St + Kd^T U, blocks outside and strips inside: each Kd fragment serves both strips
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint4 kd2 = kEarly ? kda[j] : B.kdc[j][lane];
            const bf16x4 kdf0 = as_bf4(make_uint2(kd2.x, kd2.y));
            const bf16x4 kdf1 = as_bf4(make_uint2(kd2.z, kd2.w));
#pragma unroll
            for (int m = 0; m < NS; ++m) S[m][2 * j] = mma16(kdf0, Ub[m], S[m][2 * j]);
#pragma unroll
            for (int m = 0; m < NS; ++m) S[m][2 * j + 1] = mma16(kdf1, Ub[m], S[m][2 * j + 1]);
        }
    };
    // with the fused output stage o is optional; y's lane offset within a tile's token rows
    const bool want_o = !GATED || o != nullptr;
    // y (fused output stage, two strips): lane rows lg and lg ^ 1 trade pieces so that each lane
    // stores 8 consecutive columns of its token as one 16-byte store: rows with lg even take strip
    // 0's columns 16 s + 4 lg .. + 7, rows with lg odd strip 1's 64 + 16 s + 4 (lg - 1) .. + 7.
    // Against two 8-byte stores per lane (outputs bit-identical): 1.3-4.0% faster on the
    // 16-sequence batch and 3.1-3.9% at 4 x 4096 tokens (two builds).  The same pairing for o in
    // the plain kernel measured 0.3-1.2% slower, so o keeps one 8-byte store per strip.
    const int64_t ycol = (int64_t)slice * BVT + 16 * s + 4 * (lg & ~1) + 64 * (lg & 1);
    auto pair_strips = [&](uint2 a0, uint2 a1) -> uint4 {
        const auto x = __builtin_amdgcn_permlane16_swap(a0.x, a1.x, false, false);
        const auto z = __builtin_amdgcn_permlane16_swap(a0.y, a1.y, false, false);
        return make_uint4(x[0], z[0], x[1], z[1]);
    };
    const uint32_t vo_y = (uint32_t)((ln * H + h) * D + ycol) * 2u;
    auto store_o = [&](int64_t tile, const bf16x4 (&Ot)[NS], bool masked) {
        const int64_t t0 = bos + tile * C;
        bf16_t* dst = o + ((t0 + ln) * H + h) * D + vcol0;
        if (want_o && (!masked || t0 + ln < eos)) {
#pragma unroll
            for (int m = 0; m < NS; ++m) *reinterpret_cast<uint2*>(dst + 64 * m) = as_u2(Ot[m]);
        }
    };
    // fused output stage, stage S's part.  In the period that forms tile t's o: this wave's sum of
    // o^2 per token (as rounded to bf16, as stored) into ssq.  In the next period: the four sums,
    // then y from the o kept in registers and stage B's w * sigmoid(gate).
    auto ssq_step = [&](int64_t tile, const bf16x4 (&Ot)[NS]) {
        if constexpr (GATED) {
            float ss = 0.f;
#pragma unroll
            for (int m = 0; m < NS; ++m) {
                const f32x4 of = unpack4(as_u2(Ot[m]));
#pragma unroll
                for (int r = 0; r < 4; ++r) ss += of[r] * of[r];
            }
            // the four lane groups hold the same token (columns 4 lg .. 4 lg + 3 of each strip)
            ss += __shfl_xor(ss, 16);
            ss += __shfl_xor(ss, 32);
            if (lg == 0) gsh.ssq[(uint32_t)tile & 1u][ln][s] = ss;
        }
    };
    auto y_finish = [&](int64_t tile, const bf16x4 (&Ot)[NS]) {
        if constexpr (GATED) {
            const f32x4 sq = *reinterpret_cast<const f32x4*>(&gsh.ssq[(uint32_t)tile & 1u][ln][0]);
            const float rn = __builtin_amdgcn_rsqf((sq[0] + sq[1] + sq[2] + sq[3]) / (float)D +
                                                   a.eps);
            const uint4 gwv = gsh.gw[(uint32_t)tile & 1u][s][lane];
            const uint2 gwm[2] = {make_uint2(gwv.x, gwv.y), make_uint2(gwv.z, gwv.w)};
            // stored through a buffer resource at the tile's first token row: a scalar base, the
            // lane offset computed once, and a record count that drops tokens past the end
            const int64_t t0 = bos + tile * C;
            const int nv = (int)min(max(eos - t0, (int64_t)0), (int64_t)C);
            const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(y + t0 * H * D), (short)0, nv * rb32, kBufferFlags);
            uint2 yb[NS];
#pragma unroll
            for (int m = 0; m < NS; ++m) {
                const f32x4 gw = unpack4(gwm[m]), of = unpack4(as_u2(Ot[m]));
                f32x4 yv;
#pragma unroll
                for (int r = 0; r < 4; ++r) yv[r] = of[r] * rn * gw[r];
                yb[m] = as_u2(bf4(yv));
            }
            // one 16-byte store per lane (zero scalar offset), the two strips paired as for o
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u32x4, pair_strips(yb[0], yb[1])), ry, vo_y, 0, 0);
        }
    };

    // Period q (one barrier after each) runs A(q), the first half of B1(q-1), the second half of
    // B1(q-2), B2(q-3) and S(q-4); every role passes nsteps + 4 barriers.  The stage-A loop is
    // unrolled by two so that the in-flight loads of R0 / R1 never need a register copy.  An odd
    // tile count runs one extra tile past the end, and stages A and B run up to two tiles past
    // it: those tiles read as zero (k = 0: no write; g = 0: no decay), so they leave the state
    // unchanged and store nothing.
    const int64_t nsteps = ntiles + (ntiles & 1);
    if (role == 1) {
        // with most CUs busy, stage A paces the period (its loads and exponentials start each
        // tile), and its waves then win issue ties against the other two roles on their SIMD
        if (PRIO_ROLE == 1) __builtin_amdgcn_s_setprio(1);
        Raw R0, R1;
        load_tile(R0);     // tile 0
        load_tile(R1);     // tile 1
        stage_a(0, R0);
        load_tile(R0);     // tile 2
        lds_barrier();
        stage_a(1, R1);
        load_tile(R1);     // tile 3
        lds_barrier();
        for (int64_t i = 0; i < nsteps; i += 2) {
            stage_a(i + 2, R0);
            load_tile(R0);     // tile i + 4
            lds_barrier();
            stage_a(i + 3, R1);
            load_tile(R1);     // tile i + 5
            lds_barrier();
        }
        lds_barrier();
        lds_barrier();
        if constexpr (GATED) lds_barrier();   // stage S finishes the last y one period later
    } else if (role == 2) {
        // with few workgroups the chain through stage B paces the period instead
        if (PRIO_ROLE == 2) __builtin_amdgcn_s_setprio(1);
        // every stage-B wave runs B2 of period q (tile q - 3) for its channel group, and its pair
        // alternates the two halves of B1 for the tiles of its parity
        const int par = s >> 1;            // tiles of this parity
        B2In nx;                           // the inputs of the next period's B2
        auto b2_at = [&](int64_t q) {
            if (q >= 3 && q - 3 < nsteps) stage_b2(q - 3, nx);
        };
        auto b2_pre = [&](int64_t q) {     // at the end of period q - 1, for period q
            if (q >= 3 && q - 3 < nsteps) nx = b2_in(q - 3);
        };
        int64_t q = 0;                     // period
        for (; q < 1 + par; ++q) {
            b2_at(q);
            b2_pre(q + 1);
            lds_barrier();
        }
        // The two waves of a pair would compute the same B1 and leave identical values in LDS,
        // where stage B2 reads them (the carried registers stay with the wave that formed them).
        // In the 128-column kernel the second wave skips it: 1.3-1.8% faster on the 16-sequence
        // batch with bit-identical outputs.  In the 64-column kernel both keep it, one half per
        // SIMD and period: skipping there measured 6.6% slower at H = 96 and 4.5% at 12 heads,
        // probably because B1 then becomes a branch instead of straight-line code beside B2.
        const bool do_b1 = BVT == 64 || (s & 1) == 0;
        // the gate registers: GX holds the tiles loaded in the first period of each pair below,
        // GY those of the second (the pairs keep their order into the last loop)
        GateRaw GX, GY;
        auto gate_at = [&](int64_t qq, GateRaw& G) {
            if constexpr (GATED) {
                if (qq >= 4 && qq - 4 < nsteps) gate_step(qq - 4, G);
                if (qq >= 2 && qq - 2 < nsteps) gate_load(qq - 2, G);
            }
        };
        for (int64_t j = par; j < nsteps; j += 2) {
            b2_at(q++);
            B1Carry c;
            if (do_b1) c = stage_b1a(j);
            gate_at(q - 1, GX);
            b2_pre(q);
            lds_barrier();
            b2_at(q++);
            if (do_b1) stage_b1b(j, c);
            gate_at(q - 1, GY);
            b2_pre(q);
            lds_barrier();
        }
        if constexpr (GATED) {
            // (stage S finishes the last y one period after its last tile)
            for (; q < nsteps + 5; q += 2) {
                b2_at(q);
                gate_at(q, GX);
                b2_pre(q + 1);
                lds_barrier();
                if (q + 1 < nsteps + 5) {
                    b2_at(q + 1);
                    gate_at(q + 1, GY);
                    b2_pre(q + 2);
                    lds_barrier();
                }
            }
        } else {
            for (; q < nsteps + 4; ++q) {
                b2_at(q);
                b2_pre(q + 1);
                lds_barrier();
            }
        }
    } else {
        state_in(h_in, part_m);
        lds_barrier();
        lds_barrier();
        lds_barrier();
        lds_barrier();
        // snapshots: after tile i the registers hold the state after (i + 1) * 16 tokens; every
        // snap_tiles-th full tile saves it (the next index in the snapshot array)
        int64_t snap_at = a.snaps ? a.snap_tiles : -1;
        int64_t snap_idx = a.snaps ? (a.snap_cu ? (int64_t)a.snap_cu[n] : n * a.snap_per_seq) : 0;
        // tiles whose 16 tokens all lie inside the sequence store without a mask
        const int64_t nfull = (eos - bos) / C;
        int64_t i = 0;
        bf16x4 Ot[NS], Oprev[NS];   // Oprev: the previous tile's o, whose y is finished next
        if constexpr (kPre) decay(0);
        for (; i < nfull; ++i) {
            stage_s(i, Ot);
            store_o(i, Ot, false);
            if constexpr (GATED) {
                ssq_step(i, Ot);
                if (i > 0) y_finish(i - 1, Oprev);
#pragma unroll
                for (int m = 0; m < NS; ++m) Oprev[m] = Ot[m];
            }
            if (!GATED && i + 1 == snap_at) {
                state_out(a.snaps + (snap_idx * H + h) * (int64_t)(D * D));
                ++snap_idx;
                snap_at += a.snap_tiles;
            }
            if constexpr (kPre) if (i + 1 < nsteps) decay(i + 1);
            lds_barrier();
        }
        for (; i < nsteps; ++i) {
            stage_s(i, Ot);
            store_o(i, Ot, true);
            if constexpr (GATED) {
                ssq_step(i, Ot);
                if (i > 0) y_finish(i - 1, Oprev);
#pragma unroll
                for (int m = 0; m < NS; ++m) Oprev[m] = Ot[m];
            }
            if constexpr (kPre) if (i + 1 < nsteps) decay(i + 1);
            lds_barrier();
        }
        if constexpr (GATED) {
            if (nsteps > 0) y_finish(nsteps - 1, Oprev);
            lds_barrier();
        }
        if (h_out) state_out(h_out);
    }
}

}  // namespace

hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t s) {
    // with a token-range split every (sequence, head) pair runs 2 split - 1 units
    const int64_t pairs = a.N * a.H * (a.split > 1 ? 2 * a.split - 1 : 1);
    if (pairs <= 0) return hipSuccess;
    if (a.gate) {
        // the fused output stage needs a whole head per workgroup (the caller checks pairs >= 256
        // and no split or snapshots).  Its gate work rides on the stage-B waves, which take the
        // raised priority here too: 1.7% faster on the 16-sequence batch and 3.3% at 4 x 4096
        // tokens than the same work in stage A with stage A's priority.
        if (pairs < 256 || a.split > 1 || a.snaps) return hipErrorInvalidValue;
        hipLaunchKernelGGL((kda_prefill_mfma_kernel<2, 128, true>), dim3((unsigned)pairs),
                           dim3(NT), 0, s, a);
    } else if (pairs >= 256) {
        // every CU is busy with one workgroup per (sequence, head): a workgroup takes all 128
        // columns, so stages A and B1 run once per head instead of once per 64-column half.
        // Stage B's waves take the raised priority here (1.1% faster on the 16-sequence batch and
        // 1.4% at 4 x 4096 tokens than stage A's; stage S's was slower than both).
        hipLaunchKernelGGL((kda_prefill_mfma_kernel<2, 128, false>), dim3((unsigned)pairs),
                           dim3(NT), 0, s, a);
    } else if (2 * pairs >= 128 && a.split <= 1) {
        // at least half of the 256 CUs hold a workgroup; a split's launch keeps stage B's priority
        // instead (measured 3-5% faster at 12 and 24 heads, 4,096 and 32,768 tokens)
        hipLaunchKernelGGL((kda_prefill_mfma_kernel<1, 64, false>), dim3((unsigned)(2 * pairs)),
                           dim3(NT), 0, s, a);
    } else {
        hipLaunchKernelGGL((kda_prefill_mfma_kernel<2, 64, false>), dim3((unsigned)(2 * pairs)),
                           dim3(NT), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace kda
