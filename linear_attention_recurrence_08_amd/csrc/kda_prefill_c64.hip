// KDA prefill with 64-token chunks made of four 16-token sub-tiles: the state is carried once per
// chunk, the intra-chunk coupling runs as separate diagonal and off-diagonal sub-tile products.
//
// "Kimi K3's hybrid block, from first principles", section "From linear attention to the delta
// rule": KDA is trained chunk by chunk, the tokens of a chunk together and the state passed
// between chunks, and the summed log-decay of a 16-token tile lies in (-80, 0), so every tile,
// the diagonal ones included, runs as dense products; "What's new in Kimi K3", section "KDA in one page": the
// per-token cost is quoted for chunks of 64.  Over 64 tokens the cumulative decay reaches -320,
// beyond float32's range, so every exponent below is kept within one sub-tile or is <= 0:
//
//   sub-tile s (tokens 16s .. 16s+15 of the chunk), inclusive per-channel cumsum gam_s (within
//   the sub-tile, in (-80, 0]), its total G_s = gam_s[15], and P_s = G_0 + .. + G_{s-1} (the decay
//   from the chunk start to the sub-tile start, <= 0);
//       Kq_s = K_s e^{gam_s},  Kn_s = K_s e^{-gam_s},  Qq_s = Q_s e^{gam_s},  Kd_s = K_s e^{G_s - gam_s}
//   with entering state S:
//       diagonal block      A_ss = strict_lower(Kq_s Kn_s^T),       Pd_ss = lower(Qq_s Kn_s^T)
//       off-diagonal, r < s A_sr = (Kq_s e^{P_s - P_{r+1}}) Kd_r^T,  Pd_sr = (Qq_s e^{P_s - P_{r+1}}) Kd_r^T
//       U_s = (I + Diag(beta_s) A_ss)^-1 Diag(beta_s) (V_s - (Kq_s e^{P_s}) S - sum_{r<s} A_sr U_r)
//       O_s = (Qq_s e^{P_s}) S + Pd_ss U_s + sum_{r<s} Pd_sr U_r
//       S <- e^{P_4} S + sum_s (Kd_s e^{P_4 - P_{s+1}})^T U_s
// which is the 64x64 chunk system (I + Diag(beta) A) U = Diag(beta) (V - (K e^Gam) S) solved by
// blocks (its diagonal blocks by forward substitution).  A partial last chunk holds fewer
// sub-tiles; a partial last sub-tile is padded with k = q = v = g = beta = 0 (an identity step).
//
// Float32 on the vector ALUs, one 256-thread workgroup per (sequence, head, 16 columns of dv),
// the state slice in LDS, like the general 16-token kernel.  Any dtype and head sizes that are
// multiples of 16 up to 128.
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int SUB = 16;          // sub-tile tokens
constexpr int NSUB = 4;          // sub-tiles per chunk
constexpr int BV = 16;           // dv columns per workgroup
constexpr int DKMAX = 128;
constexpr int LD = DKMAX + 1;    // padded row stride of the [token][channel] arrays

template <typename Tin>
__global__ __launch_bounds__(256) void kda_prefill_c64_kernel(PrefillArgs a) {
    __shared__ float sS[DKMAX * BV];              // state slice [dk][16] (chunk start)
    __shared__ float sKd[NSUB][SUB * LD];         // Kd_s of the chunk's sub-tiles
    __shared__ float sU[NSUB][SUB * BV];          // U_s
    __shared__ float sKq[SUB * LD], sKn[SUB * LD], sQq[SUB * LD];   // current sub-tile
    __shared__ float sG[SUB * LD];                // g, then gam (current sub-tile)
    __shared__ float sP[NSUB + 1][DKMAX];         // P_0 .. P_4 per channel (P_0 = 0)
    __shared__ float sE[NSUB + 1][DKMAX];         // e^{P_s}, e^{P_s - P_{r+1}} (r < s); carry factors
    __shared__ float sAo[NSUB - 1][SUB * SUB];    // A_sr for r < s
    __shared__ float sPo[NSUB - 1][SUB * SUB];    // Pd_sr for r < s
    __shared__ float sA[SUB * SUB], sPd[SUB * SUB];
    __shared__ float sV[SUB * BV], sB[SUB];

    const int tid = threadIdx.x;
    const int64_t H = a.H, dk = a.dk, dv = a.dv;
    const int64_t nslices = dv / BV;
    const int64_t wg = blockIdx.x;
    const int64_t cb = wg % nslices;
    const int64_t h = (wg / nslices) % H;
    const int64_t n = wg / (nslices * H);
    int64_t bos, eos;
    if (a.cu) { bos = a.cu[n]; eos = a.cu[n + 1]; }
    else { bos = n * a.T; eos = bos + a.T; }

    const Tin* q = static_cast<const Tin*>(a.q);
    const Tin* k = static_cast<const Tin*>(a.k);
    const Tin* v = static_cast<const Tin*>(a.v);
    const Tin* g = static_cast<const Tin*>(a.g);
    const Tin* beta = static_cast<const Tin*>(a.beta);
    Tin* o = static_cast<Tin*>(a.o);

    const int64_t sbase = (n * H + h) * dk * dv + cb * BV;
    for (int idx = tid; idx < dk * BV; idx += 256) {
        const int r = idx / BV, c = idx % BV;
        sS[idx] = a.h0 ? a.h0[sbase + r * dv + c] : 0.0f;
    }

    for (int64_t c0 = bos; c0 < eos; c0 += SUB * NSUB) {
        const int nsub = (int)min<int64_t>(NSUB, (eos - c0 + SUB - 1) / SUB);
        for (int c = tid; c < dk; c += 256) sP[0][c] = 0.f;
        for (int s = 0; s < nsub; ++s) {
            const int64_t t0 = c0 + s * SUB;
            const int L = (int)min<int64_t>(SUB, eos - t0);
            // 1. load the sub-tile (zero padding past the sequence end)
            for (int idx = tid; idx < SUB * dk; idx += 256) {
                const int i = idx / dk, c = idx % dk;
                float kk = 0.f, qq = 0.f, gg = 0.f;
                if (i < L) {
                    const int64_t off = ((t0 + i) * H + h) * dk + c;
                    kk = io<Tin>::load(k + off);
                    qq = io<Tin>::load(q + off);
                    gg = io<Tin>::load(g + off);
                }
                sKq[i * LD + c] = kk;
                sQq[i * LD + c] = qq;
                sG[i * LD + c] = gg;
            }
            {
                const int i = tid / BV, c = tid % BV;
                sV[tid] = (i < L) ? io<Tin>::load(v + ((t0 + i) * H + h) * dv + cb * BV + c) : 0.f;
                if (tid < SUB) sB[tid] = (tid < L) ? io<Tin>::load(beta + (t0 + tid) * H + h) : 0.f;
            }
            __syncthreads();
            // 2. inclusive cumulative log-decay within the sub-tile; P_{s+1} = P_s + G_s
            for (int c = tid; c < dk; c += 256) {
                float run = 0.f;
                for (int i = 0; i < SUB; ++i) { run += sG[i * LD + c]; sG[i * LD + c] = run; }
                sP[s + 1][c] = sP[s][c] + run;
            }
            __syncthreads();
            // 3. rescaled operands (all exponents within the sub-tile) and the per-channel decays
            //    e^{P_s} (row 0) and e^{P_s - P_{r+1}} for r < s (row 1 + r)
            for (int idx = tid; idx < (s + 1) * dk; idx += 256) {
                const int r = idx / dk, c = idx % dk;
                sE[r][c] = r == 0 ? expf(sP[s][c]) : expf(sP[s][c] - sP[r][c]);
            }
            for (int idx = tid; idx < SUB * dk; idx += 256) {
                const int i = idx / dk, c = idx % dk;
                const float gam = sG[i * LD + c], gS = sG[(SUB - 1) * LD + c];
                const float kk = sKq[i * LD + c], qq = sQq[i * LD + c];
                sKq[i * LD + c] = kk * expf(gam);
                sKn[i * LD + c] = kk * expf(-gam);
                sQq[i * LD + c] = qq * expf(gam);
                sKd[s][i * LD + c] = kk * expf(gS - gam);
            }
            __syncthreads();
            // 4. diagonal blocks (thread = (i, j)) and off-diagonal blocks against r < s
            {
                const int i = tid / SUB, j = tid % SUB;
                float accA = 0.f, accP = 0.f;
                for (int c = 0; c < dk; ++c) {
                    const float kn = sKn[j * LD + c];
                    accA += sKq[i * LD + c] * kn;
                    accP += sQq[i * LD + c] * kn;
                }
                sA[i * SUB + j] = (j < i) ? accA : 0.f;
                sPd[i * SUB + j] = (j <= i) ? accP : 0.f;
                for (int r = 0; r < s; ++r) {
                    float ao = 0.f, po = 0.f;
                    for (int c = 0; c < dk; ++c) {
                        const float dkr = sKd[r][j * LD + c] * sE[1 + r][c];
                        ao += sKq[i * LD + c] * dkr;
                        po += sQq[i * LD + c] * dkr;
                    }
                    sAo[r][i * SUB + j] = ao;
                    sPo[r][i * SUB + j] = po;
                }
            }
            __syncthreads();
            // 5. right-hand side (thread = (i, col)): beta_i (v_i - (Kq e^{P_s}) S - sum A_sr U_r)
            {
                const int i = tid / BV, col = tid % BV;
                float acc = 0.f;
                for (int c = 0; c < dk; ++c) acc += sKq[i * LD + c] * sE[0][c] * sS[c * BV + col];
                for (int r = 0; r < s; ++r)
                    for (int jj = 0; jj < SUB; ++jj)
                        acc += sAo[r][i * SUB + jj] * sU[r][jj * BV + col];
                sU[s][i * BV + col] = sB[i] * (sV[i * BV + col] - acc);
            }
            __syncthreads();
            // 6. diagonal forward substitution: u_i -= beta_i sum_{j<i} A_ij u_j (thread = column)
            if (tid < BV) {
                const int col = tid;
                for (int i = 1; i < SUB; ++i) {
                    float acc = sU[s][i * BV + col];
                    const float bi = sB[i];
                    for (int j = 0; j < i; ++j) acc -= bi * sA[i * SUB + j] * sU[s][j * BV + col];
                    sU[s][i * BV + col] = acc;
                }
            }
            __syncthreads();
            // 7. outputs O_s = (Qq e^{P_s}) S + Pd_ss U_s + sum_{r<s} Pd_sr U_r
            {
                const int i = tid / BV, col = tid % BV;
                float acc = 0.f;
                for (int c = 0; c < dk; ++c) acc += sQq[i * LD + c] * sE[0][c] * sS[c * BV + col];
                for (int jj = 0; jj <= i; ++jj) acc += sPd[i * SUB + jj] * sU[s][jj * BV + col];
                for (int r = 0; r < s; ++r)
                    for (int jj = 0; jj < SUB; ++jj)
                        acc += sPo[r][i * SUB + jj] * sU[r][jj * BV + col];
                if (i < L) io<Tin>::store(o + ((t0 + i) * H + h) * dv + cb * BV + col, acc);
            }
            __syncthreads();
        }
        // 8. one carry per chunk: S <- e^{P_n} S + sum_s (Kd_s e^{P_n - P_{s+1}})^T U_s, with the
        //    factors e^{P_n} (row nsub) and e^{P_n - P_{s+1}} (row s) per channel
        for (int idx = tid; idx < (nsub + 1) * dk; idx += 256) {
            const int r = idx / dk, c = idx % dk;
            sE[r][c] = expf(sP[nsub][c] - (r == nsub ? 0.f : sP[r + 1][c]));
        }
        __syncthreads();
        for (int idx = tid; idx < dk * BV; idx += 256) {
            const int c = idx / BV, col = idx % BV;
            float acc = sE[nsub][c] * sS[idx];
            for (int s = 0; s < nsub; ++s) {
                const float f = sE[s][c];
                float part = 0.f;
                for (int j = 0; j < SUB; ++j) part += sKd[s][j * LD + c] * sU[s][j * BV + col];
                acc += f * part;
            }
            sS[idx] = acc;
        }
        __syncthreads();
    }

    if (a.hT) {
        for (int idx = tid; idx < dk * BV; idx += 256) {
            const int r = idx / BV, c = idx % BV;
            a.hT[sbase + r * dv + c] = sS[idx];
        }
    }
}

}  // namespace

hipError_t launch_prefill_c64(const PrefillArgs& a, hipStream_t s) {
    const int64_t grid = a.N * a.H * (a.dv / BV);
    if (grid <= 0) return hipSuccess;
    if (a.dtype == 0)
        hipLaunchKernelGGL(kda_prefill_c64_kernel<bf16_t>, dim3((unsigned)grid), dim3(256), 0, s,
                           a);
    else
        hipLaunchKernelGGL(kda_prefill_c64_kernel<float>, dim3((unsigned)grid), dim3(256), 0, s,
                           a);
    return hipGetLastError();
}

}  // namespace kda
