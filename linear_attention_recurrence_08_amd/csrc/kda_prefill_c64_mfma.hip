// KDA prefill with 64-token chunks on the CDNA4 matrix cores: bf16 inputs, dk = dv = 128,
// float32 state.
//
// Method ("What's new in Kimi K3", section "KDA in one page": the per-token cost is quoted for
// chunks of 64, length-independent; "Kimi K3's hybrid block, from first principles", section "From
// linear attention to the delta rule": the tokens of a chunk are handled together and the state
// passes from chunk to chunk; the summed log-decay of 16 tokens lies in (-80, 0)).  For a chunk of L = 64 tokens with
// entering state S and Gam_t the inclusive per-channel cumsum of g from the chunk start:
//     Kg = K.e^{Gam},  Qg = Q.e^{Gam},  Kl = K.e^{Gam_L - Gam}            (every factor <= 1)
//     A = strict_lower(A_ij = sum_c k_ic k_jc e^{Gam_ic - Gam_jc}),  P = lower(same with q_i)
//     Tb = (I + Diag(beta) A)^-1 Diag(beta)                              (64 x 64, unit lower)
//     W = Tb Kg,  Ut = Tb V,  Qpp = Qg - P W,  Z = P Ut                  (independent of S)
//     U = Ut - W S,   O = Qpp S + Z,   S <- Diag(e^{Gam_L}) S + Kl^T U   (the serial carry)
// which is the token recurrence S_t = (I - b k k^T) Diag(e^g) S_{t-1} + b k v^T, o_t = S_t^T q_t
// unrolled over the chunk.  Over 64 tokens Gam reaches -320, beyond float32's range for e^{-Gam},
// so A and P are formed by 16-token sub-tile blocks: the diagonal block (s, s) with the reference
// point at the sub-tile end (factors e^{Gam_i - Gam_end(s)} <= e^80 and e^{Gam_end(s) - Gam_j} <= 1),
// an off-diagonal block (s, r < s) as (K_s e^{Gam - Gam_end(r)}) (K_r e^{Gam_end(r) - Gam})^T with both
// factors <= 1.  The inverse runs by blocks: the diagonal blocks as the finite product
// (I - N)(I + N^2)(I + N^4)(I + N^8) (N^16 = 0), the off-diagonal ones by block substitution
//     Tb_sr = -Tb_ss sum_{r <= j < s} A_sj Tb_jr.
//
// Mapping to gfx950.  Everything independent of the state runs in a prep kernel, one 4-wave
// workgroup per (chunk, head), all chunks in parallel; it leaves W, Qpp, Ut, Z, Kl and e^{Gam_L} of
// each (chunk, head) in a workspace, laid out as the matrix-core fragments the carry kernel reads.
// The carry kernel runs one 4-wave workgroup per (sequence, head): wave w keeps two 16-column
// strips of S (columns 16w and 64 + 16w) in registers for the whole sequence; per chunk it stages
// W, Qpp and Kl in LDS (double-buffered, the next chunk's copy in flight) and runs U, O and the
// update, the latter as K = 32 products over pairs of sub-tiles.  Fragment conventions as in the
// 16-token kernel: acc(X) register r holds X[4 lg + r][ln]; the A operand of Z = X Y is acc(X^T),
// the B operand acc(Y); for K = 32, slot j of lane group lg stands for index 16 (j / 4) + 4 lg +
// (j % 4).  Z and the output are formed as transposed products (operands swapped), so both come
// out token-major, the layout o is stored in.
#include "kda_internal.h"
#include "kda_mfma.h"

namespace kda {
namespace {

using namespace mfma;

constexpr int CL = 64;     // chunk tokens
constexpr int ST = 16;     // sub-tile tokens
constexpr int NSUB = 4;    // sub-tiles per chunk
constexpr int D = 128;     // dk = dv

// index of block (s, r), r <= s, of a 4 x 4 block lower triangle
__device__ __forceinline__ constexpr int tri(int s, int r) { return s * (s + 1) / 2 + r; }

// ---- workspace: one record per (chunk, head) ----
struct C64Work {
    bf16x8 w[NSUB][4][64];     // [sub-tile][32-channel group][lane]: A operands of W (token-major)
    bf16x8 qpp[NSUB][4][64];   // the same for Qpp
    uint2 kl[NSUB][8][64];     // [sub-tile][16-channel block][lane]: acc(Kl block), bf16
    uint2 ut[NSUB][8][64];     // [sub-tile][16-column block][lane]: acc(Ut block), bf16
    uint2 z[NSUB][8][64];      // acc(Z^T block), bf16 (token-major, as o is stored)
    float el[D];               // e^{Gam_L} per channel
};
static_assert(sizeof(C64Work) % 256 == 0, "workspace records stay 256-byte aligned");

// ---- prep kernel ----
// 70 KB, so that two workgroups share a CU and one's loads overlap the other's arithmetic;
// arrays whose lifetimes do not overlap share storage
struct PrepShared {
    union {
        bf16x8 kd[NSUB][4][64];   // token-major K e^{Gam_end(s) - Gam} (B operand of A, P blocks)
        bf16x8 kl[NSUB][4][64];   // then token-major Kl (transposed reads)
    };
    bf16x8 kg[NSUB][4][64];    // token-major Kg (transposed reads)
    uint2 vr[NSUB][8][64];     // token-major V per 16-column block (transposed reads)
    union {
        uint2 at[10][64];      // acc(A_sr^T), bf16 (r <= s; strict lower on the diagonal)
        uint2 y3t[10][64];     // then acc((P Tb)_sr^T), bf16
    };
    uint2 pt[10][64];          // acc(P_sr^T), bf16 (lower on the diagonal)
    uint2 tb[10][64];          // acc(Tb_sr), bf16
    uint2 tbt[10][64];         // acc(Tb_sr^T), bf16
    float G[NSUB][D];          // total log-decay of each sub-tile per channel
    float F[14][D];            // per-channel decay factors, all <= 1 (see kF*)
    float beta[CL];
};
// rows of PrepShared::F, with Gam_end(s) the chunk-relative log-decay at the end of sub-tile s:
constexpr int kFg = 0;         // kFg + s:  e^{Gam_end(s)}
constexpr int kFl = 4;         // kFl + s:  e^{Gam_L - Gam_end(s)}
constexpr int kFo = 8;         // kFo + s (s - 1) / 2 + r, r < s:  e^{Gam_end(s) - Gam_end(r)}

__global__ __launch_bounds__(256, 2) void kda_c64_prep_kernel(PrefillArgs a, C64Work* __restrict__ ws,
                                                           const int* __restrict__ coff,
                                                           int64_t nrec_chunks) {
    __shared__ PrepShared sh;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const int64_t j = blockIdx.x, h = blockIdx.y, H = a.H;

    // chunk j -> (sequence n, chunk c of n)
    int64_t n, c;
    if (a.cu) {
        if (j >= coff[a.N]) return;
        int64_t lo = 0, hi = a.N;                    // coff[lo] <= j < coff[hi]
        while (hi - lo > 1) {
            const int64_t mid = (lo + hi) >> 1;
            if (coff[mid] <= j) lo = mid; else hi = mid;
        }
        n = lo;
        c = j - coff[n];
    } else {
        const int64_t per = (a.T + CL - 1) / CL;
        n = j / per;
        c = j % per;
        if (n >= a.N) return;
    }
    int64_t bos, eos;
    if (a.cu) { bos = a.cu[n]; eos = a.cu[n + 1]; }
    else { bos = n * a.T; eos = bos + a.T; }
    const int64_t t0 = bos + c * CL;
    const int ntok = (int)min<int64_t>(CL, eos - t0);

    const bf16_t* q = static_cast<const bf16_t*>(a.q);
    const bf16_t* k = static_cast<const bf16_t*>(a.k);
    const bf16_t* v = static_cast<const bf16_t*>(a.v);
    const bf16_t* g = static_cast<const bf16_t*>(a.g);
    const bf16_t* beta = static_cast<const bf16_t*>(a.beta);

    // ---- constant fragments (as in the 16-token kernel) ----
    bf16x8 sel[2];   // selector: channel-major transpose of 32-channel-group half hh
    for (int hh = 0; hh < 2; ++hh)
        for (int jx = 0; jx < 8; ++jx)
            sel[hh][jx] = (__bf16)((lg == (ln >> 2) && jx == 4 * hh + (ln & 3)) ? 1.f : 0.f);
    bf16x4 scanHi, scanLo;   // -log2(e) above the diagonal, two-term bf16 split
    for (int jx = 0; jx < 4; ++jx) {
        const bool up = 4 * lg + jx > ln;
        scanHi[jx] = (__bf16)(up ? -L2E_HI : 0.f);
        scanLo[jx] = (__bf16)(up ? -L2E_LO : 0.f);
    }
    const bf16x8 scanHL = cat8(scanHi, scanLo);
    bf16x4 onesA;
    for (int jx = 0; jx < 4; ++jx) onesA[jx] = (__bf16)1.f;

    // ---- 1. wave s loads sub-tile s: token ln, channels / columns 16 cb + 4 lg + r ----
    const int s = wave;
    const int nv = min(max(ntok - ST * s, 0), ST);
    const int64_t row_bytes = H * D * 2;
    const int nrec = max((nv - 1) * (int)row_bytes + D * 2, 0);
    const int nrec_b = max((nv - 1) * (int)(H * 2) + 2, 0);
    const int64_t ts = t0 + ST * s;
    const int64_t e0 = (ts * H + h) * D;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)(q + e0), (short)0,
                                                                        nrec, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)(k + e0), (short)0,
                                                                        nrec, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc((void*)(g + e0), (short)0,
                                                                        nrec, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)(v + e0), (short)0,
                                                                        nrec, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(beta + (ts * H + h)), (short)0, nrec_b, kBufferFlags);
    const uint32_t vo = (uint32_t)(ln * row_bytes + 8 * lg);
    uint2 kr[8], qr[8], gr[8], vr[8];
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
        kr[cb] = ld8(rk, vo + 32 * cb);
        qr[cb] = ld8(rq, vo + 32 * cb);
        gr[cb] = ld8(rg, vo + 32 * cb);
        vr[cb] = ld8(rv, vo + 32 * cb);
    }
    const uint32_t braw = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rb, ln * H * 2, 0, 0);

    // ---- 2. log-decay within the sub-tile, X = log2(e) Gp with Gp_i = Gam_i - Gam_end(s) =
    //         -sum_{j>i} g_j >= 0 (token-major), and the sub-tile total per channel ----
    f32x4 X[8];
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
        const bf16x8 ga = cat8(as_bf4(gr[2 * gi]), as_bf4(gr[2 * gi + 1]));
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const bf16x4 gc = bf4(mma32(ga, sel[hh], zero4()));   // channel-major g (exact)
            X[2 * gi + hh] = mma32(cat8(gc, gc), scanHL, zero4());
            const f32x4 gsum = mma16(onesA, gc, zero4());
            sh.G[s][32 * gi + 16 * hh + ln] = gsum[0];           // all lane groups agree
        }
    }
    sh.beta[ST * s + ln] = __uint_as_float(braw << 16);
    // Kp = K e^{Gp} (>= 1, at most e^80), Qp = Q e^{Gp}, Kd = K e^{-Gp} (<= 1); Kd_s is the column
    // operand of every block (s', s), s' >= s
    f32x4 Kp[8], Qp[8], Kd[8];
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
        const f32x4 kf = unpack4(kr[cb]), qf = unpack4(qr[cb]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float e = __builtin_amdgcn_exp2f(X[cb][r]);
            const float d = __builtin_amdgcn_exp2f(-X[cb][r]);
            Kp[cb][r] = kf[r] * e;
            Qp[cb][r] = qf[r] * e;
            Kd[cb][r] = kf[r] * d;
        }
    }
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) sh.kd[s][gi][lane] = cat8(bf4(Kd[2 * gi]), bf4(Kd[2 * gi + 1]));
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) sh.vr[s][cb][lane] = vr[cb];
    __syncthreads();

    // per-channel factors: every chunk-level operand is a sub-tile operand times one of them (a
    // factor underflows only where the product it scales is below e^{80 - 103})
    {
        const int ch = tid & 127, half = tid >> 7;
        float E[NSUB], acc = 0.f;
#pragma unroll
        for (int sp = 0; sp < NSUB; ++sp) {
            acc += sh.G[sp][ch];
            E[sp] = acc;
        }
        if (half == 0) {
#pragma unroll
            for (int sp = 0; sp < NSUB; ++sp) {
                sh.F[kFg + sp][ch] = __builtin_amdgcn_exp2f(E[sp] * LOG2E);
                sh.F[kFl + sp][ch] = __builtin_amdgcn_exp2f((E[NSUB - 1] - E[sp]) * LOG2E);
            }
        } else {
#pragma unroll
            for (int sp = 1; sp < NSUB; ++sp)
#pragma unroll
                for (int r = 0; r < sp; ++r)
                    sh.F[kFo + sp * (sp - 1) / 2 + r][ch] =
                        __builtin_amdgcn_exp2f((E[sp] - E[r]) * LOG2E);
        }
    }
    __syncthreads();
    auto fac = [&](int row, int cb) {   // the factors of this lane's channels 16 cb + 4 lg + r
        return *reinterpret_cast<const f32x4*>(&sh.F[row][16 * cb + 4 * lg]);
    };

    // ---- 3. chunk-level operands Kg = Kp e^{Gam_end(s)}, Qg = Qp e^{Gam_end(s)} ----
    f32x4 qgr[8];          // Qg in float32, acc(Qg^T) per 16-channel block: C input of Qpp^T
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
        f32x4 kg2[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int cb = 2 * gi + hh;
            const f32x4 fg = fac(kFg + s, cb);
            kg2[hh] = Kp[cb] * fg;
            qgr[cb] = Qp[cb] * fg;
        }
        sh.kg[s][gi][lane] = cat8(bf4(kg2[0]), bf4(kg2[1]));
    }

    // ---- 4. blocks (s, r <= s) of A^T and P^T; the diagonal inverse ----
    const float bcol = sh.beta[ST * s + ln];
    const f32x4 brow = *reinterpret_cast<const f32x4*>(&sh.beta[ST * s + 4 * lg]);
    f32x4 Am = zero4();
#pragma unroll
    for (int r = 0; r < NSUB; ++r) {
        if (r > s) break;
        f32x4 At = zero4(), Pt = zero4();
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
            // row operands of block (s, r): Kp, Qp on the diagonal (the sub-tile-end reference),
            // times e^{Gam_end(s) - Gam_end(r)} for r < s (then every factor is <= 1)
            f32x4 rk2[2], rq2[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int cb = 2 * gi + hh;
                if (r == s) {
                    rk2[hh] = Kp[cb];
                    rq2[hh] = Qp[cb];
                } else {
                    const f32x4 f = fac(kFo + s * (s - 1) / 2 + r, cb);
                    rk2[hh] = Kp[cb] * f;
                    rq2[hh] = Qp[cb] * f;
                }
            }
            const bf16x8 rk8 = cat8(bf4(rk2[0]), bf4(rk2[1]));
            const bf16x8 rq8 = cat8(bf4(rq2[0]), bf4(rq2[1]));
            const bf16x8 kd8 = sh.kd[r][gi][lane];
            if (r == s) Am = mma32(rk8, kd8, Am);    // A_ss
            At = mma32(kd8, rk8, At);                // A_sr^T
            Pt = mma32(kd8, rq8, Pt);                // P_sr^T
        }
        if (r == s) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int i = 4 * lg + rr;
                At[rr] = (i < ln) ? At[rr] : 0.f;    // A^T[i][ln] = A[ln][i], strict lower
                Pt[rr] = (i <= ln) ? Pt[rr] : 0.f;   // P^T[i][ln] = P[ln][i], lower
            }
        }
        sh.at[tri(s, r)][lane] = as_u2(bf4(At));
        sh.pt[tri(s, r)][lane] = as_u2(bf4(Pt));
        if (r == s) {
            // T_ss = (I - N)(I + N^2)(I + N^4)(I + N^8), N = Diag(beta) A_ss (16 x 16)
            f32x4 N, Nt, F1t, id;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int i = 4 * lg + rr;
                N[rr] = (ln < i) ? brow[rr] * Am[rr] : 0.f;     // N[i][ln]
                Nt[rr] = bcol * At[rr];                          // N^T[i][ln] (At masked)
                F1t[rr] = ((i == ln) ? 1.f : 0.f) - Nt[rr];      // (I - N)^T
                id[rr] = (i == ln) ? 1.f : 0.f;
            }
            const bf16x4 Nb = bf4(N), Ntb = bf4(Nt);
            const f32x4 N2 = mma16(Ntb, Nb, zero4()), N2t = mma16(Nb, Ntb, zero4());
            const bf16x4 N2b = bf4(N2), N2tb = bf4(N2t);
            const f32x4 N4 = mma16(N2tb, N2b, zero4());
            const f32x4 N4t = mma16(N2b, N2tb, zero4());
            const f32x4 Gt = mma16(N2b, bf4(F1t), F1t);                  // ((I - N)(I + N^2))^T
            const f32x4 F8 = mma16(bf4(N4t), bf4(N4), id);               // I + N^8
            const f32x4 Ht = mma16(bf4(N4), bf4(Gt), Gt);                // (.. (I + N^4))^T
            const bf16x4 Htb = bf4(Ht), F8b = bf4(F8);
            const f32x4 Tm = mma16(Htb, F8b, zero4());                   // T_ss
            const f32x4 Tt = mma16(F8b, Htb, zero4());                   // T_ss^T
            f32x4 TbT, Tb;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                TbT[rr] = brow[rr] * Tt[rr];    // (T Diag(beta))^T
                Tb[rr] = bcol * Tm[rr];         // T Diag(beta)
            }
            sh.tbt[tri(s, s)][lane] = as_u2(bf4(TbT));
            sh.tb[tri(s, s)][lane] = as_u2(bf4(Tb));
        }
    }
    __syncthreads();

    // Kl = Kd e^{Gam_L - Gam_end(s)}, into the storage of Kd (no longer read)
#pragma unroll
    for (int gi = 0; gi < 4; ++gi)
        sh.kl[s][gi][lane] = cat8(bf4(Kd[2 * gi] * fac(kFl + s, 2 * gi)),
                                  bf4(Kd[2 * gi + 1] * fac(kFl + s, 2 * gi + 1)));

    // ---- 5. off-diagonal blocks of Tb, row by row: Tb_kr = -Tb_kk sum_{r <= jj < k} A_kj Tb_jr ----
#pragma unroll
    for (int kk = 1; kk < NSUB; ++kk) {
        if (s == kk) {
            const bf16x4 tkkT = as_bf4(sh.tbt[tri(kk, kk)][lane]);   // acc(Tb_kk^T)
#pragma unroll
            for (int r = 0; r < NSUB - 1; ++r) {
                if (r >= kk) break;
                f32x4 Cm = zero4();
#pragma unroll
                for (int jj = 0; jj < NSUB - 1; ++jj) {
                    if (jj < r || jj >= kk) continue;
                    const bf16x4 akj = as_bf4(sh.at[tri(kk, jj)][lane]);   // acc(A_kj^T)
                    const bf16x4 tjr = as_bf4(sh.tb[tri(jj, r)][lane]);    // acc(Tb_jr)
                    Cm = mma16(akj, tjr, Cm);     // C = sum A_kj Tb_jr
                }
                const bf16x4 nC = neg4(bf4(Cm));  // acc(-C)
                sh.tb[tri(kk, r)][lane] = as_u2(bf4(mma16(tkkT, nC, zero4())));    // -Tb_kk C
                sh.tbt[tri(kk, r)][lane] = as_u2(bf4(mma16(nC, tkkT, zero4())));   // (-Tb_kk C)^T
            }
        }
        __syncthreads();
    }

    // ---- 6. Y3 = P Tb by blocks (s, r <= s): Y3_sr^T = sum_{r <= jj <= s} Tb_jr^T P_sj^T ----
#pragma unroll
    for (int r = 0; r < NSUB; ++r) {
        if (r > s) break;
        f32x4 Y = zero4();
#pragma unroll
        for (int jj = 0; jj < NSUB; ++jj) {
            if (jj < r || jj > s) continue;
            Y = mma16(as_bf4(sh.tb[tri(jj, r)][lane]), as_bf4(sh.pt[tri(s, jj)][lane]), Y);
        }
        sh.y3t[tri(s, r)][lane] = as_u2(bf4(Y));
    }
    __syncthreads();

    // ---- 7. the chunk's products ----
    C64Work* out = ws + (j * H + h);
    const int src = 4 * lg + (ln >> 2) + 16 * (ln & 3);   // transpose-read source lane
    auto kg_acc = [&](int r, int cb) {                    // acc(Kg_r block cb)
        return lds_tr16(reinterpret_cast<const char*>(&sh.kg[r][cb >> 1][src]) + 8 * (cb & 1));
    };
    auto kl_acc = [&](int r, int cb) {
        return lds_tr16(reinterpret_cast<const char*>(&sh.kl[r][cb >> 1][src]) + 8 * (cb & 1));
    };
    auto v_acc = [&](int r, int vb) { return lds_tr16(&sh.vr[r][vb][src]); };
    const int w = wave;
    // acc(Tb_sr^T) serves as the B operand of W^T = Kg^T Tb^T and as the A operand of Ut = Tb V;
    // likewise acc(Y3_sr^T), negated for Qpp.  Operands over the tokens of sub-tile pairs (0, 1)
    // and (2, 3); blocks above the diagonal are zero.
    struct PairOps { bf16x8 tb8[2], y38[2], ny38[2]; int npairs; };
    auto pair_ops = [&](int sb) {
        PairOps po;
        auto tbt_at = [&](int r) { return r <= sb ? as_bf4(sh.tbt[tri(sb, r)][lane]) : zb4(); };
        auto y3t_at = [&](int r) { return r <= sb ? as_bf4(sh.y3t[tri(sb, r)][lane]) : zb4(); };
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
            po.tb8[pp] = cat8(tbt_at(2 * pp), tbt_at(2 * pp + 1));
            po.y38[pp] = cat8(y3t_at(2 * pp), y3t_at(2 * pp + 1));
            po.ny38[pp] = cat8(neg4(y3t_at(2 * pp)), neg4(y3t_at(2 * pp + 1)));
        }
        po.npairs = sb >= 2 ? 2 : 1;
        return po;
    };
    // W^T and Qpp^T of this wave's sub-tile, every channel block (Qg^T from registers)
    {
        const PairOps po = pair_ops(s);
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
            bf16x4 Wb[2], Qb[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int cb = 2 * gi + hh;
                f32x4 Wt = zero4(), Qt = qgr[cb];
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) {
                    if (pp >= po.npairs) break;
                    const bf16x8 A8 = cat8(kg_acc(2 * pp, cb), kg_acc(2 * pp + 1, cb));
                    Wt = mma32(A8, po.tb8[pp], Wt);       // W^T
                    Qt = mma32(A8, po.ny38[pp], Qt);      // Qpp^T = Qg^T - Kg^T (P Tb)^T
                }
                Wb[hh] = bf4(Wt);
                Qb[hh] = bf4(Qt);
            }
            out->w[s][gi][lane] = cat8(Wb[0], Wb[1]);
            out->qpp[s][gi][lane] = cat8(Qb[0], Qb[1]);
        }
    }
    // Ut and Z, value-column blocks 2w, 2w+1 of every sub-tile
#pragma unroll
    for (int sb = 0; sb < NSUB; ++sb) {
        const PairOps po = pair_ops(sb);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int vb = 2 * w + hh;
            f32x4 Ut = zero4(), Zt = zero4();
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                if (pp >= po.npairs) break;
                const bf16x8 B8 = cat8(v_acc(2 * pp, vb), v_acc(2 * pp + 1, vb));
                Ut = mma32(po.tb8[pp], B8, Ut);       // Ut = Tb V
                Zt = mma32(B8, po.y38[pp], Zt);       // Z^T = (P Tb V)^T
            }
            out->ut[sb][vb][lane] = as_u2(bf4(Ut));
            out->z[sb][vb][lane] = as_u2(bf4(Zt));
        }
    }
#pragma unroll
    for (int r = 0; r < NSUB; ++r)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) out->kl[r][2 * w + hh][lane] = as_u2(kl_acc(r, 2 * w + hh));
    if (w == 0) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int ch = lane + 64 * half;
            const float gl = sh.G[0][ch] + sh.G[1][ch] + sh.G[2][ch] + sh.G[3][ch];
            out->el[ch] = __builtin_amdgcn_exp2f(gl * LOG2E);
        }
    }
}

// ---- chunk offsets of a variable-length batch: coff[n] = sum_{m < n} ceil(len_m / 64) ----
__global__ __launch_bounds__(256) void kda_c64_offsets_kernel(const int32_t* __restrict__ cu,
                                                              int N, int* __restrict__ coff) {
    __shared__ int part[256];
    const int tid = threadIdx.x;
    const int per = (N + 255) / 256;
    const int lo = min(tid * per, N), hi = min(lo + per, N);
    int sum = 0;
    for (int i = lo; i < hi; ++i) sum += (max(cu[i + 1] - cu[i], 0) + CL - 1) / CL;
    part[tid] = sum;
    __syncthreads();
    if (tid == 0) {
        int acc = 0;
        for (int i = 0; i < 256; ++i) {
            const int t = part[i];
            part[i] = acc;
            acc += t;
        }
    }
    __syncthreads();
    int acc = part[tid];
    for (int i = lo; i < hi; ++i) {
        coff[i] = acc;
        acc += (max(cu[i + 1] - cu[i], 0) + CL - 1) / CL;
    }
    if (tid == 255) coff[N] = acc;
}

// ---- carry kernel ----
struct CarryBuf {
    bf16x8 w[NSUB][4][64];
    bf16x8 qpp[NSUB][4][64];
    uint2 kl[NSUB][8][64];
    float el[D];
};
constexpr int kCarryU4 = (int)(sizeof(CarryBuf) / 16);        // 16-byte units per chunk
static_assert(sizeof(CarryBuf) % 16 == 0, "copied in 16-byte units");
constexpr int kCarryPer = (kCarryU4 + 255) / 256;             // units per thread

// (workgroup index) -> (pair p = n * H + head, slice) with both slices of a pair on one XCD
// (workgroups are dealt to the 8 XCDs round-robin by index), so that the second slice's reads of
// the shared W, Qpp and Kl meet in that XCD's L2; one slice per pair: p = b
__device__ __forceinline__ void map_pair(int64_t b, int64_t pairs, int nslice, int64_t& p,
                                         int& slice) {
    if (nslice == 1) {
        p = b;
        slice = 0;
        return;
    }
    const int64_t full = (pairs / 8) * 16;
    if (b < full) {
        const int64_t xcd = b % 8, jx = b / 8;
        slice = (int)(jx % 2);
        p = (jx / 2) * 8 + xcd;
    } else {
        const int64_t t = b - full;
        slice = (int)(t % 2);
        p = (pairs / 8) * 8 + t / 2;
    }
}

// NS: 16-column strips per wave; NS = 2 takes a whole head per workgroup, NS = 1 one 64-column
// slice of it (two workgroups per head, for grids that would otherwise leave CUs idle)
template <int NS>
__global__ __launch_bounds__(256) void kda_c64_carry_kernel(PrefillArgs a,
                                                            const C64Work* __restrict__ ws,
                                                            const int* __restrict__ coff,
                                                            int64_t nrec_chunks) {
    __shared__ CarryBuf buf[2];
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const int64_t H = a.H;
    int64_t p;
    int slice;
    map_pair(blockIdx.x, a.N * H, 2 / NS, p, slice);
    const int64_t n = p / H, h = p % H;
    auto vblk = [&](int m) { return 4 * slice + w + 4 * m; };   // 16-column block of strip m
    int64_t bos, eos, j0;
    if (a.cu) { bos = a.cu[n]; eos = a.cu[n + 1]; j0 = coff[n]; }
    else { bos = n * a.T; eos = bos + a.T; j0 = n * ((a.T + CL - 1) / CL); }
    int64_t nch = eos > bos ? (eos - bos + CL - 1) / CL : 0;
    nch = max<int64_t>(min<int64_t>(nch, nrec_chunks - j0), 0);   // malformed offsets stay in bounds

    // state strips m: rows 16 mb + 4 lg + r, column 16 vblk(m) + ln
    const int64_t sbase = p * (int64_t)(D * D);
    f32x4 S[NS][8];
#pragma unroll
    for (int m = 0; m < NS; ++m)
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[m][mb][r] = a.h0 ? a.h0[sbase + (int64_t)(16 * mb + 4 * lg + r) * D +
                                          16 * vblk(m) + ln]
                                   : 0.f;

    // the shared part of chunk jx (W, Qpp, Kl, e^{Gam_L}) in flight in registers
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 pre[kCarryPer];
    auto fetch = [&](int64_t jx) {
        const C64Work* wk = ws + (jx * H + h);
        const u32x4* s0 = reinterpret_cast<const u32x4*>(&wk->w[0][0][0]);
        const u32x4* s1 = reinterpret_cast<const u32x4*>(&wk->el[0]);
        constexpr int n0 = (int)((sizeof(bf16x8) * 2 * NSUB * 4 * 64 + sizeof(uint2) * NSUB * 8 * 64) / 16);
#pragma unroll
        for (int i = 0; i < kCarryPer; ++i) {
            const int u = tid + 256 * i;
            if (u < n0) pre[i] = s0[u];
            else if (u < kCarryU4) pre[i] = s1[u - n0];
        }
    };
    auto stash = [&](int b) {
        u32x4* d = reinterpret_cast<u32x4*>(&buf[b]);
#pragma unroll
        for (int i = 0; i < kCarryPer; ++i) {
            const int u = tid + 256 * i;
            if (u < kCarryU4) d[u] = pre[i];
        }
    };
    bf16_t* o = static_cast<bf16_t*>(a.o);

    // this wave's columns of a chunk: Ut and Z of strips m (16-column blocks w + 4 m)
    struct Own { uint2 ut[NSUB][NS]; uint2 z[NSUB][NS]; };
    auto fetch_own = [&](int64_t jx, Own& d) {
        const C64Work* wk = ws + (jx * H + h);
#pragma unroll
        for (int sb = 0; sb < NSUB; ++sb)
#pragma unroll
            for (int m = 0; m < NS; ++m) {
                d.ut[sb][m] = wk->ut[sb][vblk(m)][lane];
                d.z[sb][m] = wk->z[sb][vblk(m)][lane];
            }
    };
    // chunk c from LDS buffer c % 2 and the wave's own registers; the next chunk's data in flight
    auto chunk = [&](int64_t c, const Own& cur, Own& nxt) {
        const int b = (int)(c & 1);
        if (c + 1 < nch) {
            fetch(j0 + c + 1);
            fetch_own(j0 + c + 1, nxt);
        }
        const CarryBuf& B = buf[b];
        // bf16 copy of the chunk-start state (B operands over 32-channel groups)
        bf16x8 Sb[NS][4];
#pragma unroll
        for (int m = 0; m < NS; ++m)
#pragma unroll
            for (int gi = 0; gi < 4; ++gi)
                Sb[m][gi] = cat8(bf4(S[m][2 * gi]), bf4(S[m][2 * gi + 1]));
        bf16x4 Ub[NSUB][NS];
        const int64_t t0 = bos + c * CL;
#pragma unroll
        for (int sb = 0; sb < NSUB; ++sb) {
            f32x4 XW[NS], XQ[NS];
#pragma unroll
            for (int m = 0; m < NS; ++m) XW[m] = XQ[m] = zero4();
#pragma unroll
            for (int gi = 0; gi < 4; ++gi) {
                const bf16x8 wf = B.w[sb][gi][lane], qf = B.qpp[sb][gi][lane];
#pragma unroll
                for (int m = 0; m < NS; ++m) {
                    XW[m] = mma32(wf, Sb[m][gi], XW[m]);
                    XQ[m] = mma32(Sb[m][gi], qf, XQ[m]);   // (Qpp S)^T: token-major
                }
            }
            const int64_t tok = t0 + ST * sb + ln;
#pragma unroll
            for (int m = 0; m < NS; ++m) {
                Ub[sb][m] = bf4(unpack4(cur.ut[sb][m]) - XW[m]);                  // U
                const bf16x4 Ot = bf4(XQ[m] + unpack4(cur.z[sb][m]));            // O^T
                if (tok < eos)
                    *reinterpret_cast<uint2*>(o + (tok * H + h) * D + 16 * vblk(m) + 4 * lg) =
                        as_u2(Ot);
            }
        }
        // S <- Diag(e^{Gam_L}) S + Kl^T U, contracted over sub-tile pairs
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
            const f32x4 e = *reinterpret_cast<const f32x4*>(&B.el[16 * mb + 4 * lg]);
            const bf16x8 k01 = cat8(as_bf4(B.kl[0][mb][lane]), as_bf4(B.kl[1][mb][lane]));
            const bf16x8 k23 = cat8(as_bf4(B.kl[2][mb][lane]), as_bf4(B.kl[3][mb][lane]));
#pragma unroll
            for (int m = 0; m < NS; ++m) {
                f32x4 acc = S[m][mb] * e;
                acc = mma32(k01, cat8(Ub[0][m], Ub[1][m]), acc);
                acc = mma32(k23, cat8(Ub[2][m], Ub[3][m]), acc);
                S[m][mb] = acc;
            }
        }
        if (c + 1 < nch) stash(b ^ 1);
        __syncthreads();
    };

    Own own0, own1;
    if (nch > 0) {
        fetch(j0);
        stash(0);
        fetch_own(j0, own0);
    }
    __syncthreads();
    // unrolled by two so that the register sets alternate without copies
    for (int64_t c = 0; c < nch; c += 2) {
        chunk(c, own0, own1);
        if (c + 1 < nch) chunk(c + 1, own1, own0);
    }
    if (a.hT) {
#pragma unroll
        for (int m = 0; m < NS; ++m)
#pragma unroll
            for (int mb = 0; mb < 8; ++mb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    a.hT[sbase + (int64_t)(16 * mb + 4 * lg + r) * D + 16 * vblk(m) + ln] =
                        S[m][mb][r];
    }
}

}  // namespace

// Workspace bytes of the 64-token-chunk matrix-core path: chunk offsets, then one record per
// (chunk, head).  nchunks bounds the chunk count (sum over sequences of ceil(len / 64)).
size_t c64_mfma_workspace_bytes(int64_t nchunks, int64_t N, int64_t H) {
    const size_t off = ((size_t)(N + 1) * sizeof(int) + 255) / 256 * 256;
    return off + (size_t)nchunks * (size_t)H * sizeof(C64Work);
}

hipError_t launch_prefill_c64_mfma(const PrefillArgs& a, void* workspace, int64_t nchunks,
                                   hipStream_t s) {
    if (a.N <= 0 || a.H <= 0) return hipSuccess;
    int* coff = static_cast<int*>(workspace);
    const size_t off = ((size_t)(a.N + 1) * sizeof(int) + 255) / 256 * 256;
    C64Work* ws = reinterpret_cast<C64Work*>(static_cast<char*>(workspace) + off);
    if (a.cu)
        hipLaunchKernelGGL(kda_c64_offsets_kernel, dim3(1), dim3(256), 0, s, a.cu, (int)a.N, coff);
    if (nchunks > 0)
        hipLaunchKernelGGL(kda_c64_prep_kernel, dim3((unsigned)nchunks, (unsigned)a.H), dim3(256),
                           0, s, a, ws, coff, nchunks);
    const int64_t pairs = a.N * a.H;
    if (pairs >= 256)   // the pairs alone fill the chip: a whole head per workgroup
        hipLaunchKernelGGL(kda_c64_carry_kernel<2>, dim3((unsigned)pairs), dim3(256), 0, s, a, ws,
                           coff, nchunks);
    else
        hipLaunchKernelGGL(kda_c64_carry_kernel<1>, dim3((unsigned)(2 * pairs)), dim3(256), 0, s,
                           a, ws, coff, nchunks);
    return hipGetLastError();
}

}  // namespace kda
