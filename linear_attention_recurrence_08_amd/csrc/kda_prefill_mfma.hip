// KDA chunkwise prefill on the CDNA4 matrix cores: bf16 inputs, dk = dv = 128, float32 state.
//
// Method ("Kimi K3's hybrid block, from first principles", section "From linear attention to the
// delta rule": parallel inside a chunk, recurrent across chunks; the cumulative log-decay over a
// 16-token tile stays within (-80, 0) so the rescaling factors stay finite and every tile runs as
// dense matrix products).  Per 16-token tile with entering state S (dk x dv), write
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
// the two slices of a head are dispatched to the same XCD so their shared q/k/g reads meet in
// that XCD's L2.  The work of a tile is split into three stages that run as a software pipeline,
// one tile apart, separated by a single workgroup barrier per tile:
//   stage A (waves 4-7, tile i+3): wave s loads key channels [32s, 32s+32) of q, k, g and value
//      columns [16s, 16s+16) of the slice, runs the cumulative log-decay as a product with a
//      triangular 0/1 matrix, and forms the decayed operands Kp, Qp, Kd (the exponentials are
//      the only transcendental work);
//   stage B (waves 8-11): B1 (tile i+2) forms A, A^T, P^T over all 128 channels and evaluates T;
//      B2 (tile i+1) forms W and Qpp for key channels [32b, 32b+32), Ut and PUt for columns
//      [16b, 16b+16), and the channel-major Kd blocks the carry consumes; the two chains belong
//      to different tiles, so they interleave;
//   stage S (waves 0-3, tile i): wave s carries its 128 x 16 strip of S, which lives in registers
//      as eight 16x16 float32 accumulator blocks for the whole sequence, and writes o.
// Three waves share each SIMD, one per stage.  Loads run two tiles ahead of their use.  All products use v_mfma_f32_16x16x{16,32}_bf16;
// changes between token-major and channel-major fragments are products with 0/1 selector
// matrices on the matrix cores (exact for bf16 data), which keeps the vector ALUs for the
// exponentials and the conversions.
//
// Fragment conventions for a 16x16 block, lane l = ln + 16 lg (ln = l % 16, lg = l / 16):
//   accumulator  acc(X): register r holds X[4 lg + r][ln]
//   A operand of Z = X Y is acc(X^T) (as bf16); B operand is acc(Y).
// For the K = 32 products over key channels, slot j of lane group lg stands for channel
// 16 (j / 4) + 4 lg + (j % 4) of the 32-channel group; A and B operands always use this order.
#include "kda_internal.h"

namespace kda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int C = 16;      // tile tokens
constexpr int D = 128;     // dk = dv
constexpr int BV = 64;     // dv columns per workgroup
constexpr int NT = 768;    // threads per workgroup (12 waves: 4 per stage)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float L2E_HI = 1.4453125f;          // bf16(log2 e)
constexpr float L2E_LO = -0.00262451171875f;  // bf16(log2 e - L2E_HI)

__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// float32 -> bf16, round to nearest even, two values per v_cvt_pk_bf16_f32.  Going through 32-bit
// integers keeps the conversions paired when the result feeds a matrix-core operand.
__device__ __forceinline__ uint32_t pk2(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ bf16x4 bf4(f32x4 x) {
    const u32x2 u = {pk2(x[0], x[1]), pk2(x[2], x[3])};
    return __builtin_bit_cast(bf16x4, u);
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f32x4 zero4() { return (f32x4){0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ bf16x4 as_bf4(uint2 u) { return __builtin_bit_cast(bf16x4, u); }
__device__ __forceinline__ uint2 as_u2(bf16x4 b) { return __builtin_bit_cast(uint2, b); }
__device__ __forceinline__ f32x4 unpack4(uint2 u) {  // bf16 x4 -> float32 x4 (exact)
    return (f32x4){__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                   __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
}
// Workgroup barrier that orders LDS only: global loads issued before it stay in flight (a full
// __syncthreads() would also wait for the prefetched tiles).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// Z = X Y given acc(X^T) and acc(Y) in float32 (rounded to bf16 for the matrix core)
__device__ __forceinline__ f32x4 mul16(f32x4 xT, f32x4 y) { return mma16(bf4(xT), bf4(y), zero4()); }

// (workgroup index) -> (pair index p = n * H + head, slice) with both slices of a pair on one XCD
// (workgroups are dealt to the 8 XCDs round-robin by index).
__device__ __forceinline__ void map_workgroup(int64_t b, int64_t pairs, int64_t& p, int& slice) {
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

// Raw inputs of one tile for one stage-A lane: token ln, key channels 32s + 16hh + 4lg + r,
// value columns 16s + 4lg + r of the slice, beta of token ln.  Lanes whose token lies past the
// sequence end load a clamped (valid) token; only their g and beta are zeroed, at the point of
// use: with beta = 0 a padded token's rows of T Diag(beta), Ut and U vanish, so its q, k and v
// never reach a stored output or the state.
struct Raw {
    uint2 q0, q1, k0, k1, g0, g1, v;
    bf16_t b;     // raw bf16 bits of beta
    bool ok;      // token inside the sequence
};

// Stage-to-stage buffers, grouped by hand-off so that one dynamic base address reaches every
// member of a group.
struct FromA {                 // stage A -> stages B1 and B2 (indexed by tile % 3)
    bf16x8 kp[4][64];          // token-major Kp per 32-channel k-step (operand fragments)
    bf16x8 kd[4][64];          // token-major Kd
    bf16x8 qp[4][64];          // token-major Qp
    f32x4 qpf[8][64];          // Qp in float32 as acc(Qp^T) per 16-channel block (C input)
    uint2 vraw[4][64];         // token-major V per 16-column strip (A operand of the transpose)
    float beta[C];
};
struct FromB {                 // stage B1 -> B2 and stage B2 -> S (indexed by tile % 2)
    uint2 kdc[8][64];          // channel-major Kd per block (A operand of Kd^T U)
    bf16x8 w[4][64];           // A operands of W per 32-channel k-step
    bf16x8 qpp[4][64];         // A operands of Qpp per 32-channel k-step
    f32x4 ut[4][64];           // Ut per strip (accumulator fragments)
    f32x4 put[4][64];          // P Ut per strip
    uint2 tbt[64];             // acc((T Diag(beta))^T) as bf16 (B1 -> B2)
    uint2 y3[64];              // acc((P T Diag(beta))^T) as bf16 (B1 -> B2)
};
struct Shared {
    FromA a[3];
    FromB b[2];
    float ec[4][D];            // e^{Gam_C} (stage A -> stage S, tile % 4)
};

__global__ __launch_bounds__(NT) void kda_prefill_mfma_kernel(PrefillArgs a) {
    __shared__ Shared sh;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
    const int lane = tid & 63, ln = lane & 15, lg = lane >> 4;
    const int role = wave >> 2;        // 0: stage S, 1: stage A, 2: stage B
    const int s = wave & 3;            // channel group / strip index of this wave
    const int64_t H = a.H;

    int64_t p;
    int slice;
    map_workgroup(blockIdx.x, a.N * H, p, slice);
    const int64_t n = p / H, h = p % H;
    int64_t bos, eos;
    if (a.cu) { bos = a.cu[n]; eos = a.cu[n + 1]; }
    else { bos = n * a.T; eos = bos + a.T; }
    const int64_t ntiles = (eos - bos + C - 1) / C;

    const bf16_t* __restrict__ q = static_cast<const bf16_t*>(a.q);
    const bf16_t* __restrict__ k = static_cast<const bf16_t*>(a.k);
    const bf16_t* __restrict__ v = static_cast<const bf16_t*>(a.v);
    const bf16_t* __restrict__ g = static_cast<const bf16_t*>(a.g);
    const bf16_t* __restrict__ beta = static_cast<const bf16_t*>(a.beta);
    bf16_t* __restrict__ o = static_cast<bf16_t*>(a.o);

    // ---- constant fragments ----
    bf16x8 sel[2];   // selector: channel-major transpose of 32-channel-group half hh (B, K = 32)
    for (int hh = 0; hh < 2; ++hh)
        for (int j = 0; j < 8; ++j)
            sel[hh][j] = (__bf16)((lg == (ln >> 2) && j == 4 * hh + (ln & 3)) ? 1.f : 0.f);
    bf16x4 eye;      // identity (B operand, K = 16)
    for (int j = 0; j < 4; ++j) eye[j] = (__bf16)((4 * lg + j == ln) ? 1.f : 0.f);
    // M^T scaled by log2(e) as a two-term bf16 split (hi + lo = log2(e) to 5e-6 relative), with
    // M[i][j] = -1 for j > i: row i of M g gives -log2(e) sum_{j>i} g_j, the exponent in base 2
    bf16x4 scanHi, scanLo;
    for (int j = 0; j < 4; ++j) {
        const bool up = 4 * lg + j > ln;
        scanHi[j] = (__bf16)(up ? -L2E_HI : 0.f);
        scanLo[j] = (__bf16)(up ? -L2E_LO : 0.f);
    }
    bf16x4 onesA;    // all ones (A operand): column c of the product is Gam_C of channel c
    for (int j = 0; j < 4; ++j) onesA[j] = (__bf16)1.f;

    // ---- stage S state: rows 16 mb + 4 lg + r, column col of this workgroup's slice ----
    const int64_t col = (int64_t)slice * BV + 16 * s + ln;
    const int64_t sbase = p * (int64_t)(D * D);
    f32x4 S[8];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) S[mb] = zero4();
    if (role == 0 && a.h0) {
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[mb][r] = a.h0[sbase + (int64_t)(16 * mb + 4 * lg + r) * D + col];
    }
    if (ntiles == 0) {
        if (role == 0 && a.hT) {
#pragma unroll
            for (int mb = 0; mb < 8; ++mb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    a.hT[sbase + (int64_t)(16 * mb + 4 * lg + r) * D + col] = S[mb][r];
        }
        return;
    }

    // ---- stage A: loads.  Offsets advance by one tile per call (tiles are loaded in order);
    //      a token past the sequence end reads the sequence's last token instead ----
    const int64_t chan0 = 32 * s + 4 * lg;
    const int64_t vcol0 = (int64_t)slice * BV + 16 * s + 4 * lg;
    const int64_t tstride = (int64_t)C * H * D;
    const int64_t last_off = ((eos - 1) * H + h) * D;
    int64_t run_off = ((bos + ln) * H + h) * D;     // element offset of this lane's next token
    int64_t run_tok = ln;                           // its index within the sequence
    const int64_t len = eos - bos;
    auto load_tile = [&](Raw& R) {
        const bool ok = run_tok < len;
        const int64_t off = ok ? run_off : last_off;
        R.q0 = *reinterpret_cast<const uint2*>(q + off + chan0);
        R.q1 = *reinterpret_cast<const uint2*>(q + off + chan0 + 16);
        R.k0 = *reinterpret_cast<const uint2*>(k + off + chan0);
        R.k1 = *reinterpret_cast<const uint2*>(k + off + chan0 + 16);
        R.g0 = *reinterpret_cast<const uint2*>(g + off + chan0);
        R.g1 = *reinterpret_cast<const uint2*>(g + off + chan0 + 16);
        R.v = *reinterpret_cast<const uint2*>(v + off + vcol0);
        R.b = beta[off / D];
        R.ok = ok;
        run_off += tstride;
        run_tok += C;
    };

    // Buffer indices of a tile: FromA by tile % 3, FromB by tile % 2, ec by tile % 4.
    auto fa = [&](int64_t tile) -> FromA& { return sh.a[(uint32_t)tile % 3u]; };
    auto fb = [&](int64_t tile) -> FromB& { return sh.b[(uint32_t)tile & 1u]; };
    auto ecb = [&](int64_t tile) -> float* { return sh.ec[(uint32_t)tile & 3u]; };

    // stage A for tile `tile`
    auto stage_a = [&](int64_t tile, const Raw& R) {
        FromA& A = fa(tile);
        float* ec = ecb(tile);
        const uint2 z = make_uint2(0u, 0u);
        const uint2 g0 = R.ok ? R.g0 : z, g1 = R.ok ? R.g1 : z;
        const float bt = R.ok ? bf16_to_f32(R.b) : 0.f;
        const bf16x8 ga = cat8(as_bf4(g0), as_bf4(g1));
        const f32x4 kf[2] = {unpack4(R.k0), unpack4(R.k1)};
        const f32x4 qf[2] = {unpack4(R.q0), unpack4(R.q1)};
        f32x4 X[2];    // log2(e) * Gp, token-major
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const bf16x4 gc = bf4(mma32(ga, sel[hh], zero4()));   // channel-major g (exact)
            X[hh] = mma16(gc, scanLo, mma16(gc, scanHi, zero4()));
            // Gam_C of channel 32s + 16hh + ln, in every register and lane group; all four lane
            // groups store the same value
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
        A.beta[ln] = bt;   // every writer of an entry holds the same value
        A.kp[s][lane] = cat8(Kpb[0], Kpb[1]);
        A.qp[s][lane] = cat8(Qpb[0], Qpb[1]);
        A.kd[s][lane] = cat8(Kdb[0], Kdb[1]);
        A.vraw[s][lane] = R.v;
    };

    // stage B1 for tile `tile`: A, A^T, P^T over all 128 channels and the inverse T; every
    // stage-B wave evaluates it (identical results) so that no wave waits for another
    auto stage_b1 = [&](int64_t tile) {
        const FromA& A = fa(tile);
        FromB& B = fb(tile);
        f32x4 Am = zero4(), At = zero4(), Pt = zero4();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 kp8 = A.kp[ks][lane], kd8 = A.kd[ks][lane], qp8 = A.qp[ks][lane];
            Am = mma32(kp8, kd8, Am);    // A  = Kp Kd^T
            At = mma32(kd8, kp8, At);    // A^T
            Pt = mma32(kd8, qp8, Pt);    // P^T = Kd Qp^T
        }
        const float bcol = A.beta[ln];
        const f32x4 brow = *reinterpret_cast<const f32x4*>(&A.beta[4 * lg]);
        f32x4 N, Nt, id;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 4 * lg + r;
            N[r] = (ln < i) ? brow[r] * Am[r] : 0.f;    // N[i][ln]
            Nt[r] = (i < ln) ? bcol * At[r] : 0.f;      // N^T[i][ln]
            Pt[r] = (i <= ln) ? Pt[r] : 0.f;            // P^T[i][ln]
            id[r] = (i == ln) ? 1.f : 0.f;
        }
        // T = (I - N)(I + N^2)(I + N^4)(I + N^8); only the transposes that are consumed as A
        // operands are formed; the identity of each factor enters as the product's C input
        const bf16x4 Nb = bf4(N), Ntb = bf4(Nt);
        const f32x4 N2 = mma16(Ntb, Nb, zero4()), N2t = mma16(Nb, Ntb, zero4());
        const bf16x4 N2b = bf4(N2), N2tb = bf4(N2t);
        const f32x4 N4 = mma16(N2tb, N2b, zero4()), N4t = mma16(N2b, N2tb, zero4());
        const f32x4 F8 = mma16(bf4(N4t), bf4(N4), id);             // I + N^8
        const f32x4 F1t = id - Nt, F2 = id + N2, F4 = id + N4;
        const f32x4 Gt = mul16(F2, F1t);               // ((I-N)(I+N^2))^T
        const f32x4 Ht = mul16(F4, Gt);                // (... (I+N^4))^T
        const bf16x4 Htb = bf4(Ht), F8b = bf4(F8);
        const f32x4 Tm = mma16(Htb, F8b, zero4());     // T
        const f32x4 Tt = mma16(F8b, Htb, zero4());     // T^T
        f32x4 TbT, Tb;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            TbT[r] = brow[r] * Tt[r];   // (T Diag(beta))^T
            Tb[r] = bcol * Tm[r];       // T Diag(beta)
        }
        B.tbt[lane] = as_u2(bf4(TbT));
        B.y3[lane] = as_u2(bf4(mma16(bf4(Tb), bf4(Pt), zero4())));   // (P Tb)^T
    };

    // stage B2 for tile `tile`, wave 8 + s: W and Qpp for channels [32s, 32s+32), Ut and PUt for
    // columns [16s, 16s+16), and the channel-major Kd blocks of those channels
    auto stage_b2 = [&](int64_t tile) {
        const FromA& A = fa(tile);
        FromB& B = fb(tile);
        const uint2 tbu = B.tbt[lane], y3u = B.y3[lane];
        const bf16x4 TbTb = as_bf4(tbu), Y3b = as_bf4(y3u);
        const bf16x4 nY3b = as_bf4(make_uint2(y3u.x ^ 0x80008000u, y3u.y ^ 0x80008000u));
        const bf16x8 kps = A.kp[s][lane], kds = A.kd[s][lane];
        bf16x4 Wf[2], Qf[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const bf16x4 kpc = bf4(mma32(kps, sel[hh], zero4()));    // channel-major Kp
            B.kdc[2 * s + hh][lane] = as_u2(bf4(mma32(kds, sel[hh], zero4())));
            Wf[hh] = bf4(mma16(kpc, TbTb, zero4()));                   // W^T
            Qf[hh] = bf4(mma16(kpc, nY3b, A.qpf[2 * s + hh][lane]));   // Qpp^T
        }
        B.w[s][lane] = cat8(Wf[0], Wf[1]);
        B.qpp[s][lane] = cat8(Qf[0], Qf[1]);
        const bf16x4 vcs = bf4(mma16(as_bf4(A.vraw[s][lane]), eye, zero4()));  // column-major V
        B.ut[s][lane] = mma16(TbTb, vcs, zero4());     // Tb V
        B.put[s][lane] = mma16(Y3b, vcs, zero4());     // P Tb V
    };

    // stage S for tile `tile`: strip s; returns the token-major o fragment (stored by the caller)
    auto stage_s = [&](int64_t tile) -> bf16x4 {
        const FromB& B = fb(tile);
        const float* ec = ecb(tile);
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
            S[mb] *= *reinterpret_cast<const f32x4*>(&ec[16 * mb + 4 * lg]);   // St
        f32x4 XW = zero4(), XQ = zero4();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 sb = cat8(bf4(S[2 * ks]), bf4(S[2 * ks + 1]));
            XW = mma32(B.w[ks][lane], sb, XW);
            XQ = mma32(B.qpp[ks][lane], sb, XQ);
        }
        const f32x4 U = B.ut[s][lane] - XW;
        const f32x4 O = XQ + B.put[s][lane];
        const bf16x4 Ub = bf4(U);
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) S[mb] = mma16(as_bf4(B.kdc[mb][lane]), Ub, S[mb]);
        return bf4(mma16(bf4(O), eye, zero4()));    // token-major o
    };
    auto store_o = [&](int64_t tile, bf16x4 Ot, bool masked) {
        const int64_t t0 = bos + tile * C;
        bf16_t* dst = o + ((t0 + ln) * H + h) * D + vcol0;
        if (!masked || t0 + ln < eos) *reinterpret_cast<uint2*>(dst) = as_u2(Ot);
    };

    // Iteration i runs A(i+3), B1(i+2), B2(i+1) and S(i) with one barrier per iteration (the
    // same count in every role).  The stage-A loop is unrolled by two so that the in-flight loads
    // of R0 / R1 never need a register copy.  An odd tile count runs one extra tile past the
    // end, and stages A and B run up to three tiles past it: those tiles' inputs are all zero
    // (k = 0: no write; g = 0: no decay), so they leave the state unchanged and store nothing.
    const int64_t nsteps = ntiles + (ntiles & 1);
    if (role == 1) {
        Raw R0, R1;
        load_tile(R0);     // tile 0
        load_tile(R1);     // tile 1
        stage_a(0, R0);
        load_tile(R0);     // tile 2
        lds_barrier();
        stage_a(1, R1);
        load_tile(R1);     // tile 3
        lds_barrier();
        stage_a(2, R0);
        load_tile(R0);     // tile 4
        lds_barrier();
        for (int64_t i = 0; i < nsteps; i += 2) {
            stage_a(i + 3, R1);
            load_tile(R1);     // tile i + 5
            lds_barrier();
            stage_a(i + 4, R0);
            load_tile(R0);     // tile i + 6
            lds_barrier();
        }
    } else if (role == 2) {
        lds_barrier();
        stage_b1(0);
        lds_barrier();
        stage_b1(1);
        stage_b2(0);
        lds_barrier();
        for (int64_t i = 0; i < nsteps; ++i) {
            stage_b1(i + 2);
            stage_b2(i + 1);
            lds_barrier();
        }
    } else {
        lds_barrier();
        lds_barrier();
        lds_barrier();
        // tiles whose 16 tokens all lie inside the sequence store without a mask
        const int64_t nfull = (eos - bos) / C;
        int64_t i = 0;
        for (; i < nfull; ++i) {
            store_o(i, stage_s(i), false);
            lds_barrier();
        }
        for (; i < nsteps; ++i) {
            store_o(i, stage_s(i), true);
            lds_barrier();
        }
    }

    if (role == 0 && a.hT) {
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                a.hT[sbase + (int64_t)(16 * mb + 4 * lg + r) * D + col] = S[mb][r];
    }
}

}  // namespace

hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t s) {
    const int64_t grid = a.N * a.H * (D / BV);
    if (grid <= 0) return hipSuccess;
    hipLaunchKernelGGL(kda_prefill_mfma_kernel, dim3((unsigned)grid), dim3(NT), 0, s, a);
    return hipGetLastError();
}

}  // namespace kda
