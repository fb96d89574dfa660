// KDA chunkwise prefill for batches with few (sequence, head) pairs, bf16 inputs, dk = dv = 128:
// each pair runs on two workgroups, a producer that computes the state-independent part of every
// tile and a consumer that carries the state, joined by a ring of tile records in L2.
//
// Method ("Kimi K3's hybrid block, from first principles", section "From linear attention to the
// delta rule": parallel inside a chunk, recurrent across chunks; over a 16-token tile the
// cumulative log-decay stays within (-80, 0), so every tile runs as dense matrix products).  The
// tile algebra is the one of kda_prefill_mfma.hip, with the decay referenced to the tile end:
//     Kp = K.E, Qp = Q.E, Kd = K.D (E = e^{Gam - Gam_C} >= 1, D = 1 / E), eC = e^{Gam_C}
//     A = strict_lower(Kp Kd^T), P = lower(Qp Kd^T), T = (I + Diag(beta) A)^-1, Tb = T Diag(beta)
//     W = Tb Kp, Ut = Tb V, Qpp = Qp - P W, PUt = P Ut                  (the tile record)
//     St = Diag(eC) S, U = Ut - W St, O = Qpp St + PUt, S <- St + Kd^T U   (the carry)
// Only the carry is serial.  The state-independent record of every tile can be formed at any
// time, so the producer's eight waves each take a whole tile (tiles w, w + 8, ... for wave w):
// loads, cumulative log-decay, decayed operands, the A / A^T / P^T products, the triangular
// inverse and W, Qpp, Ut, PUt, all without a workgroup barrier, eight tiles in flight.  Four of
// the consumer's waves carry the 128 x 128 float32 state in registers (two 16-column strips
// each), one tile per step, while its other four move records from the ring into LDS three tiles
// ahead; one workgroup barrier per step.  Stages A and B of the
// one-workgroup kernel are thus done once per head instead of once per dv half, and the two
// roles no longer share a SIMD's issue slots.
//
// The ring.  Each pair owns RING slots of one tile record (25,088 bytes, in the fragment layouts
// the consumer's products read) and a control block.  Flags carry a launch tag in their upper
// 32 bits, so that values left by earlier launches never match: ready[slot] = tag | (tile + 1)
// once the record of that tile is complete, consumed = tag | n once the consumer has copied
// records 0 .. n - 1 out of the ring.  The producer writes a record only after consumed says its
// slot is free, waits for its own stores to complete, then sets the flag; the consumer reads the
// flag and the record with device-scope loads, which miss its compute unit's L1.
// Both workgroups of a pair are dispatched to the same XCD (workgroups are dealt to the eight
// XCDs round-robin by index: producer 16 j + i, consumer 16 j + 8 + i for pair 8 j + i), so the
// record meets in that XCD's L2.  At start both roles record their XCD id through system-scope
// stores and loads; should they differ, every ring access takes system scope instead.  The
// producer's index is lower than its consumer's, so a resident consumer's producer has been
// dispatched.  Every wait is bounded (spin_limit polls); a wait that runs out marks the launch
// failed in the control block and the consumer then writes NaN to hT.
#include "kda_internal.h"
#include "kda_mfma.h"

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <mutex>

namespace kda {
namespace {

using namespace mfma;

constexpr int C = 16;       // tile tokens
constexpr int D = 128;      // dk = dv
constexpr int NW = 8;       // waves per workgroup, both roles
constexpr int NT = NW * 64;
constexpr int RING = 8;     // ring slots per pair

// One tile's record, in the operand layouts of the carry (the same as the one-workgroup kernel's
// stage B -> stage S hand-off with two strips per wave).
struct Rec {
    bf16x8 w[4][64];        // A operands of W per 32-channel k-step
    bf16x8 qpp[4][64];      // B operands of Qpp per 32-channel k-step
    uint2 kdc[8][64];       // channel-major Kd per 16-channel block (A operands of Kd^T U)
    f32x4 ut[8][64];        // Ut per 16-column strip (accumulator fragments)
    uint2 put[8][64];       // (P Ut)^T per strip, bf16 (added to o, which is bf16)
    float ec[D];            // e^{Gam_C}
};
static_assert(sizeof(Rec) == 25088, "record layout");
constexpr int kRecUnits = (int)(sizeof(Rec) / 16);   // 16-byte units per record
constexpr int kShareUnits = (kRecUnits + NT - 1) / NT;

struct Ctl {
    uint64_t ready[RING];
    uint64_t pad0[16 - RING];
    uint64_t consumed;      // separate 128-byte line from the ready flags
    uint64_t pad1[7];
    uint64_t xcc_p, xcc_c;  // tag | XCD id of the producer / consumer
    uint64_t status;        // tag | 1: a bounded wait ran out
    uint64_t pad2[5];
};
static_assert(sizeof(Ctl) == 256, "control block layout");

constexpr int64_t kMaxPairs = 128;
constexpr size_t kRingBytes = (size_t)kMaxPairs * RING * sizeof(Rec);
constexpr size_t kWsBytes = kRingBytes + (size_t)kMaxPairs * sizeof(Ctl);

static __device__ __align__(256) unsigned char pc_ws[kWsBytes];

// Producer: per-wave LDS for the layout changes of the tile it is working on.
struct PWave {
    bf16x8 kp[4][64];       // token-major Kp per 32-channel group
    bf16x8 kd[4][64];       // token-major Kd
    uint2 vraw[8][64];      // token-major V per 16-column strip
    float beta[C];
};
constexpr size_t kSmemBytes = sizeof(PWave) * NW > 3 * sizeof(Rec)
                                  ? sizeof(PWave) * NW : 3 * sizeof(Rec);

__device__ __forceinline__ uint32_t xcc_id() {
    return __builtin_amdgcn_s_getreg((20) | (0 << 6) | (15 << 11));   // HW_REG_XCC_ID, 16 bits
}

// Flag and counter accesses.  COH = false: both workgroups share one L2 (device-scope loads miss
// the L1 and find the producer's stores there); COH = true: system scope throughout.
template <bool COH> __device__ __forceinline__ uint64_t flag_load(const uint64_t* p) {
    return COH ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM)
               : __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <bool COH> __device__ __forceinline__ void flag_store(uint64_t* p, uint64_t v) {
    if (COH) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    else __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
constexpr int kAuxData(bool coh) { return coh ? 17 : 0; }     // record stores: sc0 sc1 / plain
constexpr int kAuxLoad(bool coh) { return coh ? 17 : 16; }    // record loads: sc0 sc1 / sc1
// every vector-memory access this wave issued has completed (stores included), and the compiler
// moves no memory access across this point
__device__ __forceinline__ void vm_drain() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Bounded wait until pred(flag_load(p)) holds; false when spin_limit polls ran out.
template <bool COH, typename Pred>
__device__ __forceinline__ bool wait_flag(const uint64_t* p, int64_t spin_limit, Pred pred) {
    for (int64_t i = 0; i < spin_limit; ++i) {
        if (pred(flag_load<COH>(p))) return true;
        if (i >= 64) __builtin_amdgcn_s_sleep(1);
    }
    return false;
}

// Raw inputs of one tile for one producer lane: token ln; key channels 32 s + 16 hh + 4 lg + r
// in q/k/g[2 s + hh]; value columns 16 j + 4 lg + r in v[j]; beta of token ln.
struct RawT {
    uint2 q[8], k[8], g[8], v[8];
    uint32_t b;
};

// Sequence bounds and tile count of pair p = n H + h.
__device__ __forceinline__ void pair_bounds(const PrefillArgs& a, int64_t p, int64_t& bos,
                                            int64_t& eos) {
    const int64_t n = p / a.H;
    if (a.cu) { bos = a.cu[n]; eos = a.cu[n + 1]; }
    else { bos = n * a.T; eos = bos + a.T; }
}

// Producer k (0 <= k < m) of XCD group x serves the pairs x, x + 8, ... (whose consumers run on
// XCD x).  Its items are (tile t, pair slot j), numbered i = t * nx + j for the group's nx pairs,
// and it owns i = k, k + m, k + 2 m, ...; wave w takes the owned items w, w + NW, ...  Items are
// in tile order everywhere, so the oldest outstanding record is always being worked on.
template <bool COH>
__device__ void producer(const PrefillArgs& a, PWave& L, int wave, int lane, int64_t x, int64_t k,
                         int64_t m, unsigned char* ws, uint64_t tag, int64_t spin_limit) {
    const int ln = lane & 15, lg = lane >> 4;
    const int64_t H = a.H, pairs = a.N * a.H;
    const int64_t nx = x < pairs ? (pairs - x + 7) / 8 : 0;
    if (nx == 0) return;
    int64_t max_tiles = 0;
    for (int64_t j = 0; j < nx; ++j) {
        int64_t bos, eos;
        pair_bounds(a, x + 8 * j, bos, eos);
        max_tiles = max(max_tiles, (eos - bos + C - 1) / C);
    }
    const int64_t total = max_tiles * nx;
    const int64_t step = m * NW;
    // the next item at or after index i of this wave's sequence whose tile exists, or -1
    auto next_item = [&](int64_t i) -> int64_t {
        for (; i < total; i += step) {
            int64_t bos, eos;
            pair_bounds(a, x + 8 * (i % nx), bos, eos);
            if (i / nx < (eos - bos + C - 1) / C) return i;
        }
        return -1;
    };

    const bf16_t* __restrict__ q = static_cast<const bf16_t*>(a.q);
    const bf16_t* __restrict__ k_ = static_cast<const bf16_t*>(a.k);
    const bf16_t* __restrict__ v = static_cast<const bf16_t*>(a.v);
    const bf16_t* __restrict__ g = static_cast<const bf16_t*>(a.g);
    const bf16_t* __restrict__ beta = static_cast<const bf16_t*>(a.beta);

    // constant fragments (see the one-workgroup kernel's stage A)
    bf16x8 sel[2];
    for (int hh = 0; hh < 2; ++hh)
        for (int j = 0; j < 8; ++j)
            sel[hh][j] = (__bf16)((lg == (ln >> 2) && j == 4 * hh + (ln & 3)) ? 1.f : 0.f);
    bf16x4 scanHi, scanLo;
    for (int j = 0; j < 4; ++j) {
        const bool up = 4 * lg + j > ln;
        scanHi[j] = (__bf16)(up ? -L2E_HI : 0.f);
        scanLo[j] = (__bf16)(up ? -L2E_LO : 0.f);
    }
    const bf16x8 scanHL = cat8(scanHi, scanLo);
    bf16x4 onesA;
    for (int j = 0; j < 4; ++j) onesA[j] = (__bf16)1.f;

    const int64_t row_bytes = H * D * 2;
    const int rb32 = (int)row_bytes, hb32 = (int)(H * 2);
    const uint32_t vo = (uint32_t)(ln * row_bytes + 4 * lg * 2);
    const uint32_t vo_b = (uint32_t)(ln * H * 2);
    auto load_tile = [&](RawT& R, int64_t item) {
        const int64_t pp = x + 8 * (item % nx), tile = item / nx;
        int64_t bos, eos;
        pair_bounds(a, pp, bos, eos);
        const int64_t hh_ = pp % H;
        const int64_t t0 = bos + tile * C;
        const int nv = min(max((int)(eos - bos) - (int)tile * C, 0), C);
        const int nrec = max((nv - 1) * rb32 + D * 2, 0);
        const int nrec_b = max((nv - 1) * hb32 + 2, 0);
        const int64_t e0 = (t0 * H + hh_) * D;
        const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(q + e0), (short)0, nrec, kBufferFlags);
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(k_ + e0), (short)0, nrec, kBufferFlags);
        const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(g + e0), (short)0, nrec, kBufferFlags);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(v + e0), (short)0, nrec, kBufferFlags);
        const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(beta + (t0 * H + hh_)), (short)0, nrec_b, kBufferFlags);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            R.q[i] = ld8(rq, vo + 32 * i);
            R.k[i] = ld8(rk, vo + 32 * i);
            R.g[i] = ld8(rg, vo + 32 * i);
            R.v[i] = ld8(rv, vo + 32 * i);
        }
        R.b = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rb, vo_b, 0, 0);
    };

    // B2's transposed reads: this lane addresses token 4 lg + ln / 4, values 4 (ln % 4) .. +3 of
    // each 16-wide half, which lane (token) + 16 (ln % 4) stored
    const int src = 4 * lg + (ln >> 2) + 16 * (ln & 3);

    // stage A consumes the raw registers, which then take the next item's loads while this item's
    // inverse and record are formed
    RawT R;
    int64_t cur = next_item(k + m * wave);
    if (cur >= 0) load_tile(R, cur);
    while (cur >= 0) {
        const int64_t pp = x + 8 * (cur % nx), tile = cur / nx;
        Rec* ring = reinterpret_cast<Rec*>(ws) + pp * RING;
        Ctl* ctl = reinterpret_cast<Ctl*>(ws + kRingBytes) + pp;
        const int64_t nxt = next_item(cur + step);
        // ---- stage A for the four 32-channel groups, and the A, A^T, P^T partial products ----
        const float bt = __uint_as_float(R.b << 16);
        f32x4 Am = zero4(), At = zero4(), Pt = zero4();
        f32x4 qpf[8];      // Qp in float32 as acc(Qp^T) per 16-channel block (C input of Qpp)
        float ecv[8];      // e^{Gam_C} of channel 16 i + ln
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const bf16x8 ga = cat8(as_bf4(R.g[2 * s]), as_bf4(R.g[2 * s + 1]));
            f32x4 X[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const bf16x4 gc = bf4(mma32(ga, sel[hh], zero4()));
                X[hh] = mma32(cat8(gc, gc), scanHL, zero4());
                const f32x4 gsum = mma16(onesA, gc, zero4());
                ecv[2 * s + hh] = __builtin_amdgcn_exp2f(gsum[0] * LOG2E);
            }
            bf16x4 Kpb[2], Qpb[2], Kdb[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const f32x4 kf = unpack4(R.k[2 * s + hh]), qf = unpack4(R.q[2 * s + hh]);
                f32x4 kp, kd, qp;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float e = __builtin_amdgcn_exp2f(X[hh][r]);
                    const float dd = __builtin_amdgcn_exp2f(-X[hh][r]);
                    kp[r] = kf[r] * e;
                    qp[r] = qf[r] * e;
                    kd[r] = kf[r] * dd;
                }
                Kpb[hh] = bf4(kp);
                Qpb[hh] = bf4(qp);
                Kdb[hh] = bf4(kd);
                qpf[2 * s + hh] = qp;
            }
            const bf16x8 kp8 = cat8(Kpb[0], Kpb[1]), kd8 = cat8(Kdb[0], Kdb[1]);
            const bf16x8 qp8 = cat8(Qpb[0], Qpb[1]);
            L.kp[s][lane] = kp8;
            L.kd[s][lane] = kd8;
            Am = mma32(kp8, kd8, Am);    // A  = Kp Kd^T
            At = mma32(kd8, kp8, At);    // A^T
            Pt = mma32(kd8, qp8, Pt);    // P^T = Kd Qp^T
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) L.vraw[j][lane] = R.v[j];
        L.beta[ln] = bt;   // every lane group writes the same value
        // this wave's LDS writes are complete before its lanes read each other's entries
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (nxt >= 0) load_tile(R, nxt);

        // ---- stage B1: the triangular inverse T = (I - N)(I + N^2)(I + N^4)(I + N^8) ----
        const float bcol = L.beta[ln];
        const f32x4 brow = *reinterpret_cast<const f32x4*>(&L.beta[4 * lg]);
        f32x4 N, Nt, F1t, Pm;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 4 * lg + r;
            N[r] = (ln < i) ? brow[r] * Am[r] : 0.f;     // N[i][ln]
            Nt[r] = (i < ln) ? bcol * At[r] : 0.f;       // N^T[i][ln]
            Pm[r] = (i <= ln) ? Pt[r] : 0.f;             // P^T[i][ln]
            F1t[r] = ((i == ln) ? 1.f : 0.f) - Nt[r];    // (I - N)^T
        }
        const bf16x4 Nb = bf4(N), Ntb = bf4(Nt);
        const f32x4 N2 = mma16(Ntb, Nb, zero4()), N2t = mma16(Nb, Ntb, zero4());
        const bf16x4 N2b = bf4(N2), N2tb = bf4(N2t);
        const f32x4 N4 = mma16(N2tb, N2b, zero4());
        const f32x4 N4t = mma16(N2b, N2tb, zero4());
        const f32x4 Gt = mma16(N2b, bf4(F1t), F1t);     // ((I - N)(I + N^2))^T
        f32x4 id;
#pragma unroll
        for (int r = 0; r < 4; ++r) id[r] = (4 * lg + r == ln) ? 1.f : 0.f;
        const f32x4 F8 = mma16(bf4(N4t), bf4(N4), id);              // I + N^8
        const f32x4 Ht = mma16(bf4(N4), bf4(Gt), Gt);               // ((I-N)(I+N^2)(I+N^4))^T
        const bf16x4 Htb = bf4(Ht), F8b = bf4(F8);
        const f32x4 Tm = mma16(Htb, F8b, zero4());     // T
        const f32x4 Tt = mma16(F8b, Htb, zero4());     // T^T
        f32x4 TbT, Tb;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            TbT[r] = brow[r] * Tt[r];   // (T Diag(beta))^T
            Tb[r] = bcol * Tm[r];       // T Diag(beta)
        }
        const bf16x4 TbTb = bf4(TbT);
        const bf16x4 Y3b = bf4(mma16(bf4(Tb), bf4(Pm), zero4()));   // (P Tb)^T
        const bf16x4 nY3b = neg4(Y3b);

        // ---- wait until the record's slot is free: records up to tile - RING copied out ----
        const int slot = (int)(tile % RING);
        bool ok = true;
        if (tile >= RING) {
            const uint64_t need = tag | (uint64_t)(tile - RING + 1);
            ok = wait_flag<COH>(&ctl->consumed, spin_limit, [&](uint64_t x) {
                return (x >> 32) == (tag >> 32) && x >= need;
            });
        }
        if (!ok) {
            flag_store<true>(&ctl->status, tag | 1u);
            break;
        }
        compiler_fence();

        // ---- stage B2: W, Qpp and the channel-major Kd per group, Ut and PUt per strip, written
        //      straight to the ring slot ----
        Rec* rec = ring + slot;
        const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)rec, (short)0, (int)sizeof(Rec), kBufferFlags);
        constexpr int AUX = kAuxData(COH);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x4 Wf[2], Qf[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const bf16x4 kpc = lds_tr16(reinterpret_cast<const char*>(&L.kp[s][src]) + 8 * hh);
                const bf16x4 kdc = lds_tr16(reinterpret_cast<const char*>(&L.kd[s][src]) + 8 * hh);
                Wf[hh] = bf4(mma16(kpc, TbTb, zero4()));                 // W^T
                Qf[hh] = bf4(mma16(kpc, nY3b, qpf[2 * s + hh]));         // Qpp^T
                __builtin_amdgcn_raw_buffer_store_b64(
                    __builtin_bit_cast(u32x2, kdc), rr,
                    (uint32_t)(offsetof(Rec, kdc) + ((2 * s + hh) * 64 + lane) * 8), 0, AUX);
            }
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u32x4, cat8(Wf[0], Wf[1])), rr,
                (uint32_t)(offsetof(Rec, w) + (s * 64 + lane) * 16), 0, AUX);
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u32x4, cat8(Qf[0], Qf[1])), rr,
                (uint32_t)(offsetof(Rec, qpp) + (s * 64 + lane) * 16), 0, AUX);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bf16x4 vcs = lds_tr16(&L.vraw[j][src]);          // column-major V
            const f32x4 ut = mma16(TbTb, vcs, zero4());             // Tb V
            const bf16x4 pu = bf4(mma16(vcs, Y3b, zero4()));        // (P Tb V)^T
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u32x4, ut), rr,
                (uint32_t)(offsetof(Rec, ut) + (j * 64 + lane) * 16), 0, AUX);
            __builtin_amdgcn_raw_buffer_store_b64(
                __builtin_bit_cast(u32x2, pu), rr,
                (uint32_t)(offsetof(Rec, put) + (j * 64 + lane) * 8), 0, AUX);
        }
        if (lg == 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                __builtin_amdgcn_raw_buffer_store_b32(
                    __float_as_uint(ecv[i]), rr,
                    (uint32_t)(offsetof(Rec, ec) + (16 * i + ln) * 4), 0, AUX);
        }
        // the record's stores have completed (they sit in the shared L2) before the flag says so
        vm_drain();
        flag_store<COH>(&ctl->ready[slot], tag | (uint64_t)(tile + 1));
        cur = nxt;
    }
}

// Consumer: waves 0-3 carry the state, wave w the two 128 x 16 strips of columns
// [16 w, 16 w + 16) and [16 w + 64, 16 w + 80) in registers as 16 x 16 float32 accumulator blocks
// (rows 16 mb + 4 lg + r); both strips share the operand fragments each step reads from LDS.
// Waves 4-7 move records from the ring into three LDS buffers: in step t the carry works on
// record t (and decays the state with record t + 1's factors) while the loaders write record
// t + 2 (loaded during step t - 1) and, once its flag is set, put record t + 3 in flight.  One workgroup barrier ends each step; records up to t + 2 have
// then left the ring.
constexpr int NB = 3;                         // LDS record buffers
constexpr int kLoadThreads = NT / 2;          // the loader waves
constexpr int kLoadUnits = (kRecUnits + kLoadThreads - 1) / kLoadThreads;

template <bool COH>
__device__ void consumer(const PrefillArgs& a, Rec* buf, int* fail, int wave, int lane,
                         int64_t p, int64_t h, int64_t bos, int64_t eos, int64_t ntiles,
                         const Rec* ring, Ctl* ctl, uint64_t tag, int64_t spin_limit) {
    const int ln = lane & 15, lg = lane >> 4;
    const int64_t H = a.H;
    const int64_t sbase = p * (int64_t)(D * D);
    const bool carry = wave < 4;
    bf16_t* __restrict__ o = static_cast<bf16_t*>(a.o);

    // ---- the carry's registers: strips wave and wave + 4 ----
    f32x4 S[2][8];
    if (carry) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int mb = 0; mb < 8; ++mb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    S[m][mb][r] = a.h0 ? a.h0[sbase + (int64_t)(16 * mb + 4 * lg + r) * D +
                                              16 * (wave + 4 * m) + ln]
                                       : 0.f;
    }
    // the state decayed to the end of the tile whose record B holds, St = Diag(eC) S, and its
    // bf16 copy (the products' operand), for strip m
    bf16x8 Sb[2][4];
    auto decay = [&](const Rec& B, int m) {
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
            S[m][mb] *= *reinterpret_cast<const f32x4*>(&B.ec[16 * mb + 4 * lg]);   // St
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) Sb[m][ks] = cat8(bf4(S[m][2 * ks]), bf4(S[m][2 * ks + 1]));
    };
    // one step of the carry on record B for both strips, then the decay to the end of the next
    // tile (record Bn, or none); the strips are staggered so that one strip's vector work can
    // issue while the other's products occupy the matrix core
    auto step = [&](const Rec& B, const Rec* Bn, bf16x4 (&Ot)[2]) {
        f32x4 XW[2], XQ[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) XW[m] = XQ[m] = zero4();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 wf = B.w[ks][lane], qf = B.qpp[ks][lane];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                XW[m] = mma32(wf, Sb[m][ks], XW[m]);                     // W St
                XQ[m] = mma32(Sb[m][ks], qf, XQ[m]);                     // (Qpp St)^T
            }
        }
        bf16x4 kdf[8];
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) kdf[mb] = as_bf4(B.kdc[mb][lane]);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const bf16x4 Ub = bf4(B.ut[wave + 4 * m][lane] - XW[m]);     // U
            Ot[m] = bf4(XQ[m] + unpack4(B.put[wave + 4 * m][lane]));
#pragma unroll
            for (int mb = 0; mb < 8; ++mb) S[m][mb] = mma16(kdf[mb], Ub, S[m][mb]);
            if (Bn) decay(*Bn, m);
        }
    };
    // ---- the loaders' share of a record: 16-byte units lt, lt + 256, ... ----
    const int lt = (wave - 4) * 64 + lane;
    constexpr int AUXL = kAuxLoad(COH);
    u32x4 share[kLoadUnits];
    auto load_share = [&](int64_t tile) {
        const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(ring + tile % RING), (short)0, (int)sizeof(Rec), kBufferFlags);
#pragma unroll
        for (int i = 0; i < kLoadUnits; ++i) {
            const int u = lt + kLoadThreads * i;
            if (u < kRecUnits)
                share[i] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, (uint32_t)(16 * u), 0, AUXL));
        }
    };
    auto store_share = [&](Rec& dst) {
        u32x4* d = reinterpret_cast<u32x4*>(&dst);
#pragma unroll
        for (int i = 0; i < kLoadUnits; ++i) {
            const int u = lt + kLoadThreads * i;
            if (u < kRecUnits) d[u] = share[i];
        }
    };
    // record `tile` in flight once its flag is set: `seen` is the flag's value from a load issued
    // a step earlier (no round trip when the record was already complete), else a bounded wait;
    // a wait that runs out marks the step failed for the whole workgroup
    bool failed = false;     // this loader wave gave up waiting: it waits no more
    auto fetch = [&](int64_t tile, uint64_t seen) {
        const uint64_t want = tag | (uint64_t)(tile + 1);
        if (!failed && (seen == want ||
                        wait_flag<COH>(&ctl->ready[tile % RING], spin_limit,
                                       [want](uint64_t x) { return x == want; }))) {
            compiler_fence();
            load_share(tile);
        } else {
            failed = true;
            if (lane == 0) *fail = 1;
        }
    };

    // records 0 and 1 into LDS, record 2 in flight, the flag of record 3 loading
    uint64_t seen = 0;
    if (!carry) {
        for (int64_t r = 0; r < 2 && r < ntiles; ++r) {
            fetch(r, 0);
            store_share(buf[r]);
        }
        if (ntiles > 2) fetch(2, 0);
        if (ntiles > 3) seen = flag_load<COH>(&ctl->ready[3 % RING]);
    }
    lds_barrier();
    bool ok = *fail == 0;
    if (ok && wave == 4 && lane == 0) flag_store<COH>(&ctl->consumed, tag | (uint64_t)min(ntiles, (int64_t)2));

    // the two roles run separate loops (their memory counters must not mix) that pass the same
    // barriers, one per step.  A loader that gave up waiting only stops loading, so the loops
    // always run to the end; the carry reads the failure flag once, after its last step.
    if (carry) {
        vm_drain();   // the entering state has arrived: no wait on it inside the loop
        if (ok) {
            decay(buf[0], 0);
            decay(buf[0], 1);
        }
        // step t: the products and update of tile t, then the decay of the state to the end of
        // tile t + 1, whose record has been in LDS since the previous step's barrier
        for (int64_t t = 0; ok && t < ntiles; ++t) {
            bf16x4 Ot[2];
            step(buf[t % NB], t + 1 < ntiles ? &buf[(t + 1) % NB] : nullptr, Ot);
            const int64_t t0 = bos + t * C;
            if (t0 + ln < eos) {
                bf16_t* dst = o + ((t0 + ln) * H + h) * D + 16 * wave + 4 * lg;
                *reinterpret_cast<uint2*>(dst) = as_u2(Ot[0]);
                *reinterpret_cast<uint2*>(dst + 64) = as_u2(Ot[1]);
            }
            lds_barrier();
        }
        ok = ok && *fail == 0;
    } else {
        for (int64_t t = 0; ok && t < ntiles; ++t) {
            if (t + 2 < ntiles) store_share(buf[(t + 2) % NB]);
            if (t + 3 < ntiles) fetch(t + 3, seen);
            if (t + 4 < ntiles && !failed) seen = flag_load<COH>(&ctl->ready[(t + 4) % RING]);
            lds_barrier();
            if (!failed && t + 2 < ntiles && wave == 4 && lane == 0)
                flag_store<COH>(&ctl->consumed, tag | (uint64_t)(t + 3));
            compiler_fence();
        }
        ok = ok && *fail == 0;
    }
    if (!ok && wave == 4 && lane == 0) flag_store<true>(&ctl->status, tag | 1u);
    if (carry && a.hT) {
        const float nan = __builtin_nanf("");
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int mb = 0; mb < 8; ++mb)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    a.hT[sbase + (int64_t)(16 * mb + 4 * lg + r) * D + 16 * (wave + 4 * m) + ln] =
                        ok ? S[m][mb][r] : nan;
    }
}

// Workgroups 0 .. P - 1 are producers (P a multiple of 8; producer b serves the pairs of XCD
// group b % 8, as its k = b / 8-th of m = P / 8), and workgroup P + p is the consumer of pair p,
// on XCD (P + p) % 8 = p % 8.  Producers come first in dispatch order, so every producer a resident
// consumer waits for has been dispatched.  coherent = 1 puts every ring access at system scope
// (the launcher's choice when workgroups are not dealt to XCDs round-robin by index).
__global__ __launch_bounds__(NT) void kda_prefill_pc_kernel(PrefillArgs a, unsigned char* ws,
                                                            uint32_t gen, int64_t spin_limit,
                                                            int coherent, int64_t P) {
    __shared__ __align__(16) unsigned char smem[kSmemBytes];
    __shared__ int fail;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int64_t b = blockIdx.x;
    const uint64_t tag = (uint64_t)gen << 32;
    if (b < P) {
        PWave& L = reinterpret_cast<PWave*>(smem)[wave];
        if (coherent) producer<true>(a, L, wave, lane, b % 8, b / 8, P / 8, ws, tag, spin_limit);
        else producer<false>(a, L, wave, lane, b % 8, b / 8, P / 8, ws, tag, spin_limit);
        return;
    }
    const int64_t p = b - P;
    if (p >= a.N * a.H) return;
    int64_t bos, eos;
    pair_bounds(a, p, bos, eos);
    const int64_t ntiles = (eos - bos + C - 1) / C;
    if (ntiles == 0) {                   // empty sequence: hT = h0 (zeros without h0)
        if (a.hT) {
            const int64_t sbase = p * (int64_t)(D * D);
            for (int e = tid; e < D * D; e += NT) a.hT[sbase + e] = a.h0 ? a.h0[sbase + e] : 0.f;
        }
        return;
    }
    if (tid == 0) fail = 0;
    __syncthreads();
    Rec* buf = reinterpret_cast<Rec*>(smem);
    const Rec* ring = reinterpret_cast<const Rec*>(ws) + p * RING;
    Ctl* ctl = reinterpret_cast<Ctl*>(ws + kRingBytes) + p;
    if (coherent)
        consumer<true>(a, buf, &fail, wave, lane, p, p % a.H, bos, eos, ntiles, ring, ctl, tag,
                       spin_limit);
    else
        consumer<false>(a, buf, &fail, wave, lane, p, p % a.H, bos, eos, ntiles, ring, ctl, tag,
                        spin_limit);
}

// One-time placement check: workgroup b records the XCD it runs on.
__global__ void kda_xcd_probe_kernel(uint32_t* out) {
    if (threadIdx.x == 0) out[blockIdx.x] = xcc_id();
}

// Per device: the workspace address, whether workgroups are dealt to the XCDs round-robin by
// index, the launch tag, and the event that orders launches (they share the workspace): a launch
// on another stream than the previous one waits for it.
struct PcDevice {
    std::mutex mu;
    bool init = false;
    hipError_t err = hipSuccess;
    unsigned char* ws = nullptr;
    bool round_robin = false;
    hipEvent_t done = nullptr;
    hipStream_t last = nullptr;
    bool have_last = false;
    uint32_t gen = 0;
};
constexpr int kMaxDevices = 64;
PcDevice g_pc[kMaxDevices];

bool env_is(const char* name, const char* value) {
    const char* e = std::getenv(name);
    return e && std::strcmp(e, value) == 0;
}

// Launch a 256-workgroup probe (the size of a full launch) and check that workgroup b ran on XCD
// b % 8.  Uses the workspace's ring area as its output (nothing else runs on it yet).
hipError_t check_round_robin(unsigned char* ws, hipStream_t s, bool& rr) {
    constexpr int kProbe = 256;
    uint32_t* out = reinterpret_cast<uint32_t*>(ws);
    hipLaunchKernelGGL(kda_xcd_probe_kernel, dim3(kProbe), dim3(64), 0, s, out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    uint32_t host[kProbe];
    e = hipMemcpyAsync(host, out, sizeof(host), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return e;
    rr = true;
    for (int b = 0; b < kProbe; ++b) rr = rr && host[b] == (uint32_t)(b % 8);
    return hipSuccess;
}

}  // namespace

bool prefill_pc_applicable(const PrefillArgs& a, hipStream_t s) {
    const int64_t pairs = a.N * a.H;
    if (pairs <= 0 || pairs > kMaxPairs || a.snaps || a.split > 1 || !env_is("KDA_PC", "1"))
        return false;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
        return false;   // a captured launch would replay one launch tag (and the ordering event)
    return true;
}

hipError_t launch_prefill_pc(const PrefillArgs& a, hipStream_t s) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    PcDevice& d = g_pc[dev];
    std::lock_guard<std::mutex> lock(d.mu);
    if (!d.init) {
        void* ptr = nullptr;
        d.err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(pc_ws));
        d.ws = static_cast<unsigned char*>(ptr);
        if (d.err == hipSuccess) d.err = hipEventCreateWithFlags(&d.done, hipEventDisableTiming);
        if (d.err == hipSuccess) d.err = check_round_robin(d.ws, s, d.round_robin);
        d.init = true;
    }
    if (d.err != hipSuccess) return d.err;
    if (d.have_last && d.last != s) {
        e = hipStreamWaitEvent(s, d.done, 0);
        if (e != hipSuccess) return e;
    }
    if (++d.gen == 0) d.gen = 1;
    int64_t spin = int64_t{1} << 24;
    if (const char* sl = std::getenv("KDA_PC_SPIN_LIMIT")) spin = std::max<int64_t>(1, std::atoll(sl));
    const int coherent = (!d.round_robin || env_is("KDA_PC_COHERENT", "1")) ? 1 : 0;
    // producers: the CUs the consumers leave free, a multiple of 8, at most four per pair
    const int64_t pairs = a.N * a.H;
    const int64_t P = std::max<int64_t>(8, std::min<int64_t>((256 - pairs) / 8, (4 * pairs + 7) / 8) * 8);
    const unsigned grid = (unsigned)(P + pairs);
    hipLaunchKernelGGL(kda_prefill_pc_kernel, dim3(grid), dim3(NT), 0, s, a, d.ws, d.gen, spin,
                       coherent, P);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = hipEventRecord(d.done, s);
    if (e != hipSuccess) return e;
    d.last = s;
    d.have_last = true;
    return hipSuccess;
}

}  // namespace kda
