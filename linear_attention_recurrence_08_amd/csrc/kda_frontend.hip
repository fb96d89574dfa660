// KDA input stage: turns the projected pre-activations of a token into the recurrence's inputs.
//
// "Kimi K3's hybrid block, from first principles", section "From linear attention to the delta
// rule": q and k get a four-tap causal convolution, the Swish activation and unit-length
// normalisation, v the convolution and Swish only; beta comes from a sigmoid over a projection of
// the token; the decay logit is a low-rank projection with a bias per channel, and the log-decay
// has the floor g_min and one learned scale A_h per head.  Per (token t, head h, channel c):
//     conv(x)[t,c] = sum_{i<4} w[c,i] x[t-3+i, c]      (causal, depthwise, restarts per sequence
//                                                      from the saved last three inputs or zeros)
//     q = l2(swish(conv(x_q))),  k = l2(swish(conv(x_k))),  v = swish(conv(x_v)),
//     g = g_min * sigmoid(A_h (x_z + bias_c)),  beta = sigmoid(x_b),
// with swish(y) = y sigmoid(y) and l2(y) = y / sqrt(sum_c y_c^2 + eps) over the head's dk values.
//
// The stage is HBM-bound (reads 3 dk + dv values and writes as many per (token, head)).  One
// launch streams all four tensors (blockIdx.y: q, k, v, z), a second writes the saved
// convolution state.  A group of 16 lanes owns a chunk of 32 consecutive packed tokens of one
// head; lane j holds channels 8j .. 8j+7 and, for the convolved tensors, keeps the previous three
// inputs in registers (a sliding window, so every input is read once).  The four groups of a
// wave take four consecutive chunks of one head, so their rows are addressed through one
// wave-uniform buffer resource.  A chunk inside one sequence, the common case, streams through
// two register sets of a few tokens each, the next set's rows in flight while the current one is
// computed; a chunk that crosses a sequence start (its window restarts there from the saved
// state) or ends the input goes token by token.  The L2 norms are 16-lane DPP reductions.  The
// state kernel writes the last three inputs of every sequence after the first kernel has read
// the saved state, so the state may be updated in place.
#include "kda_internal.h"

namespace kda {
namespace {

// logistic sigmoid with the hardware reciprocal (v_rcp_f32, 1 ulp)
__device__ __forceinline__ float sigm(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

// index of the sequence holding packed token t: the last n with cu[n] <= t (skips empty ones)
__device__ __forceinline__ int64_t seq_of(const FrontArgs& a, int64_t t) {
    if (!a.cu) return t / a.T;
    int64_t lo = 0, hi = a.N;            // cu[lo] <= t < cu[hi]
    while (hi - lo > 1) {
        const int64_t mid = (lo + hi) >> 1;
        if (a.cu[mid] <= t) lo = mid; else hi = mid;
    }
    return lo;
}
__device__ __forceinline__ int64_t seq_start(const FrontArgs& a, int64_t n) {
    return a.cu ? (int64_t)a.cu[n] : n * a.T;
}
__device__ __forceinline__ int64_t seq_end(const FrontArgs& a, int64_t n) {
    return a.cu ? (int64_t)a.cu[n + 1] : (n + 1) * a.T;
}

// The convolved tensors: blockIdx.y picks q, k (both with the L2 normalisation) or v (without).
// One 16-lane group per chunk of CONV_CHUNK packed tokens of head h; lane j holds
// channels 8j .. 8j+7 with their four taps and the previous three inputs (FULL: 128 channels,
// every lane holds channels).  The four groups of a wave take four consecutive chunks of one head,
// so a wave-uniform buffer resource addresses their rows (the row offset is a scalar; each lane
// keeps one 32-bit offset).  A chunk inside one sequence streams through two register sets of
// SUB tokens each: the rows of the next sub-run are in flight while the current one is computed.
template <typename Tin> constexpr int sub_of() { return sizeof(Tin) == 2 ? 8 : 4; }
constexpr int CONV_CHUNK = 32;
constexpr int kBufNT = 2;                    // buffer cache policy: non-temporal (streaming)

// eight consecutive elements through a buffer resource: one 16-byte access for bf16, two for f32.
// Loads take the row offset as the scalar offset; stores fold it into the lane offset and pass a
// zero scalar offset.  With the row offset in a scalar register, the compiler let the next vector
// instruction overwrite a 16-byte store's data registers right after the store, and the outputs
// of the last four lanes of every 16-lane row came out corrupted, differently from run to run.
// With a zero scalar offset it leaves the store its wait states, and the outputs are those of the
// earlier form (whose per-access loops kept the two apart).
template <typename Tin> struct BufRow;
template <> struct BufRow<bf16_t> {
    static __device__ __forceinline__ void load(Raw8<bf16_t>& r, __amdgpu_buffer_rsrc_t rs,
                                                uint32_t voff, uint32_t soff) {
        r.u = __builtin_bit_cast(u32v4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff,
                                                                              kBufNT));
    }
    static __device__ __forceinline__ void store(const float y[8], __amdgpu_buffer_rsrc_t rs,
                                                 uint32_t voff, uint32_t soff) {
        const u32v4 u = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                         pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32v4, u), rs, voff + soff, 0,
                                               kBufNT);
    }
};
template <> struct BufRow<float> {
    static __device__ __forceinline__ void load(Raw8<float>& r, __amdgpu_buffer_rsrc_t rs,
                                                uint32_t voff, uint32_t soff) {
        r.a = __builtin_bit_cast(f32v4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff,
                                                                              kBufNT));
        r.b = __builtin_bit_cast(f32v4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff + 16, soff,
                                                                              kBufNT));
    }
    static __device__ __forceinline__ void store(const float y[8], __amdgpu_buffer_rsrc_t rs,
                                                 uint32_t voff, uint32_t soff) {
        const f32v4 lo = {y[0], y[1], y[2], y[3]}, hi = {y[4], y[5], y[6], y[7]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32v4, lo), rs, voff + soff, 0,
                                               kBufNT);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32v4, hi), rs,
                                               voff + soff + 16, 0, kBufNT);
    }
};

template <typename Tin, bool FULL>
__global__ __launch_bounds__(256) void kda_frontend_conv_kernel(FrontArgs a) {
    constexpr int SUB = sub_of<Tin>();
    constexpr int NSUB = CONV_CHUNK / SUB;
    const int tid = threadIdx.x;
    const int j = tid & 15, grp = (tid >> 4) & 3;
    const int64_t H = a.H;
    const int64_t nchunks = (a.Ttot + CONV_CHUNK - 1) / CONV_CHUNK;
    // wave: one head, four chunks.  The wave index goes through readfirstlane so that the
    // compiler sees it (and the buffer resources built from it) as uniform; otherwise it keeps
    // the resources in vector registers and wraps every buffer access in a readfirstlane loop.
    const int64_t wv = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t h = wv % H, chunk0 = (wv / H) * 4;
    if (chunk0 >= nchunks) return;                              // the whole wave leaves
    const int64_t chunk = chunk0 + grp;
    if (chunk >= nchunks) return;                               // whole 16-lane groups leave
    const int kind = (int)blockIdx.y;                  // 0 = q, 1 = k, 2 = v, 3 = z (gates)
    const bool norm = kind < 2;                        // uniform per block
    const int64_t Cq = H * a.dk, C = H * (2 * a.dk + a.dv);
    const int64_t d = kind == 2 ? a.dv : a.dk;
    const int64_t t0 = chunk * CONV_CHUNK, t1 = min(t0 + CONV_CHUNK, a.Ttot);
    const bool on = FULL || 8 * j < d;
    const Tin* x = static_cast<const Tin*>(kind == 0 ? a.xq : kind == 1 ? a.xk :
                                           kind == 2 ? a.xv : a.xz);
    Tin* out = static_cast<Tin*>(kind == 0 ? a.q : kind == 1 ? a.k : kind == 2 ? a.v : a.g);
    const int64_t c0 = h * d + 8 * j;                  // first channel within the tensor
    const int64_t tstride = H * d;                     // elements between consecutive tokens
    const Tin* xrow = x + t0 * tstride + c0;           // this lane's slice of token t0
    Tin* orow = out + t0 * tstride + c0;

    // buffer resources over the wave's four chunks of head h (wave-uniform bases); a lane's
    // offset is its chunk's start plus its channels, a row's offset a scalar
    const int64_t wbase = chunk0 * CONV_CHUNK * tstride + h * d;        // elements
    // records: the wave's four chunks, cut at the end of the tensor
    const int64_t wlen = min(4 * CONV_CHUNK * tstride, a.Ttot * tstride - wbase);
    const uint32_t nrec = (uint32_t)(wlen * (int64_t)sizeof(Tin));
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(x + wbase), (short)0, (int)nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(out + wbase), (short)0, (int)nrec, 0x00020000);
    const uint32_t voff = (uint32_t)(((int64_t)grp * CONV_CHUNK * tstride + 8 * j) *
                                     (int64_t)sizeof(Tin));
    const uint32_t rowb = (uint32_t)(tstride * (int64_t)sizeof(Tin));  // bytes per token

    Raw8<Tin> ra[SUB], rb[SUB];
    auto load_sub = [&](Raw8<Tin> (&r)[SUB], int sub) {
#pragma unroll
        for (int i = 0; i < SUB; ++i) {
            if (on) BufRow<Tin>::load(r[i], rx, voff, (uint32_t)(sub * SUB + i) * rowb);
            else r[i].zero();
        }
    };
    // streams a whole chunk through the two register sets (the next sub-run's rows in flight
    // while the current one is computed); f(row, y) makes a token's output row
    auto stream_chunk = [&](auto&& f) {
        load_sub(ra, 0);
        load_sub(rb, 1);
        auto run_sub = [&](const Raw8<Tin> (&r)[SUB], int sub) {
#pragma unroll
            for (int i = 0; i < SUB; ++i) {
                float y[8];
                f(r[i], y);
                if (on) BufRow<Tin>::store(y, ro, voff, (uint32_t)(sub * SUB + i) * rowb);
            }
        };
#pragma unroll 1
        for (int sub = 0; sub < NSUB; sub += 2) {
            run_sub(ra, sub);
            if (sub + 2 < NSUB) load_sub(ra, sub + 2);
            run_sub(rb, sub + 1);
            if (sub + 3 < NSUB) load_sub(rb, sub + 3);
        }
    };

    if (kind == 3) {
        // g = g_min sigmoid(A_h (z + bias)), elementwise; beta = sigmoid(x_b)
        float zb[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) zb[c] = on ? a.zbias[c0 + c] : 0.f;
        const float Ah = a.A[h];
        auto gate = [&](const Raw8<Tin>& row, float y[8]) {
            float z[8];
            row.unpack(z);
#pragma unroll
            for (int c = 0; c < 8; ++c) y[c] = a.g_min * sigm(Ah * (z[c] + zb[c]));
        };
        if (t1 - t0 == CONV_CHUNK) {
            stream_chunk(gate);
        } else {
#pragma unroll 1
            for (int i = 0; i < (int)(t1 - t0); ++i) {
                Raw8<Tin> row;
                if (on) row.load(xrow + i * tstride);
                else row.zero();
                float y[8];
                gate(row, y);
                if (on) Row8<Tin>::store(orow + i * tstride, y);
            }
        }
        // lane j of the group takes tokens t0 + j, t0 + j + 16, ...
        for (int64_t t = t0 + j; t < t1; t += 16) {
            const float bl = io<Tin>::load(static_cast<const Tin*>(a.xb) + t * H + h);
            io<Tin>::store(static_cast<Tin*>(a.beta) + t * H + h, sigm(bl));
        }
        return;
    }

    const float* wsrc = kind == 0 ? a.wq : kind == 1 ? a.wk : a.wv;
    const int64_t scol = (kind == 0 ? 0 : kind == 1 ? Cq : 2 * Cq) + c0;   // state column
    const Tin* cin = static_cast<const Tin*>(a.conv_in);
    int64_t n = seq_of(a, t0);
    const int64_t bos0 = seq_start(a, n);
    int64_t eos = seq_end(a, n);
    const bool fast = t1 - t0 == CONV_CHUNK && eos >= t1;   // a whole chunk inside one sequence

    float w[8][4];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) w[c][i] = on ? wsrc[(c0 + c) * 4 + i] : 0.f;

    float win[3][8];                    // inputs at t-3, t-2, t-1
    // window of the chunk's first token: positions t0-bos-3 .. t0-bos-1 of its sequence, the
    // negative ones from the saved state (or zeros)
#pragma unroll
    for (int s = 0; s < 3; ++s) {
        const int64_t p = t0 - bos0 - 3 + s;
        float v8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (on) {
            if (p >= 0) Row8<Tin>::load(xrow + (s - 3) * tstride, v8);
            else if (cin) Row8<Tin>::load(cin + (n * 3 + (3 + p)) * C + scol, v8);
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) win[s][c] = v8[c];
    }
    // one token: convolution over the window and the current input, Swish, the L2 normalisation
    // for q and k; the window slides by one
    auto token = [&](const Raw8<Tin>& row, float y[8]) {
        float xc[8], ss = 0.f;
        row.unpack(xc);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float u = w[c][0] * win[0][c] + w[c][1] * win[1][c] + w[c][2] * win[2][c] +
                            w[c][3] * xc[c];
            y[c] = u * sigm(u);
            ss += y[c] * y[c];
            win[0][c] = win[1][c];
            win[1][c] = win[2][c];
            win[2][c] = xc[c];
        }
        if (norm) {
            const float r = __builtin_amdgcn_rsqf(sum16(ss) + a.eps);
#pragma unroll
            for (int c = 0; c < 8; ++c) y[c] *= r;
        }
    };
    if (fast) {
        stream_chunk(token);
        return;
    }
    // otherwise (the chunk crosses a sequence start, or is the last, partial one) token by token
#pragma unroll 1
    for (int i = 0; i < (int)(t1 - t0); ++i) {
        const int64_t t = t0 + i;
        if (t >= eos) {
            // a later sequence starts at token t (empty sequences skipped): its window is the
            // saved state (or zeros)
            do { ++n; } while (seq_end(a, n) <= t);
            eos = seq_end(a, n);
#pragma unroll
            for (int s = 0; s < 3; ++s) {
                float v8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                if (on && cin) Row8<Tin>::load(cin + (n * 3 + s) * C + scol, v8);
#pragma unroll
                for (int c = 0; c < 8; ++c) win[s][c] = v8[c];
            }
        }
        Raw8<Tin> row;
        if (on) row.load(xrow + i * tstride);
        else row.zero();
        float y[8];
        token(row, y);
        if (on) Row8<Tin>::store(orow + i * tstride, y);
    }
}

// conv_out[n, i, :] = input row (len_n - 3 + i) of sequence n, where rows -3 .. -1 are the saved
// state conv_in[n] (or zeros); one thread per (sequence, channel), reading all three rows before
// writing, so conv_out may alias conv_in.
template <typename Tin>
__global__ __launch_bounds__(256) void kda_frontend_state_kernel(FrontArgs a) {
    const int64_t H = a.H, dk = a.dk, dv = a.dv, Cq = H * dk, C = H * (2 * dk + dv);
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t n = blockIdx.y;
    if (c >= C) return;
    const int64_t bos = seq_start(a, n), len = seq_end(a, n) - bos;
    const Tin* cin = static_cast<const Tin*>(a.conv_in);
    float r[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int64_t p = len - 3 + i;
        if (p >= 0) {
            const int64_t t = bos + p;
            if (c < Cq) r[i] = io<Tin>::load(static_cast<const Tin*>(a.xq) + t * Cq + c);
            else if (c < 2 * Cq) r[i] = io<Tin>::load(static_cast<const Tin*>(a.xk) + t * Cq + c - Cq);
            else r[i] = io<Tin>::load(static_cast<const Tin*>(a.xv) + t * H * dv + c - 2 * Cq);
        } else {
            r[i] = cin ? io<Tin>::load(cin + (n * 3 + (3 + p)) * C + c) : 0.f;
        }
    }
    Tin* out = static_cast<Tin*>(a.conv_out);
#pragma unroll
    for (int i = 0; i < 3; ++i) io<Tin>::store(out + (n * 3 + i) * C + c, r[i]);
}

template <typename Tin, bool FULL>
hipError_t launch_frontend_t(const FrontArgs& a, hipStream_t s) {
    // conv kernels: a wave per (head, four consecutive chunks), four waves per block
    const int64_t waves = (a.Ttot + 4 * CONV_CHUNK - 1) / (4 * CONV_CHUNK) * a.H;
    const unsigned cblocks = (unsigned)((waves + 3) / 4);
    hipLaunchKernelGGL((kda_frontend_conv_kernel<Tin, FULL>), dim3(cblocks, 4), dim3(256), 0, s,
                       a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_frontend(const FrontArgs& a, hipStream_t s) {
    if (a.Ttot > 0) {
        // every lane of a 16-lane group holds 8 channels when both head sizes are 128
        const bool full = a.dk == 128 && a.dv == 128;
        const hipError_t e = a.dtype == 0
            ? (full ? launch_frontend_t<bf16_t, true>(a, s) : launch_frontend_t<bf16_t, false>(a, s))
            : (full ? launch_frontend_t<float, true>(a, s) : launch_frontend_t<float, false>(a, s));
        if (e != hipSuccess) return e;
    }
    if (a.conv_out && a.N > 0) {
        const int64_t C = a.H * (2 * a.dk + a.dv);
        const dim3 grid((unsigned)((C + 255) / 256), (unsigned)a.N);
        if (a.dtype == 0)
            hipLaunchKernelGGL(kda_frontend_state_kernel<bf16_t>, grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL(kda_frontend_state_kernel<float>, grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace kda
