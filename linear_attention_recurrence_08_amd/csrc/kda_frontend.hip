// KDA input stage: turns the projected pre-activations of a token into the recurrence's inputs.
//
// "Kimi K3's hybrid block, from first principles", section "From linear attention to the delta
// rule": queries and keys pass through a short convolution of width 4, Swish and L2 normalisation;
// values through the convolution and Swish; beta is a sigmoid of a projection of the token; the
// decay logit is a low-rank projection plus a per-channel bias, and the log-decay is bounded below
// by g_min with one learned scale A_h per head.  Per (token t, head h, channel c):
//     conv(x)[t,c] = sum_{i<4} w[c,i] x[t-3+i, c]      (causal, depthwise, restarts per sequence
//                                                      from the saved last three inputs or zeros)
//     q = l2(swish(conv(x_q))),  k = l2(swish(conv(x_k))),  v = swish(conv(x_v)),
//     g = g_min * sigmoid(A_h (x_z + bias_c)),  beta = sigmoid(x_b),
// with swish(y) = y sigmoid(y) and l2(y) = y / sqrt(sum_c y_c^2 + eps) over the head's dk values.
//
// The stage is HBM-bound (reads 3 dk + dv values and writes as many per (token, head)).  Three
// kernels run per call, one per kind of tensor (q and k with the L2 norm, v, and z with beta), so
// each executes compact code.  A group of 16 lanes owns a run of 16 consecutive packed tokens
// (8 for float32) of one head; lane j holds channels 8j .. 8j+7, keeps the previous three inputs
// in registers (a sliding window, so every input is read once) and requests all of its run's rows
// before computing the first (16 bytes per token per lane in flight).  A full run inside one
// sequence, the common case, is straight-line code; a run that crosses a sequence start (its
// window restarts there from the saved state) or ends the input goes token by token.  The L2
// norms are 16-lane DPP reductions.  A further kernel writes the saved convolution state (the last
// three inputs of every sequence) after the others have read it, so the state may be updated in
// place.
#include "kda_internal.h"

namespace kda {
namespace {

// tokens per lane group: all of a run's rows are requested before the first is used
template <typename Tin> constexpr int run_of() { return sizeof(Tin) == 2 ? 16 : 8; }
constexpr int GROUPS = 16;       // lane groups per 256-thread block

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

// g = g_min sigmoid(A_h (z + bias)) and beta = sigmoid(x_b): elementwise.  One 16-lane group per
// run of RUN packed tokens of head h; lane j holds channels 8j .. 8j+7 (FULL: dk = 128, every
// lane holds channels).
template <typename Tin, bool FULL>
__global__ __launch_bounds__(256) void kda_frontend_gate_kernel(FrontArgs a) {
    constexpr int RUN = run_of<Tin>();
    const int tid = threadIdx.x;
    const int j = tid & 15;
    const int64_t unit = (int64_t)blockIdx.x * GROUPS + (tid >> 4);
    const int64_t nruns = (a.Ttot + RUN - 1) / RUN;
    if (unit >= nruns * a.H) return;     // whole 16-lane groups leave together
    const int64_t H = a.H, d = a.dk;
    const int64_t h = unit % H, run = unit / H;
    const int64_t t0 = run * RUN, t1 = min(t0 + RUN, a.Ttot);
    const bool on = FULL || 8 * j < d;
    const int64_t c0 = h * d + 8 * j;
    const int64_t tstride = H * d;
    const Tin* xrow = static_cast<const Tin*>(a.xz) + t0 * tstride + c0;
    Tin* orow = static_cast<Tin*>(a.g) + t0 * tstride + c0;
    float zb[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) zb[c] = on ? a.zbias[c0 + c] : 0.f;
    const float Ah = a.A[h];
    Raw8<Tin> rows[RUN];
#pragma unroll
    for (int i = 0; i < RUN; ++i) {
        if (on && t0 + i < t1) rows[i].load(xrow + i * tstride);
        else rows[i].zero();
    }
#pragma unroll
    for (int i = 0; i < RUN; ++i) {
        if (t0 + i >= t1) break;
        float z[8], g8[8];
        rows[i].unpack(z);
#pragma unroll
        for (int c = 0; c < 8; ++c) g8[c] = a.g_min * sigm(Ah * (z[c] + zb[c]));
        if (on) Row8<Tin>::store(orow + i * tstride, g8);
    }
    // beta: lane j of the group takes token t0 + j
    if (t0 + j < t1) {
        const int64_t t = t0 + j;
        const float bl = io<Tin>::load(static_cast<const Tin*>(a.xb) + t * H + h);
        io<Tin>::store(static_cast<Tin*>(a.beta) + t * H + h, sigm(bl));
    }
}

// The convolved tensors: blockIdx.y picks q or k (NORM, with the L2 normalisation) or is v (no
// normalisation).  One 16-lane group per run of RUN packed tokens of head h; lane j holds
// channels 8j .. 8j+7 with their four taps and the previous three inputs (FULL: 128 channels,
// every lane holds channels).
template <typename Tin, bool NORM, bool FULL>
__global__ __launch_bounds__(256) void kda_frontend_conv_kernel(FrontArgs a) {
    constexpr int RUN = run_of<Tin>();
    const int tid = threadIdx.x;
    const int j = tid & 15;
    const int64_t unit = (int64_t)blockIdx.x * GROUPS + (tid >> 4);
    const int64_t nruns = (a.Ttot + RUN - 1) / RUN;
    if (unit >= nruns * a.H) return;     // whole 16-lane groups leave together
    const int kind = NORM ? (int)blockIdx.y : 2;      // 0 = q, 1 = k, 2 = v
    const int64_t H = a.H, Cq = H * a.dk, C = H * (2 * a.dk + a.dv);
    const int64_t d = NORM ? a.dk : a.dv;
    const int64_t h = unit % H, run = unit / H;
    const int64_t t0 = run * RUN, t1 = min(t0 + RUN, a.Ttot);
    const bool on = FULL || 8 * j < d;
    const Tin* x = static_cast<const Tin*>(kind == 0 ? a.xq : kind == 1 ? a.xk : a.xv);
    Tin* out = static_cast<Tin*>(kind == 0 ? a.q : kind == 1 ? a.k : a.v);
    const float* wsrc = kind == 0 ? a.wq : kind == 1 ? a.wk : a.wv;
    const int64_t c0 = h * d + 8 * j;                  // first channel within the tensor
    const int64_t scol = (kind == 0 ? 0 : kind == 1 ? Cq : 2 * Cq) + c0;   // state column
    const int64_t tstride = H * d;                     // elements between consecutive tokens
    const Tin* xrow = x + t0 * tstride + c0;           // this lane's slice of token t0
    Tin* orow = out + t0 * tstride + c0;
    const Tin* cin = static_cast<const Tin*>(a.conv_in);

    Raw8<Tin> rows[RUN];
#pragma unroll
    for (int i = 0; i < RUN; ++i) {
        if (on && t0 + i < t1) rows[i].load(xrow + i * tstride);
        else rows[i].zero();
    }
    float w[8][4];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) w[c][i] = on ? wsrc[(c0 + c) * 4 + i] : 0.f;

    float win[3][8];                    // inputs at t-3, t-2, t-1
    int64_t n = seq_of(a, t0);
    const int64_t bos0 = seq_start(a, n);
    int64_t eos = seq_end(a, n);
    // window of the run's first token: positions t0-bos-3 .. t0-bos-1 of its sequence, the
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
    // one token: convolution over the window and the current input, Swish, the optional L2
    // normalisation, the store; the window slides by one
    auto token = [&](const Raw8<Tin>& row, Tin* dst) {
        float xc[8], y[8], ss = 0.f;
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
        if (NORM) {
            const float r = __builtin_amdgcn_rsqf(sum16(ss) + a.eps);
#pragma unroll
            for (int c = 0; c < 8; ++c) y[c] *= r;
        }
        if (on) Row8<Tin>::store(dst, y);
    };
    if (t1 - t0 == RUN && eos >= t1) {
        // the common case: a full run inside one sequence, straight-line code
#pragma unroll
        for (int i = 0; i < RUN; ++i) token(rows[i], orow + i * tstride);
        return;
    }
    // otherwise (the run crosses a sequence start, or is the last, partial one) token by token,
    // reloading each row
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
        token(row, orow + i * tstride);
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
    const int64_t units = (a.Ttot + run_of<Tin>() - 1) / run_of<Tin>() * a.H;
    const unsigned blocks = (unsigned)((units + GROUPS - 1) / GROUPS);
    hipLaunchKernelGGL((kda_frontend_conv_kernel<Tin, true, FULL>), dim3(blocks, 2), dim3(256), 0,
                       s, a);
    hipLaunchKernelGGL((kda_frontend_conv_kernel<Tin, false, FULL>), dim3(blocks), dim3(256), 0,
                       s, a);
    hipLaunchKernelGGL((kda_frontend_gate_kernel<Tin, FULL>), dim3(blocks), dim3(256), 0, s, a);
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
