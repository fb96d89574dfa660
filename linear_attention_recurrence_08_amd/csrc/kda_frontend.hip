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
// The stage is HBM-bound (reads 3 dk + dv values and writes as many per (token, head)).  A group
// of 16 lanes owns a run of 16 consecutive packed tokens of one head; lane j holds channels
// 8j .. 8j+7 of q, k, v and z, keeps the previous three inputs of q, k and v in registers (a
// sliding window, so every input is read once) and restarts the window at each sequence start
// inside the run.  The L2 norms are 16-lane xor reductions.  A second kernel writes the saved
// convolution state (the last three inputs of every sequence) after the first has read it, so the
// state may be updated in place.
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int RUN = 16;          // tokens per lane group
constexpr int GROUPS = 16;       // lane groups per 256-thread block

__device__ __forceinline__ float sigm(float x) { return 1.f / (1.f + __expf(-x)); }

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

template <typename Tin>
struct Window {                  // inputs at tokens t-3, t-2, t-1 for this lane's 8 channels
    float w[3][8];
};

template <typename Tin>
__global__ __launch_bounds__(256) void kda_frontend_kernel(FrontArgs a) {
    const int tid = threadIdx.x;
    const int j = tid & 15;
    const int64_t unit = (int64_t)blockIdx.x * GROUPS + (tid >> 4);
    const int64_t nruns = (a.Ttot + RUN - 1) / RUN;
    if (unit >= nruns * a.H) return;     // whole 16-lane groups leave together
    const int64_t h = unit % a.H, run = unit / a.H;
    const int64_t t0 = run * RUN, t1 = min(t0 + RUN, a.Ttot);
    const int64_t H = a.H, dk = a.dk, dv = a.dv;
    const bool onk = 8 * j < dk, onv = 8 * j < dv;
    const int64_t Cq = H * dk, C = H * (2 * dk + dv);
    const int64_t cq = h * dk + 8 * j, cv = h * dv + 8 * j;     // this lane's first channel

    // taps of this lane's channels
    float wq[8][4], wk[8][4], wv[8][4], zb[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            wq[c][i] = onk ? a.wq[(cq + c) * 4 + i] : 0.f;
            wk[c][i] = onk ? a.wk[(cq + c) * 4 + i] : 0.f;
            wv[c][i] = onv ? a.wv[(cv + c) * 4 + i] : 0.f;
        }
        zb[c] = onk ? a.zbias[cq + c] : 0.f;
    }
    const float Ah = a.A[h];
    const Tin* xq = static_cast<const Tin*>(a.xq);
    const Tin* xk = static_cast<const Tin*>(a.xk);
    const Tin* xv = static_cast<const Tin*>(a.xv);
    const Tin* xz = static_cast<const Tin*>(a.xz);
    const Tin* cin = static_cast<const Tin*>(a.conv_in);

    Window<Tin> Wq, Wk, Wv;
    int64_t n = seq_of(a, t0);
    int64_t bos = seq_start(a, n), eos = seq_end(a, n);
    // value at position p (from -3) of sequence n's input for this lane's channels
    auto fill = [&](int slot, int64_t p) {
        float tq[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, tk[8], tv[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) { tk[c] = 0.f; tv[c] = 0.f; }
        if (p >= 0) {
            const int64_t t = bos + p;
            if (onk) {
                Row8<Tin>::load(xq + (t * H + h) * dk + 8 * j, tq);
                Row8<Tin>::load(xk + (t * H + h) * dk + 8 * j, tk);
            }
            if (onv) Row8<Tin>::load(xv + (t * H + h) * dv + 8 * j, tv);
        } else if (cin) {
            const Tin* row = cin + (n * 3 + (3 + p)) * C;
            if (onk) {
                Row8<Tin>::load(row + cq, tq);
                Row8<Tin>::load(row + Cq + cq, tk);
            }
            if (onv) Row8<Tin>::load(row + 2 * Cq + cv, tv);
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            Wq.w[slot][c] = tq[c];
            Wk.w[slot][c] = tk[c];
            Wv.w[slot][c] = tv[c];
        }
    };
    auto restart = [&](int64_t t) {      // window for token t of sequence n
        const int64_t p = t - bos;
        fill(0, p - 3);
        fill(1, p - 2);
        fill(2, p - 1);
    };
    restart(t0);

    Tin* oq = static_cast<Tin*>(a.q);
    Tin* ok = static_cast<Tin*>(a.k);
    Tin* ov = static_cast<Tin*>(a.v);
    Tin* og = static_cast<Tin*>(a.g);
    for (int64_t t = t0; t < t1; ++t) {
        if (t >= eos) {                  // the run crosses into a later sequence
            do { ++n; } while (seq_end(a, n) <= t);
            bos = seq_start(a, n);
            eos = seq_end(a, n);
            restart(t);
        }
        float xq8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, xk8[8], xv8[8], xz8[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) { xk8[c] = 0.f; xv8[c] = 0.f; xz8[c] = 0.f; }
        const int64_t rk = (t * H + h) * dk + 8 * j, rv = (t * H + h) * dv + 8 * j;
        if (onk) {
            Row8<Tin>::load(xq + rk, xq8);
            Row8<Tin>::load(xk + rk, xk8);
            Row8<Tin>::load(xz + rk, xz8);
        }
        if (onv) Row8<Tin>::load(xv + rv, xv8);
        float q8[8], k8[8], v8[8], g8[8], sq = 0.f, sk = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float yq = wq[c][3] * xq8[c], yk = wk[c][3] * xk8[c], yv = wv[c][3] * xv8[c];
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                yq += wq[c][i] * Wq.w[i][c];
                yk += wk[c][i] * Wk.w[i][c];
                yv += wv[c][i] * Wv.w[i][c];
            }
            q8[c] = yq * sigm(yq);
            k8[c] = yk * sigm(yk);
            v8[c] = yv * sigm(yv);
            g8[c] = a.g_min * sigm(Ah * (xz8[c] + zb[c]));
            sq += q8[c] * q8[c];
            sk += k8[c] * k8[c];
            // slide the window
            Wq.w[0][c] = Wq.w[1][c]; Wq.w[1][c] = Wq.w[2][c]; Wq.w[2][c] = xq8[c];
            Wk.w[0][c] = Wk.w[1][c]; Wk.w[1][c] = Wk.w[2][c]; Wk.w[2][c] = xk8[c];
            Wv.w[0][c] = Wv.w[1][c]; Wv.w[1][c] = Wv.w[2][c]; Wv.w[2][c] = xv8[c];
        }
#pragma unroll
        for (int m = 8; m >= 1; m >>= 1) {
            sq += __shfl_xor(sq, m, 16);
            sk += __shfl_xor(sk, m, 16);
        }
        const float rq = rsqrtf(sq + a.eps), rkn = rsqrtf(sk + a.eps);
#pragma unroll
        for (int c = 0; c < 8; ++c) { q8[c] *= rq; k8[c] *= rkn; }
        if (onk) {
            Row8<Tin>::store(oq + rk, q8);
            Row8<Tin>::store(ok + rk, k8);
            Row8<Tin>::store(og + rk, g8);
        }
        if (onv) Row8<Tin>::store(ov + rv, v8);
        if (j == 0) {
            const float b = io<Tin>::load(static_cast<const Tin*>(a.xb) + t * H + h);
            io<Tin>::store(static_cast<Tin*>(a.beta) + t * H + h, sigm(b));
        }
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

}  // namespace

hipError_t launch_frontend(const FrontArgs& a, hipStream_t s) {
    if (a.Ttot > 0) {
        const int64_t units = (a.Ttot + RUN - 1) / RUN * a.H;
        const dim3 grid((unsigned)((units + GROUPS - 1) / GROUPS));
        if (a.dtype == 0) hipLaunchKernelGGL(kda_frontend_kernel<bf16_t>, grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL(kda_frontend_kernel<float>, grid, dim3(256), 0, s, a);
        const hipError_t e = hipGetLastError();
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
