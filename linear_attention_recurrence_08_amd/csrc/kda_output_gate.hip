// KDA output stage: the mixer output, normalised per head by its root mean square, times a sigmoid
// gate of full width.
//
// "Kimi K3's hybrid block, from first principles", section "From linear attention to the delta
// rule": the layer's output is RMS-normalised per head and multiplied by a sigmoid gate of the
// token (a full-rank projection, given here as the tensor `gate`) before the output projection.
// Per (token, head) row of dv values:
//     y = o / sqrt(mean(o^2) + eps) * w * sigmoid(gate),     w: a gain per value channel (or 1)
//
// The stage is HBM-bound (three dv-wide rows per (token, head), a few flops per element).  A group
// of 16 lanes owns one row: lane j holds elements 8j .. 8j+7 (one 16-byte access for bf16, two
// for float32), the sum of squares is reduced across the group with four DPP steps, and the
// row is written back once.  Lanes past dv / 8 hold nothing (dv is a multiple of 16, <= 128).
// Each group takes eight rows and issues all their loads before the arithmetic, so every lane
// keeps 256 bytes (bf16) in flight.
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int GROUPS = 16;       // 16-lane row groups per 256-thread block
constexpr int RPG = 8;           // rows per group: all their loads are issued before any math

template <typename Tin>
__global__ __launch_bounds__(256) void kda_output_gate_kernel(GateArgs a) {
    const int tid = threadIdx.x;
    const int j = tid & 15;                                    // lane within the row group
    const int64_t row0 = ((int64_t)blockIdx.x * GROUPS + (tid >> 4)) * RPG;
    const bool lane_on = 8 * j < a.dv;
    float w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = (a.weight && lane_on) ? a.weight[8 * j + i] : 1.f;
    Raw8<Tin> xr[RPG], zr[RPG];
#pragma unroll
    for (int r = 0; r < RPG; ++r) {
        const int64_t row = row0 + r;
        if (row < a.rows && lane_on) {
            xr[r].load(static_cast<const Tin*>(a.o) + row * a.dv + 8 * j);
            zr[r].load(static_cast<const Tin*>(a.gate) + row * a.dv + 8 * j);
        } else {
            xr[r].zero();
            zr[r].zero();
        }
    }
#pragma unroll
    for (int r = 0; r < RPG; ++r) {
        float x[8], z[8];
        xr[r].unpack(x);
        zr[r].unpack(z);
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += x[i] * x[i];
        const float rn = __builtin_amdgcn_rsqf(sum16(ss) / (float)a.dv + a.eps);
        const int64_t row = row0 + r;
        if (row < a.rows && lane_on) {
            float y[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                y[i] = x[i] * rn * w[i] * __builtin_amdgcn_rcpf(1.f + __expf(-z[i]));
            Row8<Tin>::store(static_cast<Tin*>(a.y) + row * a.dv + 8 * j, y);
        }
    }
}

}  // namespace

hipError_t launch_output_gate(const GateArgs& a, hipStream_t s) {
    if (a.rows <= 0) return hipSuccess;
    const int64_t grid = (a.rows + GROUPS * RPG - 1) / (GROUPS * RPG);
    if (a.dtype == 0)
        hipLaunchKernelGGL(kda_output_gate_kernel<bf16_t>, dim3((unsigned)grid), dim3(256), 0, s,
                           a);
    else
        hipLaunchKernelGGL(kda_output_gate_kernel<float>, dim3((unsigned)grid), dim3(256), 0, s,
                           a);
    return hipGetLastError();
}

}  // namespace kda
