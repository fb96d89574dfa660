// kda_chunk_fwd_split_noalloc: the token-range split prefill with its workspace in a static
// device array of the library instead of a caller buffer, for callers that cannot allocate
// (code under stream capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array lives in this file's code object; each GPU the library runs on holds its own copy
// until the process ends.  Its device address comes from hipGetSymbolAddress, taken once per
// device on the first call made with that device current and kept per device; host code uses
// only that address (the array's name is a host-side stand-in).  The split's kernels write every
// workspace record before they read it, so nothing needs clearing between calls.  Every call on
// one GPU shares that GPU's array: calls that overlap on one GPU (two streams, two threads) race.
#include "kda.h"

#include <hip/hip_runtime.h>

#include <mutex>

namespace {

constexpr size_t kScratchBytes = size_t{32} << 20;   // 32 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// The device address of the current device's scratch array, or nullptr.
void* scratch_ptr() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::call_once(g_scratch_once[dev], [dev]() {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = p;
    });
    return g_scratch_err[dev] == hipSuccess ? g_scratch_ptr[dev] : nullptr;
}

}  // namespace

extern "C" int kda_chunk_fwd_split_noalloc(const void* q, const void* k, const void* v,
                                           const void* g, const void* beta, const float* h0,
                                           const int32_t* cu_seqlens, int num_seqs,
                                           int max_seqlen, void* o, float* hT, int B, int T,
                                           int H, int dk, int dv, int dtype, int segments,
                                           void* stream) {
    void* ws = scratch_ptr();
    if (!ws) return KDA_ERR_HIP;
    // the scratch is never NULL and is 256-byte aligned, so a workspace refusal means the call
    // needs more than the array holds
    const int st = kda_chunk_fwd_split(q, k, v, g, beta, h0, cu_seqlens, num_seqs, max_seqlen, o,
                                       hT, B, T, H, dk, dv, dtype, segments, ws, kScratchBytes,
                                       stream);
    return st == KDA_ERR_WORKSPACE ? KDA_ERR_SCRATCH : st;
}
