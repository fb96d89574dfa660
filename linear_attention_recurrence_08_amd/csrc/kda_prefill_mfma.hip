// KDA chunkwise prefill, matrix-core path (bf16, dk = dv = 128).  Placeholder: routes to the
// general tile path until the MFMA kernel lands.
#include "kda_internal.h"

namespace kda {

hipError_t launch_prefill_mfma(const PrefillArgs& a, hipStream_t s) {
    return launch_prefill_general(a, s);
}

}  // namespace kda
