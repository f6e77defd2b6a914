// MFMA prefill path (bf16, d = 128, S = 64, causal, seq_q == seq_kv).
#include "hils_common.h"
#include "hils_kernels.h"

namespace hils {

bool prefill_fast_supported(const Geometry&, int) { return false; }
size_t prefill_fast_ws(const Geometry&) { return 0; }
hipError_t launch_prefill_fast(const Geometry&, const void*, const void*, const void*, const void*,
                               const float*, void*, int32_t*, float*, void*, hipStream_t) {
  return hipErrorInvalidConfiguration;
}

}  // namespace hils
