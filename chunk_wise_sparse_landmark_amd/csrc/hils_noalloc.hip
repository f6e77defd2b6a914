// Allocation-free decode: hils_decode with its scratch memory (the per-split
// top-K lists and the per-chunk partial outputs) in a fixed device array of
// this library instead of a caller's workspace, for callers that cannot
// allocate device memory (code under graph capture, tight serving loops).
#include <hip/hip_runtime.h>

#include <mutex>

#include "hils.h"

namespace {

constexpr size_t kScratchBytes = (size_t)16 << 20;     // HILS_NOALLOC_SCRATCH_BYTES
constexpr int kMaxDevices = 64;

// One copy per GPU, alive until the process ends.  Host code never uses this
// name as an address: each device's copy is reached through the pointer that
// hipGetSymbolAddress returns on that device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The calling thread's current device's copy of `scratch` (looked up once per
// device, with that device current); null on failure.
void* device_scratch(hipError_t* err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

namespace hils {
// hils_decode itself, with the workspace passed in (defined with the other
// entry points; internal to the library)
hils_status decode_with_scratch(const hils_params* p, const void* q, const void* q_ret,
                                const void* k, const void* v, const void* lmk,
                                const float* lmk_bias, void* out, int32_t* sel_idx, float* lse,
                                void* ws, size_t ws_bytes, size_t ws_limit, void* stream);
}  // namespace hils

extern "C" size_t hils_decode_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" hils_status hils_decode_noalloc(const hils_params* p, const void* q, const void* q_ret,
                                           const void* k, const void* v, const void* lmk,
                                           const float* lmk_bias, void* out, int32_t* sel_idx,
                                           float* lse, void* stream) {
  hipError_t err = hipSuccess;
  void* ws = device_scratch(&err);
  return hils::decode_with_scratch(p, q, q_ret, k, v, lmk, lmk_bias, out, sel_idx, lse, ws,
                                   ws ? kScratchBytes : 0, kScratchBytes, stream);
}
