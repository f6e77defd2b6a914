// Small service kernels of the C ABI: the backward's copy of a caller-supplied
// selection with every id it must not use blanked out, and a zero fill (a kernel
// rather than a memset, so that a caller may capture the calls in a graph).
#include "hils_common.h"
#include "hils_kernels.h"

namespace hils {

namespace {

constexpr int kThreads = 256;

// One thread per selection entry (b, kv head, query, slot): the id is kept only
// when it is a candidate of that query (a complete chunk before its local
// window, [0, ncand)) and no earlier slot of the row holds it; anything else
// becomes -1, which every backward kernel skips.  Positions are kept (a blanked
// slot stays where it was).  The earlier slots of a row are the same cache lines
// the neighbouring threads read.
__global__ void __launch_bounds__(kThreads)
sanitize_selection(Geometry g, const int32_t* __restrict__ in, int32_t* __restrict__ out,
                   long long nent) {
  const long long e = (long long)blockIdx.x * kThreads + threadIdx.x;
  if (e >= nent) return;
  const long long r = e / g.K;
  const int s = (int)(e - r * g.K);
  const int i = (int)(r % g.Lq);
  int ncand, own, own_b;
  g.layout(i, ncand, own, own_b);
  const int32_t* src = in + r * g.K;
  const int c = src[s];
  bool keep = c >= 0 && c < ncand;
  for (int t = 0; t < s && keep; ++t) keep = src[t] != c;
  out[e] = keep ? c : -1;
}

__global__ void __launch_bounds__(kThreads)
zero_fill(uint4* __restrict__ p16, size_t n16, unsigned char* __restrict__ tail, int ntail) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  for (size_t x = (size_t)blockIdx.x * kThreads + threadIdx.x; x < n16; x += stride)
    p16[x] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

}  // namespace

size_t sanitized_selection_bytes(const Geometry& g) {
  return (size_t)g.B * g.Hkv * g.Lq * g.K * sizeof(int32_t);
}

hipError_t launch_sanitize_selection(const Geometry& g, const int32_t* in, int32_t* out,
                                     hipStream_t st) {
  const long long nent = (long long)g.B * g.Hkv * g.Lq * g.K;
  if (nent == 0) return hipSuccess;
  const unsigned nb = (unsigned)((nent + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(sanitize_selection, dim3(nb), dim3(kThreads), 0, st, g, in, out, nent);
  return hipGetLastError();
}

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t st) {
  if (!p || bytes == 0) return hipSuccess;
  const size_t n16 = bytes / 16;
  const int ntail = (int)(bytes % 16);
  const size_t want = (n16 + kThreads - 1) / kThreads;
  const unsigned nb = (unsigned)(want < 4096 ? (want > 0 ? want : 1) : 4096);
  hipLaunchKernelGGL(zero_fill, dim3(nb), dim3(kThreads), 0, st, (uint4*)p, n16,
                     (unsigned char*)p + n16 * 16, ntail);
  return hipGetLastError();
}

}  // namespace hils
