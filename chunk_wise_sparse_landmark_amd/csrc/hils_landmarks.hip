// Landmark formation: the step before retrieval scoring.
//
// Method: Hierarchical Sparse Attention Done Right (arXiv 2607.02980v1, summary
// page), §3 "Linear surrogate for chunk mass": a landmark query lq_c appended to
// chunk c induces a distribution over the chunk's keys; the weighted key sum is
// the chunk's compact summary (landmark key) and an entropy term the bias.  For
// chunk c with keys k_j (j < S):
//   l_j = scale <lq_c, k_j>,  p = softmax(l),
//   lmk_c = sum_j p_j k_j,  bias_c = -sum_j p_j log p_j = m + log z - sum_j p_j l_j
// (m = max l, z = sum e^{l - m}), i.e. the first-order Taylor expansion of the
// chunk's LogSumExp at lq_c.  Backward, with dp_j = <dlmk, k_j> - dbias (log p_j + 1):
//   dl_j = p_j (dp_j - sum_i p_i dp_i),  dlq = scale sum_j dl_j k_j,
//   dk_j = scale dl_j lq_c + p_j dlmk_c.
//
// One workgroup per (b, kv head, chunk): the chunk's S x d keys are staged in
// LDS as fp32 (row stride d + 1: conflict-free column and row reads), one thread
// per key forms its logit, block reductions give the softmax, and one thread per
// dimension forms the weighted sums.  HBM-bound (each key is read once).
#include "hils_common.h"
#include "hils_kernels.h"
#include "hils_profile.h"

namespace hils {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxElems = 16384;   // S * d bound (64 KB of fp32 keys in LDS)

template <typename T>
__device__ __forceinline__ void stage_keys(const T* __restrict__ kc, int S, int d, float* ks) {
  for (int e = threadIdx.x; e < S * d; e += kThreads) ks[(e / d) * (d + 1) + e % d] = Elem<T>::ld(kc + e);
}

// logits of the chunk's keys (thread j < S), softmax statistics; returns p_j in
// pl[j] and l_j in ll[j]; m, log z via the block reductions
template <typename T>
__device__ __forceinline__ void chunk_softmax(const float* ks, const float* qs, int S, int d,
                                              float scale, float* ll, float* pl, float* red,
                                              float& m_out, float& logz_out) {
  const int tid = threadIdx.x;
  float l = -INFINITY;
  if (tid < S) {
    float acc = 0.f;
    const float* row = ks + tid * (d + 1);
    for (int x = 0; x < d; ++x) acc = __builtin_fmaf(qs[x], row[x], acc);
    l = scale * acc;
  }
  const float m = block_max4(l, red);
  const float e = tid < S ? expf(l - m) : 0.f;
  const float z = block_sum4(e, red);
  if (tid < S) {
    pl[tid] = e / z;
    ll[tid] = l;
  }
  m_out = m;
  logz_out = logf(z);
  __syncthreads();
}

template <typename T>
__global__ void __launch_bounds__(kThreads)
landmark_forward_kernel(Geometry g, const T* __restrict__ lq, const T* __restrict__ k,
                        T* __restrict__ lmk, float* __restrict__ bias) {
  extern __shared__ float lm_smem[];
  const int S = g.S, d = g.d;
  float* ks = lm_smem;                       // S x (d + 1)
  float* qs = ks + S * (d + 1);              // d
  float* ll = qs + d;                        // S
  float* pl = ll + S;                        // S
  float* red = pl + S;                       // 4
  const int c = blockIdx.x, bkv = blockIdx.y;
  const int tid = threadIdx.x;
  T* orow = lmk + ((size_t)bkv * g.NCcap + c) * d;
  if (c >= g.NC) {                           // landmark rows past the complete chunks: 0
    for (int x = tid; x < d; x += kThreads) Elem<T>::st(orow + x, 0.f);
    if (tid == 0 && bias) bias[(size_t)bkv * g.NCcap + c] = 0.f;
    return;
  }
  stage_keys(k + ((size_t)bkv * g.Lkv + (size_t)c * S) * d, S, d, ks);
  for (int x = tid; x < d; x += kThreads) qs[x] = Elem<T>::ld(lq + ((size_t)bkv * g.NCcap + c) * d + x);
  __syncthreads();
  float m, logz;
  chunk_softmax<T>(ks, qs, S, d, g.scale, ll, pl, red, m, logz);
  const float pl_l = block_sum4(tid < S ? pl[tid] * ll[tid] : 0.f, red);
  for (int x = tid; x < d; x += kThreads) {
    float acc = 0.f;
    for (int j = 0; j < S; ++j) acc = __builtin_fmaf(pl[j], ks[j * (d + 1) + x], acc);
    Elem<T>::st(orow + x, acc);
  }
  if (tid == 0 && bias) bias[(size_t)bkv * g.NCcap + c] = m + logz - pl_l;
}

template <typename T>
__global__ void __launch_bounds__(kThreads)
landmark_backward_kernel(Geometry g, const T* __restrict__ lq, const T* __restrict__ k,
                         const T* __restrict__ dlmk, const float* __restrict__ dbias,
                         T* __restrict__ dlq, T* __restrict__ dk) {
  extern __shared__ float lm_smem[];
  const int S = g.S, d = g.d;
  float* ks = lm_smem;
  float* qs = ks + S * (d + 1);
  float* ll = qs + d;
  float* pl = ll + S;
  float* red = pl + S;
  float* dm = red + 8;                       // d
  float* dls = dm + d;                       // S
  const int c = blockIdx.x, bkv = blockIdx.y;
  const int tid = threadIdx.x;
  if (c >= g.NC) {
    // zero gradients outside the complete chunks: lq rows c >= NC and the keys
    // of an incomplete tail chunk (handled by the workgroup c == NC)
    if (c < g.NCcap)
      for (int x = tid; x < d; x += kThreads) Elem<T>::st(dlq + ((size_t)bkv * g.NCcap + c) * d + x, 0.f);
    if (c == g.NC) {
      const size_t t0 = (size_t)g.NC * S;
      for (size_t e = tid; e < ((size_t)g.Lkv - t0) * d; e += kThreads)
        Elem<T>::st(dk + ((size_t)bkv * g.Lkv + t0) * d + e, 0.f);
    }
    return;
  }
  const T* kc = k + ((size_t)bkv * g.Lkv + (size_t)c * S) * d;
  stage_keys(kc, S, d, ks);
  for (int x = tid; x < d; x += kThreads) {
    qs[x] = Elem<T>::ld(lq + ((size_t)bkv * g.NCcap + c) * d + x);
    dm[x] = Elem<T>::ld(dlmk + ((size_t)bkv * g.NCcap + c) * d + x);
  }
  __syncthreads();
  float m, logz;
  chunk_softmax<T>(ks, qs, S, d, g.scale, ll, pl, red, m, logz);
  const float db = dbias ? dbias[(size_t)bkv * g.NCcap + c] : 0.f;
  float dp = 0.f;
  if (tid < S) {
    float acc = 0.f;
    const float* row = ks + tid * (d + 1);
    for (int x = 0; x < d; ++x) acc = __builtin_fmaf(dm[x], row[x], acc);
    const float logp = ll[tid] - m - logz;
    dp = acc - db * (logp + 1.f);
  }
  const float pdp = block_sum4(tid < S ? pl[tid] * dp : 0.f, red);
  if (tid < S) dls[tid] = pl[tid] * (dp - pdp);
  __syncthreads();
  for (int x = tid; x < d; x += kThreads) {
    float acc = 0.f;
    for (int j = 0; j < S; ++j) acc = __builtin_fmaf(dls[j], ks[j * (d + 1) + x], acc);
    Elem<T>::st(dlq + ((size_t)bkv * g.NCcap + c) * d + x, g.scale * acc);
  }
  T* dkc = dk + ((size_t)bkv * g.Lkv + (size_t)c * S) * d;
  for (int e = tid; e < S * d; e += kThreads) {
    const int j = e / d, x = e % d;
    Elem<T>::st(dkc + e, __builtin_fmaf(g.scale * dls[j], qs[x], pl[j] * dm[x]));
  }
}

size_t fwd_lds(const Geometry& g) { return ((size_t)g.S * (g.d + 1) + g.d + 2 * g.S + 8) * 4; }
size_t bwd_lds(const Geometry& g) { return fwd_lds(g) + ((size_t)g.d + g.S + 8) * 4; }

template <typename T>
hipError_t launch_fwd(const Geometry& g, const void* lq, const void* k, void* lmk, float* bias,
                      hipStream_t st) {
  const int nx = g.NCcap > g.NC ? g.NCcap : g.NC;
  if (nx == 0) return hipSuccess;
  const size_t sm = fwd_lds(g);
  hipError_t e = hipFuncSetAttribute((const void*)landmark_forward_kernel<T>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
  if (e != hipSuccess) return e;
  prof_begin(kLandmarks, st);
  hipLaunchKernelGGL(landmark_forward_kernel<T>, dim3(nx, g.B * g.Hkv), dim3(kThreads), sm, st, g,
                     (const T*)lq, (const T*)k, (T*)lmk, bias);
  prof_end(kLandmarks, st);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_bwd(const Geometry& g, const void* lq, const void* k, const void* dlmk,
                      const float* dbias, void* dlq, void* dk, hipStream_t st) {
  const bool tail = (size_t)g.NC * g.S < (size_t)g.Lkv;
  int nx = g.NCcap > g.NC ? g.NCcap : g.NC;
  if (tail && nx < g.NC + 1) nx = g.NC + 1;
  if (nx == 0) return hipSuccess;
  const size_t sm = bwd_lds(g);
  hipError_t e = hipFuncSetAttribute((const void*)landmark_backward_kernel<T>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
  if (e != hipSuccess) return e;
  prof_begin(kLandmarksBwd, st);
  hipLaunchKernelGGL(landmark_backward_kernel<T>, dim3(nx, g.B * g.Hkv), dim3(kThreads), sm, st, g,
                     (const T*)lq, (const T*)k, (const T*)dlmk, dbias, (T*)dlq, (T*)dk);
  prof_end(kLandmarksBwd, st);
  return hipGetLastError();
}

}  // namespace

bool landmarks_supported(const Geometry& g) {
  return g.S >= 1 && g.S <= kThreads && g.d >= 1 && g.d <= kThreads && g.S * g.d <= kMaxElems;
}

hipError_t launch_landmarks(const Geometry& g, int bf16, const void* lq, const void* k, void* lmk,
                            float* bias, hipStream_t st) {
  return bf16 ? launch_fwd<uint16_t>(g, lq, k, lmk, bias, st)
              : launch_fwd<float>(g, lq, k, lmk, bias, st);
}

hipError_t launch_landmarks_backward(const Geometry& g, int bf16, const void* lq, const void* k,
                                     const void* dlmk, const float* dbias, void* dlq, void* dk,
                                     hipStream_t st) {
  return bf16 ? launch_bwd<uint16_t>(g, lq, k, dlmk, dbias, dlq, dk, st)
              : launch_bwd<float>(g, lq, k, dlmk, dbias, dlq, dk, st);
}

}  // namespace hils
