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
// HBM-bound: each key is read once (and its gradient written once).  Two paths:
//  * bf16, d = 128, S = 64: one wave per chunk, the chunk's keys held in
//    registers.  Lane (r = lane / 16, t = lane % 16) holds dims [8t, 8t + 8) of
//    keys r + 4i (i < 16), so every load and dk store instruction covers 1 KB of
//    contiguous rows.  Per-key dot products are reduced over the 16 lanes of a
//    row group by a butterfly that leaves lane (r, t) with key r + 4t: softmax
//    and entropy are then plain wave reductions (one key per lane).  Weighted key
//    sums broadcast p within the row group and reduce over the four groups.
//  * otherwise one workgroup per chunk: keys staged in LDS as fp32 (row stride
//    d + 1: conflict-free column and row reads), one thread per key for the
//    logits, block reductions, one thread per dimension for the weighted sums.
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

// ------------------------------------------------------------ bf16, d = 128, S = 64
constexpr int kFastD = 128, kFastS = 64, kFastWaves = 4;

__device__ __forceinline__ void unpack8(const uint4& u, float* f) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

// v[i] = <a, lane's 8 dims of key r + 4i>
__device__ __forceinline__ void partial_dots(const uint4 (&kr)[16], const float* a, float (&v)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float kf[8];
    unpack8(kr[i], kf);
    float acc = 0.f;
#pragma unroll
    for (int x = 0; x < 8; ++x) acc = __builtin_fmaf(a[x], kf[x], acc);
    v[i] = acc;
  }
}

// acc[x] (lane's 8 dims, partial over its row group's keys) summed over the four
// row groups; lane (r, t) receives dims 8t + 2r and 8t + 2r + 1.
__device__ __forceinline__ float2 reduce_groups(float (&acc)[8], int lane) {
#pragma unroll
  for (int h = 32; h >= 16; h >>= 1) {
    const bool up = (lane & h) != 0;
    const int np = h == 32 ? 2 : 1;        // pairs kept after this step
#pragma unroll
    for (int pr = 0; pr < np; ++pr) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        float lo = acc[2 * pr + e], hi = acc[2 * (pr + np) + e];
        asm("" : "+v"(lo), "+v"(hi));
        acc[2 * pr + e] = (up ? hi : lo) + lane_xor_f32(up ? lo : hi, h);
      }
    }
  }
  return make_float2(acc[0], acc[1]);
}

__device__ __forceinline__ void load_chunk(const uint16_t* __restrict__ k, size_t row0, int r, int t,
                                           uint4 (&kr)[16]) {
  const uint4* kc = reinterpret_cast<const uint4*>(k + row0 * kFastD);
#pragma unroll
  for (int i = 0; i < 16; ++i) kr[i] = kc[(r + 4 * i) * (kFastD / 8) + t];
}

// sum_j w_j k_j over the chunk, w_j of key j = r + 4t held by lane (r, t)
__device__ __forceinline__ float2 weighted_keys(const uint4 (&kr)[16], float w, int lane) {
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float wi = row_bcast_f32(w, i);
    float kf[8];
    unpack8(kr[i], kf);
#pragma unroll
    for (int x = 0; x < 8; ++x) acc[x] = __builtin_fmaf(wi, kf[x], acc[x]);
  }
  return reduce_groups(acc, lane);
}

__global__ void __launch_bounds__(kFastWaves * kWave)
landmark_forward_fast(Geometry g, int nx, const uint16_t* __restrict__ lq,
                      const uint16_t* __restrict__ k, uint16_t* __restrict__ lmk,
                      float* __restrict__ bias) {
  const int lane = threadIdx.x & (kWave - 1);
  const int c = blockIdx.x * kFastWaves + threadIdx.x / kWave, bkv = blockIdx.y;
  if (c >= nx) return;
  const int r = lane >> 4, t = lane & 15;
  const size_t row = (size_t)bkv * g.NCcap + c;
  uint32_t* orow = reinterpret_cast<uint32_t*>(lmk + row * kFastD);
  if (c >= g.NC) {
    orow[lane] = 0u;
    if (lane == 0 && bias) bias[row] = 0.f;
    return;
  }
  uint4 kr[16];
  load_chunk(k, (size_t)bkv * g.Lkv + (size_t)c * kFastS, r, t, kr);
  float qf[8];
  unpack8(reinterpret_cast<const uint4*>(lq + row * kFastD)[t], qf);
  float v[16];
  partial_dots(kr, qf, v);
  const float l = g.scale * reduce_scatter16(v, t);      // key r + 4t
  const float m = wave_max(l);
  const float e = expf(l - m);
  const float z = wave_sum(e);
  const float p = e / z;
  const float pl = wave_sum(p * l);
  const float2 o = weighted_keys(kr, p, lane);
  orow[4 * t + r] = pack2(o.x, o.y);
  if (lane == 0 && bias) bias[row] = m + logf(z) - pl;
}

__global__ void __launch_bounds__(kFastWaves * kWave)
landmark_backward_fast(Geometry g, int nx, const uint16_t* __restrict__ lq,
                       const uint16_t* __restrict__ k, const uint16_t* __restrict__ dlmk,
                       const float* __restrict__ dbias, uint16_t* __restrict__ dlq,
                       uint16_t* __restrict__ dk) {
  const int lane = threadIdx.x & (kWave - 1);
  const int c = blockIdx.x * kFastWaves + threadIdx.x / kWave, bkv = blockIdx.y;
  if (c >= nx) return;
  const int r = lane >> 4, t = lane & 15;
  const size_t row = (size_t)bkv * g.NCcap + c;
  if (c >= g.NC) {
    if (c < g.NCcap) reinterpret_cast<uint32_t*>(dlq + row * kFastD)[lane] = 0u;
    if (c == g.NC) {
      const size_t t0 = (size_t)g.NC * kFastS;
      uint32_t* tail = reinterpret_cast<uint32_t*>(dk + ((size_t)bkv * g.Lkv + t0) * kFastD);
      for (size_t e = lane; e < ((size_t)g.Lkv - t0) * (kFastD / 2); e += kWave) tail[e] = 0u;
    }
    return;
  }
  const size_t krow0 = (size_t)bkv * g.Lkv + (size_t)c * kFastS;
  uint4 kr[16];
  load_chunk(k, krow0, r, t, kr);
  float qf[8], df[8];
  unpack8(reinterpret_cast<const uint4*>(lq + row * kFastD)[t], qf);
  unpack8(reinterpret_cast<const uint4*>(dlmk + row * kFastD)[t], df);
  const float db = dbias ? dbias[row] : 0.f;
  float v[16];
  partial_dots(kr, qf, v);
  const float l = g.scale * reduce_scatter16(v, t);      // key r + 4t
  const float m = wave_max(l);
  const float e = expf(l - m);
  const float z = wave_sum(e);
  const float p = e / z;
  const float logp = l - m - logf(z);
  partial_dots(kr, df, v);
  const float dp = reduce_scatter16(v, t) - db * (logp + 1.f);
  const float pdp = wave_sum(p * dp);
  const float dl = p * (dp - pdp);
  const float2 o = weighted_keys(kr, dl, lane);
  reinterpret_cast<uint32_t*>(dlq + row * kFastD)[4 * t + r] = pack2(g.scale * o.x, g.scale * o.y);
  uint4* dkc = reinterpret_cast<uint4*>(dk + krow0 * kFastD);
  const float sdl = g.scale * dl;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float a = row_bcast_f32(sdl, i);
    const float b = row_bcast_f32(p, i);
    float y[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) y[x] = __builtin_fmaf(a, qf[x], b * df[x]);
    dkc[(r + 4 * i) * (kFastD / 8) + t] =
        make_uint4(pack2(y[0], y[1]), pack2(y[2], y[3]), pack2(y[4], y[5]), pack2(y[6], y[7]));
  }
}

bool fast_shape(const Geometry& g, int bf16) { return bf16 && g.d == kFastD && g.S == kFastS; }

// chunks each launch covers: every landmark row, and the chunk slot of a
// partial tail (backward: its keys' gradients are zeroed)
int fwd_chunks(const Geometry& g) { return g.NCcap > g.NC ? g.NCcap : g.NC; }
int bwd_chunks(const Geometry& g) {
  int nx = fwd_chunks(g);
  if ((size_t)g.NC * g.S < (size_t)g.Lkv && nx < g.NC + 1) nx = g.NC + 1;
  return nx;
}

size_t fwd_lds(const Geometry& g) { return ((size_t)g.S * (g.d + 1) + g.d + 2 * g.S + 8) * 4; }
size_t bwd_lds(const Geometry& g) { return fwd_lds(g) + ((size_t)g.d + g.S + 8) * 4; }

template <typename T>
hipError_t launch_fwd(const Geometry& g, const void* lq, const void* k, void* lmk, float* bias,
                      hipStream_t st) {
  const int nx = fwd_chunks(g);
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
  const int nx = bwd_chunks(g);
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
  if (fast_shape(g, bf16)) {
    const int nx = fwd_chunks(g);
    if (nx == 0) return hipSuccess;
    prof_begin(kLandmarks, st);
    hipLaunchKernelGGL(landmark_forward_fast, dim3((nx + kFastWaves - 1) / kFastWaves, g.B * g.Hkv),
                       dim3(kFastWaves * kWave), 0, st, g, nx, (const uint16_t*)lq,
                       (const uint16_t*)k, (uint16_t*)lmk, bias);
    prof_end(kLandmarks, st);
    return hipGetLastError();
  }
  return bf16 ? launch_fwd<uint16_t>(g, lq, k, lmk, bias, st)
              : launch_fwd<float>(g, lq, k, lmk, bias, st);
}

hipError_t launch_landmarks_backward(const Geometry& g, int bf16, const void* lq, const void* k,
                                     const void* dlmk, const float* dbias, void* dlq, void* dk,
                                     hipStream_t st) {
  if (fast_shape(g, bf16)) {
    const int nx = bwd_chunks(g);
    if (nx == 0) return hipSuccess;
    prof_begin(kLandmarksBwd, st);
    hipLaunchKernelGGL(landmark_backward_fast, dim3((nx + kFastWaves - 1) / kFastWaves, g.B * g.Hkv),
                       dim3(kFastWaves * kWave), 0, st, g, nx, (const uint16_t*)lq,
                       (const uint16_t*)k, (const uint16_t*)dlmk, dbias, (uint16_t*)dlq,
                       (uint16_t*)dk);
    prof_end(kLandmarksBwd, st);
    return hipGetLastError();
  }
  return bf16 ? launch_bwd<uint16_t>(g, lq, k, dlmk, dbias, dlq, dk, st)
              : launch_bwd<float>(g, lq, k, dlmk, dbias, dlq, dk, st);
}

}  // namespace hils
