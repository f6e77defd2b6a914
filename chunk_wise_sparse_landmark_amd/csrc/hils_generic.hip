// Shape-generic HiLS kernels: one workgroup per (query, batch x kv head) for the
// forward, and a chunk-owner pass for the key/value gradients.  They cover every
// shape the ABI accepts (fp32 or bf16, head_dim <= 256, chunk_size <= 256,
// top_k <= 64) with plain vector ALU arithmetic; the MFMA and split-decode
// paths take the bf16 d = 128, S = 64 workloads.
//
// Method: Hierarchical Sparse Attention Done Right (arXiv 2607.02980v1, summary
// page) -- §3 "Linear surrogate for chunk mass" (landmark scores), §3 "Sparse
// training" (top-K routing), §4 "Architecture" (GQA shared selection), §3
// "Hierarchical softmax" (per-chunk softmax and score-weighted fusion), §9
// (no gradient to unselected chunks).
#include "hils_common.h"
#include "hils_kernels.h"
#include "hils_profile.h"

namespace hils {

constexpr int kThreads = 256;
constexpr int kMaxD = 256;
constexpr int kMaxS = 256;
constexpr int kMaxG = 64;

// ---------------------------------------------------------------------------
// Selection: group score of every candidate, top-K, ascending ids.
// grid (Lq, B*Hkv), 256 threads.  Each wave keeps a running top-64 list.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(kThreads)
generic_select_kernel(Geometry g, const T* __restrict__ q, const T* __restrict__ lmk,
                      const float* __restrict__ bias, int32_t* __restrict__ sel_idx) {
  __shared__ float qs[kMaxG * 4 + kMaxD];          // mean query over the group
  __shared__ uint64_t lists[4][kWave];
  __shared__ uint64_t scratch[4][kWave];
  const int i = blockIdx.x;
  const int bkv = blockIdx.y;
  const int b = bkv / g.Hkv, kvh = bkv % g.Hkv;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  int ncand, own, ob;
  g.layout(i, ncand, own, ob);

  // qbar = mean_h q_h (the group score is linear in q)
  for (int e = tid; e < g.d; e += kThreads) {
    float acc = 0.f;
    for (int h = 0; h < g.G; ++h)
      acc += Elem<T>::ld(q + ((size_t)(b * g.Hq + kvh * g.G + h) * g.Lq + i) * g.d + e);
    qs[e] = acc / (float)g.G;
  }
  __syncthreads();

  const T* L = lmk + (size_t)bkv * g.NCcap * g.d;
  const float* bb = bias ? bias + (size_t)bkv * g.NCcap : nullptr;
  uint64_t run = 0;   // running top-64 of this wave, one key per lane
  for (int base = w * kWave; base < ncand; base += 4 * kWave) {
    const int c = base + lane;
    uint64_t key = 0;
    if (c < ncand) {
      float acc = 0.f;
      const T* row = L + (size_t)c * g.d;
      for (int e = 0; e < g.d; ++e) acc += qs[e] * Elem<T>::ld(row + e);
      float s = g.scale * acc + (bb ? bb[c] : 0.f);
      key = make_key(s, c);
    }
    uint64_t pair[2] = {run, key};
    run = wave_topk<2>(pair, g.K, scratch[w]);
  }
  lists[w][lane] = lane < g.K ? run : 0ull;
  __syncthreads();
  if (w == 0) {
    uint64_t top = lists[0][lane];
    for (int x = 1; x < 4; ++x) top = wave_merge_into(top, lists[x][lane], g.K, scratch[0]);
    // ascending chunk ids: sort descending on the complemented id
    uint64_t asc = (lane < g.K && top != 0) ? (0xffffffffull - (uint64_t)key_index(top)) + 1 : 0;
    asc = wave_sort64_desc(asc);
    if (lane < g.K) {
      int id = asc ? (int)(0xffffffffull - (asc - 1)) : -1;
      sel_idx[((size_t)bkv * g.Lq + i) * g.K + lane] = id;
    }
  }
}

// ---------------------------------------------------------------------------
// Shared per-member attention: logits over tokens [a, e), lse, p in LDS, o_c[d]
// for thread d.  Returns lse_c; `p` holds exp(l - lse_c).
// ---------------------------------------------------------------------------
template <typename T>
__device__ float member_attention(const Geometry& g, const float* qh, const T* Kg, const T* Vg,
                                  int a, int e, float* p, float* red, float& o_d) {
  const int tid = threadIdx.x;
  const int n = e - a;
  float l = -INFINITY;
  if (tid < n) {
    const T* kr = Kg + (size_t)(a + tid) * g.d;
    float acc = 0.f;
    for (int x = 0; x < g.d; ++x) acc += qh[x] * Elem<T>::ld(kr + x);
    l = g.scale * acc;
  }
  const float m = block_max4(l, red);
  const float ex = tid < n ? __expf(l - m) : 0.f;
  const float z = block_sum4(ex, red);
  const float lse = m + __logf(z);
  if (tid < n) p[tid] = ex / z;
  __syncthreads();
  o_d = 0.f;
  if (tid < g.d) {
    for (int j = 0; j < n; ++j) o_d += p[j] * Elem<T>::ld(Vg + (size_t)(a + j) * g.d + tid);
  }
  __syncthreads();
  return lse;
}

template <typename T>
__device__ float retrieval_score(const Geometry& g, const float* qh, const T* lrow, float bias_c,
                                 float* red) {
  const int tid = threadIdx.x;
  float part = tid < g.d ? qh[tid] * Elem<T>::ld(lrow + tid) : 0.f;
  return g.scale * block_sum4(part, red) + bias_c;
}

// ---------------------------------------------------------------------------
// Attention + fusion.  grid (Lq, B*Hkv), 256 threads; thread d owns output dim d.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(kThreads)
generic_attend_kernel(Geometry g, const T* __restrict__ q, const T* __restrict__ qr,
                      const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ lmk,
                      const float* __restrict__ bias, const int32_t* __restrict__ sel_idx,
                      T* __restrict__ out, float* __restrict__ lse_out) {
  __shared__ float qh[kMaxD];
  __shared__ float qrh[kMaxD];     // the retrieval query of the row (chunk scores)
  __shared__ float p[kMaxS];
  __shared__ float red[4];
  __shared__ int sel[kMaxTopK];
  const int i = blockIdx.x;
  const int bkv = blockIdx.y;
  const int b = bkv / g.Hkv, kvh = bkv % g.Hkv;
  const int tid = threadIdx.x;
  int ncand, own, ob;
  g.layout(i, ncand, own, ob);
  if (tid < g.K) sel[tid] = sel_idx[((size_t)bkv * g.Lq + i) * g.K + tid];
  const T* Kg = k + (size_t)bkv * g.Lkv * g.d;
  const T* Vg = v + (size_t)bkv * g.Lkv * g.d;
  const T* Lg = lmk + (size_t)bkv * g.NCcap * g.d;
  const float* bb = bias ? bias + (size_t)bkv * g.NCcap : nullptr;
  __syncthreads();

  // members: slots 0..K-1 the selection, slots K..K+win-1 the window chunks
  // (own chunk first), each window chunk fused with its exact lse
  for (int hh = 0; hh < g.G; ++hh) {
    const int h = kvh * g.G + hh;
    const size_t row = (size_t)(b * g.Hq + h) * g.Lq + i;
    if (tid < g.d) {
      qh[tid] = Elem<T>::ld(q + row * g.d + tid);
      qrh[tid] = Elem<T>::ld(qr + row * g.d + tid);
    }
    __syncthreads();
    float m = -INFINITY, z = 0.f, acc = 0.f;   // online fusion over members
    for (int slot = 0; slot < g.K + g.win; ++slot) {
      int a, e;
      float s;
      if (slot < g.K) {
        const int c = sel[slot];
        if (c < 0) continue;
        a = c * g.S;
        e = a + g.S;
        s = retrieval_score<T>(g, qrh, Lg + (size_t)c * g.d, bb ? bb[c] : 0.f, red);
        float o_d;
        member_attention<T>(g, qh, Kg, Vg, a, e, p, red, o_d);
        const float mn = fmaxf(m, s);
        const float f_old = __expf(m - mn), f_new = __expf(s - mn);
        acc = acc * f_old + f_new * o_d;
        z = z * f_old + f_new;
        m = mn;
      } else {
        if (!g.window_member(own, ob, slot - g.K, a, e)) continue;
        float o_d;
        s = member_attention<T>(g, qh, Kg, Vg, a, e, p, red, o_d);
        const float mn = fmaxf(m, s);
        const float f_old = __expf(m - mn), f_new = __expf(s - mn);
        acc = acc * f_old + f_new * o_d;
        z = z * f_old + f_new;
        m = mn;
      }
    }
    if (tid < g.d) Elem<T>::st(out + row * g.d + tid, z > 0.f ? acc / z : 0.f);
    if (tid == 0 && lse_out) lse_out[row] = z > 0.f ? m + __logf(z) : -INFINITY;
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Backward, row pass.  grid (Lq, B*Hkv).  For each head: recompute the members
// and the fusion, then
//   D = <dO, O>,  u_j = <dO, v_j>,  D_c = <dO, o_c>,
//   retrieved: dl_j = w_c p_j (u_j - D_c),  ds_c = w_c (D_c - D)
//   window:    dl_j = w_c p_j (u_j - D)      (its score is its own lse)
//   dq = scale (sum dl_j k_j + sum_c ds_c lmk_c), the second sum going to dqr
//   instead when a separate retrieval query is given (dqr non-null).
// Per (row, member) it stores (w, lse_c, Dt, ds) with Dt = D_c or D, which the
// chunk pass needs: dl_j = w p_j (u_j - Dt).
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(kThreads)
generic_bwd_rows_kernel(Geometry g, const T* __restrict__ q, const T* __restrict__ qr,
                        const T* __restrict__ k, const T* __restrict__ v,
                        const T* __restrict__ lmk, const float* __restrict__ bias,
                        const T* __restrict__ dout, const int32_t* __restrict__ sel_idx,
                        T* __restrict__ dq, T* __restrict__ dqr, float4* __restrict__ stats) {
  __shared__ float qh[kMaxD];
  __shared__ float qrh[kMaxD];
  __shared__ float gh[kMaxD];
  __shared__ float p[kMaxS];
  __shared__ float dl[kMaxS];
  __shared__ float red[4];
  __shared__ int sel[kMaxTopK];
  __shared__ float ms[kMaxTopK + kMaxLocalChunks], mlse[kMaxTopK + kMaxLocalChunks];
  __shared__ float mD[kMaxTopK + kMaxLocalChunks];
  const int nslot = g.K + g.win;
  const int i = blockIdx.x;
  const int bkv = blockIdx.y;
  const int b = bkv / g.Hkv, kvh = bkv % g.Hkv;
  const int tid = threadIdx.x;
  int ncand, own, ob;
  g.layout(i, ncand, own, ob);
  if (tid < g.K) sel[tid] = sel_idx[((size_t)bkv * g.Lq + i) * g.K + tid];
  const T* Kg = k + (size_t)bkv * g.Lkv * g.d;
  const T* Vg = v + (size_t)bkv * g.Lkv * g.d;
  const T* Lg = lmk + (size_t)bkv * g.NCcap * g.d;
  const float* bb = bias ? bias + (size_t)bkv * g.NCcap : nullptr;
  __syncthreads();

  for (int hh = 0; hh < g.G; ++hh) {
    const int h = kvh * g.G + hh;
    const size_t row = (size_t)(b * g.Hq + h) * g.Lq + i;
    if (tid < g.d) {
      qh[tid] = Elem<T>::ld(q + row * g.d + tid);
      qrh[tid] = Elem<T>::ld(qr + row * g.d + tid);
      gh[tid] = Elem<T>::ld(dout + row * g.d + tid);
    }
    __syncthreads();
    // pass 1: member scores, lse, D_c; fused output
    float m = -INFINITY, z = 0.f, acc = 0.f;
    for (int slot = 0; slot < nslot; ++slot) {
      int a = 0, e = 0;
      float s;
      bool valid;
      if (slot < g.K) {
        const int c = sel[slot];
        valid = c >= 0;
        if (valid) {
          a = c * g.S;
          e = a + g.S;
          s = retrieval_score<T>(g, qrh, Lg + (size_t)c * g.d, bb ? bb[c] : 0.f, red);
        }
      } else {
        valid = g.window_member(own, ob, slot - g.K, a, e);
      }
      if (!valid) {
        if (tid == 0) { ms[slot] = -INFINITY; mlse[slot] = 0.f; mD[slot] = 0.f; }
        continue;
      }
      float o_d;
      float lc = member_attention<T>(g, qh, Kg, Vg, a, e, p, red, o_d);
      if (slot >= g.K) s = lc;
      float Dc = block_sum4(tid < g.d ? gh[tid] * o_d : 0.f, red);
      if (tid == 0) { ms[slot] = s; mlse[slot] = lc; mD[slot] = Dc; }
      const float mn = fmaxf(m, s);
      const float f_old = __expf(m - mn), f_new = __expf(s - mn);
      acc = acc * f_old + f_new * o_d;
      z = z * f_old + f_new;
      m = mn;
    }
    __syncthreads();
    const float LSE = z > 0.f ? m + __logf(z) : -INFINITY;
    const float O_d = z > 0.f ? acc / z : 0.f;
    const float D = block_sum4(tid < g.d ? gh[tid] * O_d : 0.f, red);
    // pass 2: gradients
    float dq_d = 0.f, dqr_d = 0.f;
    for (int slot = 0; slot < nslot; ++slot) {
      float4 st = make_float4(0.f, 0.f, 0.f, 0.f);
      const float s = ms[slot];
      if (s != -INFINITY) {
        int a = 0, e = 0, c = -1;
        if (slot < g.K) {
          c = sel[slot];
          a = c * g.S;
          e = a + g.S;
        } else {
          g.window_member(own, ob, slot - g.K, a, e);
        }
        const float wgt = __expf(s - LSE);
        const float lc = mlse[slot];
        const float Dt = slot < g.K ? mD[slot] : D;
        const int n = e - a;
        if (tid < n) {
          const T* kr = Kg + (size_t)(a + tid) * g.d;
          const T* vr = Vg + (size_t)(a + tid) * g.d;
          float lq = 0.f, u = 0.f;
          for (int x = 0; x < g.d; ++x) {
            lq += qh[x] * Elem<T>::ld(kr + x);
            u += gh[x] * Elem<T>::ld(vr + x);
          }
          const float pj = __expf(g.scale * lq - lc);
          dl[tid] = wgt * pj * (u - Dt);
        }
        __syncthreads();
        if (tid < g.d) {
          float sacc = 0.f;
          for (int j = 0; j < n; ++j) sacc += dl[j] * Elem<T>::ld(Kg + (size_t)(a + j) * g.d + tid);
          dq_d += g.scale * sacc;
          if (slot < g.K) dqr_d += g.scale * wgt * (Dt - D) * Elem<T>::ld(Lg + (size_t)c * g.d + tid);
        }
        __syncthreads();
        st = make_float4(wgt, lc, Dt, slot < g.K ? wgt * (Dt - D) : 0.f);
      }
      if (tid == 0) stats[row * nslot + slot] = st;
    }
    if (tid < g.d) {
      if (dqr) {
        Elem<T>::st(dq + row * g.d + tid, dq_d);
        Elem<T>::st(dqr + row * g.d + tid, dqr_d);
      } else {
        Elem<T>::st(dq + row * g.d + tid, dq_d + dqr_d);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Backward, chunk pass.  grid (max(ceil(Lkv/S), NCcap), B*Hkv).  Workgroup c
// owns keys [cS, cS+S) and landmark c: it walks the queries in order, and for
// every (query, head) that selected c, or whose local window holds c, adds
//   dk_j += scale dl_j q,  dv_j += w p_j dO,   and for a selection
//   dlmk_c += scale ds q_r,  dbias_c += ds  (q_r: the retrieval query).
// Deterministic: one owner per output row, fixed order.
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(kThreads)
generic_bwd_chunks_kernel(Geometry g, const T* __restrict__ q, const T* __restrict__ qr,
                          const T* __restrict__ k, const T* __restrict__ v,
                          const T* __restrict__ dout,
                          const int32_t* __restrict__ sel_idx, const float4* __restrict__ stats,
                          T* __restrict__ dk, T* __restrict__ dv, T* __restrict__ dlmk,
                          float* __restrict__ dbias) {
  extern __shared__ float smem[];
  float* dkacc = smem;                      // [S][d]
  float* dvacc = smem + g.S * g.d;          // [S][d]
  __shared__ float qh[kMaxD];
  __shared__ float gh[kMaxD];
  __shared__ float pw[kMaxS];
  __shared__ float dl[kMaxS];
  __shared__ float dlm[kMaxD];
  __shared__ float qrh[kMaxD];
  __shared__ int hit;
  const int c = blockIdx.x;
  const int bkv = blockIdx.y;
  const int b = bkv / g.Hkv, kvh = bkv % g.Hkv;
  const int tid = threadIdx.x;
  const int nchunks_kv = (g.Lkv + g.S - 1) / g.S;
  const T* Kg = k + (size_t)bkv * g.Lkv * g.d;
  const T* Vg = v + (size_t)bkv * g.Lkv * g.d;
  const bool owns_keys = c < nchunks_kv;
  const int a0 = c * g.S;
  const int a1 = owns_keys ? min(a0 + g.S, g.Lkv) : a0;
  for (int x = tid; x < g.S * g.d; x += kThreads) { dkacc[x] = 0.f; dvacc[x] = 0.f; }
  if (tid < g.d) dlm[tid] = 0.f;
  float dbias_acc = 0.f;
  __syncthreads();

  if (owns_keys) {
    const int nslot = g.K + g.win;
    for (int i = 0; i < g.Lq; ++i) {
      int ncand, own, ob;
      g.layout(i, ncand, own, ob);
      // which member is chunk c for query i: a selection slot, a window slot, or none
      if (tid == 0) hit = -1;
      __syncthreads();
      if (c < g.NC && tid < g.K && sel_idx[((size_t)bkv * g.Lq + i) * g.K + tid] == c) hit = tid;
      __syncthreads();
      int slot = hit;
      int ta = a0, tb = a0 + g.S;
      if (slot < 0) {
        if (g.window_member(own, ob, own - c, ta, tb)) {
          slot = g.K + (own - c);
        } else {
          __syncthreads();
          continue;
        }
      }
      __syncthreads();
      const int n = tb - ta;
      for (int hh = 0; hh < g.G; ++hh) {
        const int h = kvh * g.G + hh;
        const size_t row = (size_t)(b * g.Hq + h) * g.Lq + i;
        const float4 st = stats[row * nslot + slot];   // w, lse_c, Dt, ds
        if (tid < g.d) {
          qh[tid] = Elem<T>::ld(q + row * g.d + tid);
          qrh[tid] = Elem<T>::ld(qr + row * g.d + tid);
          gh[tid] = Elem<T>::ld(dout + row * g.d + tid);
        }
        __syncthreads();
        if (tid < n) {
          const T* kr = Kg + (size_t)(ta + tid) * g.d;
          const T* vr = Vg + (size_t)(ta + tid) * g.d;
          float lq = 0.f, u = 0.f;
          for (int x = 0; x < g.d; ++x) {
            lq += qh[x] * Elem<T>::ld(kr + x);
            u += gh[x] * Elem<T>::ld(vr + x);
          }
          const float pj = __expf(g.scale * lq - st.y);
          pw[tid] = st.x * pj;
          dl[tid] = st.x * pj * (u - st.z);
        }
        __syncthreads();
        const int off = ta - a0;
        for (int x = tid; x < n * g.d; x += kThreads) {
          const int j = x / g.d, e = x % g.d;
          dkacc[(off + j) * g.d + e] += g.scale * dl[j] * qh[e];
          dvacc[(off + j) * g.d + e] += pw[j] * gh[e];
        }
        if (slot < g.K) {
          if (tid < g.d) dlm[tid] += g.scale * st.w * qrh[tid];
          dbias_acc += st.w;
        }
        __syncthreads();
      }
    }
    for (int x = tid; x < (a1 - a0) * g.d; x += kThreads) {
      const size_t o = ((size_t)bkv * g.Lkv + a0) * g.d + x;
      Elem<T>::st(dk + o, dkacc[x]);
      Elem<T>::st(dv + o, dvacc[x]);
    }
  }
  if (c < g.NCcap) {
    if (tid < g.d) Elem<T>::st(dlmk + ((size_t)bkv * g.NCcap + c) * g.d + tid, dlm[tid]);
    if (dbias && tid == 0) dbias[(size_t)bkv * g.NCcap + c] = dbias_acc;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename T>
hipError_t launch_generic_forward_t(const Geometry& g, const void* q, const void* qr, const void* k,
                                    const void* v, const void* lmk, const float* bias, void* out,
                                    int32_t* sel_idx, float* lse, hipStream_t st) {
  dim3 grid(g.Lq, g.B * g.Hkv);
  prof_begin(kGenericSelect, st);
  hipLaunchKernelGGL(generic_select_kernel<T>, grid, dim3(kThreads), 0, st, g, (const T*)qr,
                     (const T*)lmk, bias, sel_idx);
  prof_end(kGenericSelect, st);
  prof_begin(kGenericAttend, st);
  hipLaunchKernelGGL(generic_attend_kernel<T>, grid, dim3(kThreads), 0, st, g, (const T*)q,
                     (const T*)qr, (const T*)k, (const T*)v, (const T*)lmk, bias, sel_idx,
                     (T*)out, lse);
  prof_end(kGenericAttend, st);
  return hipGetLastError();
}

hipError_t launch_generic_forward(const Geometry& g, int bf16, const void* q, const void* qr,
                                  const void* k, const void* v, const void* lmk, const float* bias,
                                  void* out, int32_t* sel_idx, float* lse, hipStream_t st) {
  return bf16 ? launch_generic_forward_t<uint16_t>(g, q, qr, k, v, lmk, bias, out, sel_idx, lse, st)
              : launch_generic_forward_t<float>(g, q, qr, k, v, lmk, bias, out, sel_idx, lse, st);
}

size_t generic_backward_ws(const Geometry& g) {
  return (size_t)g.B * g.Hq * g.Lq * (g.K + g.win) * sizeof(float4);
}

template <typename T>
hipError_t launch_generic_backward_t(const Geometry& g, const void* q, const void* qr,
                                     const void* k, const void* v, const void* lmk,
                                     const float* bias, const void* dout, const int32_t* sel_idx,
                                     void* dq, void* dqr, void* dk, void* dv, void* dlmk,
                                     float* dbias, void* ws, hipStream_t st) {
  float4* stats = (float4*)ws;
  prof_begin(kGenericBwdRows, st);
  hipLaunchKernelGGL(generic_bwd_rows_kernel<T>, dim3(g.Lq, g.B * g.Hkv), dim3(kThreads), 0, st, g,
                     (const T*)q, (const T*)qr, (const T*)k, (const T*)v, (const T*)lmk, bias,
                     (const T*)dout, sel_idx, (T*)dq, (T*)dqr, stats);
  prof_end(kGenericBwdRows, st);
  const int nck = (g.Lkv + g.S - 1) / g.S;
  const int gx = nck > g.NCcap ? nck : g.NCcap;
  if (gx > 0) {
    const size_t sm = (size_t)2 * g.S * g.d * sizeof(float);
    if (const hipError_t e = hipFuncSetAttribute((const void*)generic_bwd_chunks_kernel<T>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
        e != hipSuccess)
      return e;
    prof_begin(kGenericBwdChunks, st);
    hipLaunchKernelGGL(generic_bwd_chunks_kernel<T>, dim3(gx, g.B * g.Hkv), dim3(kThreads), sm, st,
                       g, (const T*)q, (const T*)qr, (const T*)k, (const T*)v, (const T*)dout,
                       sel_idx, stats, (T*)dk, (T*)dv, (T*)dlmk, dbias);
    prof_end(kGenericBwdChunks, st);
  }
  return hipGetLastError();
}

hipError_t launch_generic_backward(const Geometry& g, int bf16, const void* q, const void* qr,
                                   const void* k, const void* v, const void* lmk, const float* bias,
                                   const void* dout, const int32_t* sel_idx, void* dq, void* dqr,
                                   void* dk, void* dv, void* dlmk, float* dbias, void* ws,
                                   hipStream_t st) {
  return bf16 ? launch_generic_backward_t<uint16_t>(g, q, qr, k, v, lmk, bias, dout, sel_idx, dq,
                                                    dqr, dk, dv, dlmk, dbias, ws, st)
              : launch_generic_backward_t<float>(g, q, qr, k, v, lmk, bias, dout, sel_idx, dq, dqr,
                                                 dk, dv, dlmk, dbias, ws, st);
}

}  // namespace hils
