// Split single-token decode for bf16, head_dim 128, chunk 64 (HBM-bound path).
//
// Method: Hierarchical Sparse Attention Done Right (arXiv 2607.02980v1, summary
// page): landmark scores §3 "Linear surrogate for chunk mass", top-K routing §3
// "Sparse training", GQA-shared selection §4 "Architecture", per-chunk softmax
// and score-weighted fusion §3 "Hierarchical softmax".
//
// Four launches on the caller's stream (three when one scoring workgroup per
// (b, kv head) covers every candidate):
//  1. score_select  grid (nsplit, B*Hkv): each workgroup streams a contiguous
//     range of landmark rows (16 lanes x 16 B per 256 B row, coalesced), forms
//     the group score scale*<mean_h q_h, lmk_c> + bias_c (the group mean is
//     linear in q), and keeps its local top-K as composite keys; with a
//     single split it writes the ascending chunk ids itself.
//  2. merge         grid (B*Hkv): top-K of the nsplit local lists; writes the
//     ascending chunk ids.
//  3. attend        grid (nsplit', B*Hkv): each workgroup walks one or a few
//     of the K+1 fusion slots (selected chunks and the own chunk), reading
//     each chunk's 16 KB of K and 16 KB of V once for all G heads, and folds
//     the chunk outputs into a running (max score, weight sum, weighted
//     output) per head.
//  4. fuse          one wave per (b, q head): log-sum-exp merge of the
//     nsplit' partials.  (A separate launch: on this multi-XCD part a
//     device-scope fence per workgroup -- needed for a last-workgroup
//     reduction -- writes back and invalidates L2 and costs far more than one
//     more launch.)
#include "hils_common.h"
#include "hils_mfma.h"
#include "hils_kernels.h"
#include "hils_profile.h"

namespace hils {

namespace {

constexpr int kD = 128;
constexpr int kS = 64;
constexpr int kThreads = 256;
constexpr int kMaxGd = 16;            // heads per KV group on this path

struct DecodeWs {
  uint64_t* lists;   // [B*Hkv][nsplit][K]
  float* parts;      // [B*Hkv][asplit <= K+win][G][kPartStride]: (O, M, Z) per head
};

__device__ __forceinline__ void load_bf16x8(const uint16_t* p, float (&x)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  x[0] = __uint_as_float(u.x << 16); x[1] = __uint_as_float(u.x & 0xffff0000u);
  x[2] = __uint_as_float(u.y << 16); x[3] = __uint_as_float(u.y & 0xffff0000u);
  x[4] = __uint_as_float(u.z << 16); x[5] = __uint_as_float(u.z & 0xffff0000u);
  x[6] = __uint_as_float(u.w << 16); x[7] = __uint_as_float(u.w & 0xffff0000u);
}

// ----------------------------------------------------------------------------
// 1. scores + local top-K.  A workgroup owns cps = NIT * 256 consecutive
//    candidates (NIT <= kMaxIt); in iteration i wave w scores a block of 64
//    rows (16 lanes x 16 B per 256 B row, each load instruction covering 4
//    consecutive rows = 1 KB, the next block's loads issued before
//    this one is scored) and keeps the block's keys in registers.  The wave's
//    exact top-K is then found by a bit-by-bit search for the K-th largest key
//    (wave ballots, no sorting), compacted, sorted once, and the four wave
//    lists are merged.
//    No load is predicated: a row past the split's end re-reads the split's
//    last row (its key is dropped).  A predicated load puts a branch around
//    it, and the compiler then waits for every outstanding load after the
//    branch, so the next block would no longer be in flight while one is
//    scored; the block count and the bias are template parameters for the
//    same reason.
// ----------------------------------------------------------------------------
constexpr int kMaxIt = 4;

// A floor p for the wave's valid keys (0 = empty): when there are at least K of
// them, the keys >= p are exactly the K largest (p is the K-th largest key, or
// the first prefix that exactly K keys reach: the search stops there); else p
// is no larger than the smallest valid key.  The low word of a key is the
// complemented chunk id; ids below 2^idbits leave its bits idbits..31 set, so
// only the 32 score bits and idbits id bits are searched.
template <int N>
__device__ __forceinline__ uint64_t wave_kth_key(const uint64_t (&kk)[N], int K, int idbits) {
  uint64_t p = 0;
  for (int bit = 63; bit >= 32; --bit) {
    const uint64_t t = p | (1ull << bit);
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < N; ++r) cnt += __popcll(__ballot(kk[r] >= t));
    if (cnt >= K) p = t;
    if (cnt == K) return p;
  }
  p |= (uint64_t)(0xffffffffu << idbits);
  for (int bit = idbits - 1; bit >= 0; --bit) {
    const uint64_t t = p | (1ull << bit);
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < N; ++r) cnt += __popcll(__ballot(kk[r] >= t));
    if (cnt >= K) p = t;
  }
  return p;
}

// W waves per workgroup.  kFinal: one workgroup covers every candidate of its
// (b, kv head) and writes the selection itself (ascending ids into sel_idx),
// so no merge launch follows.
template <int W, int NIT, bool kBias, bool kFinal>
__global__ void __launch_bounds__(W * kWave)
decode_score_select(Geometry g, const uint16_t* __restrict__ q, const uint16_t* __restrict__ lmk,
                    const float* __restrict__ bias, int ncand, int cps, int nsplit, int idbits,
                    uint64_t* __restrict__ lists, int32_t* __restrict__ sel_idx) {
  __shared__ uint64_t buf[W][kWave];
  __shared__ uint64_t wl[W][kWave];
  const int split = blockIdx.x, bkv = blockIdx.y;
  const int b = bkv / g.Hkv, kvh = bkv % g.Hkv;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int sub = lane & 15, grp = lane >> 4;
  const int K = g.K;

  const int c0 = split * cps;
  const int c1 = min(c0 + cps, ncand);
  uint64_t* dst = kFinal ? nullptr : lists + ((size_t)bkv * nsplit + split) * K;
  if (c1 <= c0) {                          // no candidates: an empty list
    if (w == 0 && lane < K) {
      if (kFinal) sel_idx[(size_t)bkv * K + lane] = -1;
      else dst[lane] = 0ull;
    }
    return;
  }
  const uint16_t* L = lmk + (size_t)bkv * g.NCcap * kD;
  // the row this lane scores in iteration it (x == sub below), clamped
  auto my_row = [&](int it) { return c0 + (it * W + w) * kWave + 4 * sub + grp; };
  auto load_block = [&](int it, uint4 (&raw)[16]) {
    const int base = c0 + (it * W + w) * kWave;   // this wave's block of 64
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const int c = min(base + 4 * x + grp, c1 - 1);   // 4 consecutive rows (1 KB) per load
      raw[x] = *reinterpret_cast<const uint4*>(L + (size_t)c * kD + sub * 8);
    }
  };
  // retrieval query: the first four heads' loads go out with the first block's
  const uint16_t* qg = q + (size_t)(b * g.Hq + kvh * g.G) * kD + sub * 8;
  uint4 qh[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) qh[h] = *reinterpret_cast<const uint4*>(qg + (size_t)min(h, g.G - 1) * kD);
  float qb[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int h = 4; h < g.G; ++h) {          // heads past four (G > 4 only)
    float x[8];
    load_bf16x8(qg + (size_t)h * kD, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) qb[e] += x[e];
  }
  float bv[NIT];
  if (kBias) {
    const float* bb = bias + (size_t)bkv * g.NCcap;
#pragma unroll
    for (int it = 0; it < NIT; ++it) bv[it] = bb[min(my_row(it), c1 - 1)];
  }
  uint4 cur[16], nxt[16];
  load_block(0, cur);

  // this lane's 8 dims of the mean query
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const float f = h < g.G ? 1.f : 0.f;
    const uint32_t u[4] = {qh[h].x, qh[h].y, qh[h].z, qh[h].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qb[2 * e] += f * __uint_as_float(u[e] << 16);
      qb[2 * e + 1] += f * __uint_as_float(u[e] & 0xffff0000u);
    }
  }
  const float inv = g.scale / (float)g.G;
#pragma unroll
  for (int e = 0; e < 8; ++e) qb[e] *= inv;

  uint64_t kk[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    if (it + 1 < NIT) load_block(it + 1, nxt);
    float mine = 0.f;
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const uint4 u = cur[x];
      float sc = qb[0] * __uint_as_float(u.x << 16) + qb[1] * __uint_as_float(u.x & 0xffff0000u)
               + qb[2] * __uint_as_float(u.y << 16) + qb[3] * __uint_as_float(u.y & 0xffff0000u)
               + qb[4] * __uint_as_float(u.z << 16) + qb[5] * __uint_as_float(u.z & 0xffff0000u)
               + qb[6] * __uint_as_float(u.w << 16) + qb[7] * __uint_as_float(u.w & 0xffff0000u);
      // sum over the 16 lanes of the row: rotations within a 16-lane DPP row
      sc += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(sc), 0x128, 0xf, 0xf, false));
      sc += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(sc), 0x124, 0xf, 0xf, false));
      sc += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(sc), 0x122, 0xf, 0xf, false));
      sc += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(sc), 0x121, 0xf, 0xf, false));
      if (x == sub) mine = sc;
    }
    const int c = my_row(it);
    kk[it] = c < c1 ? make_key(mine + (kBias ? bv[it] : 0.f), c) : 0ull;
    if (it + 1 < NIT) {
#pragma unroll
      for (int x = 0; x < 16; ++x) cur[x] = nxt[x];
    }
  }
  // exact top-K of the wave's keys: the keys >= the K-th largest, compacted and sorted
  const uint64_t p = wave_kth_key(kk, K, idbits);
  int cntk = 0;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const bool pred = kk[it] != 0ull && kk[it] >= p;
    const uint64_t m = __ballot(pred);
    if (pred) buf[w][cntk + mask_rank(m)] = kk[it];
    cntk += __popcll(m);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint64_t sel = lane < cntk ? buf[w][lane] : 0ull;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint64_t run = wave_rank_sort64(sel, buf[w]);
  wl[w][lane] = lane < K ? run : 0ull;
  // the wave lists merged pairwise in a tree (waves 0, 2, .. then 0, 4, ..)
#pragma unroll
  for (int st = 1; st < W; st <<= 1) {
    __syncthreads();
    if (w % (2 * st) == 0) {
      const uint64_t mg = wave_merge_into(wl[w][lane], wl[w + st][lane], K, buf[w]);
      wl[w][lane] = lane < K ? mg : 0ull;
    }
  }
  if (w == 0) {
    const uint64_t top = wl[0][lane];
    if (kFinal) {
      // ascending ids: a rank sort of the complemented ids (unique, 0 = none)
      uint64_t asc = (lane < K && top != 0) ? (0xffffffffull - (uint64_t)key_index(top)) + 1 : 0;
      asc = wave_rank_sort64(asc, buf[0]);
      if (lane < K) sel_idx[(size_t)bkv * K + lane] = asc ? (int)(0xffffffffull - (asc - 1)) : -1;
    } else if (lane < K) {
      dst[lane] = top;
    }
  }
}

template <int W, int NIT, bool kFinal>
void launch_score(dim3 grid, hipStream_t st, const Geometry& g, const uint16_t* q,
                  const uint16_t* lmk, const float* bias, int ncand, int cps, int nsplit,
                  int idbits, uint64_t* lists, int32_t* sel_idx) {
  if (bias)
    hipLaunchKernelGGL((decode_score_select<W, NIT, true, kFinal>), grid, dim3(W * kWave), 0, st, g,
                       q, lmk, bias, ncand, cps, nsplit, idbits, lists, sel_idx);
  else
    hipLaunchKernelGGL((decode_score_select<W, NIT, false, kFinal>), grid, dim3(W * kWave), 0, st,
                       g, q, lmk, bias, ncand, cps, nsplit, idbits, lists, sel_idx);
}

// ----------------------------------------------------------------------------
// 2. merge the nsplit local lists of one (b, kv head); write ascending ids.
// ----------------------------------------------------------------------------
// kMergeWaves = 1 when there are few lists: one wave merges them all, with no
// workgroup barriers.
template <int kMergeWaves>
__global__ void __launch_bounds__(kMergeWaves * kWave)
decode_merge(Geometry g, int nsplit, const uint64_t* __restrict__ lists,
             int32_t* __restrict__ sel_idx) {
  __shared__ uint64_t buf[kMergeWaves][kWave];
  __shared__ uint64_t wl[kMergeWaves][kWave];
  const int bkv = blockIdx.x;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const uint64_t* src = lists + (size_t)bkv * nsplit * g.K;
  // each wave merges every kMergeWaves-th local list (each sorted descending), with
  // the loads of eight lists issued before their merges (the merges' LDS
  // fences would otherwise hold every load back until the previous merge) ...
  uint64_t run = 0;
  for (int j0 = w; j0 < nsplit; j0 += 8 * kMergeWaves) {
    uint64_t key[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int j = j0 + x * kMergeWaves;
      key[x] = (j < nsplit && lane < g.K) ? src[(size_t)j * g.K + lane] : 0ull;
    }
#pragma unroll
    for (int x = 0; x < 8; ++x)
      if (j0 + x * kMergeWaves < nsplit)
        run = (j0 == w && x == 0) ? key[0] : wave_merge_into(run, key[x], g.K, buf[w]);
  }
  wl[w][lane] = lane < g.K ? run : 0ull;
  __syncthreads();
  // ... then the wave lists are merged pairwise in a tree
  for (int half = kMergeWaves / 2; half >= 1; half >>= 1) {
    if (w < half) {
      const uint64_t mine = wl[w][lane], other = wl[w + half][lane];
      const uint64_t mg = wave_merge_into(mine, other, g.K, buf[w]);
      wl[w][lane] = lane < g.K ? mg : 0ull;
    }
    __syncthreads();
  }
  if (w == 0) {
    // ascending ids: a rank sort of the complemented ids (unique, 0 = none)
    const uint64_t top = wl[0][lane];
    uint64_t asc = (lane < g.K && top != 0) ? (0xffffffffull - (uint64_t)key_index(top)) + 1 : 0;
    asc = wave_rank_sort64(asc, buf[0]);
    if (lane < g.K) sel_idx[(size_t)bkv * g.K + lane] = asc ? (int)(0xffffffffull - (asc - 1)) : -1;
  }
}

// ----------------------------------------------------------------------------
// 3. chunk attention with online fusion.  grid (nsplit, B*Hkv): workgroup
//    `split` walks fusion slots [split*apc, split*apc + apc) of its (b, kv
//    head) -- slot < K is the slot-th selected chunk, slot K + j the local
//    window's chunk own - j -- reading each chunk's 16 KB of K and 16 KB of V
//    once for all G heads: K into registers (thread -> key, quarter of the
//    dims), V by direct global->LDS copies, both issued before any arithmetic.
//    Per head it keeps (M, Z, O) = (max s, sum e^{s-M}, sum e^{s-M} o_c) over
//    its chunks, s the retrieval score (a window chunk: its exact lse), and
//    writes them as a partial.  No cross-chunk prefetch: with the registers
//    that frees, more workgroups stay resident and hide each other's loads.
// ----------------------------------------------------------------------------
constexpr int kPartStride = kD + 4;   // O[128], M, Z, pad  (floats)

// Any G up to 16: thread t holds a quarter of key t/4's dims and two lane
// swaps finish each (key, head) dot product.
__global__ void __launch_bounds__(kThreads)
decode_attend(Geometry g, int apc, const uint16_t* __restrict__ q, const uint16_t* __restrict__ qr,
              const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
              const uint16_t* __restrict__ lmk,
              const float* __restrict__ bias, const int32_t* __restrict__ sel_idx,
              float* __restrict__ parts) {
  __shared__ __attribute__((aligned(16))) float qs[kMaxGd][kD];
  __shared__ float lg[kMaxGd][kS];
  __shared__ __attribute__((aligned(16))) uint4 vs[kS * kD / 8];
  __shared__ float sc[kMaxGd];
  __shared__ int ca[8], cn[8], cc[8];
  const int split = blockIdx.x, bkv = blockIdx.y;
  const int nsplit = gridDim.x;
  const int b = bkv / g.Hkv, kvh = bkv % g.Hkv;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int G = g.G;
  const int t = g.Lkv - 1;

  // token ranges of this workgroup's slots
  if (tid < apc) {
    const int slot = split * apc + tid;
    int a = 0, n = 0, c = -1;
    if (slot < g.K) {
      c = sel_idx[(size_t)bkv * g.K + slot];
      if (c >= 0) { a = c * kS; n = kS; }
    } else {
      // local window slot j: chunk own - j (the own chunk's visible tokens for
      // j = 0), fused with its exact log-sum-exp
      const int j = slot - g.K, own = t / kS, cw = own - j;
      if (j < g.win && cw >= 0) {
        a = cw * kS;
        n = j == 0 ? t - a + 1 : kS;
      }
    }
    ca[tid] = a; cn[tid] = n; cc[tid] = c;
  }
  for (int x = tid; x < G * kD; x += kThreads)
    qs[x / kD][x % kD] = bf16_to_f32(q[(size_t)(b * g.Hq + kvh * G) * kD + x]);
  // retrieval query of this wave's heads (w, w+4, ..), lane -> dims 2l, 2l+1
  uint32_t qrv[kMaxGd / 4];
#pragma unroll
  for (int x = 0; x < kMaxGd / 4; ++x) {
    const int h = w + 4 * x;
    qrv[x] = h < G ? reinterpret_cast<const uint32_t*>(qr + (size_t)(b * g.Hq + kvh * G + h) * kD)[lane]
                   : 0u;
  }
  __syncthreads();

  const uint16_t* Kb = k + (size_t)bkv * g.Lkv * kD;
  const uint16_t* Vb = v + (size_t)bkv * g.Lkv * kD;
  const uint16_t* Lb = lmk + (size_t)bkv * g.NCcap * kD;
  const float* Bb = bias ? bias + (size_t)bkv * g.NCcap : nullptr;
  const int dp = tid & 63, hg = tid >> 6;      // PV: dims 2dp, 2dp+1 of heads hg, hg+4, ...
  const int wbase = w * kWave;
  float M[4], Z[4], O0[4], O1[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) { M[x] = -INFINITY; Z[x] = 0.f; O0[x] = 0.f; O1[x] = 0.f; }

  for (int s = 0; s < apc; ++s) {
    const int n = cn[s], c = cc[s];
    if (n == 0) continue;
    // all loads first: K rows into registers, V rows (full rows only: a
    // partial own chunk copies the rows it has) straight into LDS, landmark
    const uint16_t* Kc = Kb + (size_t)ca[s] * kD;
    const uint4* Vc = reinterpret_cast<const uint4*>(Vb + (size_t)ca[s] * kD);
    uint4 kr[4];
    {
      const int j = tid >> 2, qd = tid & 3;
#pragma unroll
      for (int p4 = 0; p4 < 4; ++p4)
        kr[p4] = j < n ? *reinterpret_cast<const uint4*>(Kc + (size_t)j * kD + qd * 32 + p4 * 8)
                       : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int idx = x * kThreads + tid;            // uint4 index within the chunk's V
      if (idx / (kD / 8) < n)
        __builtin_amdgcn_global_load_lds((const void*)(Vc + idx),
                                         (__attribute__((address_space(3))) void*)(vs + x * kThreads + wbase),
                                         16, 0, 0);
      else
        vs[idx] = make_uint4(0, 0, 0, 0);            // rows past a partial chunk: zero
    }
    const uint32_t lm = c >= 0 ? reinterpret_cast<const uint32_t*>(Lb + (size_t)c * kD)[tid & 63] : 0u;
    const float bc = (c >= 0 && Bb) ? Bb[c] : 0.f;
    {
      // logits: thread -> key j, 32 dims
      const int j = tid >> 2, qd = tid & 3;
      float kx[32];
#pragma unroll
      for (int p4 = 0; p4 < 4; ++p4) {
        const uint32_t u[4] = {kr[p4].x, kr[p4].y, kr[p4].z, kr[p4].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kx[p4 * 8 + 2 * e] = __uint_as_float(u[e] << 16);
          kx[p4 * 8 + 2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
        }
      }
      for (int h = 0; h < G; ++h) {
        float d4[4] = {0.f, 0.f, 0.f, 0.f};           // four independent chains
#pragma unroll
        for (int e = 0; e < 32; ++e) d4[e & 3] = __builtin_fmaf(qs[h][qd * 32 + e], kx[e], d4[e & 3]);
        float d = (d4[0] + d4[1]) + (d4[2] + d4[3]);
        d += lane_xor_f32<1>(d);
        d += lane_xor_f32<2>(d);
        if (qd == 0) lg[h][j] = j < n ? g.scale * d : -INFINITY;
      }
    }
    __syncthreads();
    // chunk softmax per head (wave w: heads w, w+4, ...) and the fusion score
#pragma unroll
    for (int x = 0; x < kMaxGd / 4; ++x) {
      const int h = w + 4 * x;
      if (h >= G) break;
      const float l = lg[h][lane];
      const float m = wave_max(l);
      const float e = __expf(l - m);
      const float z = wave_sum(e);
      lg[h][lane] = e / z;
      float sv;
      if (c >= 0) {
        const float ps = __uint_as_float(qrv[x] << 16) * __uint_as_float(lm << 16) +
                         __uint_as_float(qrv[x] & 0xffff0000u) * __uint_as_float(lm & 0xffff0000u);
        sv = g.scale * wave_sum(ps) + bc;
      } else {
        sv = m + __logf(z);   // window chunk: its exact log-sum-exp
      }
      if (lane == 0) sc[h] = sv;
    }
    __builtin_amdgcn_s_waitcnt(0);   // this thread's V copies have landed
    __syncthreads();
    // o_c = P V, folded into the running (M, Z, O) of each head
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int h = hg + 4 * x;
      if (h >= G) break;
      float a0[4] = {0.f, 0.f, 0.f, 0.f}, a1[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 16
      for (int jj = 0; jj < kS; ++jj) {   // rows past a partial chunk are zero (p too)
        const uint32_t pr = reinterpret_cast<const uint32_t*>(vs)[jj * (kD / 2) + dp];
        const float pj = lg[h][jj];
        a0[jj & 3] = __builtin_fmaf(pj, __uint_as_float(pr << 16), a0[jj & 3]);
        a1[jj & 3] = __builtin_fmaf(pj, __uint_as_float(pr & 0xffff0000u), a1[jj & 3]);
      }
      const float o0 = (a0[0] + a0[1]) + (a0[2] + a0[3]);
      const float o1 = (a1[0] + a1[1]) + (a1[2] + a1[3]);
      const float sv = sc[h];
      const float mn = fmaxf(M[x], sv);
      const float fo = __expf(M[x] - mn), fn = __expf(sv - mn);
      Z[x] = Z[x] * fo + fn;
      O0[x] = O0[x] * fo + fn * o0;
      O1[x] = O1[x] * fo + fn * o1;
      M[x] = mn;
    }
    __syncthreads();
  }
  float* part = parts + ((size_t)bkv * nsplit + split) * G * kPartStride;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int h = hg + 4 * x;
    if (h >= G) break;
    float* ph = part + (size_t)h * kPartStride;
    reinterpret_cast<float2*>(ph)[dp] = make_float2(O0[x], O1[x]);
    if (dp == 0) { ph[kD] = M[x]; ph[kD + 1] = Z[x]; }
  }
}

// G = 4: the same walk with both products on 16x16x32 bf16 MFMA, so that a
// workgroup needs few registers and 18 KB of LDS and many stay resident while
// others wait for their chunks.  Logits: wave w multiplies keys 16w .. 16w+15
// (A operand, straight from the K rows in registers) by the four queries (B
// operand columns 0..3, the other twelve zero).  Wave w then owns head w: its
// chunk softmax, the retrieval score, and P rounded to bf16.  O_c = P V: the
// four P rows sit in A rows 0, 4, 8, 12 (the rest zero), so one MFMA chain
// serves every head, and V (copied to LDS with chunk c of row r stored at
// position c ^ 2(r % 4)) comes in as the B operand by transpose reads.
// Keys r0 .. r0+3 (r0 % 4 == 0) at dim 16db + l%16 of the swizzled V rows, by
// an LDS transpose read: source lane t of a 16-lane group points at key
// r0 + t/4, dims 16db + 4(t%4) .. +3; lane i receives the four keys at dim
// 16db + i.
__device__ __forceinline__ uint2 v_rows4_at_dim(const uint4* __restrict__ vs, int r0, int db) {
  const int t = lane_id() & 15;
  const int row = r0 + (t >> 2);
  const int slot = (2 * db + ((t & 3) >> 1)) ^ (2 * (row & 3));
  const char* p = reinterpret_cast<const char*>(vs + row * (kD / 8) + slot) + 8 * (t & 1);
  const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)p);
  uint2 u;
  __builtin_memcpy(&u, &v, 8);
  return u;
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// (88 registers: five waves per SIMD, so five workgroups per CU)
__global__ void __launch_bounds__(kThreads)
decode_attend4(Geometry g, int apc, const uint16_t* __restrict__ q, const uint16_t* __restrict__ qr,
               const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
               const uint16_t* __restrict__ lmk, const float* __restrict__ bias,
               const int32_t* __restrict__ sel_idx, float* __restrict__ parts) {
  __shared__ __attribute__((aligned(16))) uint4 vs[kS * kD / 8];
  __shared__ float lg[4][kS];
  __shared__ __attribute__((aligned(16))) uint16_t pb[4][kS];
  __shared__ float sc[4];
  __shared__ int ca[8], cn[8], cc[8];
  const int split = blockIdx.x, bkv = blockIdx.y;
  const int nsplit = gridDim.x;
  const int b = bkv / g.Hkv, kvh = bkv % g.Hkv;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave, cs = tid & 15;
  const int t = g.Lkv - 1;

  if (tid < apc) {
    const int slot = split * apc + tid;
    int a = 0, n = 0, c = -1;
    if (slot < g.K) {
      c = sel_idx[(size_t)bkv * g.K + slot];
      if (c >= 0) { a = c * kS; n = kS; }
    } else {
      const int j = slot - g.K, own = t / kS, cw = own - j;
      if (j < g.win && cw >= 0) {
        a = cw * kS;
        n = j == 0 ? t - a + 1 : kS;
      }
    }
    ca[tid] = a; cn[tid] = n; cc[tid] = c;
  }
  const uint16_t* qg = q + (size_t)(b * g.Hq + kvh * 4) * kD;
  // B operand of S^T = K Q^T: column n < 4 is head n (dims 32ks + 8(l/16) ..
  // +7 in lane l), the other twelve columns zero
  bf16x8 qb[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    qb[ks] = cs < 4 ? as_bf16x8(reinterpret_cast<const uint4*>(qg + cs * kD + 32 * ks + 8 * (lane >> 4))[0])
                    : as_bf16x8(make_uint4(0, 0, 0, 0));
  const uint32_t qrv = reinterpret_cast<const uint32_t*>(qr + (size_t)(b * g.Hq + kvh * 4 + w) * kD)[lane];
  __syncthreads();

  const uint16_t* Kb = k + (size_t)bkv * g.Lkv * kD;
  const uint16_t* Vb = v + (size_t)bkv * g.Lkv * kD;
  const uint16_t* Lb = lmk + (size_t)bkv * g.NCcap * kD;
  const float* Bb = bias ? bias + (size_t)bkv * g.NCcap : nullptr;
  const int wbase = w * kWave;
  const uint32_t* vw = reinterpret_cast<const uint32_t*>(vs);
  // lane l of wave w: head l/16, dims 32w + l%16 and 32w + 16 + l%16
  float M = -INFINITY, Z = 0.f, O0 = 0.f, O1 = 0.f;

  for (int s = 0; s < apc; ++s) {
    const int n = cn[s], c = cc[s];
    if (n == 0) continue;
    const uint4* Kc = reinterpret_cast<const uint4*>(Kb + (size_t)ca[s] * kD);
    const uint4* Vc = reinterpret_cast<const uint4*>(Vb + (size_t)ca[s] * kD);
    // A operand: wave w's keys 16w + l%16, dims 32ks + 8(l/16) .. +7
    bf16x8 kr[4];
    {
      const int key = 16 * w + (lane & 15);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        kr[ks] = key < n ? as_bf16x8(Kc[key * (kD / 8) + 4 * ks + (lane >> 4)]) : as_bf16x8(make_uint4(0, 0, 0, 0));
    }
    // V rows into LDS row-major, chunk j of row r at position j ^ 2(r%4) (so
    // that the transpose reads below hit distinct banks); rows past a partial
    // chunk are zero
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int idx = x * kThreads + tid;             // LDS position: row idx/16, slot idx%16
      const int row = idx / (kD / 8);
      if (row < n)
        __builtin_amdgcn_global_load_lds((const void*)(Vc + row * (kD / 8) + ((idx & 15) ^ (2 * (row & 3)))),
                                         (__attribute__((address_space(3))) void*)(vs + x * kThreads + wbase),
                                         16, 0, 0);
      else
        vs[idx] = make_uint4(0, 0, 0, 0);
    }
    const uint32_t lm = c >= 0 ? reinterpret_cast<const uint32_t*>(Lb + (size_t)c * kD)[lane] : 0u;
    const float bc = (c >= 0 && Bb) ? Bb[c] : 0.f;
    {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = mfma(kr[ks], qb[ks], acc);
      // lane l: head l%16 (valid below 4), keys 16w + 4(l/16) + i
      if (cs < 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * w + 4 * (lane >> 4) + i;
          lg[cs][row] = row < n ? g.scale * acc[i] : -INFINITY;
        }
      }
    }
    __syncthreads();
    // head w: chunk softmax, P as bf16, retrieval score (window chunk: its lse)
    const float l = lg[w][lane];
    const float m = wave_max(l);
    const float e = __expf(l - m);
    const float z = wave_sum(e);
    pb[w][lane] = f32_to_bf16(e * __builtin_amdgcn_rcpf(z));
    const float sv = c >= 0 ? g.scale * wave_sum(dot2_bf16(qrv, lm, 0.f)) + bc : m + __logf(z);
    if (lane == 0) sc[w] = sv;
    __builtin_amdgcn_s_waitcnt(0);   // this thread's V copies have landed
    __syncthreads();
    // o_c = P V by MFMA: head h is row 4h of the 16 (the other rows zero), so
    // it comes out in lane group h; k = keys, columns = this wave's dims 32w ..
    // 32w + 31.  P (A operand) from the bf16 rows above; V (B operand: 8 keys
    // at one dim per lane) from LDS transpose reads, each handing a lane four
    // consecutive keys at its dim
    bf16x8 pa[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      pa[ks] = (lane & 3) == 0
                   ? as_bf16x8(*reinterpret_cast<const uint4*>(&pb[(lane & 15) >> 2][32 * ks + 8 * (lane >> 4)]))
                   : as_bf16x8(make_uint4(0, 0, 0, 0));
    f32x4 oc[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      oc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int r0 = 32 * ks + 8 * (lane >> 4);
        const uint2 lo = v_rows4_at_dim(vs, r0, 2 * w + nt);
        const uint2 hi = v_rows4_at_dim(vs, r0 + 4, 2 * w + nt);
        oc[nt] = mfma(pa[ks], as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), oc[nt]);
      }
    }
    // lane l holds o_c[head l/16][dim 32w + 16nt + l%16] in oc[nt][0]
    {
      const float svh = sc[lane >> 4];
      const float mn = fmaxf(M, svh);
      const float fo = __expf(M - mn), fn = __expf(svh - mn);
      Z = Z * fo + fn;
      O0 = O0 * fo + fn * oc[0][0];
      O1 = O1 * fo + fn * oc[1][0];
      M = mn;
    }
    __syncthreads();
  }
  float* ph = parts + (((size_t)bkv * nsplit + split) * 4 + (lane >> 4)) * kPartStride;
  ph[32 * w + (lane & 15)] = O0;
  ph[32 * w + 16 + (lane & 15)] = O1;
  if (w == 0 && (lane & 15) == 0) { ph[kD] = M; ph[kD + 1] = Z; }
}

// ----------------------------------------------------------------------------
// 4. merge of the nsplit partials of each (b, q head): one workgroup per row;
//    wave w of W takes splits w, w + W, ...; lane -> dims 2l, 2l+1.  With few
//    rows (fewer workgroups than CUs) sixteen waves keep each wave's chain of
//    partial loads short (at most five of the 65 partials of a decode_4m row);
//    with many rows four waves per row launch faster.
//    O = sum_s e^{M_s - M} O_s / sum_s e^{M_s - M} Z_s,  LSE = M + log(...).
// ----------------------------------------------------------------------------
template <int W>
__global__ void __launch_bounds__(W * kWave)
decode_fuse(Geometry g, int nsplit, const float* __restrict__ parts, uint16_t* __restrict__ out,
            float* __restrict__ lse_out) {
  constexpr int kFuseWaves = W;
  __shared__ float red[kFuseWaves][2 * kWave + 2];
  const int row = blockIdx.x;                  // b * Hq + hq
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int b = row / g.Hq, hq = row % g.Hq;
  const int kvh = hq / g.G, h = hq % g.G;
  const int bkv = b * g.Hkv + kvh;
  const size_t sstride = (size_t)g.G * kPartStride;
  const float* pb = parts + (size_t)bkv * nsplit * sstride + (size_t)h * kPartStride;
  float m = -INFINITY;
  for (int s0 = 0; s0 < nsplit; s0 += kWave) {
    const int si = s0 + lane;
    m = fmaxf(m, wave_max(si < nsplit ? pb[si * sstride + kD] : -INFINITY));
  }
  float z = 0.f, o0 = 0.f, o1 = 0.f;
  if (m != -INFINITY) {
#pragma unroll 4
    for (int s = w; s < nsplit; s += kFuseWaves) {
      const float* ps = pb + s * sstride;
      const float2 ov = reinterpret_cast<const float2*>(ps)[lane];
      const float ms = ps[kD];
      const float f = ms == -INFINITY ? 0.f : __expf(ms - m);
      z = __builtin_fmaf(f, ps[kD + 1], z);
      o0 = __builtin_fmaf(f, ov.x, o0);
      o1 = __builtin_fmaf(f, ov.y, o1);
    }
  }
  red[w][2 * lane] = o0;
  red[w][2 * lane + 1] = o1;
  if (lane == 0) red[w][2 * kWave] = z;
  __syncthreads();
  if (w == 0) {
    float zt = 0.f, a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int x = 0; x < kFuseWaves; ++x) {
      zt += red[x][2 * kWave];
      a0 += red[x][2 * lane];
      a1 += red[x][2 * lane + 1];
    }
    const float inv = zt > 0.f ? 1.f / zt : 0.f;
    const uint32_t pk = (uint32_t)f32_to_bf16(a0 * inv) | ((uint32_t)f32_to_bf16(a1 * inv) << 16);
    reinterpret_cast<uint32_t*>(out + (size_t)row * kD)[lane] = pk;
    if (lane == 0 && lse_out) lse_out[row] = zt > 0.f ? m + __logf(zt) : -INFINITY;
  }
}

struct DecodePlan {
  int ncand, nit, cps, nsplit, idbits;
  bool fused;           // one 8-wave scoring workgroup per (b, kv head) writes the selection
  int apc, asplit;      // attention: fusion slots per workgroup, workgroups per (b, kv head)
};

DecodePlan plan(const Geometry& g) {
  DecodePlan p;
  const int t = g.Lkv - 1;
  p.ncand = max(0, min(t / kS - max(g.win - 1, 0), g.NC));   // chunks before the window
  const int bkv = g.B * g.Hkv;
  // scoring, fused: when eight waves of up to kMaxIt blocks cover a pair's
  // candidates and the pairs fill at least half the CUs, one workgroup per
  // pair scores, selects and writes the ascending ids itself (no list merge
  // launch).  Split: about 256 workgroups (one per CU), each streaming up to
  // kMaxIt blocks of 64 candidates per wave; fewer, longer splits leave fewer
  // lists to merge (at 16 x 8 (b, kv head) pairs and 2047 candidates, two
  // splits of four blocks per wave beat four splits of two by about 2 us).
  p.fused = p.ncand <= 8 * kMaxIt * kWave && bkv >= 128;
  if (p.fused) {
    p.nit = max(1, (p.ncand + 8 * kWave - 1) / (8 * kWave));
    p.cps = 8 * kWave * p.nit;
    p.nsplit = 1;
  } else {
    const int want_splits = max(1, 256 / max(1, bkv));
    const int per = (p.ncand + want_splits - 1) / want_splits;
    p.nit = min(kMaxIt, max(1, (per + 255) / 256));
    p.cps = 256 * p.nit;
    p.nsplit = max(1, (p.ncand + p.cps - 1) / p.cps);
  }
  p.idbits = 1;
  while (p.idbits < 32 && (1ll << p.idbits) < (long long)max(p.ncand, 1)) ++p.idbits;
  // attention: one fusion slot per workgroup (latency hidden by parallelism)
  // unless that gives fewer than 256 workgroups; then up to 8 per workgroup
  const int nslot = max(1, g.K + g.win);
  p.apc = min(8, max(1, 256 / max(1, nslot * bkv)));
  p.asplit = (nslot + p.apc - 1) / p.apc;
  return p;
}

DecodeWs carve(const Geometry& g, const DecodePlan& p, void* ws) {
  DecodeWs d;
  char* c = reinterpret_cast<char*>(ws);
  size_t off = 0;
  d.lists = reinterpret_cast<uint64_t*>(c + off);
  off += ((size_t)g.B * g.Hkv * p.nsplit * g.K * 8 + 255) & ~(size_t)255;
  d.parts = reinterpret_cast<float*>(c + off);
  return d;
}

}  // namespace

bool decode_fast_supported(const Geometry& g, int bf16) {
  return bf16 && g.d == kD && g.S == kS && g.G <= kMaxGd && g.K <= kMaxTopK && g.Lq == 1 &&
         g.causal;
}

size_t decode_fast_ws(const Geometry& g) {
  DecodePlan p = plan(g);
  size_t off = ((size_t)g.B * g.Hkv * p.nsplit * g.K * 8 + 255) & ~(size_t)255;
  off += ((size_t)g.B * g.Hkv * (g.K + g.win + 1) * g.G * kPartStride * 4 + 255) & ~(size_t)255;
  return off;
}

hipError_t launch_decode_fast(const Geometry& g, const void* q, const void* qr, const void* k,
                              const void* v, const void* lmk, const float* bias, void* out,
                              int32_t* sel_idx, float* lse, void* ws, hipStream_t st) {
  DecodePlan p = plan(g);
  DecodeWs d = carve(g, p, ws);
  const int bkv = g.B * g.Hkv;
  const uint16_t* Q = (const uint16_t*)q;
  const uint16_t* QR = (const uint16_t*)qr;
  const uint16_t* Lm = (const uint16_t*)lmk;
  dim3 g1(p.nsplit, bkv);
  prof_begin(kDecodeScore, st);
  static_assert(kMaxIt == 4, "one scoring instance per block count");
  if (p.fused) {
    switch (p.nit) {
      case 1: launch_score<8, 1, true>(g1, st, g, QR, Lm, bias, p.ncand, p.cps, 1, p.idbits, d.lists, sel_idx); break;
      case 2: launch_score<8, 2, true>(g1, st, g, QR, Lm, bias, p.ncand, p.cps, 1, p.idbits, d.lists, sel_idx); break;
      case 3: launch_score<8, 3, true>(g1, st, g, QR, Lm, bias, p.ncand, p.cps, 1, p.idbits, d.lists, sel_idx); break;
      default: launch_score<8, 4, true>(g1, st, g, QR, Lm, bias, p.ncand, p.cps, 1, p.idbits, d.lists, sel_idx); break;
    }
  } else {
    switch (p.nit) {
      case 1: launch_score<4, 1, false>(g1, st, g, QR, Lm, bias, p.ncand, p.cps, p.nsplit, p.idbits, d.lists, sel_idx); break;
      case 2: launch_score<4, 2, false>(g1, st, g, QR, Lm, bias, p.ncand, p.cps, p.nsplit, p.idbits, d.lists, sel_idx); break;
      case 3: launch_score<4, 3, false>(g1, st, g, QR, Lm, bias, p.ncand, p.cps, p.nsplit, p.idbits, d.lists, sel_idx); break;
      default: launch_score<4, 4, false>(g1, st, g, QR, Lm, bias, p.ncand, p.cps, p.nsplit, p.idbits, d.lists, sel_idx); break;
    }
  }
  prof_end(kDecodeScore, st);
  if (!p.fused) {
    prof_begin(kDecodeMerge, st);
    if (p.nsplit <= 8)
      hipLaunchKernelGGL(decode_merge<1>, dim3(bkv), dim3(kWave), 0, st, g, p.nsplit, d.lists, sel_idx);
    else
      hipLaunchKernelGGL(decode_merge<16>, dim3(bkv), dim3(16 * kWave), 0, st, g, p.nsplit, d.lists,
                         sel_idx);
    prof_end(kDecodeMerge, st);
  }
  prof_begin(kDecodeAttend, st);
  if (g.G == 4)
    hipLaunchKernelGGL(decode_attend4, dim3(p.asplit, bkv), dim3(kThreads), 0, st, g, p.apc,
                       Q, QR, (const uint16_t*)k, (const uint16_t*)v, Lm, bias, sel_idx, d.parts);
  else
    hipLaunchKernelGGL(decode_attend, dim3(p.asplit, bkv), dim3(kThreads), 0, st, g, p.apc,
                       Q, QR, (const uint16_t*)k, (const uint16_t*)v, Lm, bias, sel_idx, d.parts);
  prof_end(kDecodeAttend, st);
  if (g.B * g.Hq < 256)
    hipLaunchKernelGGL(decode_fuse<16>, dim3(g.B * g.Hq), dim3(16 * kWave), 0, st, g, p.asplit, d.parts,
                       (uint16_t*)out, lse);
  else
    hipLaunchKernelGGL(decode_fuse<4>, dim3(g.B * g.Hq), dim3(4 * kWave), 0, st, g, p.asplit, d.parts,
                       (uint16_t*)out, lse);
  return hipGetLastError();
}

}  // namespace hils
