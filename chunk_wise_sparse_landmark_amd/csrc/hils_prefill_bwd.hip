// MFMA backward of the prefill path: bf16, head_dim 128, chunk 64, GQA group
// of 4, causal, seq_q == seq_kv (the shapes the MFMA forward covers), up to 256
// chunks with K <= 32 and up to 512 chunks (32K tokens) with K <= 16.
//
// Method: Hierarchical Sparse Attention Done Right (arXiv 2607.02980v1, summary
// page), §3 "Hierarchical softmax" (gradients of the LM loss reach the chunk
// retrieval scores through the fusion weights) and §9 (unselected chunks get no
// gradient).  With the selection fixed, for a query row with fusion weights w_c
// (w_c = exp(s_c - LSE); a local-window chunk's score is its exact lse_c) and
// chunk softmaxes p:
//   D   = <dO, O>,  u_j = <dO, v_j>,  D_c = sum_j p_j u_j
//   retrieved chunk: dl_j = w_c p_j (u_j - D_c),  ds_c = w_c (D_c - D)
//   window chunk:    dl_j = w_c p_j (u_j - D)
//   dq = scale (sum_j dl_j k_j + sum_c ds_c lmk_c),  dk_j += scale dl_j q,
//   dv_j += w p_j dO,  dlmk_c += scale ds_c q,  dbias_c += ds_c.
//
// Three launches:
//  1. prefill_bwd_prep    per (b, kv head, 64-query window): the window's
//     chunk of K and V in operand-fragment order, D per row, and the (query,
//     chunk) -> slot map with per-window query masks.
//  2. prefill_bwd_rows    per window (like the forward's attention kernel):
//     for every chunk of the window's union, S^T = K Q^T and U^T = V dO^T by
//     MFMA, the chunk softmax, D_c, dl, and dQ += dL K in MFMA accumulators;
//     each (row, slot)'s (w, log2 lse_c, D_c) goes to a table; after the loop
//     dq gains scale * sum ds_c lmk_c.
//  3. prefill_bwd_chunks  per (b, kv head, chunk): gathers the queries that
//     selected the chunk (and those whose local window holds it) in tiles of 8 queries x
//     4 heads = 32 rows (q and dO read once, straight from the inputs; the
//     transposed operands come from LDS transpose reads), recomputes S = Q K^T
//     and U = dO V^T for the wave's 16
//     keys, turns them into w p and dl with the row table (no reductions), and
//     accumulates dV += (w P)^T dO and dK += dL^T Q by MFMA over the rows, plus
//     dlmk and dbias.  Each chunk is owned by one workgroup: no atomics.
#include "hils_mfma.h"
#include "hils_kernels.h"
#include "hils_profile.h"

namespace hils {

namespace {

constexpr int kD = 128;
constexpr int kS = 64;
constexpr int kG = 4;
constexpr int kWin = 64;
constexpr int kMaxKb = 32;
constexpr int kMaxNCb = 512;                       // chunks bound on this path (L <= 32768)
// the rows pass keeps per-(query, slot) and per-(query, chunk) tables in LDS
// next to two 48 KB chunk buffers: up to 256 chunks with K <= 32, up to 512
// chunks with K <= 16
constexpr int kRowsNarrowNC = 256;
constexpr int kRowsWideK = 16;
constexpr int kFragE = kWave * 8;                  // bf16 per fragment
constexpr int kBwdFrags = 48;                      // K (A), V (A), K (B, P order)
constexpr int kBwdChunkElems = kBwdFrags * kFragE; // 48 KB per chunk
constexpr int kRowWaves = 8;
constexpr int kRowThreads = kRowWaves * kWave;
constexpr int kRowBlocks = kWin / 4 / kRowWaves;   // query blocks per wave
constexpr int kPrepThreads = 256;
constexpr int kChunkThreads = 256;
constexpr int kPlanThreads = kMaxNCb;              // one thread per chunk
constexpr int kTilesPerItem = 64;                  // 512 (query, chunk) pairs per work item
constexpr int kPartFloats = 2 * kS * kD + kD + 4;  // dV, dK, dlmk, dbias (+pad to 16 B)

// Upper bound of the work items of one (b, kv head): a query selects at most K
// chunks, so the retrieved tiles number at most L*K/8 plus one partial tile per
// chunk; each chunk adds the tiles of the local windows that hold it (8 per
// window) and at most one short item.
int max_items_of(const Geometry& g) {
  const long tiles = (long)g.Lq * g.K / 8 + g.NC + (long)g.NC * (kWin / 8) * max(g.win, 1);
  return (int)(tiles / kTilesPerItem + 2 * g.NC + 1);
}

struct BwdWs {
  uint16_t* frags;   // [bkv][NC][48 fragments][64 lanes][8]
  float* Drow;       // [B][Hq][L]
  float4* stats;     // [B][Hq][L][K+win]: (w, log2 lse_c, D_c (window: D), ds_c (window: 0))
  uint64_t* qm;      // [bkv][NW][NC]: window queries that selected chunk c
  uint8_t* slot;     // [bkv][L][NC]: slot of chunk c in query i's selection, 0xff if none
  int4* items;       // [bkv][max_items]: (chunk, first tile, end tile, partial slot or -1)
  int* nitems;       // [bkv]
  int2* chunkseg;    // [bkv][NC]: (first partial slot, number of items)
  float* part;       // [bkv * max_items][kPartFloats]: partial dV, dK, dlmk, dbias
  int max_items;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

BwdWs carve(const Geometry& g, void* base, size_t* total) {
  const size_t nbkv = (size_t)g.B * g.Hkv, L = g.Lq, NW = L / kWin;
  size_t off = 0;
  char* c = reinterpret_cast<char*>(base);
  BwdWs w;
  w.frags = reinterpret_cast<uint16_t*>(c + off);
  off += align256(nbkv * g.NC * kBwdChunkElems * 2);
  w.Drow = reinterpret_cast<float*>(c + off);
  off += align256((size_t)g.B * g.Hq * L * 4);
  w.stats = reinterpret_cast<float4*>(c + off);
  off += align256((size_t)g.B * g.Hq * L * (g.K + g.win) * 16);
  w.qm = reinterpret_cast<uint64_t*>(c + off);
  off += align256(nbkv * NW * g.NC * 8);
  w.slot = reinterpret_cast<uint8_t*>(c + off);
  off += align256(nbkv * L * g.NC);
  w.max_items = max_items_of(g);
  w.items = reinterpret_cast<int4*>(c + off);
  off += align256(nbkv * w.max_items * 16);
  w.nitems = reinterpret_cast<int*>(c + off);
  off += align256(nbkv * 4);
  w.chunkseg = reinterpret_cast<int2*>(c + off);
  off += align256(nbkv * g.NC * 8);
  w.part = reinterpret_cast<float*>(c + off);
  off += align256(nbkv * (size_t)w.max_items * kPartFloats * 4);
  if (total) *total = off;
  return w;
}

// ----------------------------------------------------------------------------
// 1. prep
//    fragment f, lane l, element j:
//      f <  16 (mt*4+ks):   K[16mt + l%16][32ks + 8(l/16) + j]   A of S^T = K Q^T
//      f <  32 (16+mt*4+ks): V, same                              A of U^T = V dO^T
//      f <  48 (32+db*2+ks): K[32ks + 16(j/4) + 4(l/16) + j%4][16db + l%16]
//                            B of dQ = dL K, keys in the order dL leaves S^T
// ----------------------------------------------------------------------------
template <int NCB>
__global__ void __launch_bounds__(kPrepThreads)
prefill_bwd_prep(Geometry g, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                 const uint16_t* __restrict__ v, const uint16_t* __restrict__ out,
                 const uint16_t* __restrict__ dout, const int32_t* __restrict__ sel_idx,
                 BwdWs ws) {
  __shared__ __attribute__((aligned(16))) uint16_t ks_[kS * kD];
  __shared__ __attribute__((aligned(16))) uint16_t vs_[kS * kD];
  __shared__ uint64_t qmask[NCB];
  __shared__ uint8_t slots[kWin * NCB];
  const int nbkv = g.B * g.Hkv;
  const int bkv = blockIdx.x % nbkv, win = blockIdx.x / nbkv;
  const int b = bkv / g.Hkv, kvh = bkv % g.Hkv;
  const int tid = threadIdx.x;
  const int L = g.Lq, NW = L / kWin;
  const size_t row0 = (size_t)bkv * L + (size_t)win * kS;
  for (int x = tid; x < kS * kD / 8; x += kPrepThreads) {
    reinterpret_cast<uint4*>(ks_)[x] = reinterpret_cast<const uint4*>(k + row0 * kD)[x];
    reinterpret_cast<uint4*>(vs_)[x] = reinterpret_cast<const uint4*>(v + row0 * kD)[x];
  }
  for (int c = tid; c < NCB; c += kPrepThreads) qmask[c] = 0ull;
  for (int x = tid; x < kWin * NCB / 4; x += kPrepThreads)
    reinterpret_cast<uint32_t*>(slots)[x] = 0xffffffffu;
  __syncthreads();

  uint16_t* fd = ws.frags + ((size_t)bkv * g.NC + win) * kBwdChunkElems;
  for (int e = tid; e < kBwdFrags * kWave; e += kPrepThreads) {
    const int f = e / kWave, l = e % kWave;
    uint4 val;
    if (f < 32) {
      const uint16_t* src = f < 16 ? ks_ : vs_;
      const int mt = (f % 16) / 4, kk = f % 4;
      val = *reinterpret_cast<const uint4*>(src + (16 * mt + l % 16) * kD + 32 * kk + 8 * (l / 16));
    } else {
      const int db = (f - 32) / 2, kk = (f - 32) % 2;
      uint32_t wd[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        uint32_t h2[2];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const int j = jj * 2 + x;
          const int key = 32 * kk + 16 * (j / 4) + 4 * (l / 16) + (j % 4);
          h2[x] = ks_[key * kD + 16 * db + (l % 16)];
        }
        wd[jj] = h2[0] | (h2[1] << 16);
      }
      val = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    }
    reinterpret_cast<uint4*>(fd)[e] = val;
  }

  // D = <dO, O> per (query, head)
  {
    const int qq = tid >> 2, h = tid & 3;
    const size_t row = (size_t)(b * g.Hq + kvh * kG + h) * L + win * kWin + qq;
    const uint4* po = reinterpret_cast<const uint4*>(out + row * kD);
    const uint4* pd = reinterpret_cast<const uint4*>(dout + row * kD);
    float acc = 0.f;
#pragma unroll
    for (int x = 0; x < kD / 8; ++x) {
      const uint4 a = po[x], c = pd[x];
      const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, cw[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc += __uint_as_float(aw[e] << 16) * __uint_as_float(cw[e] << 16);
        acc += __uint_as_float(aw[e] & 0xffff0000u) * __uint_as_float(cw[e] & 0xffff0000u);
      }
    }
    ws.Drow[row] = acc;
  }

  // selection masks and slots of this window's queries
  for (int x = tid; x < kWin * g.K; x += kPrepThreads) {
    const int qq = x / g.K, s = x % g.K;
    const int c = sel_idx[((size_t)bkv * L + win * kWin + qq) * g.K + s];
    if (c >= 0) {
      atomicOr((unsigned long long*)&qmask[c], 1ull << qq);
      slots[qq * NCB + c] = (uint8_t)s;
    }
  }
  __syncthreads();
  for (int c = tid; c < g.NC; c += kPrepThreads)
    ws.qm[((size_t)bkv * NW + win) * g.NC + c] = qmask[c];
  // the window's 64 x NC slot bytes are one contiguous range that starts at a
  // multiple of 64 bytes (L and the window start are multiples of 64): four
  // bytes per store
  uint32_t* sw = reinterpret_cast<uint32_t*>(ws.slot + ((size_t)bkv * L + win * kWin) * g.NC);
  for (int x4 = tid; x4 < kWin * g.NC / 4; x4 += kPrepThreads) {
    uint32_t wd = 0;
    int qq = (4 * x4) / g.NC, c = 4 * x4 - qq * g.NC;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      wd |= (uint32_t)slots[qq * NCB + c] << (8 * e);
      if (++c == g.NC) { c = 0; ++qq; }
    }
    sw[x4] = wd;
  }
}

// ----------------------------------------------------------------------------
// 2. rows: dq and the per-(row, slot) table
// ----------------------------------------------------------------------------
template <int KB, int NCB>
struct RowsSmem {
  uint4 kv[2][kBwdFrags * kWave];     // 2 x 48 KB of chunk fragments
  float wts[kWin * KB * kG];          // (query, slot, head): weight, then ds
  uint8_t slotmap[kWin * NCB];        // (query, chunk) -> slot
  int sel[kWin * KB];
  uint64_t qmask[NCB];
  uint16_t ulist[NCB];
  float Dr[kWin * kG];
  float LSE2[kWin * kG];              // forward LSE in log2 units
  int wcount[kRowWaves];
};
static_assert(sizeof(RowsSmem<kMaxKb, kRowsNarrowNC>) <= 160 * 1024, "rows pass LDS");
static_assert(sizeof(RowsSmem<kRowsWideK, kMaxNCb>) <= 160 * 1024, "rows pass LDS");

__device__ __forceinline__ void stage48(const uint16_t* __restrict__ src, uint4* __restrict__ dst) {
  const uint4* s = reinterpret_cast<const uint4*>(src);
  const int wbase = (threadIdx.x / kWave) * kWave;
#pragma unroll
  for (int x = 0; x < kBwdFrags * kWave / kRowThreads; ++x)
    __builtin_amdgcn_global_load_lds((const void*)(s + x * kRowThreads + threadIdx.x),
                                     (__attribute__((address_space(3))) void*)(dst + x * kRowThreads + wbase),
                                     16, 0, 0);
}

__device__ __forceinline__ void stage_wait_all() { __builtin_amdgcn_s_waitcnt(0); }

__device__ __forceinline__ void load16(const uint4* __restrict__ src, bf16x8 (&f)[16]) {
  const int lane = lane_id();
#pragma unroll
  for (int x = 0; x < 16; ++x) f[x] = as_bf16x8(src[x * kWave + lane]);
}

// X^T = F Y^T for one block: F fragments (A, 64 keys) against the block's B
// fragments; lane l gets keys 16mt + 4(l/16) + i of row l%16.
__device__ __forceinline__ void keys_by_rows(const bf16x8 (&f)[16], const bf16x8 (&y)[4],
                                             f32x4 (&x)[4]) {
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = mfma(f[mt * 4 + ks], y[ks], acc);
    x[mt] = acc;
  }
  __builtin_amdgcn_s_setprio(0);
}

// dl (scaled values as bf16) in the A layout of dQ = dL K: k-slot (g4, j) <->
// key 32ks + 16(j/4) + 4g4 + j%4.
__device__ __forceinline__ void pack_keys(const f32x4 (&x)[4], bf16x8 (&pa)[2]) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    uint32_t w4[4];
    w4[0] = pack_bf16x2(x[2 * ks][0], x[2 * ks][1]);
    w4[1] = pack_bf16x2(x[2 * ks][2], x[2 * ks][3]);
    w4[2] = pack_bf16x2(x[2 * ks + 1][0], x[2 * ks + 1][1]);
    w4[3] = pack_bf16x2(x[2 * ks + 1][2], x[2 * ks + 1][3]);
    __builtin_memcpy(&pa[ks], w4, 16);
  }
}

// One block against one staged chunk.  Keys >= vis are hidden.  A local-window
// chunk (local): D_c := D and the weight exp(lse_c - LSE) is computed here from
// the chunk's lse; otherwise the weight is w_in.  Returns the row's
// (w, log2 lse_c, D_c) in lanes l < 16 (and in all lanes of the row group).
__device__ __forceinline__ float4 block_bwd(const uint4* kvb, const bf16x8 (&qf)[4],
                                            const bf16x8 (&df)[4], float sc2, int vis, bool local,
                                            float w_in, float Drow, float lse2_row,
                                            f32x4 (&dq)[8]) {
  const int g4 = lane_id() >> 4;
  f32x4 s[4], u[4];
  // one fragment set in registers at a time (the barriers keep the compiler
  // from hoisting the next set's loads)
  {
    bf16x8 f[16];
    load16(kvb, f);
    keys_by_rows(f, qf, s);
  }
  __builtin_amdgcn_sched_barrier(0);
  {
    bf16x8 f[16];
    load16(kvb + 16 * kWave, f);
    keys_by_rows(f, df, u);
  }
  __builtin_amdgcn_sched_barrier(0);
  if (vis < kS) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (mt * 16 + g4 * 4 + i >= vis) s[mt][i] = -INFINITY;
  }
  const float t0 = fmax3(s[0][0], s[0][1], s[0][2]), t1 = fmax3(s[0][3], s[1][0], s[1][1]);
  const float t2 = fmax3(s[1][2], s[1][3], s[2][0]), t3 = fmax3(s[2][1], s[2][2], s[2][3]);
  const float t4 = fmax3(s[3][0], s[3][1], s[3][2]);
  float mx = fmax3(fmax3(t0, t1, t2), fmax3(t3, t4, s[3][3]), -INFINITY);
  mx = rowgroup_max(mx);
  const float mb = mx * sc2;
  float z = 0.f, y = 0.f;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][i], sc2, -mb));
      s[mt][i] = e;
      z += e;
      y = __builtin_fmaf(e, u[mt][i], y);
    }
  z = rowgroup_sum(z);
  y = rowgroup_sum(y);
  const float rz = __builtin_amdgcn_rcpf(z);
  const float lse2 = mb + __log2f(z);
  const float Dc = y * rz;                               // sum_j p_j u_j
  const float w = local ? __builtin_amdgcn_exp2f(lse2 - lse2_row) : w_in;
  const float ref = local ? Drow : Dc;
  const float f = w * rz;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) s[mt][i] = f * s[mt][i] * (u[mt][i] - ref);   // dl
  bf16x8 pa[2];
  pack_keys(s, pa);
  __builtin_amdgcn_sched_barrier(0);
  bf16x8 kb[16];
  load16(kvb + 32 * kWave, kb);
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) dq[db] = mfma(pa[ks], kb[db * 2 + ks], dq[db]);
  __builtin_amdgcn_s_setprio(0);
  return make_float4(w, lse2, ref, 0.f);
}

// One step of the rows pass over a staged chunk c: first the next chunk's copy
// into `nxt` starts (the chunk buffers and LDS tables are restrict, so the reads
// of `kvb` need not wait for it).  jwin >= 0: member jwin of the local window
// (chunk own - jwin, table slot K + jwin; only the own chunk, jwin = 0, is
// masked), every block takes part.  jwin < 0: a union chunk; blocks none of
// whose queries selected it are skipped, and each selecting row's ds_c replaces
// its weight in `wts`.
template <int NCB>
__device__ __forceinline__ void rows_step(
    const Geometry& g, const uint4* __restrict__ kvb, uint4* __restrict__ nxt,
    const uint16_t* __restrict__ nsrc, const uint8_t* __restrict__ slotmap,
    float* __restrict__ wts, const float* __restrict__ Dr, const float* __restrict__ LSE2,
    uint64_t qmk, int c, int jwin, const bf16x8 (&qf)[kRowBlocks][4],
    const bf16x8 (&df)[kRowBlocks][4], float sc2, const BwdWs& ws, int b, int kvh, int i0, int w,
    f32x4 (&dq)[kRowBlocks][8]) {
  const int lane = lane_id(), r16 = lane & 15;
  const int K = g.K, L = g.Lq;
  const bool local = jwin >= 0;
  if (nsrc) stage48(nsrc, nxt);
#pragma unroll
  for (int j = 0; j < kRowBlocks; ++j) {
    const int blk = w * kRowBlocks + j;
    if (((qmk >> (blk * 4)) & 0xfull) == 0) continue;
    const int qi = blk * 4 + (r16 >> 2), h = r16 & 3;
    const int slot = local ? K + jwin : slotmap[qi * NCB + c];
    const float wv = (!local && slot != 0xff) ? wts[(qi * K + slot) * kG + h] : 0.f;
    const float dr = Dr[qi * kG + h];
    float4 st = block_bwd(kvb, qf[j], df[j], sc2, jwin == 0 ? qi + 1 : kS, local, wv, dr,
                          LSE2[qi * kG + h], dq[j]);
    if (!local) st.w = wv * (st.z - dr);                           // ds_c
    if (lane < 16 && slot != 0xff) {
      ws.stats[((size_t)(b * g.Hq + kvh * kG + h) * L + i0 + qi) * (size_t)(K + g.win) + slot] = st;
      if (!local) wts[(qi * K + slot) * kG + h] = st.w;
    }
  }
}

template <int KB, int NCB>
__global__ void __launch_bounds__(kRowThreads)
prefill_bwd_rows(Geometry g, const uint16_t* __restrict__ q, const uint16_t* __restrict__ qr,
                 const uint16_t* __restrict__ dout, const uint16_t* __restrict__ lmk,
                 const float* __restrict__ bias, const int32_t* __restrict__ sel_idx,
                 const float* __restrict__ lse, BwdWs ws, uint16_t* __restrict__ dq_out,
                 uint16_t* __restrict__ dqr_out) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  RowsSmem<KB, NCB>& sm = *reinterpret_cast<RowsSmem<KB, NCB>*>(smem_raw);
  static_assert(NCB <= kRowThreads, "one thread per chunk in the union list");
  const int nbkv = g.B * g.Hkv;
  const int bkv = blockIdx.x % nbkv;
  const int win = (g.Lq / kWin - 1) - blockIdx.x / nbkv;
  const int b = bkv / g.Hkv, kvh = bkv % g.Hkv;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int K = g.K, L = g.Lq;
  const int i0 = win * kWin, own = win;
  // local window: chunks own, own - 1, .., own - nwin + 1; candidates precede it
  const int nwin = g.win > 0 ? 1 + min(g.win - 1, own) : 0;
  const int ncand = max(0, min(own - max(g.win - 1, 0), g.NC));
  const uint16_t* Fg = ws.frags + (size_t)bkv * g.NC * kBwdChunkElems;
  const uint16_t* Lg = lmk + (size_t)bkv * g.NCcap * kD;
  const float* bb = bias ? bias + (size_t)bkv * g.NCcap : nullptr;
  const float scale = g.scale;
  const float sc2 = scale * 1.4426950408889634f;

  // ---- selection tables and the window's chunk union
  for (int x = tid; x < kWin * K; x += kRowThreads)
    sm.sel[x] = sel_idx[((size_t)bkv * L + i0 + x / K) * K + x % K];
  for (int x = tid; x < kWin * NCB / 4; x += kRowThreads)
    reinterpret_cast<uint32_t*>(sm.slotmap)[x] = 0xffffffffu;
  for (int c = tid; c < NCB; c += kRowThreads) sm.qmask[c] = 0ull;
  if (tid < kWin * kG) {
    const int qq = tid >> 2, h = tid & 3;
    const size_t row = (size_t)(b * g.Hq + kvh * kG + h) * L + i0 + qq;
    sm.Dr[tid] = ws.Drow[row];
    sm.LSE2[tid] = lse[row] * 1.4426950408889634f;
  }
  __syncthreads();
  for (int x = tid; x < kWin * K; x += kRowThreads) {
    const int c = sm.sel[x];
    if (c >= 0) {
      atomicOr((unsigned long long*)&sm.qmask[c], 1ull << (x / K));
      sm.slotmap[(x / K) * NCB + c] = (uint8_t)(x % K);
    }
  }
  __syncthreads();
  {
    const int c = tid;
    const bool f = c < ncand && c < NCB && sm.qmask[c < NCB ? c : 0] != 0ull;
    const uint64_t m = __ballot(f);
    if (lane == 0) sm.wcount[w] = __popcll(m);
    __syncthreads();
    int off = 0;
    for (int x = 0; x < w; ++x) off += sm.wcount[x];
    if (f) sm.ulist[off + mask_rank(m)] = (uint16_t)c;
  }
  int nunion = 0;
  for (int x = 0; x < kRowWaves; ++x) nunion += sm.wcount[x];

  // B fragments of q and dO of this wave's blocks: row r16 = (query 4*blk + r16/4, head r16%4)
  bf16x8 qf[kRowBlocks][4], df[kRowBlocks][4];
#pragma unroll
  for (int j = 0; j < kRowBlocks; ++j) {
    const int blk = w * kRowBlocks + j;
    const int qi = blk * 4 + (r16 >> 2), h = r16 & 3;
    const size_t row = ((size_t)(b * g.Hq + kvh * kG + h) * L + i0 + qi) * kD + g4 * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      qf[j][ks] = ld8(q + row + ks * 32);
      df[j][ks] = ld8(dout + row + ks * 32);
    }
  }

  // staged chunk sequence: the window chunks, then the union
  const int nseq = nwin + nunion;
  __syncthreads();                        // the union list is complete
  auto seq_src = [&](int x) -> const uint16_t* {
    if (x >= nseq) return nullptr;
    const int c = x < nwin ? own - x : sm.ulist[x - nwin];
    return Fg + (size_t)c * kBwdChunkElems;
  };
  if (nseq > 0) stage48(seq_src(0), sm.kv[0]);

  // ---- fusion weights of (row, selected chunk): exp(scale q_r.lmk + bias - LSE),
  //      q_r the retrieval query (the query itself unless a separate one is given)
  bf16x8 rf[kRowBlocks][4];
#pragma unroll
  for (int j = 0; j < kRowBlocks; ++j) {
    const int blk = w * kRowBlocks + j;
    const int qi = blk * 4 + (r16 >> 2), h = r16 & 3;
    const size_t row = ((size_t)(b * g.Hq + kvh * kG + h) * L + i0 + qi) * kD + g4 * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) rf[j][ks] = ld8(qr + row + ks * 32);
  }
  for (int nt = 0; nt * 16 < nunion; ++nt) {
    const int uu = nt * 16 + r16;
    const int c = sm.ulist[uu < nunion ? uu : 0];
    bf16x8 bl[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) bl[ks] = ld8(Lg + (size_t)c * kD + g4 * 8 + ks * 32);
    const float bc = bb ? bb[c] : 0.f;
#pragma unroll
    for (int j = 0; j < kRowBlocks; ++j) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = mfma(rf[j][ks], bl[ks], acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = g4 * 4 + i;
        const int qi = (w * kRowBlocks + j) * 4 + (rr >> 2), h = rr & 3;
        const int slot = uu < nunion ? sm.slotmap[qi * NCB + c] : 0xff;
        if (slot != 0xff)
          sm.wts[(qi * K + slot) * kG + h] = __builtin_amdgcn_exp2f(
              (scale * acc[i] + bc) * 1.4426950408889634f - sm.LSE2[qi * kG + h]);
      }
    }
  }
  stage_wait_all();
  __syncthreads();

  f32x4 dq[kRowBlocks][8];
#pragma unroll
  for (int j = 0; j < kRowBlocks; ++j)
#pragma unroll
    for (int db = 0; db < 8; ++db) dq[j][db] = f32x4{0.f, 0.f, 0.f, 0.f};

  int cur = 0;
  int x0 = 0;
  if (nwin > 0) {   // the own chunk (straight-line: its mode is known here)
    rows_step<NCB>(g, sm.kv[0], sm.kv[1], seq_src(1), sm.slotmap, sm.wts, sm.Dr, sm.LSE2, ~0ull, own, 0,
              qf, df, sc2, ws, b, kvh, i0, w, dq);
    stage_wait_all();
    __syncthreads();
    cur = 1;
    x0 = 1;
  }
  for (int x = x0; x < nwin; ++x, cur ^= 1) {
    rows_step<NCB>(g, sm.kv[cur], sm.kv[cur ^ 1], seq_src(x + 1), sm.slotmap, sm.wts, sm.Dr, sm.LSE2,
              ~0ull, own - x, x, qf, df, sc2, ws, b, kvh, i0, w, dq);
    stage_wait_all();
    __syncthreads();
  }
  for (int x = nwin; x < nseq; ++x, cur ^= 1) {
    const int c = sm.ulist[x - nwin];
    rows_step<NCB>(g, sm.kv[cur], sm.kv[cur ^ 1], seq_src(x + 1), sm.slotmap, sm.wts, sm.Dr, sm.LSE2,
              sm.qmask[c], c, -1, qf, df, sc2, ws, b, kvh, i0, w, dq);
    stage_wait_all();
    __syncthreads();
  }

  // ---- the score gradients sum_c ds_c lmk_c: into dq, or into dq_r when a
  //      separate retrieval query is given; then scale.  Lane holds
  //      dQ[row 4*g4 + i][16*db + r16], row 4*g4 + i = (query 4*blk + g4, head i)
#pragma unroll
  for (int j = 0; j < kRowBlocks; ++j) {
    const int qi = (w * kRowBlocks + j) * 4 + g4;
    f32x4 dr[8];
#pragma unroll
    for (int db = 0; db < 8; ++db) dr[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < K; ++s) {
      const int c = sm.sel[qi * K + s];
      if (c < 0) continue;
      float lv[8];
#pragma unroll
      for (int db = 0; db < 8; ++db) lv[db] = bf16_to_f32(Lg[(size_t)c * kD + 16 * db + r16]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ds = sm.wts[(qi * K + s) * kG + i];
#pragma unroll
        for (int db = 0; db < 8; ++db) dr[db][i] = __builtin_fmaf(ds, lv[db], dr[db][i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t ro = ((size_t)(b * g.Hq + kvh * kG + i) * L + i0 + qi) * kD + r16;
      if (dqr_out) {
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          dq_out[ro + 16 * db] = f32_to_bf16(scale * dq[j][db][i]);
          dqr_out[ro + 16 * db] = f32_to_bf16(scale * dr[db][i]);
        }
      } else {
#pragma unroll
        for (int db = 0; db < 8; ++db)
          dq_out[ro + 16 * db] = f32_to_bf16(scale * (dq[j][db][i] + dr[db][i]));
      }
    }
  }
}

// ----------------------------------------------------------------------------
// 3. chunks: dk, dv, dlmk, dbias
// ----------------------------------------------------------------------------
// (tile staging helpers and the chunk kernel follow the planner)

// ---- work items: each chunk's tiles (the local windows that hold it first, 8
//      tiles per window, then the retrieving queries in query order, 8 per
//      tile) cut into items of kTilesPerItem.
//      One workgroup per (b, kv head).
__global__ void __launch_bounds__(kPlanThreads)
prefill_bwd_plan(Geometry g, BwdWs ws) {
  __shared__ int scan[kPlanThreads];
  const int bkv = blockIdx.x, tid = threadIdx.x;
  const int NW = g.Lq / kWin;
  int nseg = 0, tiles = 0;
  if (tid < g.NC) {
    int n = 0;
#pragma unroll 8
    for (int wdw = tid + max(g.win, 1); wdw < NW; ++wdw)
      n += __popcll(ws.qm[((size_t)bkv * NW + wdw) * g.NC + tid]);
    tiles = (n + 7) / 8 + (kWin / 8) * min(g.win, NW - tid);
    nseg = max(1, (tiles + kTilesPerItem - 1) / kTilesPerItem);
  }
  scan[tid] = nseg;
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {
    const int t = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += t;
    __syncthreads();
  }
  if (tid < g.NC) {
    const int base = scan[tid] - nseg;
    for (int sgi = 0; sgi < nseg; ++sgi) {
      const int t0 = sgi * kTilesPerItem, t1 = min(tiles, t0 + kTilesPerItem);
      ws.items[(size_t)bkv * ws.max_items + base + sgi] =
          make_int4(tid, t0, t1, nseg > 1 ? base + sgi : -1);
    }
    ws.chunkseg[(size_t)bkv * g.NC + tid] = make_int2(base, nseg);
  }
  if (tid == 0) ws.nitems[bkv] = scan[kPlanThreads - 1];
}

// One tile of 8 queries x 4 heads = 32 rows, staged in LDS by the four waves
// with direct global->LDS loads:
//   qn, dn  q and dO rows, row r = (query r/4, head r%4), 128 dims = 16 chunks
//           of 16 B; chunk c of row r sits at position c ^ 2(r%4) of the row
//           (so that four consecutive rows of one 32-B column band fall in
//           different banks).  The A operands of S = Q K^T and U = dO V^T are
//           16-B reads of a row; the B operands of dV and dK (four heads of a
//           query at one dim) come out of LDS transpose reads.
//   st      [32 rows] (w, log2 lse_c, D_c, ds_c)
struct TileBuf {
  uint4 qn[32 * kD / 8];
  uint4 dn[32 * kD / 8];
  float4 st[32];
};
struct ChunkSmem {
  TileBuf tb[4];                    // two tiles computed while the next two are copied in
  uint16_t eq[kTilesPerItem * 8];   // tile entries: query
  uint8_t es[kTilesPerItem * 8];    // slot (K + j = window member j), 0xff = padding
  int scan[kChunkThreads];
};

__device__ __forceinline__ void lds_load16(const void* gsrc, void* ldst_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void*)ldst_wave_base,
                                   16, 0, 0);
}

__device__ __forceinline__ int tile_pos(int r, int c) { return r * (kD / 8) + (c ^ (2 * (r & 3))); }

// wave w stages its share of tile t into buffer tb: waves 0, 1 the q rows,
// waves 2, 3 the dO rows (four rows = 1 KB per load instruction), wave 2 also
// the row table
__device__ __forceinline__ void stage_tile(const Geometry& g, const uint16_t* __restrict__ q,
                                           const uint16_t* __restrict__ dout, const BwdWs& ws,
                                           int b, int kvh, int bkv, const uint16_t* eq,
                                           const uint8_t* es, int t, TileBuf& tb) {
  const int lane = lane_id(), w = threadIdx.x / kWave;
  const int L = g.Lq;
  const int e0 = t * 8;
  const uint16_t* src = w < 2 ? q : dout;
  uint4* dst = w < 2 ? tb.qn : tb.dn;
#pragma unroll
  for (int x4 = 0; x4 < 4; ++x4) {
    const int x = (w & 1) * 4 + x4;            // rows 4x .. 4x + 3
    const int r = 4 * x + (lane >> 4);         // this lane's slot: row r, position lane % 16
    const int c = (lane & 15) ^ (2 * (r & 3)); // the chunk that belongs there
    const int e = e0 + (r >> 2);
    const int qq = eq[es[e] != 0xff ? e : e0];
    lds_load16(src + ((size_t)(b * g.Hq + kvh * kG + (r & 3)) * L + qq) * kD + 8 * c, dst + 64 * x);
  }
  if (w == 2 && lane < 32) {   // the row table: row r = (query r/4, head r%4)
    const int ee = e0 + (lane >> 2);
    const int sl = es[ee];
    const int qq = eq[sl != 0xff ? ee : e0];
    const int slot = sl != 0xff ? sl : es[e0];
    const float4* p = ws.stats + ((size_t)(b * g.Hq + kvh * kG + (lane & 3)) * L + qq) * (g.K + g.win) + slot;
    lds_load16(p, tb.st);
  }
}

// B operand half of dV / dK for dims 16db..16db+15: the four heads of query
// slot qs (rows 4qs .. 4qs+3) at dim 16db + l%16, by an LDS transpose read:
// source lane t of a 16-lane group points at row 4qs + t/4, dims 16db + 4(t%4)
// .. +3; lane i then holds the four rows at dim 16db + i.
__device__ __forceinline__ uint2 tile_heads_at_dim(const uint4* __restrict__ tile, int qs, int db) {
  const int t = lane_id() & 15;
  const int r = 4 * qs + (t >> 2);
  const int c = 2 * db + ((t & 3) >> 1);
  const char* p = reinterpret_cast<const char*>(tile + tile_pos(r, c)) + 8 * (t & 1);
  const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)p);
  uint2 u;
  __builtin_memcpy(&u, &v, 8);
  return u;
}

// Accumulate one staged tile.
__device__ __forceinline__ void chunk_tile_compute(
    const Geometry& g, int w, int lane, int key, float sc2, int t,
    const TileBuf* __restrict__ tbp, const uint16_t* __restrict__ eq,
    const uint8_t* __restrict__ es, const bf16x8 (&kB)[4], const bf16x8 (&vB)[4],
    f32x4 (&dv)[8], f32x4 (&dk)[8], float (&dlm)[2], float& dbt) {
  const TileBuf& tb = *tbp;
  // S and U for this wave's keys; D layout rows (mt, qq = l/16, h = i), key l%16
  f32x4 s[2], u[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    f32x4 as = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int pos = tile_pos(16 * mt + (lane & 15), 4 * ks + (lane >> 4));
      as = mfma(as_bf16x8(tb.qn[pos]), kB[ks], as);
      au = mfma(as_bf16x8(tb.dn[pos]), vB[ks], au);
    }
    s[mt] = as;
    u[mt] = au;
  }
  float a8[8], d8[8], ds[2][4];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int e = t * 8 + 4 * mt + (lane >> 4);
    const int sl = es[e];
    const bool valid = sl != 0xff;
    const bool local = sl >= g.K;            // a window member (keys after the query hidden)
    const int qq = eq[valid ? e : t * 8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 st = tb.st[(4 * mt + (lane >> 4)) * 4 + i];
      float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][i], sc2, -st.y));
      if (!valid || (local && key > qq)) p = 0.f;
      const float wp = st.x * p;
      a8[4 * mt + i] = wp;
      d8[4 * mt + i] = wp * (u[mt][i] - st.z);
      ds[mt][i] = (valid && !local) ? st.w : 0.f;
    }
  }
  const bf16x8 Awp = pack_bf16x8(a8), Adl = pack_bf16x8(d8);
  const int qs0 = lane >> 4, qs1 = 4 + (lane >> 4);   // k-slots: rows of query slots l/16 and 4 + l/16
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    const uint2 q0 = tile_heads_at_dim(tb.qn, qs0, db);
    const uint2 q1 = tile_heads_at_dim(tb.qn, qs1, db);
    const uint2 d0 = tile_heads_at_dim(tb.dn, qs0, db);
    const uint2 d1 = tile_heads_at_dim(tb.dn, qs1, db);
    dv[db] = mfma(Awp, as_bf16x8(make_uint4(d0.x, d0.y, d1.x, d1.y)), dv[db]);
    dk[db] = mfma(Adl, as_bf16x8(make_uint4(q0.x, q0.y, q1.x, q1.y)), dk[db]);
    if ((db >> 1) == w) {                 // wave w: landmark-gradient dims 32w .. 32w + 31
      const uint32_t qw[4] = {q0.x, q0.y, q1.x, q1.y};
      float tacc = dlm[db & 1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        tacc = __builtin_fmaf(ds[e / 2][(e % 2) * 2], __uint_as_float(qw[e] << 16), tacc);
        tacc = __builtin_fmaf(ds[e / 2][(e % 2) * 2 + 1], __uint_as_float(qw[e] & 0xffff0000u), tacc);
      }
      dlm[db & 1] = tacc;
    }
  }
  if (w == 0 && (lane & 15) == 0) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) dbt += ds[mt][i];
  }
}

// Tiles t and t + 1 (staged in a, b) are accumulated while tiles t + 2 and
// t + 3 are copied into c, d: two tiles of each workgroup in flight while it
// computes (with one, the gather of q and dO waits on its latency).  All four
// buffers are restrict, so the LDS reads of a and b need not wait for the
// copies into c and d.
__device__ __forceinline__ void chunk_pair_step(
    const Geometry& g, const uint16_t* __restrict__ q, const uint16_t* __restrict__ dout,
    const BwdWs& ws, int b, int kvh, int bkv, int w, int lane, int key, float sc2, int t,
    int ntile, const TileBuf* __restrict__ ta, const TileBuf* __restrict__ tb,
    TileBuf* __restrict__ tc, TileBuf* __restrict__ td, const uint16_t* __restrict__ eq,
    const uint8_t* __restrict__ es, const bf16x8 (&kB)[4], const bf16x8 (&vB)[4],
    f32x4 (&dv)[8], f32x4 (&dk)[8], float (&dlm)[2], float& dbt) {
  if (t + 2 < ntile) stage_tile(g, q, dout, ws, b, kvh, bkv, eq, es, t + 2, *tc);
  if (t + 3 < ntile) stage_tile(g, q, dout, ws, b, kvh, bkv, eq, es, t + 3, *td);
  chunk_tile_compute(g, w, lane, key, sc2, t, ta, eq, es, kB, vB, dv, dk, dlm, dbt);
  __builtin_amdgcn_sched_barrier(0);     // one tile's registers at a time
  if (t + 1 < ntile) chunk_tile_compute(g, w, lane, key, sc2, t + 1, tb, eq, es, kB, vB, dv, dk, dlm, dbt);
}

// WPT: query windows listed per thread (one up to 256 windows, two up to 512)
template <int WPT>
__global__ void __launch_bounds__(kChunkThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_bwd_chunks(Geometry g, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                   const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout, BwdWs ws,
                   uint16_t* __restrict__ dk_out, uint16_t* __restrict__ dv_out,
                   uint16_t* __restrict__ dlmk_out, float* __restrict__ dbias_out) {
  __shared__ ChunkSmem sm;
  const int nbkv = g.B * g.Hkv;
  const int bkv = blockIdx.x % nbkv, item = blockIdx.x / nbkv;
  if (item >= ws.nitems[bkv]) return;
  const int4 it = ws.items[(size_t)bkv * ws.max_items + item];
  const int c = it.x, t0 = it.y, t1 = it.z, part = it.w;
  const int b = bkv / g.Hkv, kvh = bkv % g.Hkv;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int L = g.Lq, NW = L / kWin;
  const float scale = g.scale, sc2 = scale * 1.4426950408889634f;
  // the local windows c, c+1, .., c+win-1 (those that exist) hold chunk c
  const int own_tiles = (kWin / 8) * min(g.win, NW - c);
  const int ntile = t1 - t0;

  // ---- tile entries of this item: the queries of the windows that hold the
  //      chunk (window c + j: slot K + j), then the retrieving queries of later
  //      windows in query order
  for (int e = tid; e < kTilesPerItem * 8; e += kChunkThreads) sm.es[e] = 0xff;
  __syncthreads();
  for (int e = tid; e < ntile * 8; e += kChunkThreads) {
    const int t = t0 + e / 8;
    if (t < own_tiles) {
      const int jw = t / (kWin / 8);
      sm.eq[e] = (uint16_t)((c + jw) * kWin + (t % (kWin / 8)) * 8 + e % 8);
      sm.es[e] = (uint8_t)(g.K + jw);
    }
  }
  const int r0 = 8 * max(0, t0 - own_tiles), r1 = 8 * max(0, t1 - own_tiles);
  const int rbase = 8 * max(0, own_tiles - t0);   // entry index of the first retrieved query
  const int wret = c + max(g.win, 1);        // first window that may retrieve chunk c
  const int nlater = NW - wret;
  // thread t lists windows wret + WPT t .. + WPT - 1
  uint64_t m[WPT];
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    const int wi = tid * WPT + j;
    m[j] = (wi < nlater && r1 > r0) ? ws.qm[((size_t)bkv * NW + wret + wi) * g.NC + c] : 0ull;
    cnt += __popcll(m[j]);
  }
  sm.scan[tid] = cnt;
  __syncthreads();
  for (int off = 1; off < kChunkThreads; off <<= 1) {
    const int tt = tid >= off ? sm.scan[tid - off] : 0;
    __syncthreads();
    sm.scan[tid] += tt;
    __syncthreads();
  }
  {
    int pos = sm.scan[tid] - cnt;
    if (pos < r1 && pos + cnt > r0) {
#pragma unroll
      for (int j = 0; j < WPT; ++j) {
        uint64_t mm = m[j];
        while (mm) {
          const int bit = __ffsll((long long)mm) - 1;
          mm &= mm - 1;
          if (pos >= r0 && pos < r1) {
            const int qq = (wret + tid * WPT + j) * kWin + bit;
            sm.eq[rbase + pos - r0] = (uint16_t)qq;
          }
          ++pos;
        }
      }
    }
  }
  __syncthreads();
  // the retrieved entries' slots: one independent load per entry, all in
  // flight together (a load inside the per-window bit loop above would wait
  // for each one in turn)
  // (entries past the last retrieving query pad the last tile and keep 0xff)
  const int rend = rbase + min(r1, sm.scan[kChunkThreads - 1]) - r0;
  for (int e = rbase + tid; e < rend; e += kChunkThreads)
    sm.es[e] = ws.slot[((size_t)bkv * L + sm.eq[e]) * g.NC + c];
  __syncthreads();

  // this wave's 16 keys of the chunk as B fragments of S = Q K^T and U = dO V^T
  bf16x8 kB[4], vB[4];
  {
    const size_t row = ((size_t)bkv * L + c * kS + 16 * w + (lane & 15)) * kD + 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      kB[ks] = ld8(k + row + 32 * ks);
      vB[ks] = ld8(v + row + 32 * ks);
    }
  }
  f32x4 dv[8], dk[8];
  float dlm[2];                       // landmark gradient, dims 16 (2w + x) + l % 16
  float dbt = 0.f;
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    dv[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    dk[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  dlm[0] = dlm[1] = 0.f;
  const int key = c * kS + 16 * w + (lane & 15);

  if (ntile > 0) stage_tile(g, q, dout, ws, b, kvh, bkv, sm.eq, sm.es, 0, sm.tb[0]);
  if (ntile > 1) stage_tile(g, q, dout, ws, b, kvh, bkv, sm.eq, sm.es, 1, sm.tb[1]);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int t = 0; t < ntile; t += 2) {
    const int s = t & 2;                  // tiles t, t + 1 in buffers s, s + 1
    chunk_pair_step(g, q, dout, ws, b, kvh, bkv, w, lane, key, sc2, t, ntile, &sm.tb[s],
                    &sm.tb[s + 1], &sm.tb[s ^ 2], &sm.tb[(s ^ 2) + 1], sm.eq, sm.es, kB, vB, dv,
                    dk, dlm, dbt);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // ---- outputs: lane holds dX[key 16w + 4(l/16) + i][16db + l%16]
#pragma unroll
  for (int x = 0; x < 2; ++x) dlm[x] = rowgroup_sum(dlm[x]);
  if (w == 0) dbt = rowgroup_sum(dbt);
  if (part < 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t row = ((size_t)bkv * L + c * kS + 16 * w + 4 * (lane >> 4) + i) * kD + (lane & 15);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        dv_out[row + 16 * db] = f32_to_bf16(dv[db][i]);
        dk_out[row + 16 * db] = f32_to_bf16(scale * dk[db][i]);
      }
    }
#pragma unroll
    for (int x = 0; x < 2; ++x)
      if (lane < 16) dlmk_out[((size_t)bkv * g.NCcap + c) * kD + 16 * (2 * w + x) + lane] = f32_to_bf16(scale * dlm[x]);
    if (w == 0 && lane == 0 && dbias_out) dbias_out[(size_t)bkv * g.NCcap + c] = dbt;
  } else {
    float* pp = ws.part + ((size_t)bkv * ws.max_items + part) * kPartFloats;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kr = 16 * w + 4 * (lane >> 4) + i;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        pp[kr * kD + 16 * db + (lane & 15)] = dv[db][i];
        pp[kS * kD + kr * kD + 16 * db + (lane & 15)] = dk[db][i];
      }
    }
#pragma unroll
    for (int x = 0; x < 2; ++x)
      if (lane < 16) pp[2 * kS * kD + 16 * (2 * w + x) + lane] = dlm[x];
    if (w == 0 && lane == 0) pp[2 * kS * kD + kD] = dbt;
  }
}

// ---- sums the partial items of chunks split over several workgroups, in item
//      order; zeroes the landmark rows past the complete chunks.
__global__ void __launch_bounds__(kChunkThreads)
prefill_bwd_reduce(Geometry g, BwdWs ws, uint16_t* __restrict__ dk_out,
                   uint16_t* __restrict__ dv_out, uint16_t* __restrict__ dlmk_out,
                   float* __restrict__ dbias_out) {
  const int nbkv = g.B * g.Hkv;
  const int bkv = blockIdx.x % nbkv, c = blockIdx.x / nbkv;
  const int tid = threadIdx.x;
  const float scale = g.scale;
  if (c >= g.NC) {
    if (tid < kD) dlmk_out[((size_t)bkv * g.NCcap + c) * kD + tid] = 0;
    if (tid == 0 && dbias_out) dbias_out[(size_t)bkv * g.NCcap + c] = 0.f;
    return;
  }
  const int2 cs = ws.chunkseg[(size_t)bkv * g.NC + c];
  if (cs.y <= 1) return;
  const float* pb = ws.part + ((size_t)bkv * ws.max_items + cs.x) * kPartFloats;
  const size_t row0 = ((size_t)bkv * g.Lq + c * kS) * kD;
  for (int x = tid * 4; x < kS * kD; x += kChunkThreads * 4) {
    float4 sv = make_float4(0.f, 0.f, 0.f, 0.f), sk = sv;
    for (int sgi = 0; sgi < cs.y; ++sgi) {
      const float4 a = *reinterpret_cast<const float4*>(pb + (size_t)sgi * kPartFloats + x);
      const float4 bq = *reinterpret_cast<const float4*>(pb + (size_t)sgi * kPartFloats + kS * kD + x);
      sv.x += a.x; sv.y += a.y; sv.z += a.z; sv.w += a.w;
      sk.x += bq.x; sk.y += bq.y; sk.z += bq.z; sk.w += bq.w;
    }
    const uint2 ov = make_uint2((uint32_t)f32_to_bf16(sv.x) | ((uint32_t)f32_to_bf16(sv.y) << 16),
                                (uint32_t)f32_to_bf16(sv.z) | ((uint32_t)f32_to_bf16(sv.w) << 16));
    const uint2 ok = make_uint2((uint32_t)f32_to_bf16(scale * sk.x) | ((uint32_t)f32_to_bf16(scale * sk.y) << 16),
                                (uint32_t)f32_to_bf16(scale * sk.z) | ((uint32_t)f32_to_bf16(scale * sk.w) << 16));
    *reinterpret_cast<uint2*>(dv_out + row0 + x) = ov;
    *reinterpret_cast<uint2*>(dk_out + row0 + x) = ok;
  }
  if (tid <= kD) {
    float sl = 0.f;
    for (int sgi = 0; sgi < cs.y; ++sgi) sl += pb[(size_t)sgi * kPartFloats + 2 * kS * kD + tid];
    if (tid < kD) dlmk_out[((size_t)bkv * g.NCcap + c) * kD + tid] = f32_to_bf16(scale * sl);
    else if (dbias_out) dbias_out[(size_t)bkv * g.NCcap + c] = sl;
  }
}

// ---- landmark gradients when a separate retrieval query is given: dlmk_c =
//      scale sum ds_c q_r over the rows that retrieved chunk c, overwriting the
//      chunk pass's values (which used the query itself).  One workgroup per
//      (b, kv head, chunk): the retrieving queries are listed in query order
//      (one window per thread, a prefix sum places them), wave w takes entries
//      w, w + 4, .. with lane l on dims 2l, 2l + 1, and the four wave sums are
//      added in wave order, so the result does not depend on timing.
constexpr int kQrThreads = 256;

template <int NCB>
__global__ void __launch_bounds__(kQrThreads)
prefill_bwd_dlmk_qret(Geometry g, const uint16_t* __restrict__ qr, BwdWs ws,
                      uint16_t* __restrict__ dlmk_out) {
  // the chunk's retrieving queries (at most L <= 64 NCB): ids and slots
  __shared__ uint16_t eq[NCB * kS];
  __shared__ uint8_t es[NCB * kS];
  __shared__ int scan[kQrThreads];
  __shared__ float red[kQrThreads / kWave][kD];
  const int nbkv = g.B * g.Hkv;
  const int bkv = blockIdx.x % nbkv, c = blockIdx.x / nbkv;
  const int b = bkv / g.Hkv, kvh = bkv % g.Hkv;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int L = g.Lq, NW = L / kWin;
  const size_t nslot = (size_t)(g.K + g.win);
  const int wret = c + max(g.win, 1);       // first window that may retrieve chunk c
  const int nlater = NW - wret;
  // thread t lists windows wret + kWpt t .. + kWpt - 1
  constexpr int kWpt = NCB / kQrThreads;
  uint64_t m[kWpt];
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < kWpt; ++j) {
    const int wi = tid * kWpt + j;
    m[j] = wi < nlater ? ws.qm[((size_t)bkv * NW + wret + wi) * g.NC + c] : 0ull;
    cnt += __popcll(m[j]);
  }
  scan[tid] = cnt;
  __syncthreads();
  for (int off = 1; off < kQrThreads; off <<= 1) {
    const int t = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += t;
    __syncthreads();
  }
  {
    int pos = scan[tid] - cnt;
#pragma unroll
    for (int j = 0; j < kWpt; ++j) {
      uint64_t mm = m[j];
      while (mm) {
        const int bit = __ffsll((long long)mm) - 1;
        mm &= mm - 1;
        eq[pos] = (uint16_t)((wret + tid * kWpt + j) * kWin + bit);
        ++pos;
      }
    }
  }
  const int total = scan[kQrThreads - 1];
  __syncthreads();
  // slots: one independent load per entry, all in flight together
  for (int n = tid; n < total; n += kQrThreads)
    es[n] = ws.slot[((size_t)bkv * L + eq[n]) * g.NC + c];
  __syncthreads();
  float a0 = 0.f, a1 = 0.f;
#pragma unroll 4
  for (int n = w; n < total; n += kQrThreads / kWave) {
    const int qq = eq[n], slot = es[n];
#pragma unroll
    for (int h = 0; h < kG; ++h) {
      const size_t row = (size_t)(b * g.Hq + kvh * kG + h) * L + qq;
      const float ds = ws.stats[row * nslot + slot].w;
      const uint32_t pr = reinterpret_cast<const uint32_t*>(qr + row * kD)[lane];
      a0 = __builtin_fmaf(ds, __uint_as_float(pr << 16), a0);
      a1 = __builtin_fmaf(ds, __uint_as_float(pr & 0xffff0000u), a1);
    }
  }
  red[w][2 * lane] = a0;
  red[w][2 * lane + 1] = a1;
  __syncthreads();
  if (tid < kD) {
    float acc = 0.f;
#pragma unroll
    for (int x = 0; x < kQrThreads / kWave; ++x) acc += red[x][tid];
    dlmk_out[((size_t)bkv * g.NCcap + c) * kD + tid] = f32_to_bf16(g.scale * acc);
  }
}

}  // namespace

bool prefill_bwd_fast_supported(const Geometry& g, int bf16) {
  return bf16 && g.d == kD && g.S == kS && g.G == kG && g.causal && g.Lq == g.Lkv &&
         g.Lq % kWin == 0 && g.K <= kMaxKb && g.NC <= kMaxNCb && g.NC >= 1 &&
         (g.NC <= kRowsNarrowNC || g.K <= kRowsWideK) && g.K + g.win < 0xff;
}

size_t prefill_bwd_fast_ws(const Geometry& g) {
  size_t total = 0;
  carve(g, nullptr, &total);
  return total;
}

hipError_t launch_prefill_bwd_fast(const Geometry& g, const void* q, const void* qr, const void* k,
                                   const void* v, const void* lmk, const float* bias,
                                   const void* out, const void* dout, const int32_t* sel_idx,
                                   const float* lse, void* dq, void* dqr, void* dk, void* dv,
                                   void* dlmk, float* dbias, void* wsp, hipStream_t st) {
  BwdWs ws = carve(g, wsp, nullptr);
  const int nbkv = g.B * g.Hkv, NW = g.Lq / kWin;
  const uint16_t* Q = (const uint16_t*)q;
  const uint16_t* DO = (const uint16_t*)dout;
  const bool narrow = g.NC <= kRowsNarrowNC;
  if (narrow)
    hipLaunchKernelGGL(prefill_bwd_prep<kRowsNarrowNC>, dim3(nbkv * NW), dim3(kPrepThreads), 0, st, g, Q,
                       (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)out, DO, sel_idx, ws);
  else
    hipLaunchKernelGGL(prefill_bwd_prep<kMaxNCb>, dim3(nbkv * NW), dim3(kPrepThreads), 0, st, g, Q,
                       (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)out, DO, sel_idx, ws);
  // dynamic LDS above 64 KB must be enabled for each kernel (per device; cheap)
  const void* rows_fn = narrow ? (const void*)prefill_bwd_rows<kMaxKb, kRowsNarrowNC>
                               : (const void*)prefill_bwd_rows<kRowsWideK, kMaxNCb>;
  const size_t rows_lds = narrow ? sizeof(RowsSmem<kMaxKb, kRowsNarrowNC>)
                                 : sizeof(RowsSmem<kRowsWideK, kMaxNCb>);
  hipError_t e = hipFuncSetAttribute(rows_fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)rows_lds);
  if (e != hipSuccess) return e;
  prof_begin(kPrefillBwdRows, st);
  if (narrow)
    hipLaunchKernelGGL((prefill_bwd_rows<kMaxKb, kRowsNarrowNC>), dim3(nbkv * NW), dim3(kRowThreads),
                       rows_lds, st, g, Q, (const uint16_t*)qr, DO, (const uint16_t*)lmk, bias, sel_idx,
                       lse, ws, (uint16_t*)dq, (uint16_t*)dqr);
  else
    hipLaunchKernelGGL((prefill_bwd_rows<kRowsWideK, kMaxNCb>), dim3(nbkv * NW), dim3(kRowThreads),
                       rows_lds, st, g, Q, (const uint16_t*)qr, DO, (const uint16_t*)lmk, bias, sel_idx,
                       lse, ws, (uint16_t*)dq, (uint16_t*)dqr);
  prof_end(kPrefillBwdRows, st);
  hipLaunchKernelGGL(prefill_bwd_plan, dim3(nbkv), dim3(kPlanThreads), 0, st, g, ws);
  prof_begin(kPrefillBwdChunks, st);
  if (narrow)
    hipLaunchKernelGGL(prefill_bwd_chunks<1>, dim3(nbkv * ws.max_items), dim3(kChunkThreads), 0, st,
                       g, Q, (const uint16_t*)k, (const uint16_t*)v, DO, ws, (uint16_t*)dk,
                       (uint16_t*)dv, (uint16_t*)dlmk, dbias);
  else
    hipLaunchKernelGGL(prefill_bwd_chunks<kMaxNCb / kChunkThreads>, dim3(nbkv * ws.max_items),
                       dim3(kChunkThreads), 0, st, g, Q, (const uint16_t*)k, (const uint16_t*)v, DO,
                       ws, (uint16_t*)dk, (uint16_t*)dv, (uint16_t*)dlmk, dbias);
  prof_end(kPrefillBwdChunks, st);
  hipLaunchKernelGGL(prefill_bwd_reduce, dim3(nbkv * g.NCcap), dim3(kChunkThreads), 0, st, g, ws,
                     (uint16_t*)dk, (uint16_t*)dv, (uint16_t*)dlmk, dbias);
  if (dqr) {
    if (narrow)
      hipLaunchKernelGGL(prefill_bwd_dlmk_qret<kRowsNarrowNC>, dim3(nbkv * g.NC), dim3(kQrThreads), 0,
                         st, g, (const uint16_t*)qr, ws, (uint16_t*)dlmk);
    else
      hipLaunchKernelGGL(prefill_bwd_dlmk_qret<kMaxNCb>, dim3(nbkv * g.NC), dim3(kQrThreads), 0, st, g,
                         (const uint16_t*)qr, ws, (uint16_t*)dlmk);
  }
  return hipGetLastError();
}

}  // namespace hils
