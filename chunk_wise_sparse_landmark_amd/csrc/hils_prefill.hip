// MFMA prefill path: bf16, head_dim 128, chunk 64, GQA group of 4, causal,
// seq_q == seq_kv.
//
// Method: Hierarchical Sparse Attention Done Right (arXiv 2607.02980v1, summary
// page): landmark scores §3 "Linear surrogate for chunk mass", top-K routing §3
// "Sparse training", GQA-shared selection §4 "Architecture", per-chunk softmax
// and fusion by the retrieval scores §3 "Hierarchical softmax".  The page's own
// kernel batches M adjacent queries over the union of their chunks so that a
// loaded chunk feeds an (M x G, d) x (d, S) product (§4 "Kernel design"); here
// the idea is rebuilt for 64-wide waves and 16x16x32 bf16 MFMA:
//
//  1. prefill_select  grid (L/64, B*Hkv), one workgroup per chunk-aligned
//     64-query window.  Group scores sum_h q_h . lmk_c are one MFMA chain (the
//     G heads extend the reduction), then each query's top-K is found without
//     sorting: tau = K-th largest lane maximum, keys >= tau are compacted in
//     chunk order and a rank count keeps K, which come out in ascending id.
//     The same workgroup also rewrites its chunk of V in MFMA B-operand order
//     (16 B per lane per fragment), so the attention kernel loads V fully
//     coalesced and never transposes it.
//  2. prefill_attend  grid (L/32, B*Hkv).  A 32-query window (128 rows) walks
//     the union of its queries' selected chunks.  For each chunk only the
//     queries that selected it are gathered, four per 16-row tile (rows ordered
//     head-major, so in the MFMA result the register index is the query slot
//     and the lane group is the head).  The four waves split the work of a
//     chunk by keys for S^T = K Q^T (16 keys each; row max and sum go through
//     LDS) and by output columns for O = P V (32 columns each), so the fp32
//     accumulators of all 128 rows live in registers, each wave owning its 32
//     columns: no LDS accumulation, no atomics, a fixed summation order.
//     Retrieval scores of the window's rows against its union come from one
//     MFMA pass; the own chunk is attended first, so every fusion weight is
//     final before the retrieved chunks are added.
#include "hils_common.h"
#include "hils_kernels.h"
#include "hils_profile.h"

namespace hils {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kD = 128;
constexpr int kS = 64;
constexpr int kG = 4;            // query heads per KV group on this path
constexpr int kThreads = 256;
constexpr int kSelWin = 64;      // queries per selection window (one chunk)
constexpr int kW = 32;           // queries per attention window
constexpr int kRows = kW * kG;   // 128 rows
constexpr int kMaxT = kW / 4;    // 16-row tiles per chunk at most
constexpr int kMaxKf = 32;       // top-K bound on this path
constexpr int kMaxNC = 256;      // chunks bound on this path (L <= 16384)
constexpr int kQStride = 136;    // bf16 per staged Q row (272 B: 2-way bank spread)
constexpr int kFragsPerChunk = 16;   // V fragments per chunk: 8 column blocks x 2 key steps

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  bf16x8 r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) {
  bf16x8 r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}
__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
// two fp32 -> packed bf16, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// ----------------------------------------------------------------------------
// Top-K of R keys per lane (candidate c = r*64 + lane), written as ascending
// chunk ids (-1 padded) to dst[0..K).  Keys are unique apart from 0 (empty).
// K * R <= 64: order-preserving compaction + rank count, no sort.
// ----------------------------------------------------------------------------
template <int R>
__device__ void select_ascending(uint64_t (&keys)[R], int K, uint64_t* buf, uint64_t* buf2,
                                 int32_t* dst) {
  const int lane = lane_id();
  if (K * R > kWave) {
    const uint64_t top = wave_topk<R>(keys, K, buf);
    const uint64_t asc = (lane < K && top != 0) ? (0xffffffffull - (uint64_t)key_index(top)) + 1 : 0;
    const uint64_t srt = wave_rank_sort64(asc, buf);
    if (lane < K) dst[lane] = srt ? (int)(0xffffffffull - (srt - 1)) : -1;
    return;
  }
  uint64_t lm = keys[0];
#pragma unroll
  for (int r = 1; r < R; ++r) lm = keys[r] > lm ? keys[r] : lm;
  buf[lane] = lm;
  wave_sync_lds();
  int rank = 0;
  const ulonglong2* b2 = reinterpret_cast<const ulonglong2*>(buf);
#pragma unroll
  for (int j = 0; j < kWave / 2; ++j) {
    const ulonglong2 kk = b2[j];
    rank += (kk.x > lm) + (kk.y > lm);
  }
  const uint64_t hit = __ballot(rank == K - 1 && lm != 0);
  uint64_t tau = 1;
  if (hit) tau = shfl_u64(lm, __ffsll((long long)hit) - 1);
  int base = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool pred = keys[r] >= tau;
    const uint64_t m = __ballot(pred);
    if (pred) buf2[base + mask_rank(m)] = keys[r];
    base += __popcll(m);
  }
  wave_sync_lds();
  const uint64_t key = lane < base ? buf2[lane] : 0ull;
  int rank2 = 0;
  const ulonglong2* c2 = reinterpret_cast<const ulonglong2*>(buf2);
  for (int j = 0; j < (base + 1) / 2; ++j) {
    const ulonglong2 kk = c2[j];
    rank2 += (kk.x > key) + ((2 * j + 1 < base) && (kk.y > key));
  }
  const uint64_t sel_key = (key != 0 && rank2 < K) ? key : 0ull;
  wave_sync_lds();
  const uint64_t m = __ballot(sel_key != 0);
  const int nsel = __popcll(m);
  if (sel_key != 0) dst[mask_rank(m)] = key_index(sel_key);
  if (lane >= nsel && lane < K) dst[lane] = -1;
}

// ----------------------------------------------------------------------------
// 1. selection (+ V of this window's chunk in B-operand fragment order)
//    Vf[bkv][chunk][db 0..7][ks 0..1][lane 0..63][8]: lane l, element j holds
//    V[32ks + 16(j/4) + 4(l/16) + j%4][16db + l%16].
// ----------------------------------------------------------------------------
template <int R>
__global__ void __launch_bounds__(kThreads)
prefill_select(Geometry g, const uint16_t* __restrict__ q, const uint16_t* __restrict__ v,
               const uint16_t* __restrict__ lmk, const float* __restrict__ bias,
               int32_t* __restrict__ sel_idx, uint16_t* __restrict__ vf) {
  constexpr int NCP = R * kWave;
  __shared__ float gs[kSelWin][NCP + 1];
  __shared__ uint64_t buf[4][kWave];
  __shared__ uint64_t buf2[4][kWave];
  __shared__ __attribute__((aligned(16))) uint16_t vs[kS * kD];
  const int nbkv = g.B * g.Hkv;            // (b, kv head) fastest: one head per XCD
  const int bkv = blockIdx.x % nbkv;
  const int win = (g.Lq / kSelWin - 1) - blockIdx.x / nbkv;
  const int b = bkv / g.Hkv, kvh = bkv % g.Hkv;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int i0 = win * kSelWin;
  const int ncand = min(i0 / kS, g.NC);
  const int r16 = lane & 15, g4 = lane >> 4;

  // V of chunk `win` -> LDS (coalesced), later rewritten in fragment order
  const uint16_t* Vc = v + ((size_t)bkv * g.Lkv + (size_t)win * kS) * kD;
#pragma unroll
  for (int x = tid; x < kS * kD / 8; x += kThreads)
    reinterpret_cast<uint4*>(vs)[x] = reinterpret_cast<const uint4*>(Vc)[x];

  // A operand: 16 queries of this wave x 4 heads x 4 k-steps
  bf16x8 a[kG][4];
#pragma unroll
  for (int h = 0; h < kG; ++h) {
    const uint16_t* qr = q + ((size_t)(b * g.Hq + kvh * kG + h) * g.Lq + i0 + w * 16 + r16) * kD + g4 * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) a[h][ks] = ld8(qr + ks * 32);
  }
  const uint16_t* L = lmk + (size_t)bkv * g.NCcap * kD;
  const float* bb = bias ? bias + (size_t)bkv * g.NCcap : nullptr;
  const float sc = g.scale / (float)kG;
  const int ntile = (ncand + 15) / 16;
  for (int nt0 = 0; nt0 < ntile; nt0 += 8) {
    bf16x8 bv[8][4];   // all loads of up to 8 column tiles in flight together
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int c = (nt0 + x) * 16 + r16;
      const int cl = c < ncand ? c : 0;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) bv[x][ks] = ld8(L + (size_t)cl * kD + g4 * 8 + ks * 32);
    }
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int nt = nt0 + x;
      if (nt >= ntile) break;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int h = 0; h < kG; ++h)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mfma(a[h][ks], bv[x][ks], acc);
      const int c = nt * 16 + r16;
      const float bc = (bb && c < ncand) ? bb[c] : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) gs[w * 16 + g4 * 4 + i][c] = acc[i] * sc + bc;
    }
  }
  __syncthreads();

  // V fragments of this chunk (1024 x 16 B, four per thread)
  uint16_t* vdst = vf + ((size_t)bkv * g.NC + win) * kFragsPerChunk * kWave * 8;
#pragma unroll
  for (int f = tid; f < kFragsPerChunk * kWave; f += kThreads) {
    const int fl = f % kWave, ks = (f / kWave) % 2, db = f / (2 * kWave);
    uint32_t wd[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      uint32_t h2[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int j = jj * 2 + e;
        const int key = 32 * ks + 16 * (j / 4) + 4 * (fl / 16) + (j % 4);
        h2[e] = vs[key * kD + 16 * db + (fl % 16)];
      }
      wd[jj] = h2[0] | (h2[1] << 16);
    }
    reinterpret_cast<uint4*>(vdst)[f] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  }

  for (int qq = 0; qq < 16; ++qq) {
    const int qrow = w * 16 + qq;
    uint64_t keys[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int c = r * kWave + lane;
      keys[r] = c < ncand ? make_key(gs[qrow][c], c) : 0ull;
    }
    select_ascending<R>(keys, g.K, buf[w], buf2[w],
                        sel_idx + ((size_t)bkv * g.Lq + i0 + qrow) * g.K);
  }
}

// ----------------------------------------------------------------------------
// 2. attention
// ----------------------------------------------------------------------------
constexpr int kTB = 4;          // tiles per batch (P, row max and row sums in LDS)
constexpr int kAccStride = 144; // floats per accumulator row (576 B: head rows on other banks)

struct ChunkFrags {
  bf16x8 k[4];        // A operand: keys 16w + lane%16, k-step ks
  bf16x8 v[2][2];     // B operand: column block 2w + nb, key step ks
};

__device__ __forceinline__ void load_chunk_frags(const uint16_t* Kc, const uint16_t* Vfc, int w,
                                                 ChunkFrags& f) {
  const int lane = lane_id();
  const uint16_t* kr = Kc + (size_t)(w * 16 + (lane & 15)) * kD + (lane >> 4) * 8;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) f.k[ks] = ld8(kr + ks * 32);
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      f.v[nb][ks] = ld8(Vfc + ((size_t)((2 * w + nb) * 2 + ks) * kWave + lane) * 8);
}

struct AttendSmem {
  float acc[kRows * kAccStride];                 // fp32 output rows (row = qi*4 + h)
  uint16_t qs[kRows * kQStride];                 // window Q, row = qi*4 + h; reused for output
  uint4 pf[kTB][2][kWave];                       // unnormalised P, in A-operand fragment order
  float smax[kTB][4][16];
  float ssum[kTB][4][16];
  float wts[kW * kMaxKf * kG];                   // (query, slot, head): score, then weight
  int sel[kW * kMaxKf];
  uint8_t slotmap[kW * kMaxNC];                  // (query, chunk) -> slot, 0xff if not selected
  uint32_t qmask[kMaxNC];
  uint16_t ulist[kMaxNC];
  float lseown[kRows];
  float wown[kRows];
  float wsl[4][kW][kG];                          // per wave: fusion weight of (slot, head)
  int wcount[4];
};

// Phase A for tiles tbase .. tbase+ntl-1 (ntl <= kTB) of one chunk: S^T for this
// wave's 16 keys and the wave-partial row max.  Row r16 of a tile = (head
// r16/4, query slot r16%4); slot n of the chunk is query list[n].  vis_own >= 0
// marks the own chunk: key kk of query qi is visible when kk <= qi + vis_own.
__device__ __forceinline__ void phase_a(AttendSmem& sm, const ChunkFrags& f, int w, int tbase,
                                        int ntl, int lq, int nlist, float scale, int vis_own,
                                        float (&s)[kTB][4]) {
  const int lane = lane_id(), r16 = lane & 15, g4 = lane >> 4;
#pragma unroll
  for (int tl = 0; tl < kTB; ++tl) {
    if (tl >= ntl) break;
    const int slot = (tbase + tl) * 4 + (r16 & 3);
    const int qi = __shfl(lq, slot < nlist ? slot : 0, kWave);
    const uint16_t* qr = sm.qs + (qi * kG + (r16 >> 2)) * kQStride + g4 * 8;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 qb = as_bf16x8(*reinterpret_cast<const uint4*>(qr + ks * 32));
      acc = mfma(f.k[ks], qb, acc);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kk = w * 16 + g4 * 4 + i;
      const bool vis = vis_own < 0 || kk <= qi + vis_own;
      const float x = vis ? acc[i] * scale : -INFINITY;
      s[tl][i] = x;
      mx = fmaxf(mx, x);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    if (lane < 16) sm.smax[tl][w][r16] = mx;
  }
}

// Phase B: row max over the four waves, exponentials, P (bf16) and partial
// sums; s[tl][0] keeps the row max of row r16.
__device__ __forceinline__ void phase_b(AttendSmem& sm, int w, int ntl, float (&s)[kTB][4]) {
  const int lane = lane_id(), r16 = lane & 15, g4 = lane >> 4;
#pragma unroll
  for (int tl = 0; tl < kTB; ++tl) {
    if (tl >= ntl) break;
    const float m = fmaxf(fmaxf(sm.smax[tl][0][r16], sm.smax[tl][1][r16]),
                          fmaxf(sm.smax[tl][2][r16], sm.smax[tl][3][r16]));
    float e[4], z = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      e[i] = __expf(s[tl][i] - m);
      z += e[i];
    }
    z += __shfl_xor(z, 16, kWave);
    z += __shfl_xor(z, 32, kWave);
    if (lane < 16) sm.ssum[tl][w][r16] = z;
    // keys 16w + 4*g4 + i are elements 4*(w&1) + i of this lane's fragment for k-step w>>1
    reinterpret_cast<uint2*>(&sm.pf[tl][w >> 1][lane])[w & 1] =
        make_uint2(pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]));
    s[tl][0] = m;
  }
}

// Phase C for tile tl of the batch: O = P V for this wave's 32 columns; lane
// holds O[row 4*g4 + i][column 32w + 16nb + lane%16] in o[nb][i], and 1/rowsum
// of those rows in zi[i].
__device__ __forceinline__ void phase_c(const AttendSmem& sm, const ChunkFrags& f, int tl,
                                        f32x4 (&o)[2], float (&zi)[4]) {
  const int lane = lane_id(), r16 = lane & 15, g4 = lane >> 4;
  bf16x8 pa[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) pa[ks] = as_bf16x8(sm.pf[tl][ks][lane]);
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) acc = mfma(pa[ks], f.v[nb][ks], acc);
    o[nb] = acc;
  }
  const float z = sm.ssum[tl][0][r16] + sm.ssum[tl][1][r16] + sm.ssum[tl][2][r16] + sm.ssum[tl][3][r16];
  const float inv = 1.f / z;
#pragma unroll
  for (int i = 0; i < 4; ++i) zi[i] = __shfl(inv, g4 * 4 + i, kWave);
}

// acc[row of (query of slot i, head lane/16)][this wave's 32 columns] +=
// wgt[i] * O[.][i] for the nv valid slots of a tile.  No other wave writes these
// columns and the slots of a tile hold distinct queries, so all reads are issued
// before any write.
__device__ __forceinline__ void acc_update_tile(AttendSmem& sm, int w, const int (&qi)[4], int nv,
                                                const f32x4 (&o)[2], const float (&wgt)[4]) {
  const int lane = lane_id();
  float* a[4];
  float x0[4], x1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = sm.acc + (qi[i] * kG + (lane >> 4)) * kAccStride + 32 * w + (lane & 15);
    if (i < nv) { x0[i] = a[i][0]; x1[i] = a[i][16]; }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i < nv) {
      a[i][0] = x0[i] + wgt[i] * o[0][i];
      a[i][16] = x1[i] + wgt[i] * o[1][i];
    }
}

__global__ void __launch_bounds__(kThreads)
prefill_attend(Geometry g, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
               const uint16_t* __restrict__ vf, const uint16_t* __restrict__ lmk,
               const float* __restrict__ bias, const int32_t* __restrict__ sel_idx,
               uint16_t* __restrict__ out, float* __restrict__ lse_out) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  AttendSmem& sm = *reinterpret_cast<AttendSmem*>(smem_raw);
  // Workgroups are dispatched round-robin over the XCDs: with (b, kv head)
  // varying fastest, each XCD's L2 keeps serving the K/V of the same heads.
  // Windows run last-to-first (the late ones have the largest unions).
  const int nbkv = g.B * g.Hkv;
  const int bkv = blockIdx.x % nbkv;
  const int win = (g.Lq / kW - 1) - blockIdx.x / nbkv;
  const int b = bkv / g.Hkv, kvh = bkv % g.Hkv;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int K = g.K;
  const int i0 = win * kW;
  const int own = i0 / kS;
  const int ncand = min(own, g.NC);
  const uint16_t* Kg = k + (size_t)bkv * g.Lkv * kD;
  const uint16_t* Vfg = vf + (size_t)bkv * g.NC * kFragsPerChunk * kWave * 8;
  const uint16_t* Lg = lmk + (size_t)bkv * g.NCcap * kD;
  const float* bb = bias ? bias + (size_t)bkv * g.NCcap : nullptr;
  const float scale = g.scale;

  // ---- setup: window Q in LDS, selections, chunk -> query masks, union list
  for (int x = tid; x < kRows * 16; x += kThreads) {
    const int row = x >> 4, seg = x & 15;
    const int qi = row >> 2, h = row & 3;
    const uint4 u = *reinterpret_cast<const uint4*>(
        q + ((size_t)(b * g.Hq + kvh * kG + h) * g.Lq + i0 + qi) * kD + seg * 8);
    *reinterpret_cast<uint4*>(sm.qs + row * kQStride + seg * 8) = u;
  }
  for (int x = tid; x < kRows * kAccStride; x += kThreads) sm.acc[x] = 0.f;
  for (int x = tid; x < kW * K; x += kThreads)
    sm.sel[x] = sel_idx[((size_t)bkv * g.Lq + i0 + x / K) * K + x % K];
  for (int x = tid; x < kW * kMaxNC / 4; x += kThreads)
    reinterpret_cast<uint32_t*>(sm.slotmap)[x] = 0xffffffffu;
  for (int c = tid; c < kMaxNC; c += kThreads) sm.qmask[c] = 0u;
  __syncthreads();
  for (int x = tid; x < kW * K; x += kThreads) {
    const int c = sm.sel[x];
    if (c >= 0) {
      atomicOr(&sm.qmask[c], 1u << (x / K));
      sm.slotmap[(x / K) * kMaxNC + c] = (uint8_t)(x % K);
    }
  }
  __syncthreads();
  {
    const int c = tid;
    const bool f = c < ncand && sm.qmask[c] != 0u;
    const uint64_t m = __ballot(f);
    if (lane == 0) sm.wcount[w] = __popcll(m);
    __syncthreads();
    int off = 0;
    for (int x = 0; x < w; ++x) off += sm.wcount[x];
    if (f) sm.ulist[off + mask_rank(m)] = (uint16_t)c;
  }
  const int nunion = sm.wcount[0] + sm.wcount[1] + sm.wcount[2] + sm.wcount[3];

  // ---- retrieval scores of (row, selected chunk) by MFMA: rows x union columns
  {
    bf16x8 aq[2][4];
#pragma unroll
    for (int m2 = 0; m2 < 2; ++m2) {
      const int row = (2 * w + m2) * 16 + r16;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        aq[m2][ks] = as_bf16x8(*reinterpret_cast<const uint4*>(sm.qs + row * kQStride + g4 * 8 + ks * 32));
    }
    for (int nt = 0; nt * 16 < nunion; ++nt) {
      const int u = nt * 16 + r16;
      const int c = sm.ulist[u < nunion ? u : 0];
      bf16x8 bl[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) bl[ks] = ld8(Lg + (size_t)c * kD + g4 * 8 + ks * 32);
      const float bc = bb ? bb[c] : 0.f;
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mfma(aq[m2][ks], bl[ks], acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = (2 * w + m2) * 16 + g4 * 4 + i;
          const int qi = row >> 2, h = row & 3;
          const int slot = u < nunion ? sm.slotmap[qi * kMaxNC + c] : 0xff;
          if (slot != 0xff) sm.wts[(qi * K + slot) * kG + h] = scale * acc[i] + bc;
        }
      }
    }
  }
  __syncthreads();

  float s[kTB][4];
  ChunkFrags fr;

  // ---- own chunk, pass 1: row statistics -> lse_own (tile t = queries 4t..4t+3)
  if (g.keep_own) {
    load_chunk_frags(Kg + (size_t)own * kS * kD, Vfg + (size_t)own * kFragsPerChunk * kWave * 8, w, fr);
    for (int tb = 0; tb < kMaxT; tb += kTB) {
      phase_a(sm, fr, w, tb, kTB, lane, kW, scale, i0 - own * kS, s);
      __syncthreads();
      phase_b(sm, w, kTB, s);
      __syncthreads();
      if (w == 0) {
#pragma unroll
        for (int tl = 0; tl < kTB; ++tl) {
          const float z = sm.ssum[tl][0][r16] + sm.ssum[tl][1][r16] + sm.ssum[tl][2][r16] + sm.ssum[tl][3][r16];
          if (lane < 16) {
            const int qi = (tb + tl) * 4 + (r16 & 3), h = r16 >> 2;
            sm.lseown[qi * kG + h] = s[tl][0] + __logf(z);
          }
        }
      }
      __syncthreads();
    }
  }
  // ---- fusion weights: LSE over the retrieval scores and the own chunk's lse
  if (tid < kRows) {
    const int qi = tid >> 2, h = tid & 3;
    float m = g.keep_own ? sm.lseown[tid] : -INFINITY;
    for (int slot = 0; slot < K; ++slot)
      if (sm.sel[qi * K + slot] >= 0) m = fmaxf(m, sm.wts[(qi * K + slot) * kG + h]);
    float z = g.keep_own ? __expf(sm.lseown[tid] - m) : 0.f;
    for (int slot = 0; slot < K; ++slot)
      if (sm.sel[qi * K + slot] >= 0) z += __expf(sm.wts[(qi * K + slot) * kG + h] - m);
    const float LSE = z > 0.f ? m + __logf(z) : -INFINITY;
    for (int slot = 0; slot < K; ++slot)
      if (sm.sel[qi * K + slot] >= 0)
        sm.wts[(qi * K + slot) * kG + h] = __expf(sm.wts[(qi * K + slot) * kG + h] - LSE);
    sm.wown[tid] = (g.keep_own && z > 0.f) ? __expf(sm.lseown[tid] - LSE) : 0.f;
    if (lse_out) lse_out[(size_t)(b * g.Hq + kvh * kG + h) * g.Lq + i0 + qi] = LSE;
  }
  __syncthreads();
  // ---- own chunk, pass 2: P V weighted by w_own
  if (g.keep_own) {
    for (int tb = 0; tb < kMaxT; tb += kTB) {
      phase_a(sm, fr, w, tb, kTB, lane, kW, scale, i0 - own * kS, s);
      __syncthreads();
      phase_b(sm, w, kTB, s);
      __syncthreads();
#pragma unroll
      for (int tl = 0; tl < kTB; ++tl) {
        f32x4 o[2];
        float zi[4];
        phase_c(sm, fr, tl, o, zi);
        int qi[4];
        float wg[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          qi[i] = (tb + tl) * 4 + i;
          wg[i] = sm.wown[qi[i] * kG + g4] * zi[i];
        }
        acc_update_tile(sm, w, qi, 4, o, wg);
      }
      __syncthreads();
    }
  }

  // ---- retrieved chunks, all waves in step over the union
  if (nunion > 0)
    load_chunk_frags(Kg + (size_t)sm.ulist[0] * kS * kD,
                     Vfg + (size_t)sm.ulist[0] * kFragsPerChunk * kWave * 8, w, fr);
  for (int u = 0; u < nunion; ++u) {
    const int c = sm.ulist[u];
    const uint32_t qmk = sm.qmask[c];
    const int p = __popc(qmk);
    const int ntiles = (p + 3) >> 2;
    // slot n (n < p) of this chunk is the n-th selecting query: lane n holds it
    // in lq and its four fusion weights in wsl[w][n][*]
    int lq;
    {
      const bool bit = lane < kW && ((qmk >> (lane & 31)) & 1u);
      const uint64_t m = __ballot(bit);
      const int pos = mask_rank(m);
      // lane n takes the query of the n-th set bit (inverse of the rank map, via LDS)
      if (bit) sm.wsl[w][pos][0] = __int_as_float(lane);
      wave_sync_lds();
      lq = lane < p ? __float_as_int(sm.wsl[w][lane][0]) : 0;
      wave_sync_lds();
      if (lane < p) {
        const int ks = sm.slotmap[lq * kMaxNC + c];
        const float4 wv = *reinterpret_cast<const float4*>(&sm.wts[(lq * K + ks) * kG]);
        *reinterpret_cast<float4*>(&sm.wsl[w][lane][0]) = wv;
      }
    }
    ChunkFrags nx;
    const bool more = u + 1 < nunion;
    if (more) {   // prefetch the next chunk's fragments before this chunk's MFMA work
      const int cn = sm.ulist[u + 1];
      load_chunk_frags(Kg + (size_t)cn * kS * kD, Vfg + (size_t)cn * kFragsPerChunk * kWave * 8, w, nx);
    }
    for (int tb = 0; tb < ntiles; tb += kTB) {
      const int ntl = min(kTB, ntiles - tb);
      __syncthreads();   // previous batch's P, maxima and sums are consumed
      phase_a(sm, fr, w, tb, ntl, lq, p, scale, -1, s);
      __syncthreads();
      phase_b(sm, w, ntl, s);
      __syncthreads();
      for (int tl = 0; tl < ntl; ++tl) {
        f32x4 o[2];
        float zi[4];
        phase_c(sm, fr, tl, o, zi);
        const int s0 = (tb + tl) * 4;
        const int nv = min(4, p - s0);
        int qi[4];
        float wg[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int sl = i < nv ? s0 + i : s0;
          qi[i] = __builtin_amdgcn_readlane(lq, sl);
          wg[i] = sm.wsl[w][sl][g4] * zi[i];
        }
        acc_update_tile(sm, w, qi, nv, o, wg);
      }
    }
    if (more) fr = nx;
  }
  __syncthreads();

  // ---- output rows (bf16), 16 B per thread
  for (int x = tid; x < kRows * 16; x += kThreads) {
    const int row = x >> 4, seg = x & 15;
    const int qi = row >> 2, h = row & 3;
    const float* a = sm.acc + row * kAccStride + seg * 8;
    uint4 pk;
    pk.x = pack_bf16x2(a[0], a[1]);
    pk.y = pack_bf16x2(a[2], a[3]);
    pk.z = pack_bf16x2(a[4], a[5]);
    pk.w = pack_bf16x2(a[6], a[7]);
    *reinterpret_cast<uint4*>(out + ((size_t)(b * g.Hq + kvh * kG + h) * g.Lq + i0 + qi) * kD + seg * 8) = pk;
  }
}

}  // namespace

bool prefill_fast_supported(const Geometry& g, int bf16) {
  return bf16 && g.d == kD && g.S == kS && g.causal && g.Lq == g.Lkv && g.Lq % kSelWin == 0 &&
         g.G == kG && g.K <= kMaxKf && g.NC <= kMaxNC && g.Lq > 0;
}

size_t prefill_fast_ws(const Geometry& g) {
  return (size_t)g.B * g.Hkv * g.NC * kFragsPerChunk * kWave * 16;
}

hipError_t launch_prefill_fast(const Geometry& g, const void* q, const void* k, const void* v,
                               const void* lmk, const float* bias, void* out, int32_t* sel_idx,
                               float* lse, void* ws, hipStream_t st) {
  const uint16_t* Q = (const uint16_t*)q;
  const uint16_t* Lm = (const uint16_t*)lmk;
  uint16_t* vfrag = (uint16_t*)ws;
  const int R = g.NC <= 64 ? 1 : g.NC <= 128 ? 2 : 4;
  dim3 gsel((g.Lq / kSelWin) * g.B * g.Hkv);
  prof_begin(kPrefillSelect, st);
  switch (R) {
    case 1: hipLaunchKernelGGL(prefill_select<1>, gsel, dim3(kThreads), 0, st, g, Q, (const uint16_t*)v, Lm, bias, sel_idx, vfrag); break;
    case 2: hipLaunchKernelGGL(prefill_select<2>, gsel, dim3(kThreads), 0, st, g, Q, (const uint16_t*)v, Lm, bias, sel_idx, vfrag); break;
    default: hipLaunchKernelGGL(prefill_select<4>, gsel, dim3(kThreads), 0, st, g, Q, (const uint16_t*)v, Lm, bias, sel_idx, vfrag); break;
  }
  prof_end(kPrefillSelect, st);
  prof_begin(kPrefillAttend, st);
  // dynamic LDS above 64 KB must be enabled for the kernel (per device; cheap)
  hipFuncSetAttribute((const void*)prefill_attend, hipFuncAttributeMaxDynamicSharedMemorySize,
                      (int)sizeof(AttendSmem));
  hipLaunchKernelGGL(prefill_attend, dim3((g.Lq / kW) * g.B * g.Hkv), dim3(kThreads), sizeof(AttendSmem), st, g, Q,
                     (const uint16_t*)k, vfrag, Lm, bias, sel_idx, (uint16_t*)out, lse);
  prof_end(kPrefillAttend, st);
  return hipGetLastError();
}

}  // namespace hils
