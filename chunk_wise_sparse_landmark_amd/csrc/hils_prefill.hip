// MFMA prefill path: bf16, head_dim 128, chunk 64, GQA group of 4, causal,
// seq_q == seq_kv.
//
// Method: Hierarchical Sparse Attention Done Right (arXiv 2607.02980v1, summary
// page): landmark scores §3 "Linear surrogate for chunk mass", top-K routing §3
// "Sparse training", GQA-shared selection §4 "Architecture", per-chunk softmax
// and fusion by the retrieval scores §3 "Hierarchical softmax"; the attention
// kernel follows the page's kernel design (§4 "Kernel design": M adjacent
// queries x G heads as one (M x G, d) x (d, S) product over the union of their
// chunks, M x G >= 16), rebuilt for 64-wide waves and 16x16x32 bf16 MFMA.
//
//  1. prefill_select  one workgroup per chunk-aligned 64-query window (two,
//     one per 32-query half, from 256 candidates on).  Group scores
//     sum_h q_h . lmk_c are one MFMA chain (the G heads extend the reduction),
//     then each query's top-K is found without sorting (narrow rows: a bit
//     search four lanes per row; wide rows: tau = K-th largest lane maximum,
//     keys >= tau compacted in chunk order and a rank count keeps K, which come
//     out in ascending id).  The (first) workgroup also rewrites the window's
//     chunk of K and V in MFMA operand-fragment order (16 B per lane per
//     fragment), so the attention kernel stages a chunk with plain coalesced
//     copies and reads conflict-free 16-B fragments from LDS.
//  2. prefill_attend  one workgroup per 64-query window = 16 query blocks of
//     M = 4 queries x G = 4 heads = 16 rows.  Each of the eight waves owns two
//     blocks and keeps their fp32 output tiles in MFMA accumulators across all
//     chunks; the two waves of a SIMD run out of phase (one does its O += P V
//     a step late), so one's softmax overlaps the other's MFMA work.
//     For every chunk of the window's union it computes S^T = K Q^T, the chunk
//     softmax, and O += (w/Z) P V, where w is the row's fusion weight (0 for a
//     row whose query did not select the chunk) and Z the chunk's softmax sum;
//     a block none of whose queries selected the chunk is skipped.  Retrieval
//     scores of the window's rows against its union come from one MFMA pass and
//     the local window's exact lse from a statistics pass over its chunks, so
//     every fusion weight is final before any chunk is accumulated; the window
//     chunks then enter with P = exp(l - LSE).  Chunk fragments are staged
//     in LDS while the previous chunk is computed (K in two buffers, V in
//     three for the lagging waves): one barrier per chunk.
#include "hils_mfma.h"
#include "hils_kernels.h"
#include "hils_profile.h"

namespace hils {

namespace {

constexpr int kD = 128;
constexpr int kS = 64;
constexpr int kG = 4;            // query heads per KV group on this path
// prefill_select: with 4+ candidate blocks per row the score table fills the
// LDS (one workgroup per CU), so sixteen waves (four per SIMD) interleave their
// serial searches; with fewer, three workgroups of four waves share a CU
// prefill_select: four waves over a whole window below four candidate blocks
// per lane; eight waves over half a window (32 rows) from four blocks up, so
// that two workgroups (each with a 66 KB score table) share a CU
constexpr int sel_threads(int R) { return R >= 4 ? 512 : 256; }
constexpr int sel_rows(int R) { return R >= 4 ? 32 : 64; }
constexpr int kAttWaves = 8;             // prefill_attend: two waves per SIMD
constexpr int kAttThreads = kAttWaves * 64;
constexpr int kWin = 64;         // queries per window (one chunk), both kernels
constexpr int kBlocks = kWin / 4;          // 16 query blocks of 4 queries
constexpr int kBlocksPerWave = kBlocks / kAttWaves;
constexpr int kMaxKf = 32;       // top-K bound on this path
constexpr int kMaxNC = 512;      // chunks bound on this path (L <= 32768)
constexpr int kFrag = kWave * 8;           // bf16 per operand fragment (64 lanes x 16 B)
constexpr int kChunkFrags = 32;            // 16 K + 16 V fragments per chunk
constexpr int kChunkElems = kChunkFrags * kFrag;   // 16384 bf16 = 32 KB

// ----------------------------------------------------------------------------
// Top-K of R composite keys per lane (candidate c = r*64 + lane, key 0 =
// empty), written as ascending chunk ids (-1 padded) to dst[n*dstride ..).  The K-th
// largest key is found bit by bit from the top with wave ballots (count of
// keys >= prefix); keys are unique, so exactly the keys >= it are selected.
// The 32 score bits are searched first with 32-bit compares of the keys' high
// words; only a tie at the K-th score (or a zero score word among the top K)
// needs the id bits: with chunk ids below R*64 = 2^b the low word of every key
// is ~id with bits b..31 set, so b bits are searched.
// ----------------------------------------------------------------------------
// NR rows are searched together: their ballot and scalar chains are
// independent, so they overlap where a single row's chain would wait.
// The floor p[n] of row n's top K: the nonzero keys >= p[n] are exactly its
// min(K, valid) largest.  kIdBits: the id bits a key's low word can vary in.
template <int R, int NR, int kIdBits>
__device__ __forceinline__ void floor_search(const uint64_t (&keys)[NR][R], int K, uint64_t (&p)[NR]) {
  // the score word first, with 32-bit compares of the keys' high words
  // A prefix that exactly K keys reach already decides the row (the keys at or
  // above it are its top K), so the search stops there; for scores that are
  // not tied near the K-th that happens well before the last bit.  A search
  // that runs through bit 0 without that ended on a tie at the K-th score word
  // (the count at its floor is above K), or found no nonzero floor.
  uint32_t ph[NR];
  bool done[NR];
#pragma unroll
  for (int n = 0; n < NR; ++n) { ph[n] = 0u; done[n] = false; }
#pragma unroll
  for (int bit = 31; bit >= 0; --bit) {
    bool all = true;
#pragma unroll
    for (int n = 0; n < NR; ++n) {
      if (done[n]) continue;
      const uint32_t th = ph[n] | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int r = 0; r < R; ++r) cnt += __popcll(__ballot(static_cast<uint32_t>(keys[n][r] >> 32) >= th));
      if (cnt >= K) ph[n] = th;
      done[n] = cnt == K;
      all = all && done[n];
    }
    if (all) break;
  }
#pragma unroll
  for (int n = 0; n < NR; ++n) {
    p[n] = static_cast<uint64_t>(ph[n]) << 32;
    bool tie = !done[n];
    if (ph[n] == 0u) {
      // fewer than K valid keys (then all of them), or a zero score word among the top K
      p[n] = 1ull;
      int nvalid = 0;
#pragma unroll
      for (int r = 0; r < R; ++r) nvalid += __popcll(__ballot(keys[n][r] != 0ull));
      tie = nvalid > K;
    }
    if (tie) {
      // a tie at the K-th score word: the id bits decide
      uint64_t q = (p[n] == 1ull ? 0ull : p[n]) | static_cast<uint64_t>(0xffffffffu << kIdBits);
      for (int bit = kIdBits - 1; bit >= 0; --bit) {
        const uint64_t t = q | (1ull << bit);
        int cnt = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) cnt += __popcll(__ballot(keys[n][r] >= t));
        if (cnt >= K) q = t;
      }
      p[n] = q;
    }
  }
}

// The largest 32-bit floor th with at least K of the words >= th (0 when fewer
// than K words are nonzero), from the top bit down with wave ballots; stops at
// the first prefix that exactly K words reach.
template <int NR>
__device__ __forceinline__ void word_floor(const uint32_t (&h)[NR], int K, uint32_t (&ph)[NR]) {
  bool done[NR];
#pragma unroll
  for (int n = 0; n < NR; ++n) { ph[n] = 0u; done[n] = false; }
#pragma unroll
  for (int bit = 31; bit >= 0; --bit) {
    bool all = true;
#pragma unroll
    for (int n = 0; n < NR; ++n) {
      if (done[n]) continue;
      const uint32_t th = ph[n] | (1u << bit);
      const int cnt = __popcll(__ballot(h[n] >= th));
      if (cnt >= K) ph[n] = th;
      done[n] = cnt == K;
      all = all && done[n];
    }
    if (all) break;
  }
}

// The nonzero keys >= p of R keys per lane (candidate r*64 + lane), in
// ascending candidate order, as chunk ids into d[0, K); -1 past the last.
template <int R>
__device__ __forceinline__ void write_ascending(const uint64_t (&keys)[R], uint64_t p, int K, int32_t* d,
                                                int lane) {
  int base = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool pred = keys[r] != 0ull && keys[r] >= p;
    const uint64_t m = __ballot(pred);
    const int at = base + mask_rank(m);
    if (pred && at < K) d[at] = key_index(keys[r]);   // (exactly min(K, valid) keys pass)
    base += __popcll(m);
  }
  for (int x = base + lane; x < K; x += kWave) d[x] = -1;
}

template <int R, int NR>
__device__ __forceinline__ void select_ascending(const uint64_t (&keys)[NR][R], int K, int32_t* dst,
                                                 size_t dstride, uint64_t* buf) {
  const int lane = lane_id();
  constexpr int kIdBits = R == 1 ? 6 : (R == 2 ? 7 : (R == 4 ? 8 : 9));
  uint64_t p[NR];
  if constexpr (R >= 4) {
    static_assert(NR == 1, "one row at a time with wide rows");
    // Prefilter: every top-K key has a score word >= the K-th largest of the 64
    // lanes' maximum score words (at least K lanes hold a key that reaches it).
    // The keys that reach it (about K for untied scores) are compacted in
    // candidate order and, when at most 64 do, each one's rank among them is
    // counted from LDS broadcasts: the top K are those of rank < K, with no
    // further bit search.  Lanes that hold no key of a batch write it to a slot
    // of their own at 64 + lane, so that no store is predicated.
    uint32_t lm[1];
    lm[0] = static_cast<uint32_t>(keys[0][0] >> 32);
#pragma unroll
    for (int r = 1; r < R; ++r) lm[0] = max(lm[0], static_cast<uint32_t>(keys[0][r] >> 32));
    uint32_t ph[1];
    word_floor<1>(lm, K, ph);
    const uint64_t tau = ph[0] ? static_cast<uint64_t>(ph[0]) << 32 : 1ull;
    uint64_t m[R];
    int pre[R];
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      m[r] = __ballot(keys[0][r] >= tau);
      pre[r] = cnt;
      cnt += __popcll(m[r]);
    }
    if (cnt <= kWave) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const bool pr = keys[0][r] >= tau;
        const int at = pre[r] + mask_rank(m[r]);
        buf[pr ? at : kWave + lane] = keys[0][r];
      }
      if (lane >= cnt) buf[lane] = 0ull;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // keys are unique, so the ranks are distinct; empty slots (0) rank nothing
      const uint64_t mine = buf[lane];
      int rank = 0;
      const ulonglong2* b2 = reinterpret_cast<const ulonglong2*>(buf);
      for (int j = 0; j < cnt; j += 8) {
        ulonglong2 kk[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) kk[x] = b2[j / 2 + x];
#pragma unroll
        for (int x = 0; x < 4; ++x) rank += (kk[x].x > mine) + (kk[x].y > mine);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const bool sel = mine != 0ull && rank < K;
      const uint64_t ms = __ballot(sel);
      if (sel) dst[mask_rank(ms)] = key_index(mine);
      for (int x = __popcll(ms) + lane; x < K; x += kWave) dst[x] = -1;
      return;
    }
  }
  floor_search<R, NR, kIdBits>(keys, K, p);
#pragma unroll
  for (int n = 0; n < NR; ++n) write_ascending<R>(keys[n], p[n], K, dst + n * dstride, lane);
}

// Sums over the four lanes of a quad (lane & ~3 .. lane | 3) by DPP quad
// permutes: every lane of the quad receives the total, or the sum over the
// quad's lanes below its own (q = lane % 4).
__device__ __forceinline__ int quad_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xf, 0xf, false);   // lanes [1,0,3,2]
  x += __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xf, 0xf, false);   // lanes [2,3,0,1]
  return x;
}
__device__ __forceinline__ int quad_below(int x, int q) {
  const int v0 = __builtin_amdgcn_update_dpp(0, x, 0x00, 0xf, 0xf, false);   // lane 0 of the quad
  const int v1 = __builtin_amdgcn_update_dpp(0, x, 0x55, 0xf, 0xf, false);   // lane 1
  const int v2 = __builtin_amdgcn_update_dpp(0, x, 0xAA, 0xf, 0xf, false);   // lane 2
  return (q > 0 ? v0 : 0) + (q > 1 ? v1 : 0) + (q > 2 ? v2 : 0);
}

// Top K of the 64R (R <= 2) candidates of 16 score rows (rows 0..15 at `row0`,
// `stride` floats apart), written as ascending chunk ids (-1 past the last) to
// the 16 consecutive K-entry rows at `dst`.  Four lanes share a row: lane part
// q holds candidates q*n .. q*n + n - 1 as order-preserving score words in
// registers.  The K-th largest word is found bit by bit, each row's count of
// words >= the trial floor summed over its quad; the rows' searches run side
// by side in the lanes, so a round costs two vector instructions per word and
// no scalar chain.  A floor that exactly K words reach stays so as the search
// goes on, and the search stops once every row of the wave has met one.  The
// words above the floor are taken, then the lowest-id words at it up to K,
// which is the composite-key order.  `stage` is 16*32 + 64 ints of LDS private
// to the wave.
template <int R>
__device__ __forceinline__ void narrow_rows_topk(const float* row0, int stride, int ncand, int K, int32_t* dst,
                                                 int* stage) {
  constexpr int P = 4, kRows = kWave / P, n = R * kWave / P;
  const int lane = lane_id(), rl = lane / P, q = lane % P;
  const float* src = row0 + rl * stride + q * n;
  uint32_t wd[n];
#pragma unroll
  for (int j = 0; j < n; ++j) {
    // read unconditionally (a predicated read is waited for before the next);
    // valid words are kept nonzero (word 0 is one NaN pattern, ranked with the
    // NaN next to it) so that 0 marks the candidates past ncand
    const uint32_t u = __float_as_uint(src[j]);
    const uint32_t o = max(u ^ (static_cast<uint32_t>(static_cast<int32_t>(u) >> 31) | 0x80000000u), 1u);
    wd[j] = q * n + j < ncand ? o : 0u;
  }
  // the words are in registers before `stage` (which may be the rows just
  // read) is written
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  int* st = stage + rl * K;
  if (ncand <= K) {
    // every candidate is taken
    for (int x = q; x < K; x += P) st[x] = x < ncand ? x : -1;
  } else {
    // ph: the largest floor that at least K of the row's words reach
    uint32_t ph = 0u;
    uint64_t done = 0ull;
#pragma unroll
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t th = ph | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < n; ++j) cnt += wd[j] >= th ? 1 : 0;
      cnt = quad_sum(cnt);
      ph = cnt >= K ? th : ph;
      done |= __ballot(cnt == K);
      if (done == ~0ull) break;
    }
    int ngt = 0, neq = 0;
#pragma unroll
    for (int j = 0; j < n; ++j) {
      ngt += wd[j] > ph ? 1 : 0;
      neq += wd[j] == ph ? 1 : 0;
    }
    const int need = K - quad_sum(ngt);
    const int teq = min(max(need - quad_below(neq, q), 0), neq);
    const int mine = ngt + teq;
    const int total = quad_sum(mine);
    for (int x = total + q; x < K; x += P) st[x] = -1;
    int pos = quad_below(mine, q), eqs = 0;
    int* trash = stage + kRows * kMaxKf + lane;
    // the same floor through an identity lane permute, so that the compares
    // are made again here rather than 2n lane masks kept in scalar registers
    const uint32_t pf = static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(ph), 0xE4, 0xf, 0xf, false));
#pragma unroll
    for (int j = 0; j < n; ++j) {
      const bool e = wd[j] == pf;
      const bool t = wd[j] > pf || (e && eqs < teq);
      *(t ? st + pos : trash) = q * n + j;
      pos += t ? 1 : 0;
      eqs += e ? 1 : 0;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  for (int x = lane; x < kRows * K; x += kWave) dst[x] = stage[x];
}

// ----------------------------------------------------------------------------
// 1. selection (+ this window's chunk of K and V in operand-fragment order)
//    KVf[bkv][chunk] = 16 K fragments then 16 V fragments, 64 lanes x 16 B each:
//    K fragment f = mt*4 + ks, lane l, element j: K[16mt + l%16][32ks + 8(l/16) + j]
//      (A operand of S^T = K Q^T for keys 16mt.., k-step ks);
//    V fragment f = db*2 + ks, lane l, element j:
//      V[32ks + 16(j/4) + 4(l/16) + j%4][16db + l%16]
//      (B operand of O = P V for columns 16db.., keys 32ks.., in the key order
//      in which P leaves the S^T accumulators).
// ----------------------------------------------------------------------------
template <int R>
__global__ void __launch_bounds__(sel_threads(R), R >= 4 ? 2 : 3)
prefill_select(Geometry g, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
               const uint16_t* __restrict__ v, const uint16_t* __restrict__ lmk,
               const float* __restrict__ bias, int32_t* __restrict__ sel_idx,
               uint16_t* __restrict__ kvf) {
  constexpr int NCP = R * kWave;
  constexpr int kRows = sel_rows(R);          // score rows (queries) of this workgroup
  constexpr int kHalves = kWin / kRows;
  constexpr bool kStageV = R < 4;             // V rewritten through LDS (else gathered)
  __shared__ __attribute__((aligned(16))) float gs[kRows][NCP + 1];
  __shared__ __attribute__((aligned(16))) uint16_t vs[kStageV ? kS * kD : 8];
  // wide rows: each wave's work buffer for its row searches (128 keys)
  __shared__ __attribute__((aligned(16))) uint64_t wbuf[kStageV ? 1 : sel_threads(R) / kWave][2 * kWave];
  const int nbkv = g.B * g.Hkv;            // (b, kv head) fastest: one head per XCD
  const int bkv = blockIdx.x % nbkv;
  const int wh = blockIdx.x / nbkv;
  const int win = (g.Lq / kWin - 1) - wh / kHalves, half = wh % kHalves;
  const int b = bkv / g.Hkv, kvh = bkv % g.Hkv;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int i0 = win * kWin + half * kRows;
  // the window's own chunk is rewritten in fragment order by its first half
  const bool rewrite = half == 0;
  // candidates: complete chunks before the local window (own chunk `win` and the
  // g.win - 1 chunks before it)
  const int ncand = max(0, min(win - max(g.win - 1, 0), g.NC));
  const int r16 = lane & 15, g4 = lane >> 4;

  // V of chunk `win` -> LDS (coalesced), later rewritten in fragment order
  const size_t row0 = (size_t)bkv * g.Lkv + (size_t)win * kS;
  const uint16_t* Vc = v + row0 * kD;
  const uint16_t* Kc = k + row0 * kD;
  constexpr int kThreads = sel_threads(R);
  constexpr int kSelWaves = kThreads / kWave;
  // the loads of the chunk's own K and V go out first, so that their latency
  // overlaps the query and landmark loads of the scores: V by direct
  // global->LDS copies (lane i of a wave lands at the wave's base + 16 i; they
  // have landed at the wait before the V rewrite below), K into registers for
  // its fragment rewrite (below 8 candidate blocks per lane; at 8 the
  // registers are taken by the landmark batches, and K is loaded at the
  // rewrite)
  if constexpr (kStageV) {
    const int wbase = w * kWave;
#pragma unroll
    for (int j = 0; j < kS * kD / 8 / kThreads; ++j)
      __builtin_amdgcn_global_load_lds(
          (const void*)(reinterpret_cast<const uint4*>(Vc) + j * kThreads + tid),
          (__attribute__((address_space(3))) void*)(reinterpret_cast<uint4*>(vs) + j * kThreads + wbase),
          16, 0, 0);
  }
  constexpr int kKf = 16 * kWave / kThreads;   // K fragment words per thread
  constexpr bool kEarlyK = R < 8;
  // K word i of this thread: fragment f = tid + i * kThreads, lane fl, k-step
  // ks, key tile mt
  auto kf_src = [&](int i) {
    const int f = tid + i * kThreads;
    const int fl = f % kWave, ks = (f / kWave) % 4, mt = f / (4 * kWave);
    return reinterpret_cast<const bf16x8*>(Kc + (size_t)(16 * mt + fl % 16) * kD + 32 * ks + 8 * (fl / 16));
  };
  bf16x8 kfr[kKf];
  if (kEarlyK && rewrite) {
#pragma unroll
    for (int i = 0; i < kKf; ++i) kfr[i] = *kf_src(i);
  }

  // scores: with nw waves over kRows rows (kRG row groups of 16), wave w
  // computes the rows of row group w % kRG against batches w / kRG,
  // w / kRG + nw / kRG, ... of the column tiles, and each wave then selects
  // for its own kRows / nw rows below
  // A operand: 16 queries of this row group x 4 heads x 4 k-steps
  constexpr int kRG = kRows / 16;           // row groups of 16 queries
  const int rg = w % kRG, ch = w / kRG;     // (four waves over 64 rows: ch = 0)
  bf16x8 a[kG][4];
#pragma unroll
  for (int h = 0; h < kG; ++h) {
    const uint16_t* qr = q + ((size_t)(b * g.Hq + kvh * kG + h) * g.Lq + i0 + rg * 16 + r16) * kD + g4 * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) a[h][ks] = ld8(qr + ks * 32);
  }
  const uint16_t* L = lmk + (size_t)bkv * g.NCcap * kD;
  // the biases are read with the landmark rows, unpredicated (without a bias
  // the loads read a landmark word and are discarded): a predicated load would
  // make the compiler wait for every load in flight after it
  const bool use_bias = bias != nullptr;
  const float* bsrc = use_bias ? bias + (size_t)bkv * g.NCcap : reinterpret_cast<const float*>(L);
  const float sc = g.scale / (float)kG;
  const int ntile = (ncand + 15) / 16;
  // column tiles per batch: 2 with sixteen waves (128 registers each), 4 with
  // small tables, so that three workgroups fit a CU's registers
  constexpr int kTiles = R >= 4 ? 2 : 4;
  for (int nt0 = kTiles * ch; nt0 < ntile; nt0 += kTiles * (kSelWaves / kRG)) {
    bf16x8 bv[kTiles][4];   // the loads of up to kTiles column tiles in flight together
    float bx[kTiles];
#pragma unroll
    for (int x = 0; x < kTiles; ++x) {
      const int c = (nt0 + x) * 16 + r16;
      const int cl = c < ncand ? c : 0;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) bv[x][ks] = ld8(L + (size_t)cl * kD + g4 * 8 + ks * 32);
      bx[x] = bsrc[use_bias ? cl : 0];
    }
    // every tile of the batch is multiplied and stored, a tile past the last
    // one (clamped rows) into the padding column: no branch, so that no load
    // of the batch is sunk after one
#pragma unroll
    for (int x = 0; x < kTiles; ++x) {
      const int nt = nt0 + x;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int h = 0; h < kG; ++h)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mfma(a[h][ks], bv[x][ks], acc);
      const int c = nt * 16 + r16;
      const float bc = (use_bias && c < ncand) ? bx[x] : 0.f;
      const int cs = nt < ntile ? c : NCP;
#pragma unroll
      for (int i = 0; i < 4; ++i) gs[rg * 16 + g4 * 4 + i][cs] = acc[i] * sc + bc;
    }
  }

  constexpr int kRowsPerWave = kRows / (kThreads / kWave);
  if constexpr (R <= 2) {
    // Narrow rows: wave w scored its own 16 rows against every column tile, so
    // it searches them now, without waiting for the other waves or the chunk
    // rewrite below; its table rows, dead once their words are in registers,
    // are its work space.
    static_assert(kSelWaves == kRG && kRowsPerWave == kWave / 4, "a wave owns its rows");
    static_assert(kRowsPerWave * kMaxKf + kWave <= kRowsPerWave * (NCP + 1), "staging");
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    narrow_rows_topk<R>(&gs[w * kRowsPerWave][0], NCP + 1, ncand, g.K,
                        sel_idx + ((size_t)bkv * g.Lq + i0 + w * kRowsPerWave) * g.K,
                        reinterpret_cast<int*>(&gs[w * kRowsPerWave][0]));
  }

  // K fragments of this chunk: straight 16-B copies
  uint16_t* kdst = kvf + ((size_t)bkv * g.NC + win) * kChunkElems;
  uint16_t* vdst = kdst + 16 * kFrag;
  // V fragment f, lane fl, element j: V[32ks + 16(j/4) + 4(fl/16) + j%4][16db + fl%16]
  auto v_key = [](int f, int j) {
    const int fl = f % kWave, ks = (f / kWave) % 2;
    return 32 * ks + 16 * (j / 4) + 4 * (fl / 16) + (j % 4);
  };
  auto v_col = [](int f) { return 16 * (f / (2 * kWave)) + (f % kWave) % 16; };
  if constexpr (kStageV) {
    if constexpr (!kEarlyK) {
#pragma unroll
      for (int i = 0; i < kKf; ++i) kfr[i] = *kf_src(i);
    }
#pragma unroll
    for (int i = 0; i < kKf; ++i) reinterpret_cast<bf16x8*>(kdst)[tid + i * kThreads] = kfr[i];
    __builtin_amdgcn_s_waitcnt(0);           // this thread's V copies have landed
    __syncthreads();
    // V fragments of this chunk, from the LDS copy
    for (int f = tid; f < 16 * kWave; f += kThreads) {
      uint32_t wd[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        wd[jj] = (uint32_t)vs[v_key(f, 2 * jj) * kD + v_col(f)] |
                 ((uint32_t)vs[v_key(f, 2 * jj + 1) * kD + v_col(f)] << 16);
      reinterpret_cast<uint4*>(vdst)[f] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    }
  } else if (rewrite) {
    if constexpr (!kEarlyK) {
#pragma unroll
      for (int i = 0; i < kKf; ++i) kfr[i] = *kf_src(i);
    }
#pragma unroll
    for (int i = 0; i < kKf; ++i) reinterpret_cast<bf16x8*>(kdst)[tid + i * kThreads] = kfr[i];
    // V fragments gathered straight from the V rows (a wave's 2-byte loads
    // cover 32 contiguous bytes of each of four rows), all issued together
    constexpr int kVf = 16 * kWave / kThreads;
    uint16_t hv[kVf][8];
#pragma unroll
    for (int i = 0; i < kVf; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) hv[i][j] = Vc[v_key(tid + i * kThreads, j) * kD + v_col(tid + i * kThreads)];
#pragma unroll
    for (int i = 0; i < kVf; ++i) {
      uint32_t wd[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) wd[jj] = (uint32_t)hv[i][2 * jj] | ((uint32_t)hv[i][2 * jj + 1] << 16);
      reinterpret_cast<uint4*>(vdst)[tid + i * kThreads] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    }
  }

  // the selection of the wide rows (the narrow ones are done above)
  if constexpr (R >= 4) {
    __syncthreads();
    // one row at a time over the whole wave
    for (int q0 = 0; q0 < kRowsPerWave; ++q0) {
      const int row = w * kRowsPerWave + q0;
      uint64_t keys[1][R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        // read unconditionally (the table is NCP + 1 wide), masked after: a
        // predicated read would be waited for before the next one is issued
        const int c = r * kWave + lane;
        const uint64_t kk = make_key(gs[row][c], c);
        keys[0][r] = kk & (c < ncand ? ~0ull : 0ull);
      }
      select_ascending<R, 1>(keys, g.K, sel_idx + ((size_t)bkv * g.Lq + i0 + row) * g.K,
                             (size_t)g.K, &wbuf[w][0]);
    }
  }
}

// ----------------------------------------------------------------------------
// 2. attention
// ----------------------------------------------------------------------------
struct AttendSmem {
  // staged chunk t: its K fragments in kb[t % 2], its V fragments in vb[t % 3]
  // (a V buffer lives one step longer: the lagging waves multiply it in the
  // step after its scores)
  uint4 kb[2][16 * kWave];
  uint4 vb[3][16 * kWave];
  float wts[kWin * kMaxKf * kG];          // (query, slot, head): score, then weight
  int sel[kWin * kMaxKf];
  uint8_t slotmap[kWin * kMaxNC];         // (query, chunk) -> slot, 0xff if not selected
  uint64_t qmask[kMaxNC];                 // chunk -> window queries that selected it
  uint16_t ulist[kMaxNC];
  float lsewin[kWin * kG];                // (query, head): lse of the local window's tokens
  float lse2[kWin * kG];                  // (query, head): the row's LSE in log2 units
  int wcount[kAttWaves];
};
static_assert(sizeof(AttendSmem) <= 160 * 1024, "attention LDS exceeds one CU's 160 KB");

// Start copying one chunk's 16 KB of K fragments and 16 KB of V fragments
// into two LDS buffers with direct global->LDS loads (16 B per lane; lane i of
// a wave lands at the wave's LDS base + 16 i).  Completion: s_waitcnt
// vmcnt(0), then a barrier.
__device__ __forceinline__ void stage_async(const uint16_t* __restrict__ src, uint4* __restrict__ kdst,
                                            uint4* __restrict__ vdst) {
  static_assert(16 * kWave == 2 * kAttThreads, "two copies per thread for each half");
  const uint4* s = reinterpret_cast<const uint4*>(src);
  const int wbase = (threadIdx.x / kWave) * kWave;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    uint4* dst = x < 2 ? kdst + x * kAttThreads : vdst + (x - 2) * kAttThreads;
    __builtin_amdgcn_global_load_lds((const void*)(s + x * kAttThreads + threadIdx.x),
                                     (__attribute__((address_space(3))) void*)(dst + wbase), 16, 0, 0);
  }
}
__device__ __forceinline__ void stage_wait() { __builtin_amdgcn_s_waitcnt(0); }

// S^T = K Q^T of one block: 64 keys x 16 rows; lane l holds keys
// 16mt + 4(l/16) + i of row l%16.
__device__ __forceinline__ void block_scores(const bf16x8 (&kf)[16], const bf16x8 (&qf)[4],
                                             f32x4 (&s)[4]) {
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc = mfma(kf[mt * 4 + ks], qf[ks], acc);
    s[mt] = acc;
  }
}

// Chunk softmax of one block in place: s <- exp2(sc2*s - m); returns the row
// max m (log2 units) and the row sum z.  kMasked hides keys >= vis.
template <bool kMasked>
__device__ __forceinline__ void block_softmax(f32x4 (&s)[4], float sc2, int vis, float& m_out,
                                              float& z_out) {
  const int g4 = lane_id() >> 4;
  if (kMasked) {
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
  float z = 0.f;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][i], sc2, -mb));
      s[mt][i] = e;
      z += e;
    }
  m_out = mb;
  z_out = rowgroup_sum(z);
}

// Window chunks enter the fusion with their exact lse, so their tokens' fused
// weight is exp(l - LSE): s <- exp2(sc2*s - lse2) with the row's final LSE in
// log2 units, no per-chunk statistics.  kMasked hides keys >= vis.
template <bool kMasked>
__device__ __forceinline__ void block_direct(f32x4 (&s)[4], float sc2, int vis, float lse2) {
  const int g4 = lane_id() >> 4;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[mt][i], sc2, -lse2));
      s[mt][i] = (kMasked && mt * 16 + g4 * 4 + i >= vis) ? 0.f : e;
    }
}

// P (scaled by f) as the A operand of O += P V: k-slot (g4, j) <-> key
// 32ks + 16(j/4) + 4g4 + j%4, which is how S^T left the keys in the lane.
__device__ __forceinline__ void pack_p(const f32x4 (&s)[4], float f, bf16x8 (&pa)[2]) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    uint32_t w4[4];
    w4[0] = pack_bf16x2(s[2 * ks][0] * f, s[2 * ks][1] * f);
    w4[1] = pack_bf16x2(s[2 * ks][2] * f, s[2 * ks][3] * f);
    w4[2] = pack_bf16x2(s[2 * ks + 1][0] * f, s[2 * ks + 1][1] * f);
    w4[3] = pack_bf16x2(s[2 * ks + 1][2] * f, s[2 * ks + 1][3] * f);
    __builtin_memcpy(&pa[ks], w4, 16);
  }
}

__device__ __forceinline__ void load_frags(const uint4* __restrict__ src, bf16x8 (&f)[16]) {
  const int lane = lane_id();
#pragma unroll
  for (int x = 0; x < 16; ++x) f[x] = as_bf16x8(src[x * kWave + lane]);
}

// Scores, chunk softmax and P of one staged chunk for the wave's active query
// blocks (`act` bit j: block j takes part, uniform over the wave); S^T of
// every active block first, then the softmaxes, so the MFMA work of one block
// overlaps the softmax of another.  rw[j] is this lane's row weight; P leaves
// scaled by rw / z.  kDirect (a local-window chunk): P = exp(l - LSE) with
// rw[j] = the row's LSE in log2 units.
template <bool kMasked, bool kDirect>
__device__ __forceinline__ void chunk_probs(const uint4* __restrict__ kbuf,
                                            const bf16x8 (&qf)[kBlocksPerWave][4], float sc2,
                                            unsigned act, const int (&vis)[kBlocksPerWave],
                                            const float (&rw)[kBlocksPerWave],
                                            bf16x8 (&pa)[kBlocksPerWave][2]) {
  f32x4 s[kBlocksPerWave][4];
  {
    bf16x8 kf[16];
    load_frags(kbuf, kf);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int j = 0; j < kBlocksPerWave; ++j)
      if (act & (1u << j)) block_scores(kf, qf[j], s[j]);
    __builtin_amdgcn_s_setprio(0);
  }
#pragma unroll
  for (int j = 0; j < kBlocksPerWave; ++j) {
    if (act & (1u << j)) {
      if (kDirect) {
        block_direct<kMasked>(s[j], sc2, vis[j], rw[j]);
        pack_p(s[j], 1.f, pa[j]);
      } else {
        float m, z;
        block_softmax<kMasked>(s[j], sc2, vis[j], m, z);
        pack_p(s[j], rw[j] * __builtin_amdgcn_rcpf(z), pa[j]);
      }
    }
  }
}

// O += P V for the active blocks of `act`, V from one staged chunk.
__device__ __forceinline__ void chunk_pv(const uint4* __restrict__ vbuf, unsigned act,
                                         const bf16x8 (&pa)[kBlocksPerWave][2],
                                         f32x4 (&o)[kBlocksPerWave][8]) {
  bf16x8 vf[16];
  load_frags(vbuf, vf);
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int j = 0; j < kBlocksPerWave; ++j)
    if (act & (1u << j)) {
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) o[j][db] = mfma(pa[j][ks], vf[db * 2 + ks], o[j][db]);
    }
  __builtin_amdgcn_s_setprio(0);
}

// One accumulation step.  The two waves that share a SIMD run it out of phase:
// a leading wave does this chunk's scores and softmax, then its O += P V; a
// lagging wave first does O += P V of the previous step's chunk (P and the
// block mask kept in pa / pact, V still staged), then this chunk's scores and
// softmax.  So one wave's softmax (vector ALU) runs against the other's MFMA
// work instead of both waves doing the same phase between two barriers.  The
// next chunk's copy is started first, into buffers no wave reads in this step.
template <bool kMasked, bool kDirect>
__device__ __forceinline__ void chunk_step(bool lag, const uint4* __restrict__ kbuf,
                                           const uint4* __restrict__ vbuf,
                                           const uint4* __restrict__ vprev,
                                           uint4* __restrict__ knx, uint4* __restrict__ vnx,
                                           const uint16_t* __restrict__ nsrc,
                                           const bf16x8 (&qf)[kBlocksPerWave][4], float sc2,
                                           unsigned act, const int (&vis)[kBlocksPerWave],
                                           const float (&rw)[kBlocksPerWave], unsigned& pact,
                                           bf16x8 (&pa)[kBlocksPerWave][2],
                                           f32x4 (&o)[kBlocksPerWave][8]) {
  if (nsrc) stage_async(nsrc, knx, vnx);
  // a wave none of whose blocks takes part reads no fragments
  if (lag) {
    if (pact) chunk_pv(vprev, pact, pa, o);
    __builtin_amdgcn_sched_barrier(0);
    if (act) chunk_probs<kMasked, kDirect>(kbuf, qf, sc2, act, vis, rw, pa);
  } else if (act) {
    chunk_probs<kMasked, kDirect>(kbuf, qf, sc2, act, vis, rw, pa);
    // keep the V fragment loads after the softmax (register pressure)
    __builtin_amdgcn_sched_barrier(0);
    chunk_pv(vbuf, act, pa, o);
  }
  pact = act;
}

// Statistics of one staged local-window chunk for every block of the wave: the
// chunk's row max (log2 units) and sum are folded into the running (M2, Z).
template <bool kMasked>
__device__ __forceinline__ void window_stats_step(const uint4* __restrict__ kbuf,
                                                  uint4* __restrict__ knx, uint4* __restrict__ vnx,
                                                  const uint16_t* __restrict__ nsrc,
                                                  const bf16x8 (&qf)[kBlocksPerWave][4], float sc2,
                                                  const int (&vis)[kBlocksPerWave],
                                                  float (&M2)[kBlocksPerWave],
                                                  float (&Z)[kBlocksPerWave]) {
  if (nsrc) stage_async(nsrc, knx, vnx);
  bf16x8 kf[16];
  load_frags(kbuf, kf);
#pragma unroll
  for (int j = 0; j < kBlocksPerWave; ++j) {
    f32x4 st[4];
    float m2, z;
    block_scores(kf, qf[j], st);
    block_softmax<kMasked>(st, sc2, vis[j], m2, z);
    const float mn = fmax2(M2[j], m2);
    Z[j] = Z[j] * __builtin_amdgcn_exp2f(M2[j] - mn) + z * __builtin_amdgcn_exp2f(m2 - mn);
    M2[j] = mn;
  }
}

__global__ void __launch_bounds__(kAttThreads)
prefill_attend(Geometry g, const uint16_t* __restrict__ q, const uint16_t* __restrict__ qr,
               const uint16_t* __restrict__ kvf,
               const uint16_t* __restrict__ lmk, const float* __restrict__ bias,
               const int32_t* __restrict__ sel_idx, uint16_t* __restrict__ out,
               float* __restrict__ lse_out) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  AttendSmem& sm = *reinterpret_cast<AttendSmem*>(smem_raw);
  // (b, kv head) fastest over the workgroup id: consecutive workgroups go to
  // different XCDs, so each XCD's L2 keeps serving the same heads.  Windows run
  // last to first (late windows have the largest unions).
  const int nbkv = g.B * g.Hkv;
  const int bkv = blockIdx.x % nbkv;
  const int win = (g.Lq / kWin - 1) - blockIdx.x / nbkv;
  const int b = bkv / g.Hkv, kvh = bkv % g.Hkv;
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int K = g.K;
  const int i0 = win * kWin;
  const int own = win;                    // the window is exactly chunk `win`
  // local window: chunks own, own - 1, .., own - nwin + 1; candidates precede it
  const int nwin = g.win > 0 ? 1 + min(g.win - 1, own) : 0;
  const int ncand = max(0, min(own - max(g.win - 1, 0), g.NC));
  const uint16_t* KVg = kvf + (size_t)bkv * g.NC * kChunkElems;
  const uint16_t* Lg = lmk + (size_t)bkv * g.NCcap * kD;
  const float* bb = bias ? bias + (size_t)bkv * g.NCcap : nullptr;
  const float scale = g.scale;

  // ---- setup: selections, chunk -> query masks, union list
  for (int x = tid; x < kWin * K; x += kAttThreads)
    sm.sel[x] = sel_idx[((size_t)bkv * g.Lq + i0 + x / K) * K + x % K];
  for (int x = tid; x < kWin * kMaxNC / 4; x += kAttThreads)
    reinterpret_cast<uint32_t*>(sm.slotmap)[x] = 0xffffffffu;
  for (int c = tid; c < kMaxNC; c += kAttThreads) sm.qmask[c] = 0ull;
  __syncthreads();
  for (int x = tid; x < kWin * K; x += kAttThreads) {
    const int c = sm.sel[x];
    if (c >= 0) {
      atomicOr((unsigned long long*)&sm.qmask[c], 1ull << (x / K));
      sm.slotmap[(x / K) * kMaxNC + c] = (uint8_t)(x % K);
    }
  }
  __syncthreads();
  int nunion = 0;
  for (int c0 = 0; c0 < kMaxNC; c0 += kAttThreads) {
    const int c = c0 + tid;
    const bool f = c < ncand && sm.qmask[c] != 0ull;
    const uint64_t m = __ballot(f);
    if (lane == 0) sm.wcount[w] = __popcll(m);
    __syncthreads();
    int off = nunion;
    for (int x = 0; x < w; ++x) off += sm.wcount[x];
    if (f) sm.ulist[off + mask_rank(m)] = (uint16_t)c;
    for (int x = 0; x < kAttWaves; ++x) nunion += sm.wcount[x];
    __syncthreads();                      // wcount is rewritten by the next group
  }

  // Q fragments of this wave's four blocks (B operand of S^T, also the A operand
  // of the retrieval scores): row r16 = (query 4*blk + r16/4, head r16%4)
  bf16x8 qf[kBlocksPerWave][4];
#pragma unroll
  for (int j = 0; j < kBlocksPerWave; ++j) {
    const int blk = w * kBlocksPerWave + j;
    const int qi = blk * 4 + (r16 >> 2), h = r16 & 3;
    const uint16_t* qr = q + ((size_t)(b * g.Hq + kvh * kG + h) * g.Lq + i0 + qi) * kD + g4 * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[j][ks] = ld8(qr + ks * 32);
  }

  // staged chunks: the window chunks own, own - 1, .., own - nwin + 1
  // (statistics pass), then the same chunks in the reverse order (the first of
  // them is still staged), then the union
  auto csrc = [&](int c) -> const uint16_t* { return KVg + (size_t)c * kChunkElems; };
  __syncthreads();                        // the union list is complete
  const uint16_t* first_src = nwin > 0 ? csrc(own) : (nunion > 0 ? csrc(sm.ulist[0]) : nullptr);
  if (first_src) stage_async(first_src, sm.kb[0], sm.vb[0]);

  // ---- retrieval scores of (row, selected chunk) by MFMA: rows x union columns,
  //      from the retrieval query's fragments (the query itself unless a
  //      separate retrieval query is given)
  bf16x8 rf[kBlocksPerWave][4];
#pragma unroll
  for (int j = 0; j < kBlocksPerWave; ++j) {
    const int blk = w * kBlocksPerWave + j;
    const int qi = blk * 4 + (r16 >> 2), h = r16 & 3;
    const uint16_t* qrr = qr + ((size_t)(b * g.Hq + kvh * kG + h) * g.Lq + i0 + qi) * kD + g4 * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) rf[j][ks] = ld8(qrr + ks * 32);
  }
  for (int nt = 0; nt * 16 < nunion; ++nt) {
    const int u = nt * 16 + r16;
    const int c = sm.ulist[u < nunion ? u : 0];
    bf16x8 bl[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) bl[ks] = ld8(Lg + (size_t)c * kD + g4 * 8 + ks * 32);
    const float bc = bb ? bb[c] : 0.f;
#pragma unroll
    for (int j = 0; j < kBlocksPerWave; ++j) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = mfma(rf[j][ks], bl[ks], acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = g4 * 4 + i;                 // block row: query rr/4, head rr%4
        const int qi = (w * kBlocksPerWave + j) * 4 + (rr >> 2), h = rr & 3;
        const int slot = u < nunion ? sm.slotmap[qi * kMaxNC + c] : 0xff;
        if (slot != 0xff) sm.wts[(qi * K + slot) * kG + h] = scale * acc[i] + bc;
      }
    }
  }
  stage_wait();
  __syncthreads();

  f32x4 o[kBlocksPerWave][8];
#pragma unroll
  for (int j = 0; j < kBlocksPerWave; ++j)
#pragma unroll
    for (int db = 0; db < 8; ++db) o[j][db] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- local window, pass 1: lse of its visible tokens (key kk of the own
  //      chunk visible to query qi when kk <= qi, as the window is the chunk;
  //      the other window chunks are complete: vis = kS)
  const float sc2 = scale * 1.4426950408889634f;   // scale * log2(e)
  int t = 0;                              // staged chunk: K in kb[t % 2], V in vb[t % 3]
  if (nwin > 0) {
    float M2[kBlocksPerWave], Z[kBlocksPerWave];
    int vis_own[kBlocksPerWave], vis_full[kBlocksPerWave];
#pragma unroll
    for (int j = 0; j < kBlocksPerWave; ++j) {
      M2[j] = -INFINITY;
      Z[j] = 0.f;
      vis_own[j] = (w * kBlocksPerWave + j) * 4 + (r16 >> 2) + 1;
      vis_full[j] = kS;
    }
    for (int x = 0; x < nwin; ++x) {
      const bool last = x + 1 == nwin;
      window_stats_step<true>(sm.kb[t & 1], sm.kb[(t + 1) & 1], sm.vb[(t + 1) % 3],
                              last ? nullptr : csrc(own - x - 1), qf, sc2,
                              x == 0 ? vis_own : vis_full, M2, Z);
      stage_wait();
      __syncthreads();
      if (!last) ++t;
    }
    // natural-log lse of the window's visible tokens: (M2 + log2 Z) * ln 2
#pragma unroll
    for (int j = 0; j < kBlocksPerWave; ++j) {
      const int qi = (w * kBlocksPerWave + j) * 4 + (r16 >> 2);
      if (lane < 16) sm.lsewin[qi * kG + (r16 & 3)] = (M2[j] + __log2f(Z[j])) * 0.6931471805599453f;
    }
  }
  __syncthreads();
  // ---- fusion weights: LSE over the retrieval scores and the window's lse
  //      (the window chunks' own lse values combine into it exactly)
  if (tid < kWin * kG) {
    const int qi = tid >> 2, h = tid & 3;     // 64 queries x 4 heads
    const float lo = nwin > 0 ? sm.lsewin[tid] : -INFINITY;
    // the row's selection and scores read once, all reads in flight together
    // (slots past K re-read slot 0 and are dropped)
    float sv[kMaxKf];
    uint32_t valid = 0u;
#pragma unroll
    for (int slot = 0; slot < kMaxKf; ++slot) {
      const int ss = slot < K ? slot : 0;
      const bool ok = slot < K && sm.sel[qi * K + ss] >= 0;
      sv[slot] = sm.wts[(qi * K + ss) * kG + h];
      valid |= ok ? 1u << slot : 0u;
    }
    float m = lo;
#pragma unroll
    for (int slot = 0; slot < kMaxKf; ++slot)
      if ((valid >> slot) & 1u) m = fmaxf(m, sv[slot]);
    float z = nwin > 0 ? __expf(lo - m) : 0.f;
#pragma unroll
    for (int slot = 0; slot < kMaxKf; ++slot)
      if ((valid >> slot) & 1u) z += __expf(sv[slot] - m);
    const float LSE = z > 0.f ? m + __logf(z) : -INFINITY;
#pragma unroll
    for (int slot = 0; slot < kMaxKf; ++slot)
      if ((valid >> slot) & 1u) sm.wts[(qi * K + slot) * kG + h] = __expf(sv[slot] - LSE);
    sm.lse2[tid] = LSE * 1.4426950408889634f;
    if (lse_out) lse_out[(size_t)(b * g.Hq + kvh * kG + h) * g.Lq + i0 + qi] = LSE;
  }
  __syncthreads();

  // ---- the window chunks (P = exp(l - LSE)) from own - nwin + 1 (still
  //      staged) up to the own chunk, then the union; the next chunk is copied
  //      into free buffers while one is computed.  Waves 4..7 lag one step
  //      behind in their O += P V (each SIMD holds one leading and one lagging
  //      wave when waves are placed round-robin).
  const bool lag = w >= kAttWaves / 2;
  unsigned pact = 0;
  bf16x8 pa[kBlocksPerWave][2];
  if (nwin > 0) {
    int vis_own[kBlocksPerWave], vis_full[kBlocksPerWave];
    float rw[kBlocksPerWave];
#pragma unroll
    for (int j = 0; j < kBlocksPerWave; ++j) {
      const int qi = (w * kBlocksPerWave + j) * 4 + (r16 >> 2);
      vis_own[j] = qi + 1;                   // key kk of the own chunk visible when kk <= qi
      vis_full[j] = kS;
      rw[j] = sm.lse2[qi * kG + (r16 & 3)];
    }
    const unsigned all = (1u << kBlocksPerWave) - 1;
    for (int y = nwin - 1; y >= 0; --y, ++t) {
      const uint16_t* nsrc = y > 0 ? csrc(own - y + 1) : (nunion > 0 ? csrc(sm.ulist[0]) : nullptr);
      chunk_step<true, true>(lag, sm.kb[t & 1], sm.vb[t % 3], sm.vb[(t + 2) % 3], sm.kb[(t + 1) & 1],
                             sm.vb[(t + 1) % 3], nsrc, qf, sc2, all, y == 0 ? vis_own : vis_full,
                             rw, pact, pa, o);
      stage_wait();
      __syncthreads();
    }
  }
  for (int u = 0; u < nunion; ++u, ++t) {
    const int c = sm.ulist[u];
    const uint64_t qmk = sm.qmask[c];
    unsigned act = 0;
    int vis[kBlocksPerWave];
    float rw[kBlocksPerWave];
#pragma unroll
    for (int j = 0; j < kBlocksPerWave; ++j) {
      const int blk = w * kBlocksPerWave + j;
      if ((qmk >> (blk * 4)) & 0xfull) act |= 1u << j;    // some query of the block selected c
      const int qi = blk * 4 + (r16 >> 2);
      const int slot = sm.slotmap[qi * kMaxNC + c];
      vis[j] = kS;
      rw[j] = slot != 0xff ? sm.wts[(qi * K + slot) * kG + (r16 & 3)] : 0.f;
    }
    const uint16_t* nsrc = u + 1 < nunion ? csrc(sm.ulist[u + 1]) : nullptr;
    chunk_step<false, false>(lag, sm.kb[t & 1], sm.vb[t % 3], sm.vb[(t + 2) % 3],
                             sm.kb[(t + 1) & 1], sm.vb[(t + 1) % 3], nsrc, qf, sc2, act, vis, rw,
                             pact, pa, o);
    stage_wait();
    __syncthreads();
  }
  // the lagging waves' last O += P V (the last chunk's V is still staged)
  if (lag && pact) chunk_pv(sm.vb[(t + 2) % 3], pact, pa, o);

  // ---- output: lane holds O[row 4*g4 + i][16*db + r16] of each block;
  //      row 4*g4 + i = (query 4*blk + g4, head i)
#pragma unroll
  for (int j = 0; j < kBlocksPerWave; ++j) {
    const int qi = (w * kBlocksPerWave + j) * 4 + g4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint16_t* orow = out + ((size_t)(b * g.Hq + kvh * kG + i) * g.Lq + i0 + qi) * kD + r16;
#pragma unroll
      for (int db = 0; db < 8; ++db) orow[16 * db] = f32_to_bf16(o[j][db][i]);
    }
  }
}

template <int R>
void launch_select(const Geometry& g, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                   const uint16_t* lmk, const float* bias, int32_t* sel_idx, uint16_t* kvf,
                   hipStream_t st) {
  hipLaunchKernelGGL(prefill_select<R>, dim3((g.Lq / kWin) * (kWin / sel_rows(R)) * g.B * g.Hkv),
                     dim3(sel_threads(R)), 0, st,
                     g, q, k, v, lmk, bias, sel_idx, kvf);
}

}  // namespace

bool prefill_fast_supported(const Geometry& g, int bf16) {
  return bf16 && g.d == kD && g.S == kS && g.causal && g.Lq == g.Lkv && g.Lq % kWin == 0 &&
         g.G == kG && g.K <= kMaxKf && g.NC <= kMaxNC && g.Lq > 0;
}

size_t prefill_fast_ws(const Geometry& g) {
  return (size_t)g.B * g.Hkv * g.NC * kChunkElems * sizeof(uint16_t);
}

hipError_t launch_prefill_fast(const Geometry& g, const void* q, const void* qr, const void* k,
                               const void* v, const void* lmk, const float* bias, void* out,
                               int32_t* sel_idx, float* lse, void* ws, hipStream_t st) {
  const uint16_t* Q = (const uint16_t*)q;
  const uint16_t* QR = (const uint16_t*)qr;
  const uint16_t* Kp = (const uint16_t*)k;
  const uint16_t* Vp = (const uint16_t*)v;
  const uint16_t* Lm = (const uint16_t*)lmk;
  uint16_t* kvf = (uint16_t*)ws;
  prof_begin(kPrefillSelect, st);
  if (g.NC <= 64) launch_select<1>(g, QR, Kp, Vp, Lm, bias, sel_idx, kvf, st);
  else if (g.NC <= 128) launch_select<2>(g, QR, Kp, Vp, Lm, bias, sel_idx, kvf, st);
  else if (g.NC <= 256) launch_select<4>(g, QR, Kp, Vp, Lm, bias, sel_idx, kvf, st);
  else launch_select<8>(g, QR, Kp, Vp, Lm, bias, sel_idx, kvf, st);
  prof_end(kPrefillSelect, st);
  // dynamic LDS above 64 KB must be enabled for the kernel (per device; cheap)
  if (const hipError_t e = hipFuncSetAttribute((const void*)prefill_attend,
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)sizeof(AttendSmem));
      e != hipSuccess)
    return e;
  prof_begin(kPrefillAttend, st);
  hipLaunchKernelGGL(prefill_attend, dim3((g.Lq / kWin) * g.B * g.Hkv), dim3(kAttThreads),
                     sizeof(AttendSmem), st, g, Q, QR, kvf, Lm, bias, sel_idx, (uint16_t*)out, lse);
  prof_end(kPrefillAttend, st);
  return hipGetLastError();
}

}  // namespace hils
