// Device helpers shared by the HiLS kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hils {

constexpr int kWave = 64;
constexpr int kMaxTopK = 64;
constexpr int kMaxLocalChunks = 64;   // local window width bound, in chunk slots

// ---------------------------------------------------------------- bf16 <-> fp32
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Round to nearest, ties to even (hardware conversion); NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static __forceinline__ float ld(const float* p) { return *p; }
  __device__ static __forceinline__ void st(float* p, float x) { *p = x; }
};
template <> struct Elem<uint16_t> {
  __device__ static __forceinline__ float ld(const uint16_t* p) { return bf16_to_f32(*p); }
  __device__ static __forceinline__ void st(uint16_t* p, float x) { *p = f32_to_bf16(x); }
};

// Workgroup barrier for LDS data only: this wave's LDS operations complete,
// then s_barrier.  Unlike __syncthreads() it leaves outstanding global loads,
// stores and global->LDS copies in flight (their waits are the caller's).  The
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---------------------------------------------------------------- wave primitives
__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Value held by lane l ^ J for J = 1, 2, 4, 8, by DPP: quad permutes for 1
// and 2, a rotation by 8 within each 16-lane row for 8, and for 4 a shift by
// four lanes up or down within the row, chosen by the lane's bit 2.
template <int J>
__device__ __forceinline__ uint32_t dpp_xor_u32(uint32_t x) {
  const int v = static_cast<int>(x);
  if constexpr (J == 1) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, v, 0xB1, 0xf, 0xf, false));
  } else if constexpr (J == 2) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, v, 0x4E, 0xf, 0xf, false));
  } else if constexpr (J == 8) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, v, 0x128, 0xf, 0xf, false));
  } else {
    static_assert(J == 4, "lane distance");
    const int up = __builtin_amdgcn_update_dpp(0, v, 0x104, 0xf, 0xf, false);   // from lane + 4
    const int dn = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // from lane - 4
    return static_cast<uint32_t>((lane_id() & 4) ? dn : up);
  }
}

// Value held by lane l ^ J (J a power of two): the lane-swap VALU
// instructions for J = 32 and 16, DPP below.
template <int J>
__device__ __forceinline__ uint32_t lane_xor_u32(uint32_t x) {
  if constexpr (J == 32 || J == 16) {
    const auto a = J == 32 ? __builtin_amdgcn_permlane32_swap(x, x, false, false)
                           : __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (lane_id() & J) ? a[0] : a[1];
  } else {
    return dpp_xor_u32<J>(x);
  }
}
template <int J>
__device__ __forceinline__ float lane_xor_f32(float x) {
  return __uint_as_float(lane_xor_u32<J>(__float_as_uint(x)));
}
// The same for a 64-bit key, word by word.
template <int J>
__device__ __forceinline__ uint64_t lane_xor_u64(uint64_t x) {
  const uint32_t lo = lane_xor_u32<J>(static_cast<uint32_t>(x));
  const uint32_t hi = lane_xor_u32<J>(static_cast<uint32_t>(x >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
// The same with the distance as an argument; it must fold to a constant (an
// unrolled loop over the distances).
__device__ __forceinline__ uint64_t lane_xor_u64(uint64_t x, int j) {
  switch (j) {
    case 32: return lane_xor_u64<32>(x);
    case 16: return lane_xor_u64<16>(x);
    case 8: return lane_xor_u64<8>(x);
    case 4: return lane_xor_u64<4>(x);
    case 2: return lane_xor_u64<2>(x);
    default: return lane_xor_u64<1>(x);
  }
}
__device__ __forceinline__ float lane_xor_f32(float x, int j) {
  switch (j) {
    case 32: return lane_xor_f32<32>(x);
    case 16: return lane_xor_f32<16>(x);
    case 8: return lane_xor_f32<8>(x);
    case 4: return lane_xor_f32<4>(x);
    case 2: return lane_xor_f32<2>(x);
    default: return lane_xor_f32<1>(x);
  }
}
// Lane i (0..15) of this lane's 16-lane row, by DPP (row broadcast); i must
// fold to a constant (an unrolled loop).
template <int I>
__device__ __forceinline__ float row_bcast_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + I, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_bcast_f32(float x, int i) {
  switch (i) {
    case 0: return row_bcast_f32<0>(x);
    case 1: return row_bcast_f32<1>(x);
    case 2: return row_bcast_f32<2>(x);
    case 3: return row_bcast_f32<3>(x);
    case 4: return row_bcast_f32<4>(x);
    case 5: return row_bcast_f32<5>(x);
    case 6: return row_bcast_f32<6>(x);
    case 7: return row_bcast_f32<7>(x);
    case 8: return row_bcast_f32<8>(x);
    case 9: return row_bcast_f32<9>(x);
    case 10: return row_bcast_f32<10>(x);
    case 11: return row_bcast_f32<11>(x);
    case 12: return row_bcast_f32<12>(x);
    case 13: return row_bcast_f32<13>(x);
    case 14: return row_bcast_f32<14>(x);
    default: return row_bcast_f32<15>(x);
  }
}
// Lane `src`'s key in every lane; `src` must be the same in all lanes.
__device__ __forceinline__ uint64_t bcast_u64(uint64_t x, int src) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), src));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x >> 32), src));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
// Butterfly reductions over the wave (lane distances 32, 16, ..., 1, every lane
// receiving the result), without LDS permutes.
__device__ __forceinline__ float wave_sum(float x) {
  x += lane_xor_f32<32>(x);
  x += lane_xor_f32<16>(x);
  x += lane_xor_f32<8>(x);
  x += lane_xor_f32<4>(x);
  x += lane_xor_f32<2>(x);
  x += lane_xor_f32<1>(x);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, lane_xor_f32<32>(x));
  x = fmaxf(x, lane_xor_f32<16>(x));
  x = fmaxf(x, lane_xor_f32<8>(x));
  x = fmaxf(x, lane_xor_f32<4>(x));
  x = fmaxf(x, lane_xor_f32<2>(x));
  x = fmaxf(x, lane_xor_f32<1>(x));
  return x;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint64_t y = lane_xor_u64(x, m);
    x = y > x ? y : x;
  }
  return x;
}
// number of set bits of `mask` below this lane
__device__ __forceinline__ int mask_rank(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
}

// ---------------------------------------------------------------- selection keys
// Composite key: order-preserving fp32 score bits in the high word, and the
// complemented chunk id in the low word, so that the larger key is the higher
// score and, on equal scores, the lower chunk id.  Valid keys are never 0.
__device__ __forceinline__ uint64_t make_key(float score, int idx) {
  uint32_t u = __float_as_uint(score);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(u) << 32) | (0xffffffffu - static_cast<uint32_t>(idx));
}
__device__ __forceinline__ int key_index(uint64_t key) {
  return static_cast<int>(0xffffffffu - static_cast<uint32_t>(key));
}
__device__ __forceinline__ float key_score(uint64_t key) {
  uint32_t u = static_cast<uint32_t>(key >> 32);
  u = (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u;
  return __uint_as_float(u);
}

// Bitonic sort of one key per lane, descending (lane 0 = largest).
__device__ __forceinline__ uint64_t wave_sort64_desc(uint64_t key) {
  const int lane = lane_id();
#pragma unroll
  for (int k = 2; k <= kWave; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      uint64_t other = lane_xor_u64(key, j);
      bool lower = (lane & j) == 0;
      bool keep_max = lower == ((lane & k) == 0);
      uint64_t mx = other > key ? other : key;
      uint64_t mn = other > key ? key : other;
      key = keep_max ? mx : mn;
    }
  }
  return key;
}

// Bitonic sort of R keys per lane (element e = r * 64 + lane), descending in e.
template <int R>
__device__ __forceinline__ void wave_sort_desc(uint64_t (&keys)[R]) {
  const int lane = lane_id();
  constexpr int N = R * kWave;
#pragma unroll
  for (int k = 2; k <= N; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= kWave) {
        const int jr = j / kWave;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if ((r & jr) == 0) {
            const int e = r * kWave + lane;
            const bool asc_blk = (e & k) == 0;   // lower element keeps the max
            uint64_t a = keys[r], b = keys[r | jr];
            uint64_t mx = a > b ? a : b, mn = a > b ? b : a;
            keys[r] = asc_blk ? mx : mn;
            keys[r | jr] = asc_blk ? mn : mx;
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int e = r * kWave + lane;
          uint64_t other = lane_xor_u64(keys[r], j);
          bool lower = (e & j) == 0;
          bool keep_max = lower == ((e & k) == 0);
          uint64_t mx = other > keys[r] ? other : keys[r];
          uint64_t mn = other > keys[r] ? keys[r] : other;
          keys[r] = keep_max ? mx : mn;
        }
      }
    }
  }
}

// Sort one key per lane, descending, by rank counting: every lane counts the
// keys larger than its own (all 64 are read back from LDS as broadcasts) and
// scatters its key to that rank.  Keys must be unique apart from 0 (empty),
// which sorts last.  `buf` is 64 uint64 of LDS private to the calling wave.
// The reads are independent, so the latency is one LDS round trip plus ~130
// vector instructions, instead of the 21 dependent exchanges of a bitonic net.
__device__ __forceinline__ uint64_t wave_rank_sort64(uint64_t key, uint64_t* buf) {
  const int lane = lane_id();
  buf[lane] = key;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  int rank = 0;
  const ulonglong2* b2 = reinterpret_cast<const ulonglong2*>(buf);
#pragma unroll
  for (int j = 0; j < kWave / 2; ++j) {
    ulonglong2 kk = b2[j];
    rank += (kk.x > key) + (kk.y > key);
  }
  const int nvalid = __popcll(__ballot(key != 0));
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (key != 0) buf[rank] = key;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint64_t out = lane < nvalid ? buf[lane] : 0ull;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  return out;
}

template <int J>
__device__ __forceinline__ uint64_t bitonic_step_desc(uint64_t c) {
  const uint64_t o = lane_xor_u64<J>(c);
  const bool lower = (lane_id() & J) == 0;
  const uint64_t mx = o > c ? o : c, mn = o > c ? c : o;
  return lower ? mx : mn;
}
// Top 64 of two wave-wide lists sorted descending, sorted descending: the
// elementwise max of a and reversed b is bitonic and holds the top 64; six
// compare-exchange stages sort it.  (`buf`: 64 keys of LDS for the reversal.)
__device__ __forceinline__ uint64_t wave_merge_sorted(uint64_t a, uint64_t b, uint64_t* buf) {
  const int lane = lane_id();
  buf[lane] = b;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint64_t br = buf[kWave - 1 - lane];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint64_t c = a > br ? a : br;
  c = bitonic_step_desc<32>(c);
  c = bitonic_step_desc<16>(c);
  c = bitonic_step_desc<8>(c);
  c = bitonic_step_desc<4>(c);
  c = bitonic_step_desc<2>(c);
  c = bitonic_step_desc<1>(c);
  return c;
}

// Top-K (K <= 64) of R keys per lane (keys unique apart from 0 = empty).
// Returns, in lane l < K, the l-th largest key (0 where fewer than l+1 valid
// keys exist); lanes >= K hold the following keys in order.  `buf` is 64
// uint64 of LDS private to the calling wave.
//
// K * R <= 64: tau = K-th largest of the lane maxima.  The K lanes owning the
// largest maxima hold every key >= tau (at most K * R <= 64 of them), and the
// top K are among them, so one compaction and one rank sort finish the job.
// Otherwise the R columns are merged into a running sorted list; a column
// whose maximum does not beat the current K-th key is skipped.
template <int R>
__device__ __forceinline__ uint64_t wave_topk(uint64_t (&keys)[R], int K, uint64_t* buf) {
  const int lane = lane_id();
  if (R == 1) return wave_rank_sort64(keys[0], buf);
  if (K * R <= kWave) {
    uint64_t lm = keys[0];
#pragma unroll
    for (int r = 1; r < R; ++r) lm = keys[r] > lm ? keys[r] : lm;
    uint64_t srt = wave_rank_sort64(lm, buf);
    uint64_t tau = bcast_u64(srt, K - 1);
    if (tau == 0) tau = 1;
    int base = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      bool pred = keys[r] >= tau;
      uint64_t m = __ballot(pred);
      if (pred) buf[base + mask_rank(m)] = keys[r];
      base += __popcll(m);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    uint64_t key = lane < base ? buf[lane] : 0ull;
    return wave_rank_sort64(key, buf);
  }
  uint64_t run = wave_rank_sort64(keys[0], buf);
#pragma unroll
  for (int r = 1; r < R; ++r) {
    const uint64_t kth = bcast_u64(run, K - 1);
    if (wave_max_u64(keys[r]) > kth) run = wave_merge_sorted(run, wave_rank_sort64(keys[r], buf), buf);
  }
  return run;
}

// Merge a list sorted descending (lanes >= K hold 0) into the running sorted
// top list `run`, unless its head cannot beat the current K-th key.
__device__ __forceinline__ uint64_t wave_merge_into(uint64_t run, uint64_t list, int K,
                                                    uint64_t* buf) {
  const uint64_t kth = bcast_u64(run, K - 1);
  const uint64_t head = bcast_u64(list, 0);
  return head > kth ? wave_merge_sorted(run, list, buf) : run;
}

// ---------------------------------------------------------------- lane reductions
// Sum of v[i] over 16 lanes (the lanes that differ only in bits 0..3, i.e. an
// aligned group of 16), returned to the lane whose bits 0..3 equal i (t = lane & 15).
// At the step with mask h the lane keeps the half of its values whose index bit
// matches its own lane bit and adds the partner's copy of that half.
__device__ __forceinline__ float reduce_scatter16(float (&v)[16], int t) {
#pragma unroll
  for (int h = 8; h >= 1; h >>= 1) {
    const bool up = (t & h) != 0;
#pragma unroll
    for (int i = 0; i < h; ++i) {
      float a = v[i], b = v[i + h];
      asm("" : "+v"(a), "+v"(b));   // keep the selects on registers (no indexed array access)
      v[i] = (up ? b : a) + lane_xor_f32(up ? a : b, h);
    }
  }
  return v[0];
}

// ---------------------------------------------------------------- block reductions
// 256-thread (4-wave) block sum / max; `red` is 4 floats of LDS.  All threads
// receive the result.
__device__ __forceinline__ float block_sum4(float x, float* red) {
  x = wave_sum(x);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if (lane_id() == 0) red[w] = x;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}
__device__ __forceinline__ float block_max4(float x, float* red) {
  x = wave_max(x);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if (lane_id() == 0) red[w] = x;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// ---------------------------------------------------------------- geometry
struct Geometry {
  // win: chunk slots of the local window (0 none, 1 the own chunk); keep_own = win > 0
  int B, Hq, Hkv, G, d, Lq, Lkv, S, K, NC, NCcap, causal, keep_own, win;
  float scale;
  // Query i: own slot `own` (causal: its chunk; non-causal: the trailing partial
  // chunk NC), the end `own_b` of its visible tokens, and the candidate count
  // (complete chunks before the local window).
  __device__ __forceinline__ void layout(int i, int& ncand, int& own, int& own_b) const {
    if (causal) {
      const int t = Lkv - Lq + i;
      own = t / S;
      own_b = t + 1;
    } else {
      own = NC;
      own_b = Lkv;
    }
    const int first = own - (win > 1 ? win - 1 : 0);
    ncand = first < 0 ? 0 : (first < NC ? first : NC);
  }
  // Token range [a, b) of window member j (chunk own - j); false when absent or empty.
  __device__ __forceinline__ bool window_member(int own, int own_b, int j, int& a, int& b) const {
    const int c = own - j;
    if (j < 0 || j >= win || c < 0) return false;
    a = c * S;
    b = j == 0 ? own_b : a + S;
    return b > a;
  }
};

}  // namespace hils
