// Device fill for the seeded synthetic inputs: the same counter-based
// generator as hils_inputs/gen.py (SplitMix64 finaliser, Irwin-Hall sum of four
// 16-bit fields, one correctly rounded fp32 multiply, bf16 round-to-nearest-
// even), so any slice can be regenerated on the host bit for bit.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kTidMul = 0xD1B54A32D192ED03ull;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ inline float draw(uint64_t key, uint64_t n, float inv_sd, float scale, int scaled) {
  const uint64_t u = mix64(key + (n + 1) * kGolden);
  const int64_t s = (int64_t)(u & 0xffff) + (int64_t)((u >> 16) & 0xffff) +
                    (int64_t)((u >> 32) & 0xffff) + (int64_t)((u >> 48) & 0xffff) - 131070;
  float x = __fmul_rn((float)s, inv_sd);
  if (scaled) x = __fmul_rn(x, scale);
  return x;
}

__device__ inline uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__global__ void fill_bf16(uint16_t* dst, uint64_t n, uint64_t key, uint64_t offset, float inv_sd,
                          float scale, int scaled) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x * 8;
  for (uint64_t base = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8; base < n;
       base += stride) {
    if (base + 8 <= n) {
      uint32_t w[4];
      for (int e = 0; e < 4; ++e) {
        const uint16_t lo = to_bf16(draw(key, offset + base + 2 * e, inv_sd, scale, scaled));
        const uint16_t hi = to_bf16(draw(key, offset + base + 2 * e + 1, inv_sd, scale, scaled));
        w[e] = (uint32_t)lo | ((uint32_t)hi << 16);
      }
      *reinterpret_cast<uint4*>(dst + base) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      for (uint64_t e = base; e < n; ++e) dst[e] = to_bf16(draw(key, offset + e, inv_sd, scale, scaled));
    }
  }
}

__global__ void fill_f32(float* dst, uint64_t n, uint64_t key, uint64_t offset, float inv_sd,
                         float scale, int scaled) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t e = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride)
    dst[e] = draw(key, offset + e, inv_sd, scale, scaled);
}

}  // namespace

extern "C" int hils_inputs_fill_normal(void* dst, uint64_t n, uint64_t seed, uint64_t tid,
                                       uint64_t offset, float inv_sd, float scale, int as_bf16,
                                       void* stream) {
  const uint64_t key = mix64(seed * kGolden + tid * kTidMul);
  const int scaled = scale != 1.0f;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int blocks = 8192;
  if (n == 0) return 0;
  if (as_bf16)
    hipLaunchKernelGGL(fill_bf16, dim3(blocks), dim3(256), 0, st, (uint16_t*)dst, n, key, offset,
                       inv_sd, scale, scaled);
  else
    hipLaunchKernelGGL(fill_f32, dim3(blocks), dim3(256), 0, st, (float*)dst, n, key, offset,
                       inv_sd, scale, scaled);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// Plain device copy of whole 16-byte words (grid-stride).  Its HBM byte counters
// are the calibration for the per-kernel traffic figures: it reads and writes
// exactly 16 * n bytes.
__global__ void copy_u4(const uint4* __restrict__ src, uint4* __restrict__ dst, uint64_t n) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = src[i];
}

extern "C" int hils_inputs_copy(void* dst, const void* src, uint64_t bytes, void* stream) {
  if (bytes % 16 != 0 || ((uintptr_t)dst | (uintptr_t)src) % 16 != 0) return 1;
  const uint64_t n = bytes / 16;
  if (n == 0) return 0;
  hipLaunchKernelGGL(copy_u4, dim3(4096), dim3(256), 0, (hipStream_t)stream, (const uint4*)src,
                     (uint4*)dst, n);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// Plain streaming read of whole 16-byte words: workgroup g reads the g-th of
// `nwg` equal contiguous segments, four 16-byte loads in flight per thread, and
// writes one word per thread to `sink` (nwg * 256 words) so the loads are kept.
// It measures the read bandwidth the part sustains on its own, next to which the
// kernels' own rates are read.
__global__ void __launch_bounds__(256) read_u4(const uint4* __restrict__ src, uint64_t seg,
                                               uint32_t* __restrict__ sink) {
  const uint4* p = src + (uint64_t)blockIdx.x * seg;
  uint32_t acc = 0;
  for (uint64_t i = threadIdx.x; i < seg; i += 4 * 256) {
    const uint4 a = p[i], b = p[i + 256], c = p[i + 512], d = p[i + 768];
    acc ^= a.x ^ b.y ^ c.z ^ d.w;
  }
  sink[(uint64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

extern "C" int hils_inputs_read(const void* src, uint64_t bytes, void* sink, int nwg, void* stream) {
  // whole segments of 4 x 256 words per workgroup, 16-byte aligned
  if (nwg <= 0 || ((uintptr_t)src % 16) != 0 || bytes % ((uint64_t)nwg * 4 * 256 * 16) != 0) return 1;
  const uint64_t seg = bytes / 16 / (uint64_t)nwg;
  hipLaunchKernelGGL(read_u4, dim3(nwg), dim3(256), 0, (hipStream_t)stream, (const uint4*)src, seg,
                     (uint32_t*)sink);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// Plain matrix-core loop: every wave of 256 workgroups x 8 waves runs `iters`
// rounds of eight independent 16x16x32 bf16 MFMA chains on register operands
// and writes one word per thread to `sink` (256 * 512 words).  It measures the
// dense bf16 rate the part sustains by itself, beside the 2.5 PFLOP/s peak.
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 probe_bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float probe_f32x4;
__global__ void __launch_bounds__(512) mfma_loop(int iters, float seed, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  probe_bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (float)(lane + i));
    b[i] = (__bf16)(seed * (float)(lane - i));
  }
  probe_f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = probe_f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][3];
  sink[(uint64_t)blockIdx.x * 512 + threadIdx.x] = s;
}

extern "C" int hils_inputs_mfma_loop(int iters, void* sink, void* stream) {
  if (iters <= 0) return 1;
  hipLaunchKernelGGL(mfma_loop, dim3(256), dim3(512), 0, (hipStream_t)stream, iters, 1e-3f,
                     (float*)sink);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
