// MFMA-side helpers shared by the prefill forward and backward kernels
// (gfx950: v_mfma_f32_16x16x32_bf16, wave64).
//
// Operand layout of the 16x16x32 bf16 MFMA (lane l, element j = 0..7):
//   A[m][k]: m = l % 16, k = 8 (l / 16) + j
//   B[k][n]: k = 8 (l / 16) + j, n = l % 16
//   D[m][n]: m = 4 (l / 16) + i (i = 0..3), n = l % 16
#pragma once
#include "hils_common.h"

namespace hils {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

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
// two fp32 -> packed bf16, round to nearest even (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ bf16x8 pack_bf16x8(const float (&x)[8]) {
  uint32_t w4[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) w4[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
  bf16x8 r;
  __builtin_memcpy(&r, w4, 16);
  return r;
}

// max(a, b) and max(a, b, c) as single instructions: inputs are finite values
// or -inf, never NaN, so no canonicalising of the MFMA results (which the
// compiler inserts before a max it builds itself) is needed
__device__ __forceinline__ float fmax2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float fmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// reductions over the four lanes l, l^16, l^32, l^48 (one MFMA D column) with
// the lane-swap VALU instructions instead of LDS permutes
__device__ __forceinline__ float rowgroup_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = fmax2(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t v = __float_as_uint(x);
  const auto c = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return fmax2(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float rowgroup_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t v = __float_as_uint(x);
  const auto c = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

}  // namespace hils
