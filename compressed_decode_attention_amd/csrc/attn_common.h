// Pieces shared by the attention kernels (single-token decode and
// multi-query chunk attention): wave-level reductions across the 16-lane
// rows of a 64-lane wave, the q-operand layout of the MFMA products, and
// small conversions.
#pragma once

#include "cda_device.h"

namespace cda {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Reductions across the 16-lane rows of a wave: partner lanes l ^ 16 and
// l ^ 32 via the row-swap permutes (no LDS round trip).
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// d of the first of the 8 q values lane (g, kg) supplies at k-step s: the d
// the K operand of that lane holds there (the order of the bytes of its K
// chunk: 16 FP8 elements = 2 k-steps, 32 FP4 elements = 4, 8 bf16 = 1).
template <int KV>
__device__ __forceinline__ int q_d0(int s, int kg) {
  if (KV == kKvFP8) return 64 * (s >> 1) + 16 * kg + 8 * (s & 1);
  if (KV == kKvFP4) return 32 * kg + 8 * s;
  return 32 * s + 8 * kg;
}

__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

// Mask of the bytes of dword w (bytes 4w .. 4w+3) that lie below `lim`.
__device__ __forceinline__ uint32_t bytes_below(int lim, int w) {
  const int k = lim - 4 * w;
  return k >= 4 ? 0xFFFFFFFFu : (k <= 0 ? 0u : (1u << (8 * k)) - 1u);
}

}  // namespace cda
