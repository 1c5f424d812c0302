// Device-side types and helpers shared by the gfx950 kernels of the compact
// decode-attention library.  Nothing here is shared with the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/cda.h"

namespace cda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kTile = CDA_SEG_ALIGN;   // rows per V tile and per segment granule
constexpr int kBlock = 256;            // threads per workgroup of every kernel

// Stored formats (the cda_kv_dtype values), as template arguments.
constexpr int kKvBF16 = CDA_KV_BF16, kKvFP8 = CDA_KV_FP8_E4M3, kKvFP4 = CDA_KV_FP4_E2M1;
// Bytes of one stored row of D elements (FP4: two elements per byte).
__host__ __device__ constexpr int kv_row_bytes(int kv, int D) {
  return kv == kKvBF16 ? 2 * D : kv == kKvFP8 ? D : D / 2;
}

// Byte offset, inside its 64-row tile, of the 16-byte chunk c of row r of a
// K pool whose rows are rb = D * e bytes.  The permutation puts the data one
// 64-lane load instruction of the attention kernel needs (16 rows x 64 bytes,
// in MFMA operand order) into 1 KB of consecutive bytes:
//   instruction (m, j) = ((r >> 2) & 3, c >> 2), lane = (c & 3) * 16 + g,
//   g = ((r >> 4) << 2) | (r & 3).
__host__ __device__ __forceinline__ int k_chunk_offset(int r, int c, int rb) {
  const int m = (r >> 2) & 3, g = ((r >> 4) << 2) | (r & 3);
  return ((m * (rb >> 6) + (c >> 2)) << 10) + ((c & 3) << 8) + (g << 4);
}

// Byte offset of the 8 consecutive elements starting at d0 (a multiple of
// 8) of pool row `row` in a K pool of D-element rows of e-byte elements.
__device__ __forceinline__ int64_t k_elem8(int64_t row, int d0, int D, int e) {
  const int rb = D * e, b = d0 * e;
  return (row / kTile) * kTile * rb + k_chunk_offset((int)(row % kTile), b >> 4, rb) + (b & 15);
}

// Byte offset of byte `byte` of pool row `row` in a K pool of rb-byte rows.
__device__ __forceinline__ int64_t k_byte(int64_t row, int byte, int rb) {
  return (row / kTile) * kTile * rb + k_chunk_offset((int)(row % kTile), byte >> 4, rb) + (byte & 15);
}

// BF16 and FP8 V pool: a 64-row tile is four blocks of 16 rows, each block
// column-major, so element (r, d) of a tile is at byte
//   ((r / 16) * D + d) * 16 * e + (r % 16) * e.
// One lane's 16 consecutive rows of one column (a PV operand) stay one run
// of 16 * e bytes, and the D values of one row fall in D * 16 * e / 128
// cache lines instead of one line per 128 / (64 * e) columns.
__host__ __device__ __forceinline__ int v_tile_off(int r, int d, int D, int e) {
  return (((r >> 4) * D + d) * 16 + (r & 15)) * e;
}
// Column d and first row row0 of the 16-byte run at tile byte vb (a multiple
// of 16) of such a tile: 16 / e rows of one column.
__host__ __device__ __forceinline__ void v_tile_run(int vb, int D, int e, int& d, int& row0) {
  const int blk = vb / (16 * D * e), o = vb - blk * 16 * D * e;
  d = o / (16 * e);
  row0 = blk * 16 + (o - d * 16 * e) / e;
}

// FP4 V pool: the same 16-row blocks, two rows per byte: element (r, d) of
// a tile is nibble r & 1 (low for even rows) of tile byte
//   ((r / 16) * D + d) * 8 + (r % 16) / 2.
__host__ __device__ __forceinline__ int v_nib_off(int r, int d, int D) {
  return ((r >> 4) * D + d) * 8 + ((r & 15) >> 1);
}
// The pool byte of element (row, d).
__device__ __forceinline__ int64_t v_nib_byte(int64_t row, int d, int D) {
  return (row / kTile) * kTile * (D / 2) + v_nib_off((int)(row % kTile), d, D);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// OCP E4M3FN encode of one f32, round-to-nearest-even, saturating at +-448,
// NaN -> 0x7F with the input's sign.  Integer arithmetic on the binary32
// fields: the 3 kept mantissa bits are rounded on the 20 dropped ones, with
// the carry running into the exponent field; values below 2^-6 are rounded
// to a multiple of 2^-9 from the full 24-bit significand.
__device__ __forceinline__ uint32_t e4m3_from_f32(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;   // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;  // >= 448 or infinite
  const uint32_t e = a >> 23;
  if (e >= 121u) {                            // >= 2^-6: normal code
    const uint32_t m = a & 0x7FFFFFu;
    uint32_t code = ((e - 120u) << 3) | (m >> 20);
    const uint32_t rem = m & 0xFFFFFu;
    code += (rem > 0x80000u || (rem == 0x80000u && (code & 1u))) ? 1u : 0u;
    return sign | code;
  }
  if (e < 110u) return sign;                  // below 2^-17: rounds to zero
  const uint32_t full = (a & 0x7FFFFFu) | 0x800000u;  // value = full * 2^(e-150)
  const uint32_t shift = 141u - e;                     // in units of 2^-9
  uint32_t q = full >> shift;
  const uint32_t rem = full & ((1u << shift) - 1u);
  const uint32_t half = 1u << (shift - 1u);
  q += (rem > half || (rem == half && (q & 1u))) ? 1u : 0u;
  return sign | q;
}

// The same encode of two values (codes in bits 0-7 and 8-15) with the
// gfx950 conversion instruction: inputs clamped to [-448, 448] first (the
// instruction alone gives NaN for magnitudes that round past 448), NaN
// mapped to 0x7F with its sign after it (the instruction does not keep the
// sign of every NaN).  Equal to e4m3_from_f32 on every binary32 input, in
// the default round-to-nearest-even mode.
__device__ __forceinline__ uint32_t e4m3x2_from_f32(float a, float b) {
  uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(a, -448.0f, 448.0f),
                                                         __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f),
                                                         0, false) & 0xFFFFu;
  if (__builtin_isnan(a)) w = (w & 0xFF00u) | 0x7Fu | ((__float_as_uint(a) >> 24) & 0x80u);
  if (__builtin_isnan(b)) w = (w & 0x00FFu) | ((0x7Fu | ((__float_as_uint(b) >> 24) & 0x80u)) << 8);
  return w;
}

// Nibble `odd` of the FP4 V byte at q set to code c, the other kept (a
// read-modify-write of the byte; its other row must not be written at the
// same time).
__device__ __forceinline__ void nib_store(uint8_t* q, int odd, uint32_t c) {
  const uint32_t cur = *q;
  *q = (uint8_t)(odd ? ((cur & 0x0Fu) | (c << 4)) : ((cur & 0xF0u) | c));
}

// OCP MX FP4 E2M1 encode of two values into one byte (a in the low nibble):
// round-to-nearest-even, saturating at +-6, NaN -> +-6 with its sign -- what
// the gfx950 conversion instruction computes for every binary32 input at
// scale 1 (checked exhaustively on the device against the definition).
__device__ __forceinline__ uint32_t e2m1x2_from_f32(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0) & 0xFFu;
}

// Dequantisation and quantisation factors from a per-head absmax.
__device__ __forceinline__ float fp8_scale(float amax) {
  return (amax > 0.0f && amax <= 3.402823466e38f) ? __fdiv_rn(amax, 448.0f) : 1.0f;
}
__device__ __forceinline__ float fp8_inv_scale(float amax) {
  return (amax > 0.0f && amax <= 3.402823466e38f) ? __fdiv_rn(448.0f, amax) : 1.0f;
}
// The same for the 4-bit store (largest magnitude 6); 1 for BF16.
template <int KV>
__device__ __forceinline__ float kv_scale(float amax) {
  if (KV == kKvFP8) return fp8_scale(amax);
  if (KV == kKvFP4) return (amax > 0.0f && amax <= 3.402823466e38f) ? __fdiv_rn(amax, 6.0f) : 1.0f;
  return 1.0f;
}
template <int KV>
__device__ __forceinline__ float kv_inv_scale(float amax) {
  if (KV == kKvFP8) return fp8_inv_scale(amax);
  if (KV == kKvFP4) return (amax > 0.0f && amax <= 3.402823466e38f) ? __fdiv_rn(6.0f, amax) : 1.0f;
  return 1.0f;
}

// Four FP8 codes (one dword) -> four bf16 / f16 values, exact.
__device__ __forceinline__ void fp8x4_to_bf16(uint32_t w, bf16x2& lo, bf16x2& hi) {
  lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
}
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  bf16x2 a, b, c, d;
  fp8x4_to_bf16(w0, a, b);
  fp8x4_to_bf16(w1, c, d);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
__device__ __forceinline__ f16x8 fp8x8_to_f16x8(uint32_t w0, uint32_t w1) {
  f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
  f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
  f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
  f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Eight FP4 codes (one dword, element 2j in the low nibble of byte j) ->
// eight bf16 / f16 values, exact.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16x8(uint32_t w) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
__device__ __forceinline__ f16x8 fp4x8_to_f16x8(uint32_t w) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Exclusive prefix sum over the 256 threads of a workgroup.  smem: >= 4 ints.
// Every thread of the workgroup must call it.
__device__ __forceinline__ int block_exclusive_scan(int v, int* total, int* smem) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) smem[wid] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kBlock / 64; ++w) {
    int s = smem[w];
    before += (w < wid) ? s : 0;
    all += s;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

__device__ __forceinline__ int block_sum(int v, int* smem) {
  int total;
  block_exclusive_scan(v, &total, smem);
  return total;
}

}  // namespace cda
