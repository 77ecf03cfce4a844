// pa_mfma.h -- matrix-core helpers shared by the gfx950 attention kernels:
// 16-bit narrowing, the hi + lo split of softmax weights, the two MFMA
// shapes used (16x16x32 and 16x16x16, bf16 and f16 inputs, fp32
// accumulators), the gfx950 transposing LDS read, and 4-lane row reductions.
//
// Lane layouts of v_mfma_f32_16x16x{32,16} (K = 32 or 16, KL = K / 4 values
// of each operand per lane): lane l holds A[l % 16][KL * (l / 16) + e],
// B[KL * (l / 16) + e][l % 16] (e < KL) and C[4 * (l / 16) + r][l % 16]
// (r < 4).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa.h"

namespace pa {
namespace mx {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// round-to-nearest-even narrowing and exact widening of the 16-bit types
template <int DT>
__device__ inline uint16_t narrow16(float x) {
  if constexpr (DT == PA_F16) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  } else {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x0040u);
    return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
  }
}
// Two weights p0, p1 (finite, >= 0) as a 16-bit pair hi plus the pair of
// remainders lo = p - hi, so hi + lo carries about 17 significant bits (the
// remainder p - hi is exact in fp32).
template <int DT>
__device__ inline void split_pair(float p0, float p1, uint32_t& hi, uint32_t& lo) {
  if constexpr (DT == PA_F16) {
    const f16x2 h = __builtin_convertvector(f32x2{p0, p1}, f16x2);
    const f32x2 r = f32x2{p0, p1} - __builtin_convertvector(h, f32x2);
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, f16x2));
  } else {
    const bf16x2 h = __builtin_convertvector(f32x2{p0, p1}, bf16x2);
    const uint32_t hb = __builtin_bit_cast(uint32_t, h);
    const float r0 = p0 - __uint_as_float(hb << 16);
    const float r1 = p1 - __uint_as_float(hb & 0xffff0000u);
    hi = hb;
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{r0, r1}, bf16x2));
  }
}

// 16 keys x 32 dims (A) times 32 dims x 16 rows (B), accumulated in c
template <int DT>
__device__ inline f32x4 mma_k32(uint4 a, uint4 b, f32x4 c) {
  if constexpr (DT == PA_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// 16 dims x 16 keys (A) times 16 keys x 16 rows (B)
template <int DT>
__device__ inline f32x4 mma_k16(uint2 a, uint2 b, f32x4 c) {
  if constexpr (DT == PA_F16)
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// max / sum over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lanes of one row)
// with the CDNA4 row swaps: v_permlane16_swap(x, x) returns x[l] and
// x[l ^ 16] in its two results, v_permlane32_swap x[l] and x[l ^ 32].
__device__ inline float row4_max(float x) {
  const uint32_t b = __float_as_uint(x);
  const auto r16 = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  x = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const uint32_t c = __float_as_uint(x);
  const auto r32 = __builtin_amdgcn_permlane32_swap(c, c, false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}
__device__ inline float row4_sum(float x) {
  const uint32_t b = __float_as_uint(x);
  const auto r16 = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  x = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  const uint32_t c = __float_as_uint(x);
  const auto r32 = __builtin_amdgcn_permlane32_swap(c, c, false, false);
  return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

// ds_read_b64_tr_b16: in each 16-lane group, lane i receives element i % 4
// of the 8-byte units addressed by lanes i / 4, i / 4 + 4, i / 4 + 8 and
// i / 4 + 12, in that order.  With lane a of the group addressing row
// r0 + a / 4, columns c0 + 4 (a % 4) .. + 3 of a row-major 16-bit tile, lane
// i gets column c0 + i of rows r0 .. r0 + 3: a 4-element column of the tile.
__device__ inline uint2 ds_read_tr16(const void* lds_ptr) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(const_cast<void*>(lds_ptr)));
  return __builtin_bit_cast(uint2, v);
}

}  // namespace mx
}  // namespace pa
