// gfx950 matrix-core helpers shared by the decode and prefill kernels:
// 16x16x32 and 16x16x16 MFMAs on 16-bit operands held as packed words,
// float32 <-> 16-bit conversions, and exact FP8 -> 16-bit widening.
//
// Lane layouts (checked on the hardware): for a 16x16xK MFMA with K/4 elements
// per lane, lane l holds A[i = l % 16][k = (K/4)(l / 16) + e] and
// B[k = (K/4)(l / 16) + e][j = l % 16]; the float32 result has lane l holding
// C[i = 4 (l / 16) + r][j = l % 16], r = 0..3.
#pragma once

#include "pa_device.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// C += A·B over 32 k (8 elements of A and of B per lane, 4 words each).
template <int QK>
__device__ __forceinline__ f32x4_t mma_k32(const uint32_t* a, const uint32_t* b, f32x4_t c) {
  const u32x4_t av = {a[0], a[1], a[2], a[3]};
  const u32x4_t bv = {b[0], b[1], b[2], b[3]};
  if constexpr (QK == kBF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bv),
                                                   c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, av), __builtin_bit_cast(f16x8_t, bv), c,
                                                  0, 0, 0);
}

// C += A·B over 16 k (4 elements of A and of B per lane, 2 words each).
template <int QK>
__device__ __forceinline__ f32x4_t mma_k16(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f32x4_t c) {
  const u32x2_t av = {a0, a1};
  const u32x2_t bv = {b0, b1};
  if constexpr (QK == kBF16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, av), __builtin_bit_cast(i16x4_t, bv),
                                                     c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, av), __builtin_bit_cast(f16x4_t, bv), c,
                                                 0, 0, 0);
}

// Two float32 -> two 16-bit values of the query's type (nearest-even), packed.
template <int QK>
__device__ __forceinline__ uint32_t pack2(float x, float y) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  if constexpr (QK == kBF16) {
    typedef __bf16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){x, y}, h2));
  } else {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){x, y}, h2));
  }
}

template <int QK> __device__ __forceinline__ float lo16_to_f32(uint32_t w) {
  return QK == kBF16 ? bf16_lo(w) : f16_lo(w);
}
template <int QK> __device__ __forceinline__ float hi16_to_f32(uint32_t w) {
  return QK == kBF16 ? bf16_hi(w) : f16_hi(w);
}

// Four FP8 codes -> four values of the query's 16-bit type (exact), as two words.
template <int QK>
__device__ __forceinline__ void fp8x4_to_16(uint32_t w, uint32_t& lo, uint32_t& hi) {
  if constexpr (QK == kBF16) {
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false));
    hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true));
  } else {
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, false));
    hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, true));
  }
}

// The B operand of a 16x16x16 product O += P·V (or half of a 16x16x32 one
// over two tiles) from a row-major V tile in LDS (16 rows of `stride` 16-bit
// elements): lane l gets V[4(l/16) + e][c0 + l % 16] for e = 0..3, i.e. four
// tokens of one column, as two packed words.
// One transposing LDS read (ds_read_b64_tr_b16) does it: within each 16-lane
// group, output lane i element e comes from lane 4e + i/4, element i % 4, so
// lane l supplies the 8 bytes at row 4(l/16) + (l%16)/4, column
// c0 + 4((l%16) % 4).
__device__ __forceinline__ u32x2_t v_operand_tr(const uint16_t* tile, int stride, int c0, int lane) {
  const int g = lane >> 4, n = lane & 15;
  const uint16_t* p = tile + (4 * g + (n >> 2)) * stride + c0 + 4 * (n & 3);
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)p);
  return __builtin_bit_cast(u32x2_t, v);
}

}  // namespace pa
