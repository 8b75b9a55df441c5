// Device helpers for the gfx950 paged-attention kernels: storage kinds,
// conversions, 16-byte loads, wave-level reductions, the E4M3 encoder.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Storage kinds. The numeric values match pa_dtype in include/pa.h.
enum Kind : int { kF32 = 0, kF16 = 1, kBF16 = 2, kFP8 = 3 };

template <int K> struct KindBytes;
template <> struct KindBytes<kF32> { static constexpr int value = 4; };
template <> struct KindBytes<kF16> { static constexpr int value = 2; };
template <> struct KindBytes<kBF16> { static constexpr int value = 2; };
template <> struct KindBytes<kFP8> { static constexpr int value = 1; };

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// Geometry of one (block, kv head) tile of 16 token rows as seen by one wave:
// each lane loads 16 contiguous bytes per instruction, so a wave-load covers
// 1 KiB = RPL whole token rows, each row split over LPR lanes holding E
// elements apiece, and the tile takes NL wave-loads.
template <int CK, int D> struct TileGeo {
  static constexpr int kBytes = KindBytes<CK>::value;
  static constexpr int E = 16 / kBytes;
  static constexpr int LPR = D / E;
  static constexpr int RPL = 64 / LPR;
  static constexpr int NL = 16 / RPL;
  static_assert(LPR >= 4 && LPR <= 32 && RPL * LPR == 64 && NL * RPL == 16, "unsupported tile geometry");
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xffffu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
}

// Round float32 to bf16, nearest-even; NaN becomes the canonical quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)(0x7fc0u | ((u >> 16) & 0x8000u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint16_t f32_to_f16_rne(float x) {
  return __builtin_bit_cast(unsigned short, (_Float16)x);
}

// float32 -> OCP E4M3 code: nearest value, ties to even; |y| > 448 (and
// infinity) saturates to +-448; NaN -> S.1111.111; the sign bit is kept.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;
  if (a > 0x43e00000u) return sign | 0x7eu;   // 448 = 1.75 * 2^8
  if (a < 0x3c800000u) {                      // below 2^-6: subnormal grid of step 2^-9
    const float t = __uint_as_float(a) * 512.0f;  // exact power-of-two scaling
    return sign | (uint32_t)__builtin_rintf(t);   // 0..8, and 8 is the code of 2^-6
  }
  // Normal range: keep 3 mantissa bits, nearest-even on the 20 dropped bits;
  // a carry out of the mantissa moves into the exponent as it should.
  const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
  return sign | ((r >> 20) - (120u << 3));
}

// x / scale rounded once (float32 division of |x|, the sign put back, so a NaN keeps its sign).
__device__ __forceinline__ float e4m3_quotient(float x, float scale) { return __builtin_copysignf(__builtin_fabsf(x) / scale, x); }

// Eight 16-bit source elements -> eight E4M3 bytes.
// The 8 16-bit values of a 16-byte chunk (SRC = kF16 or kBF16) as 8 E4M3 codes.
template <int SRC>
__device__ __forceinline__ uint2 e4m3_chunk16(const uint4& v, float scale) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float lo, hi;
    if constexpr (SRC == kBF16) {
      lo = bf16_lo(w[i]);
      hi = bf16_hi(w[i]);
    } else {
      lo = f16_lo(w[i]);
      hi = f16_hi(w[i]);
    }
    const uint32_t b = e4m3_encode(e4m3_quotient(lo, scale)) | (e4m3_encode(e4m3_quotient(hi, scale)) << 8);
    o[i >> 1] |= b << ((i & 1) * 16);
  }
  return make_uint2(o[0], o[1]);
}

// Four float32 source elements -> four E4M3 bytes.
// The 4 float32 values of a 16-byte chunk as 4 E4M3 codes.
__device__ __forceinline__ uint32_t e4m3_chunk32(const uint4& v, float scale) {
  return e4m3_encode(e4m3_quotient(__uint_as_float(v.x), scale)) | (e4m3_encode(e4m3_quotient(__uint_as_float(v.y), scale)) << 8) |
         (e4m3_encode(e4m3_quotient(__uint_as_float(v.z), scale)) << 16) |
         (e4m3_encode(e4m3_quotient(__uint_as_float(v.w), scale)) << 24);
}

// Wave-level sum over groups of N consecutive lanes (N = 4, 8, 16 or 32);
// every lane of a group ends with the same value.
template <int Ctrl> __device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), Ctrl, 0xf, 0xf, false));
}
constexpr int kDppQuadXor1 = 0xb1;       // quad_perm(1,0,3,2)
constexpr int kDppQuadXor2 = 0x4e;       // quad_perm(2,3,0,1)
constexpr int kDppRowHalfMirror = 0x141; // lane i <-> 7-i within each 8
constexpr int kDppRowMirror = 0x140;     // lane i <-> 15-i within each 16

template <int N> __device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32, "group size");
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  if constexpr (N >= 8) x += dpp<kDppRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppRowMirror>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16, 64);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pa
