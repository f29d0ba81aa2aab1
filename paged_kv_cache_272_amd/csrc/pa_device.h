// Device-side helpers shared by the libpa kernels (gfx950).
//
// Number formats:
//  * bf16 is the upper half of an IEEE binary32; widening is a 16-bit shift,
//    narrowing rounds to nearest even.
//  * e4m3 is the OCP "E4M3FN" 8-bit float: sign, 4 exponent bits (bias 7),
//    3 mantissa bits, subnormals m * 2^-9, NaN = S.1111.111, max 448.
//  * int4 is a signed integer in [-8, 7] stored as the 4-bit code value + 8.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kBlockTokens = 16;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // quiet NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Exact value of one e4m3 code (low 8 bits of `c`), from the field layout.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t sign = (c & 0x80u) << 24;
  const uint32_t e = (c >> 3) & 0xfu;
  const uint32_t m = c & 0x7u;
  float v;
  if (e == 0) {
    v = __uint_as_float(sign | __float_as_uint((float)m * 0x1p-9f));
  } else if (e == 0xfu && m == 0x7u) {
    v = __uint_as_float(sign | 0x7fc00000u);
  } else {
    v = __uint_as_float(sign | ((e + 120u) << 23) | (m << 20));  // 2^(e-7) * (1 + m/8)
  }
  return v;
}

// Saturating round-to-nearest-even encode of a binary32 value to e4m3.
// The quantum in the binade [2^E, 2^(E+1)) is 2^(E-3) for E >= -6, and
// 2^-9 for the subnormal range below 2^-6.
__device__ __forceinline__ uint32_t f32_to_e4m3_sat_rne(float x) {
  const uint32_t bits = __float_as_uint(x);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = __uint_as_float(bits & 0x7fffffffu);
  if (a != a) return sign | 0x7fu;
  if (a >= 448.0f) return sign | 0x7eu;
  if (a < 0x1p-6f) {
    // multiples of 2^-9; r == 8 is 2^-6, whose code (exponent 1, mantissa 0) is also 8
    const float r = __builtin_rintf(a * 512.0f);
    return sign | (uint32_t)r;
  }
  int E = (int)((bits >> 23) & 0xffu) - 127;
  float r = __builtin_rintf(__builtin_ldexpf(a, 3 - E));  // in [8, 16]
  uint32_t ri = (uint32_t)r;
  if (ri == 16u) { ri = 8u; E += 1; }
  return sign | ((uint32_t)(E + 7) << 3) | (ri - 8u);
}

// int4 code of a binary32 value: round half to even (the default rounding
// of rint), clamp to [-8, 7], offset by 8.  NaN gives code 0.
__device__ __forceinline__ uint32_t f32_to_int4_code(float x) {
  const float r = fminf(fmaxf(__builtin_rintf(x), -8.0f), 7.0f);
  return (uint32_t)(int)(r + 8.0f);
}

// --- wave-level reductions (64 lanes) ---------------------------------------

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace pa
