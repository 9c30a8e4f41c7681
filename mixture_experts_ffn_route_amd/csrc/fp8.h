// OCP 8-bit and 4-bit float helpers of the FP4 -> FP8 re-dequantisation
// (redequant.hip).
//   E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; normals
//         1.m x 2^(e-7) for e = 1..15 except the NaN codes S.1111.111,
//         subnormals m/8 x 2^-6; largest finite 448.
//   E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit: 0, 0.5, 1, 1.5, 2,
//         3, 4, 6.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Nearest E4M3 code to v, ties to even mantissa, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t code;
  if (!(a < 448.f)) {
    code = 0x7Eu;                              // 1.75 x 2^8
  } else if (a < 0.015625f) {                  // below 2^-6: multiples of 2^-9
    code = (uint32_t)__builtin_rintf(a * 512.f);   // 8 -> 0x08 = 2^-6
  } else {
    const uint32_t f = __float_as_uint(a);
    uint32_t q = f >> 20;                      // fp32 exponent and top 3 mantissa bits
    const uint32_t rem = f & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ++q;
    code = q - (120u << 3);                    // rebias 127 -> 7
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return sign | code;
}

// Value of a finite E4M3 code (exact in fp32).
__device__ __forceinline__ float e4m3_value(uint32_t code) {
  const uint32_t e = (code >> 3) & 0xFu, m = code & 7u;
  const float mag = e == 0 ? (float)m * 0x1p-9f : ldexpf(1.f + (float)m * 0.125f, (int)e - 7);
  return (code & 0x80u) ? -mag : mag;
}

// Value of an E2M1 code (low 4 bits of c).
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  const float mag = e == 0 ? 0.5f * (float)m : ldexpf(1.f + 0.5f * (float)m, (int)e - 1);
  return (c & 8u) ? -mag : mag;
}

}  // namespace moe
