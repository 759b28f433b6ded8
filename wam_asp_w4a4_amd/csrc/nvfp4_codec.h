// NVFP4 element/scale codecs shared by the host packer and the gfx950 kernels.
//
// Format (model card "FastWAM UR3 3-task -- 4-bit quantisations", method
// table): E2M1 elements, blocks of 16, E4M3 block scales.  Readings:
// scale = E4M3FN(amax/6), round to nearest even, saturating at 448; element
// magnitude = E2M1(|v|/scale), round to nearest with ties to the even code,
// saturating at 6; sign bit copied from v; a zero scale zeroes the block.
//
// Exactness (no fast-math anywhere in this library):
//  * amax/6 is formed by IEEE float32 division (correctly rounded).  An E4M3
//    tie point has at most 5 significant bits, so the exact quotient of a
//    float32 amax is either exactly a tie (then float32 holds it) or at least
//    2^-23/6 * 2^e(amax) away from it, more than float32 rounding can move it:
//    rounding the float32 quotient gives the same E4M3 code as the exact one.
//  * Element codes use no division at all: |v| is compared against the grid
//    midpoints times the scale, products of <= 3 and <= 4 significant bits,
//    exact in float32.  (Multiplying by a rounded 1/scale is not exact: e.g.
//    4.6875 * fl(1/1.875) lands above the 2|3 midpoint.)
#pragma once

#include <stdint.h>
#include <string.h>

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define ASP_HD __host__ __device__ __forceinline__
#else
#include <math.h>
#define ASP_HD static inline
#endif

namespace asp {

ASP_HD uint32_t f32_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

ASP_HD float bits_f32(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

// E4M3FN code (0x00..0x7E) of a non-negative float, RNE, saturating.  Both
// the subnormal and the normal path are evaluated and the result selected, so
// the function compiles to straight-line code on the GPU.
ASP_HD uint32_t e4m3_encode(float q) {
  // below 2^-6 the step is 2^-9: q * 512 is exact (power-of-two scaling of a
  // float32), rint rounds half to even, and a result of 8 is the smallest
  // normal, code 0x08.  The clamp keeps the conversion in range for large q.
  const uint32_t sub = (uint32_t)rintf(fminf(q, 0.015625f) * 512.0f);
  const uint32_t b = f32_bits(q);
  const uint32_t exp = (b >> 23) - 120u;  // E4M3 exponent field: (e - 127) + 7
  const uint32_t man = b & 0x7FFFFFu;
  const uint32_t keep = man >> 20;        // top 3 mantissa bits
  const uint32_t rest = man & 0xFFFFFu;   // 20 dropped bits
  const uint32_t up = (uint32_t)(rest > 0x80000u) | ((uint32_t)(rest == 0x80000u) & keep & 1u);
  uint32_t nrm = (exp << 3) + keep + up;  // a carry out of keep bumps the exponent
  nrm = nrm > 0x7Eu ? 0x7Eu : nrm;
  const uint32_t code = q < 0.015625f ? sub : nrm;
  return q < 448.0f ? code : 0x7Eu;       // saturate (NaN too)
}

// Value of a non-negative E4M3FN code (0x00..0x7E) as float32 (exact).
ASP_HD float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float sub = (float)m * 0.001953125f;  // m * 2^-9
  const float nrm = bits_f32(((e + 120u) << 23) | (m << 20));
  return e == 0 ? sub : nrm;
}

// E2M1 magnitude code (0..7) of a = |v| for a block whose scale decodes to sd.
// Each comparison decides one step of the grid 0,.5,1,1.5,2,3,4,6; at a
// midpoint, '>' keeps the lower (even) code and '>=' takes the upper (even).
// A zero scale (the block's maximum underflowed) gives magnitude 0.
ASP_HD uint32_t e2m1_magnitude(float a, float sd) {
  uint32_t m = 0;
  m += a > 0.25f * sd;   // 0 | 1, tie -> 0
  m += a >= 0.75f * sd;  // 1 | 2, tie -> 2
  m += a > 1.25f * sd;   // 2 | 3, tie -> 2
  m += a >= 1.75f * sd;  // 3 | 4, tie -> 4
  m += a > 2.5f * sd;    // 4 | 5, tie -> 4
  m += a >= 3.5f * sd;   // 5 | 6, tie -> 6
  m += a > 5.0f * sd;    // 6 | 7, tie -> 6
  return sd > 0.0f ? m : 0u;
}

// 4-bit code of v (sign bit | magnitude) in a block with decoded scale sd.
ASP_HD uint32_t e2m1_code(float v, float sd) {
  return ((f32_bits(v) >> 31) << 3) | e2m1_magnitude(fabsf(v), sd);
}

// Value of a 4-bit E2M1 code as float32 (exact).
ASP_HD float e2m1_decode(uint32_t c) {
  uint32_t e = (c >> 1) & 3u, m = c & 1u;
  float mag = e == 0 ? 0.5f * (float)m : bits_f32(((e + 126u) << 23) | (m << 22));
  return (c & 8u) ? -mag : mag;
}

// Block scale code for a block maximum magnitude.
ASP_HD uint32_t block_scale_code(float amax) { return e4m3_encode(amax / 6.0f); }

// Round a float32 to bfloat16 bits, nearest even (finite inputs).
ASP_HD uint16_t f32_to_bf16_rne(float f) {
  uint32_t b = f32_bits(f);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

}  // namespace asp
