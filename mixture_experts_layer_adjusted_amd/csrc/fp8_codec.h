// E4M3FN (OCP OFP8) encoding shared by the quantisers and the FP8 GEMM epilogue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Round-to-nearest-even E4M3FN code of y, saturating at +-448 (bias 7, 3 mantissa bits,
// S.1111.111 is NaN), computed in integer arithmetic from the fp32 bit pattern.
__device__ __forceinline__ uint32_t e4m3_from_f32(float y) {
  const uint32_t bits = __float_as_uint(y);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = fabsf(y);
  if (a != a) return 0x7Fu;                    // NaN
  uint32_t code;
  if (a < 0.015625f) {                         // below 2^-6: subnormal grid, spacing 2^-9
    code = (uint32_t)__builtin_rintf(a * 512.0f);   // exact scaling, round half to even; 8 -> min normal
  } else {
    const uint32_t ab = bits & 0x7FFFFFFFu;
    const int e = (int)(ab >> 23) - 127;       // >= -6 here
    const uint32_t frac = ab & 0x7FFFFFu;
    uint32_t m = frac >> 20;                   // top 3 mantissa bits
    const uint32_t rem = frac & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (m & 1u))) ++m;
    int ee = e + 7;
    if (m == 8u) {
      m = 0u;
      ++ee;
    }
    code = ee > 15 ? 0x7Fu : ((uint32_t)ee << 3) | m;
    if (code > 0x7Eu) code = 0x7Eu;            // saturate at 448
  }
  return sign | code;
}

// Four values to their E4M3FN codes, packed lowest first, by gfx950's packed conversion
// instruction (round to nearest even).  For |v| <= 464 it gives exactly e4m3_from_f32's codes
// (checked on the GPU for every fp32 bit pattern of that range, both signs); every quantiser here
// divides values by amax / 448, so its inputs stay within 448 (1 + 2^-23).
__device__ __forceinline__ uint32_t e4m3x4_from_f32(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

}  // namespace moe
