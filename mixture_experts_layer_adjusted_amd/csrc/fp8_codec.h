// E4M3FN (OCP OFP8) encoding shared by the quantisers and the FP8 GEMM epilogue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Four fp32 values to their E4M3FN codes (bias 7, 3 mantissa bits, S.1111.111 is NaN), packed
// lowest first, by gfx950's packed conversion instruction v_cvt_pk_fp8_f32: round to nearest
// even, saturating at +-448.  Every caller divides by amax / 448 first, so its inputs lie within
// 448 (1 + 2^-23) in magnitude.  The quantisers built on it are compared bit for bit with the
// CPU quantiser of the E4M3FN definition by the GPU tests (activations, weights, and the gate/up
// epilogue's H through the quantisation-faithful layer).
__device__ __forceinline__ uint32_t e4m3x4_from_f32(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

}  // namespace moe
