// encode_hw.h -- the quantizers' division and rounding steps on gfx950
// hardware (device code, shared by the row quantizers and the encoder
// probe that tests these steps against the rule on their whole domain).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// x / d rounded to nearest, from y = 1/d (rounded to nearest) with one
// product and one FMA correction of its exact residual: the correctly
// rounded quotient whenever x, d, y, the quotient and the residual are
// normal (Markstein's theorem on division by a correctly rounded
// reciprocal).  The quantizers take it for divisors in [2^-90, 2^100]
// (recip_div_ok), where every quotient that can change a code (2^-10 and
// above, so x >= 2^-100) qualifies; a smaller quotient may differ in its
// last bits but encodes to a signed zero either way.  The sign is x's, as
// in the division (the FMA steps would turn -0 into +0).
__device__ __forceinline__ bool recip_div_ok(float d) { return d >= 0x1p-90f && d <= 0x1p100f; }
__device__ __forceinline__ float div_by_recip(float x, float d, float y) {
  const float q0 = x * y;
  const float r = fmaf(-q0, d, x);
  return __builtin_copysignf(fmaf(r, y, q0), x);
}

// fp32 values -> E2M1 codes by the hardware conversion at unit scale: the
// nearest grid value with ties to the even code, saturating at 6, sign
// kept, for every non-NaN input (nvfp4_probe_encode runs it for the tests,
// which compare it with the CPU encoder); element 2s of q goes to the low
// nibble of byte s.
__device__ __forceinline__ uint32_t e2m1x8_hw(const float *q) {
  uint32_t w = 0u;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[0], q[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[2], q[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[4], q[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[6], q[7], 1.0f, 3);
  return w;
}
// fp32 quadruple -> E4M3 bytes: the sign and the nearest E4M3FN magnitude,
// ties to even, saturating at 448, for every non-NaN input (tested like
// the E2M1 step).  The hardware conversion does not saturate (past 448 it
// gives the NaN code), so the input is clamped to +-448 first.
typedef short s16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t e4m3x4_hw(const float *q) {
  s16x2 w = {0, 0};
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, __builtin_amdgcn_fmed3f(q[0], -448.0f, 448.0f),
                                               __builtin_amdgcn_fmed3f(q[1], -448.0f, 448.0f), 1.0f, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, __builtin_amdgcn_fmed3f(q[2], -448.0f, 448.0f),
                                               __builtin_amdgcn_fmed3f(q[3], -448.0f, 448.0f), 1.0f, true);
  return __builtin_bit_cast(uint32_t, w);
}

}  // namespace nvfp4
