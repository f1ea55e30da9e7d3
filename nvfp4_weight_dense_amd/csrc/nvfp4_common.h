// nvfp4_common.h -- device helpers shared by the gfx950 kernels of the
// NVFP4 dense SwiGLU FFN library.
//
// NVFP4 value of one element: e2m1(code) * e4m3(block scale) * tensor scale,
// one E4M3 ("FN") scale per 16 consecutive K elements.  Codes are packed two
// per byte along K, element 2j in the low nibble.
//
// Dequantization to bf16 is exact: an E2M1 value has at most 2 significant
// bits and an E4M3 value at most 4, so their product (<= 6 bits, magnitude
// in [2^-10, 2688]) is a bf16 value.  The tensor scale is applied to the
// fp32 accumulators instead.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float f32x2 __attribute__((__vector_size__(2 * sizeof(float))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));

constexpr int kWave = 64;

// E4M3FN byte -> fp32.  Normal bytes move their 7 magnitude bits into the
// fp32 exponent/mantissa fields and rebias the exponent (7 -> 127);
// exponent-0 bytes are m * 2^-9; S.1111.111 is NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  uint32_t em = b & 0x7Fu;
  float mag = em >= 8u ? __uint_as_float((em << 20) + (120u << 23))
                       : (float)em * 0x1p-9f;
  mag = em == 0x7Fu ? __builtin_nanf("") : mag;
  return (b & 0x80u) ? -mag : mag;
}

// Eight E2M1 codes (one 32-bit word, K order from the low nibble) times a
// block scale -> the eight bf16 values of one MFMA operand fragment.  The
// hardware fp4 conversion yields the exact E2M1 values in fp32 (its scale
// operand is a power of two, 1.0 here); the E4M3 scale multiply and the
// bf16 pack are exact.
__device__ __forceinline__ bf16x8 dequant8(uint32_t w, float s) {
  f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  bf16x8 r;
  r[0] = (__bf16)(p0[0] * s);
  r[1] = (__bf16)(p0[1] * s);
  r[2] = (__bf16)(p1[0] * s);
  r[3] = (__bf16)(p1[1] * s);
  r[4] = (__bf16)(p2[0] * s);
  r[5] = (__bf16)(p2[1] * s);
  r[6] = (__bf16)(p3[0] * s);
  r[7] = (__bf16)(p3[1] * s);
  return r;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// silu(t) = t * sigmoid(t), with the sigmoid built from exp(-|t|) in (0, 1]:
// nothing overflows, so for very negative t the result stays the tiny (but
// representable) t*e^t instead of t divided by an overflowed exp(-t).
__device__ __forceinline__ float silu_f32(float t) {
  const float e = expf(-fabsf(t));
  const float sig = t >= 0.0f ? 1.0f / (1.0f + e) : e / (1.0f + e);
  return t * sig;
}

// bf16(silu(bf16(g)) * bf16(u)): gate and up are rounded to bf16 first,
// as they are when they pass through bf16 buffers between launches.
__device__ __forceinline__ __bf16 swiglu_bf16(float g, float u) {
  float gb = (float)(__bf16)g;
  float ub = (float)(__bf16)u;
  return (__bf16)(silu_f32(gb) * ub);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

__host__ __device__ constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

}  // namespace nvfp4
