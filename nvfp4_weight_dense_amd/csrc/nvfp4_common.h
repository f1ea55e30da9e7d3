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
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// E4M3FN byte -> fp32 with the gfx950 OCP fp8 conversion (exact for all 256
// bytes, NaN for S.1111.111).  `sel` picks the byte of `w`.
template <int sel>
__device__ __forceinline__ float e4m3_to_f32_sel(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8(w, sel);
}
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) { return e4m3_to_f32_sel<0>(b); }

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

// The same eight values as fp16, for operands that are NVFP4 on both sides.
// An E2M1 value (at most 2 significant bits) times an E4M3 scale (at most
// 4) needs at most 6 significant bits and lies in [2^-10, 2688], so it is
// exact in fp16, and so is every E4M3 value.  The hardware conversions run
// with a unit scale (fp4 -> the exact E2M1 values, fp8 -> the exact E4M3
// values); the block scale then follows as one packed fp16 multiply per
// pair, its operand selected from the scale pair by op_sel.
__device__ __forceinline__ f16x2 e4m3x2_to_f16x2(uint32_t w) {  // bytes 0, 1 of w
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
}
__device__ __forceinline__ f16x8 dequant8_f16(uint32_t w, _Float16 s) {
  const f16x2 ss = {s, s};
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * ss;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * ss;
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * ss;
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * ss;
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Eight E4M3 bytes (K order from the low byte of lo) -> eight exact fp16
// values (the hardware conversion with a unit scale).
__device__ __forceinline__ f16x8 fp8x8_to_f16(uint32_t lo, uint32_t hi) {
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// silu(t) = t * sigmoid(t), with the sigmoid built from exp(-|t|) in (0, 1]:
// nothing overflows, so for very negative t the result stays the tiny (but
// representable) t*e^t instead of t divided by an overflowed exp(-t).
__device__ __forceinline__ float silu_f32(float t) {
  // sigma(t) from e = exp(-|t|) <= 1, so nothing overflows for large |t|.
  // e = 2^(64 - |t| log2 e) * 2^-64: v_exp_f32 (about 1 ulp) only ever sees
  // normal results, and the exact power-of-two multiply rounds e into the
  // fp32 subnormal range once (silu(t) for t < -87 is a bf16 subnormal).
  // v_rcp_f32 on [1, 2] is within about 1 ulp; both errors sit far below the
  // resolution of the bf16 result.
  const float e = __builtin_amdgcn_exp2f(64.0f - fabsf(t) * 1.44269504088896341f) *
                  5.42101086242752217e-20f;  // log2(e); 2^-64
  const float r = __builtin_amdgcn_rcpf(1.0f + e);
  return t * (t >= 0.0f ? r : e * r);
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

// Packed-Q2 weights (page layers/dense_ffn_prefill.rs, `prefill_q2`: Q2_0
// weights with a group size, dequantized to BF16 for the BF16 GEMM; the code
// is this library's reading): a 2-bit code q per element, four per byte from
// the low bits, one fp16 scale d per row and group of K; the value is
// bf16((q - 2) * d).  A lane's 32 K values of a step lie in one group
// (group >= 32), so the four values it can meet form a table, T_q =
// bf16(fma(q, d, -2d)) -- exact in fp32 and rounded once, the bits of the
// dequantized BF16 weight -- packed two per dword: lo = T0 | T1 << 16,
// hi = T2 | T3 << 16.
__device__ __forceinline__ void q2_table(uint32_t d_bits16, uint32_t &lo, uint32_t &hi) {
  const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)d_bits16);
  const float m2d = -2.0f * d;
  const bf16x2 t01 = {(__bf16)__builtin_fmaf(0.0f, d, m2d), (__bf16)__builtin_fmaf(1.0f, d, m2d)};
  const bf16x2 t23 = {(__bf16)__builtin_fmaf(2.0f, d, m2d), (__bf16)__builtin_fmaf(3.0f, d, m2d)};
  lo = __builtin_bit_cast(uint32_t, t01);
  hi = __builtin_bit_cast(uint32_t, t23);
}

// Eight codes (16 bits, element e in bits 2e..2e+1) -> their eight table
// values.  z = cw | cw << 14 puts the codes of elements 2i and 2i+1 at bits
// 4i and 4i+16, so (z >> 4i) & 0x30003 = q_2i + q_2i+1 << 16; times 0x0202
// plus 0x01000100 that is the byte selector {2q, 2q+1} of each half for
// v_perm_b32 over the 8-byte table {hi, lo} (bytes 0-3 lo, 4-7 hi).
__device__ __forceinline__ bf16x8 q2_dequant8(uint32_t cw, uint32_t lo, uint32_t hi) {
  const uint32_t z = cw | (cw << 14);
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t y = (z >> (4 * i)) & 0x00030003u;
    o[i] = __builtin_amdgcn_perm(hi, lo, y * 0x0202u + 0x01000100u);
  }
  return __builtin_bit_cast(bf16x8, uint4{o[0], o[1], o[2], o[3]});
}


// ---- buffer loads -------------------------------------------------------------
// A raw buffer resource over [base, base + bytes): loads at offsets beyond
// the range return zero instead of touching memory, which handles ragged
// rows, columns and K without branches.  Ranges are capped below 2^31 and
// kOOB is an offset outside every range.
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, size_t bytes) {
  const uint32_t nrec = bytes < (size_t)0x7FFFFFFF ? (uint32_t)bytes : 0x7FFFFFFFu;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)nrec,
                                           0x00020000);
}
// The same, for a base and size the caller knows to be wave-uniform: the
// pieces go through readfirstlane, so the descriptor stays in scalar
// registers (instructions that need it there, such as LDS-DMA loads, are
// otherwise wrapped in a per-lane loop).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_uniform(const void *base, size_t bytes) {
  const uint64_t a = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t nrec = __builtin_amdgcn_readfirstlane(
      bytes < (size_t)0x7FFFFFFF ? (uint32_t)bytes : 0x7FFFFFFFu);
  return __builtin_amdgcn_make_buffer_rsrc((void *)(((uint64_t)hi << 32) | lo), (short)0, (int)nrec,
                                           0x00020000);
}
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// The same with a wave-uniform part of the offset in the instruction's
// scalar offset register (keeps per-lane offset arrays out of VGPRs).
__device__ __forceinline__ uint4 ld16s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// Streaming variants for data read once per call (weights): the
// non-temporal policy keeps them from displacing reused lines in the caches.
constexpr int kStreamPolicy = 2;  // nt
__device__ __forceinline__ uint4 ld16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kStreamPolicy));
}
__device__ __forceinline__ uint32_t ld2_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_bit_cast(uint16_t,
                                      __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, kStreamPolicy));
}
__device__ __forceinline__ uint32_t ld4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t ld2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_bit_cast(uint16_t, __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
}

// ---- row-contiguous weight loads ------------------------------------------------
// In the 16x16 MFMA operand layout lane (c, g) = (lane%16, lane/16) holds
// row c, so four neighbouring lanes read four different rows, and a
// streaming kernel is then held by the texture addresser rather than by
// HBM.  The load layout instead gives lane s row s/4 and piece s%4 of it
// (four neighbours read one contiguous run); one ds_bpermute per dword then
// hands lane (c, g) the registers of lane 4c + g, i.e. row c, piece g.
__device__ __forceinline__ int load_layout_src_addr(int lane) {
  return (((lane & 15) << 2) | (lane >> 4)) << 2;  // byte address of lane 4c + g
}
__device__ __forceinline__ uint32_t from_load_layout(uint32_t v, int src_addr) {
  return (uint32_t)__builtin_amdgcn_ds_bpermute(src_addr, (int)v);
}
__device__ __forceinline__ uint4 from_load_layout(const uint4 &v, int src_addr) {
  return uint4{from_load_layout(v.x, src_addr), from_load_layout(v.y, src_addr),
               from_load_layout(v.z, src_addr), from_load_layout(v.w, src_addr)};
}

// A 16-bit store through a buffer resource: offsets beyond its range are
// dropped, so rows past the end need no branch.
__device__ __forceinline__ void st2(__amdgpu_buffer_rsrc_t r, uint32_t off, __bf16 v) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, v), r, off, 0, 0);
}
__device__ __forceinline__ void st2s(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, __bf16 v) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, v), r, voff, soff, 0);
}

// ---- split-K partials shared between workgroups on different XCDs ----------
// Partials are written and read with the system-coherent cache policy
// (sc0 sc1): those accesses bypass the XCDs' non-coherent L2 state, so the
// hand-off needs no cache-wide writeback or invalidate (which an agent-scope
// fence would emit), only the completion of the writer's stores before it
// bumps the arrival counter.  The loads are ordinary (not atomic), so a
// lane's loads of all splits are in flight together.
constexpr int kCoherent = 17;  // sc0 | sc1

__device__ __forceinline__ void st_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, kCoherent);
}
__device__ __forceinline__ float ld_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kCoherent));
}
// All of this wave's memory operations have completed.
__device__ __forceinline__ void wait_all_memory() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// 16 bytes per lane from a buffer straight into LDS (gfx950 LDS-DMA): lane l
// writes lds + 16 l (lds must be wave-uniform).  Completion is tracked by
// the wave's vector-memory counter, like any load.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void *lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, off,
                                           0, 0, 0);
}

// Workgroup barrier for LDS hand-offs only: this wave's LDS operations
// complete (lgkmcnt 0), then s_barrier.  Unlike __syncthreads it does not
// wait for outstanding global loads, so prefetches stay in flight.  The
// signal fences keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

}  // namespace nvfp4
