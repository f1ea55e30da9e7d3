// k_probe.hip -- measurement aids, not steps of the FFN: the bf16 matrix
// throughput and the HBM read rate this part reaches in practice, to print
// beside the specification's peaks (2.5 PFLOP/s, 8 TB/s) when a kernel's
// fraction of its roofline is reported.
//
// MFMA probe:
// Each wave runs `iters` rounds of four independent
// v_mfma_f32_32x32x16_bf16 (32x32x16 multiply-adds, 32768 flops each) on
// register operands: no memory traffic, no LDS, no dependence between the
// four accumulators within a round, so the matrix pipe never waits on a
// result.  Workgroups of four waves (one per SIMD).
#include "encode_hw.h"
#include "launchers.h"
#include "nvfp4_common.h"

namespace nvfp4 {

namespace {

__global__ __launch_bounds__(256) void k_mfma_probe(int iters, float *sink) {
  const int lane = (int)(threadIdx.x & 63);
  // operands from the lane index, so nothing folds at compile time
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1.0f + 0.0078125f * (float)((lane + i) & 7));
    b[i] = (__bf16)(0.5f + 0.0078125f * (float)((lane * 3 + i) & 7));
  }
  f32x16 acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {};
  for (int it = 0; it < iters; ++it) {
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc1, 0, 0, 0);
    acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc2, 0, 0, 0);
    acc3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += acc0[e] + acc1[e] + acc2[e] + acc3[e];
  // every operand is positive, so s > 0 and the store never happens; the
  // compiler cannot know that, so the loop stays
  if (s == -1.0f) sink[threadIdx.x] = s;
}

// Read probe: one pass over n16 16-byte items with nothing else to do.
// Workgroup b reads items [b * 1024, (b + 1) * 1024): each lane has four
// 16-byte loads in flight (256 lanes x 4, consecutive lanes on consecutive
// items), folds them with xor and stores only if the fold equals a value
// the caller's buffer is never filled with -- so the loads stay, and the
// probe writes nothing in practice.
constexpr int kReadPerLane = 4;
__global__ __launch_bounds__(256) void k_read_probe(const uint4 *src, size_t n16, uint32_t never, float *sink) {
  const size_t base = (size_t)blockIdx.x * (256 * kReadPerLane) + threadIdx.x;
  uint4 v[kReadPerLane];
#pragma unroll
  for (int i = 0; i < kReadPerLane; ++i) {
    const size_t idx = base + (size_t)i * 256;
    v[i] = idx < n16 ? src[idx] : uint4{0u, 0u, 0u, 0u};
  }
  uint32_t f = 0;
#pragma unroll
  for (int i = 0; i < kReadPerLane; ++i) f ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  if (f == never) sink[threadIdx.x] = 1.0f;
}

// Encoder probe: the quantizers' quotient and rounding steps on arbitrary
// inputs, for the tests.  Thread t takes elements 8t .. 8t + 7 (n % 8 == 0):
// q = x / d as the quantizers divide, and the E2M1 and E4M3 codes of x
// itself, one byte per element.
__global__ __launch_bounds__(256) void k_encode_probe(const float *x, int64_t n8, float d, float *q,
                                                      uint8_t *e2m1, uint8_t *e4m3) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n8) return;
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = x[8 * t + i];
  const bool fast = recip_div_ok(d);
  const float y = 1.0f / d;
#pragma unroll
  for (int i = 0; i < 8; ++i) q[8 * t + i] = fast ? div_by_recip(v[i], d, y) : v[i] / d;
  const uint32_t c4 = e2m1x8_hw(v);
  const uint32_t c8[2] = {e4m3x4_hw(v), e4m3x4_hw(v + 4)};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    e2m1[8 * t + i] = (uint8_t)((c4 >> (4 * i)) & 0xFu);
    e4m3[8 * t + i] = (uint8_t)(c8[i >> 2] >> (8 * (i & 3)));
  }
}

}  // namespace

hipError_t launch_encode_probe(const float *x, int64_t n, float d, float *q, uint8_t *e2m1, uint8_t *e4m3,
                               hipStream_t stream) {
  const int64_t n8 = n / 8;
  hipLaunchKernelGGL(k_encode_probe, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream, x, n8, d, q,
                     e2m1, e4m3);
  return hipGetLastError();
}

hipError_t launch_read_probe(const void *src, size_t bytes, uint32_t never, float *sink, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  const size_t per_wg = 256 * kReadPerLane;
  hipLaunchKernelGGL(k_read_probe, dim3((unsigned)((n16 + per_wg - 1) / per_wg)), dim3(256), 0, stream,
                     (const uint4 *)src, n16, never, sink);
  return hipGetLastError();
}

hipError_t launch_mfma_probe(int workgroups, int iters, float *sink, hipStream_t stream) {
  hipLaunchKernelGGL(k_mfma_probe, dim3(workgroups), dim3(256), 0, stream, iters, sink);
  return hipGetLastError();
}

}  // namespace nvfp4
