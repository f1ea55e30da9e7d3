// k_probe.hip -- a measurement aid, not a step of the FFN: the bf16 matrix
// throughput this part reaches in practice, to print beside the 2.5 PFLOP/s
// specification when a many-row kernel's fraction of the peak is reported.
//
// Each wave runs `iters` rounds of four independent
// v_mfma_f32_32x32x16_bf16 (32x32x16 multiply-adds, 32768 flops each) on
// register operands: no memory traffic, no LDS, no dependence between the
// four accumulators within a round, so the matrix pipe never waits on a
// result.  Workgroups of four waves (one per SIMD).
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

}  // namespace

hipError_t launch_mfma_probe(int workgroups, int iters, float *sink, hipStream_t stream) {
  hipLaunchKernelGGL(k_mfma_probe, dim3(workgroups), dim3(256), 0, stream, iters, sink);
  return hipGetLastError();
}

}  // namespace nvfp4
