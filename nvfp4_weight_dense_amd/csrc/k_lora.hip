// k_lora.hip -- the LoRA overlay's delta on the NVFP4 FFN (gfx950):
// base[m][n] += scale * (x . A^T) . B^T for a low-rank pair A [r][k],
// B [n][r] (page layers/dense_ffn_overlays.rs, `apply_lora_gate_up` and
// `apply_lora_down`: gate/up deltas before the activation, the output's
// after the down projection; the overlay works through an x.A^T buffer and
// a delta buffer).
//
// Two passes, both bound by reading A and B once:
//   * k_lora_xa: xa[m][r] = x . A^T in fp32.  A workgroup takes one row of x
//     and eight rows of A; each thread walks 8-element K chunks (16-byte
//     loads of x and of the eight A rows), then the eight partial sums are
//     reduced over the workgroup in a fixed order (wave butterfly, then the
//     four waves in order).
//   * k_lora_add: each thread owns one output column c of one row: the
//     row's xa sits in LDS, B[c][0..r) is read with 16-byte loads, the dot
//     product runs in j order, and base = bf16(base + scale * dot).
// r is a multiple of 8 (at most kMaxRank); k a multiple of 8.
#include "launchers.h"
#include "nvfp4_common.h"

namespace nvfp4 {

namespace {

constexpr int kRB = 8;  // A rows per workgroup

__device__ __forceinline__ float bf_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

__global__ __launch_bounds__(256) void k_lora_xa(const uint16_t *__restrict__ x, int k,
                                                 const uint16_t *__restrict__ a, int r,
                                                 float *__restrict__ xa) {
  const int row = blockIdx.y;
  const int j0 = blockIdx.x * kRB;
  const int t = threadIdx.x;
  const uint4 *xr = (const uint4 *)(x + (size_t)row * k);
  float acc[kRB];
#pragma unroll
  for (int j = 0; j < kRB; ++j) acc[j] = 0.f;
  for (int c = t; c < (k >> 3); c += 256) {
    const uint4 xv = xr[c];
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
    for (int j = 0; j < kRB; ++j) {
      if (j0 + j >= r) break;
      const uint4 av = ((const uint4 *)(a + (size_t)(j0 + j) * k))[c];
      const uint32_t aw[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[j] = fmaf(bf_lo(xw[q]), bf_lo(aw[q]), acc[j]);
        acc[j] = fmaf(bf_hi(xw[q]), bf_hi(aw[q]), acc[j]);
      }
    }
  }
  __shared__ float part[4][kRB];
#pragma unroll
  for (int j = 0; j < kRB; ++j) {
    float v = acc[j];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if ((t & 63) == 0) part[t >> 6][j] = v;
  }
  __syncthreads();
  if (t < kRB && j0 + t < r)
    xa[(size_t)row * r + j0 + t] = ((part[0][t] + part[1][t]) + part[2][t]) + part[3][t];
}

__global__ __launch_bounds__(256) void k_lora_add(const float *__restrict__ xa, int r,
                                                  const uint16_t *__restrict__ b, int n,
                                                  float scale, uint16_t *base) {
  const int row = blockIdx.y;
  __shared__ float xs[kMaxRank];
  for (int j = threadIdx.x; j < r; j += 256) xs[j] = xa[(size_t)row * r + j];
  __syncthreads();
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= n) return;
  const uint4 *bc = (const uint4 *)(b + (size_t)c * r);
  float d = 0.f;
  for (int j8 = 0; j8 < (r >> 3); ++j8) {
    const uint4 bv = bc[j8];
    const uint32_t bw[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      d = fmaf(xs[8 * j8 + 2 * q], bf_lo(bw[q]), d);
      d = fmaf(xs[8 * j8 + 2 * q + 1], bf_hi(bw[q]), d);
    }
  }
  uint16_t *p = base + (size_t)row * n + c;
  const float v = __builtin_bit_cast(float, (uint32_t)*p << 16) + scale * d;
  *p = __builtin_bit_cast(uint16_t, (__bf16)v);
}

}  // namespace

size_t lora_xa_floats(int m, int r) { return (size_t)m * r; }

hipError_t launch_lora_delta(const void *x, int m, int k, const void *a, const void *b, int r, int n,
                             float scale, void *base, float *xa, hipStream_t stream) {
  if (m == 0 || r == 0) return hipSuccess;
  hipLaunchKernelGGL(k_lora_xa, dim3((r + kRB - 1) / kRB, m), dim3(256), 0, stream,
                     (const uint16_t *)x, k, (const uint16_t *)a, r, xa);
  hipLaunchKernelGGL(k_lora_add, dim3((n + 255) / 256, m), dim3(256), 0, stream, (const float *)xa, r,
                     (const uint16_t *)b, n, scale, (uint16_t *)base);
  return hipGetLastError();
}

}  // namespace nvfp4
