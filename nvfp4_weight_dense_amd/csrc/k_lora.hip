// k_lora.hip -- the LoRA overlay's deltas on the NVFP4 FFN (gfx950):
// base[m][n] += scale * (x . A^T) . B^T for a low-rank pair A [r][k],
// B [n][r] (page layers/dense_ffn_overlays.rs, `apply_lora_gate_up` and
// `apply_lora_down`: gate/up deltas before the activation, the output's
// after the down projection; the overlay works through an x.A^T buffer and
// a delta buffer).
//
// Passes, each bound by reading A and B once:
//   * k_lora_xa: fp32 partials of x . A^T over K chunks of kKC elements,
//     for one or two pairs that read the same x (gate and up).  A
//     workgroup takes one row of x, one K chunk and eight rows of A; each
//     thread walks 8-element pieces (16-byte loads), then the eight partial
//     sums are reduced over the workgroup in a fixed order (wave butterfly,
//     then the four waves in order).  Partials: [pair][chunk][m][r].
//   * k_lora_add: base = bf16(base + scale * xa . B^T), one thread per
//     output column; the row's xa (chunk partials summed in chunk order)
//     sits in LDS, B[c][0..r) comes by 16-byte loads, the dot runs in j
//     order.
//   * k_lora_silu: the gate and up deltas and silu_mul in one pass:
//     g' = bf16(g + sg * dg), u' = bf16(u + su * du), act = bf16(silu(g') u')
//     -- the same roundings as adding each delta into its bf16 buffer and
//     then running silu_mul.
// r is a multiple of 8 (at most kMaxRank); k a multiple of 8.
#include "launchers.h"
#include "nvfp4_common.h"

namespace nvfp4 {

namespace {

constexpr int kRB = 8;     // A rows per workgroup
constexpr int kKC = 1024;  // K elements per chunk

__device__ __forceinline__ float bf_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
  return __builtin_bit_cast(float, (uint32_t)v << 16);
}

struct XaArgs {
  const uint16_t *x;  // [m][k]
  int m, k, nkc;
  const uint16_t *a[2];
  int r[2];
  float *part;  // [pair][nkc][m][rmax]
  int rmax;
};

__global__ __launch_bounds__(256) void k_lora_xa(XaArgs p) {
  const int pair = blockIdx.z % 2, row = blockIdx.z / 2;
  const int r = p.r[pair];
  const int j0 = blockIdx.x * kRB;
  if (j0 >= r) return;  // uniform per workgroup
  const int kc = blockIdx.y;
  const int t = threadIdx.x;
  const uint16_t *a = p.a[pair];
  const int c_begin = kc * (kKC / 8), c_end = min((kc + 1) * (kKC / 8), p.k / 8);
  const uint4 *xr = (const uint4 *)(p.x + (size_t)row * p.k);
  float acc[kRB];
#pragma unroll
  for (int j = 0; j < kRB; ++j) acc[j] = 0.f;
  for (int c = c_begin + t; c < c_end; c += 256) {
    const uint4 xv = xr[c];
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
    for (int j = 0; j < kRB; ++j) {
      const uint4 av = ((const uint4 *)(a + (size_t)(j0 + j) * p.k))[c];
      const uint32_t aw[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[j] = fmaf(bf_lo(xw[q]), bf_lo(aw[q]), acc[j]);
        acc[j] = fmaf(bf_hi(xw[q]), bf_hi(aw[q]), acc[j]);
      }
    }
  }
  __shared__ float red[4][kRB];
#pragma unroll
  for (int j = 0; j < kRB; ++j) {
    float v = acc[j];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if ((t & 63) == 0) red[t >> 6][j] = v;
  }
  __syncthreads();
  if (t < kRB)
    p.part[(((size_t)pair * p.nkc + kc) * p.m + row) * p.rmax + j0 + t] =
        ((red[0][t] + red[1][t]) + red[2][t]) + red[3][t];
}

// the row's xa of one pair into LDS: partials summed in chunk order
__device__ __forceinline__ void gather_xa(const float *part, int pair, int nkc, int m, int rmax,
                                          int row, int r, float *xs) {
  for (int j = threadIdx.x; j < r; j += 256) {
    float v = 0.f;
    for (int kc = 0; kc < nkc; ++kc) v += part[(((size_t)pair * nkc + kc) * m + row) * rmax + j];
    xs[j] = v;
  }
}

__device__ __forceinline__ float dot_b(const float *xs, const uint16_t *b, int c, int r) {
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
  return d;
}

struct AddArgs {
  const float *part;
  int nkc, m, rmax, r;
  const uint16_t *b;  // [n][r]
  int n;
  float scale;
  uint16_t *base;  // [m][n]
};

__global__ __launch_bounds__(256) void k_lora_add(AddArgs p) {
  const int row = blockIdx.y;
  __shared__ float xs[kMaxRank];
  gather_xa(p.part, 0, p.nkc, p.m, p.rmax, row, p.r, xs);
  __syncthreads();
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= p.n) return;
  const float d = dot_b(xs, p.b, c, p.r);
  uint16_t *q = p.base + (size_t)row * p.n + c;
  *q = __builtin_bit_cast(uint16_t, (__bf16)(bf16_to_f32(*q) + p.scale * d));
}

struct SiluArgs {
  const float *part;
  int nkc, m, rmax;
  const uint16_t *b[2];  // gate, up: [n][r]
  int r[2];
  float scale[2];
  int n;
  uint16_t *g;        // [m][n], receives act
  const uint16_t *u;  // [m][n]
};

__global__ __launch_bounds__(256) void k_lora_silu(SiluArgs p) {
  const int row = blockIdx.y;
  __shared__ float xs[2][kMaxRank];
#pragma unroll
  for (int i = 0; i < 2; ++i)
    if (p.r[i] > 0) gather_xa(p.part, i, p.nkc, p.m, p.rmax, row, p.r[i], xs[i]);
  __syncthreads();
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= p.n) return;
  const size_t e = (size_t)row * p.n + c;
  float gv = bf16_to_f32(p.g[e]), uv = bf16_to_f32(p.u[e]);
  if (p.r[0] > 0) gv = (float)(__bf16)(gv + p.scale[0] * dot_b(xs[0], p.b[0], c, p.r[0]));
  if (p.r[1] > 0) uv = (float)(__bf16)(uv + p.scale[1] * dot_b(xs[1], p.b[1], c, p.r[1]));
  p.g[e] = __builtin_bit_cast(uint16_t, (__bf16)(silu_f32(gv) * uv));
}

int chunks(int k) { return (k + kKC - 1) / kKC; }

hipError_t launch_xa(const void *x, int m, int k, const void *a0, int r0, const void *a1, int r1,
                     float *part, hipStream_t stream) {
  XaArgs p{};
  p.x = (const uint16_t *)x;
  p.m = m;
  p.k = k;
  p.nkc = chunks(k);
  p.a[0] = (const uint16_t *)a0;
  p.a[1] = (const uint16_t *)a1;
  p.r[0] = r0;
  p.r[1] = r1;
  p.rmax = r0 > r1 ? r0 : r1;
  p.part = part;
  if (p.rmax == 0) return hipSuccess;  // no pair reads x
  hipLaunchKernelGGL(k_lora_xa, dim3((p.rmax + kRB - 1) / kRB, p.nkc, 2 * m), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

int lora_chunks(int k) { return chunks(k); }

hipError_t launch_lora_xa_pair(const void *x, int m, int k, const LoraRef &lg, const LoraRef &lu, float *xa,
                               hipStream_t stream) {
  if (m == 0) return hipSuccess;
  return launch_xa(x, m, k, lg.a, lg.r, lu.a, lu.r, xa, stream);
}

size_t lora_xa_floats(int m, int k, int npairs) { return (size_t)npairs * chunks(k) * m * kMaxRank; }

hipError_t launch_lora_delta(const void *x, int m, int k, const void *a, const void *b, int r, int n,
                             float scale, void *base, float *xa, hipStream_t stream) {
  if (m == 0 || r == 0) return hipSuccess;
  hipError_t e = launch_xa(x, m, k, a, r, nullptr, 0, xa, stream);
  if (e != hipSuccess) return e;
  AddArgs p{};
  p.part = xa;
  p.nkc = chunks(k);
  p.m = m;
  p.rmax = r;
  p.r = r;
  p.b = (const uint16_t *)b;
  p.n = n;
  p.scale = scale;
  p.base = (uint16_t *)base;
  hipLaunchKernelGGL(k_lora_add, dim3((n + 255) / 256, m), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_lora_gate_up_silu(const void *x, int m, int k, const LoraRef &lg, const LoraRef &lu,
                                    int n, void *g, const void *u, float *xa, hipStream_t stream) {
  if (m == 0) return hipSuccess;
  hipError_t e = launch_xa(x, m, k, lg.a, lg.r, lu.a, lu.r, xa, stream);
  if (e != hipSuccess) return e;
  SiluArgs p{};
  p.part = xa;
  p.nkc = chunks(k);
  p.m = m;
  p.rmax = lg.r > lu.r ? lg.r : lu.r;
  p.b[0] = (const uint16_t *)lg.b;
  p.b[1] = (const uint16_t *)lu.b;
  p.r[0] = lg.r;
  p.r[1] = lu.r;
  p.scale[0] = lg.scale;
  p.scale[1] = lu.scale;
  p.n = n;
  p.g = (uint16_t *)g;
  p.u = (const uint16_t *)u;
  hipLaunchKernelGGL(k_lora_silu, dim3((n + 255) / 256, m), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace nvfp4
