// k_stream.hip -- weight-streaming NVFP4 projection for few rows (gfx950).
//
// Regime: the page layers/dense_ffn_prefill.rs (`w4a16_prefill_gemm`) runs
// a dedicated small-m path for up to 64 rows; with so few rows the FFN is
// bound by streaming the 4.5-bit weights from HBM once.
//
// Work decomposition
//   * A workgroup owns 16 output columns (one MFMA tile width) and a range of
//     K; its NW waves split that range into interleaved 128-element steps.
//   * In one step, lane (c = lane%16, g = lane/16) loads 16 bytes of codes
//     (32 K elements of weight row col0+c, K offset 32g) plus their 2 scale
//     bytes with one 128-bit and one 16-bit load; a wave's load covers 16
//     rows x 64 contiguous bytes.  The codes are dequantized in registers to
//     four bf16 B fragments and fed to v_mfma_f32_16x16x32_bf16, whose K
//     order inside a step is (g, element) -- the same permutation is used for
//     the activation fragment, so the sum is unchanged.
//   * The activation fragment of row r in a step is the 32 contiguous K
//     values starting at the same offset (bf16, 64 bytes), or, for W4A4, the
//     row's NVFP4 codes dequantized exactly like the weight.
//   * Waves reduce through LDS in fixed wave order; with ksplit > 1 the
//     workgroups write fp32 partials that a second kernel sums in split
//     order.  The K order of every output therefore depends only on (n, k),
//     never on m -- the property the W4A4 arm needs.
//   * Up to 64 rows (MT tiles of 16) share each dequantized weight fragment;
//     more rows use more row blocks (grid.z).
#include "launchers.h"
#include "nvfp4_common.h"

namespace nvfp4 {

namespace {

constexpr int kNW = 4;            // waves per workgroup (K split inside it)
constexpr int kTargetBlocks = 512;

struct StreamArgs {
  const void *x;          // bf16 [m][k] (W4A16)
  const uint8_t *xc;      // NVFP4 codes [m][k/2] (W4A4)
  const uint8_t *xs;      // [m][k/16]
  const float *xr;        // [m]
  int m, k, n;
  const uint8_t *codes0, *scales0;
  const uint8_t *codes1, *scales1;
  float ts0, ts1;
  void *y;
  float *partial;
  int ksplit, steps_per_split;
};

template <int MT>
struct Batch {  // steps loaded together per wave
  static constexpr int U = MT == 1 ? 8 : (MT == 2 ? 4 : 2);
};

template <int MT, int NMAT, bool AFP4>
__global__ __launch_bounds__(kNW * 64) void k_stream(StreamArgs p) {
  constexpr int U = Batch<MT>::U;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c16 = lane & 15;
  const int g = lane >> 4;
  const int k = p.k;
  const int col = blockIdx.x * 16 + c16;
  const bool col_ok = col < p.n;
  const int row0 = blockIdx.z * 64;
  const int nsteps = (k + 127) >> 7;
  const int s_begin = blockIdx.y * p.steps_per_split;
  const int s_end = min(nsteps, s_begin + p.steps_per_split);

  const size_t wrow = (size_t)(col_ok ? col : 0);
  const uint8_t *crow0 = p.codes0 + wrow * (size_t)(k >> 1);
  const uint8_t *srow0 = p.scales0 + wrow * (size_t)(k >> 4);
  const uint8_t *crow1 = NMAT > 1 ? p.codes1 + wrow * (size_t)(k >> 1) : nullptr;
  const uint8_t *srow1 = NMAT > 1 ? p.scales1 + wrow * (size_t)(k >> 4) : nullptr;

  // activation rows this lane feeds (A operand row = lane % 16)
  bool a_ok[MT];
  size_t arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int r = row0 + mt * 16 + c16;
    a_ok[mt] = r < p.m;
    arow[mt] = (size_t)(a_ok[mt] ? r : 0);
  }

  f32x4 acc[NMAT][MT];
#pragma unroll
  for (int i = 0; i < NMAT; ++i)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[i][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint4 z4 = make_uint4(0, 0, 0, 0);
  for (int base = s_begin + wave; base < s_end; base += kNW * U) {
    uint4 bw[U][NMAT];
    uint32_t bsc[U][NMAT];
    uint4 aw[U][MT][AFP4 ? 1 : 4];
    uint32_t asc[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = base + u * kNW;
      const int kk = t * 128 + 32 * g;
      const bool ok = t < s_end && kk < k;
      const bool wok = ok && col_ok;
      bw[u][0] = wok ? *(const uint4 *)(crow0 + (kk >> 1)) : z4;
      bsc[u][0] = wok ? (uint32_t)*(const uint16_t *)(srow0 + (kk >> 4)) : 0u;
      if constexpr (NMAT > 1) {
        bw[u][1] = wok ? *(const uint4 *)(crow1 + (kk >> 1)) : z4;
        bsc[u][1] = wok ? (uint32_t)*(const uint16_t *)(srow1 + (kk >> 4)) : 0u;
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bool aok = ok && a_ok[mt];
        if constexpr (AFP4) {
          aw[u][mt][0] = aok ? *(const uint4 *)(p.xc + arow[mt] * (size_t)(k >> 1) + (kk >> 1)) : z4;
          asc[u][mt] = aok ? (uint32_t)*(const uint16_t *)(p.xs + arow[mt] * (size_t)(k >> 4) + (kk >> 4)) : 0u;
        } else {
          const uint4 *src = (const uint4 *)((const uint16_t *)p.x + arow[mt] * (size_t)k + kk);
#pragma unroll
          for (int q = 0; q < 4; ++q) aw[u][mt][q] = aok ? src[q] : z4;
          asc[u][mt] = 0;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      bf16x8 bf[NMAT][4];
#pragma unroll
      for (int i = 0; i < NMAT; ++i) {
        const float s0 = e4m3_to_f32(bsc[u][i] & 0xFFu);
        const float s1 = e4m3_to_f32(bsc[u][i] >> 8);
        bf[i][0] = dequant8(bw[u][i].x, s0);
        bf[i][1] = dequant8(bw[u][i].y, s0);
        bf[i][2] = dequant8(bw[u][i].z, s1);
        bf[i][3] = dequant8(bw[u][i].w, s1);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        bf16x8 af[4];
        if constexpr (AFP4) {
          const float s0 = e4m3_to_f32(asc[u][mt] & 0xFFu);
          const float s1 = e4m3_to_f32(asc[u][mt] >> 8);
          af[0] = dequant8(aw[u][mt][0].x, s0);
          af[1] = dequant8(aw[u][mt][0].y, s0);
          af[2] = dequant8(aw[u][mt][0].z, s1);
          af[3] = dequant8(aw[u][mt][0].w, s1);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) af[q] = as_bf16x8(aw[u][mt][q]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < NMAT; ++i)
            acc[i][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[j], bf[i][j], acc[i][mt], 0, 0, 0);
      }
    }
  }

  // fixed-order reduction over the workgroup's waves
  __shared__ float red[kNW][NMAT][MT][4][64];
#pragma unroll
  for (int i = 0; i < NMAT; ++i)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[wave][i][mt][e][lane] = acc[i][mt][e];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int i = 0; i < NMAT; ++i)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float s = red[0][i][mt][e][lane];
#pragma unroll
        for (int w = 1; w < kNW; ++w) s += red[w][i][mt][e][lane];
        acc[i][mt][e] = s;
      }

  if (!col_ok) return;
  // output element (row0 + mt*16 + 4g + e, col) of the 16x16 tile
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = row0 + mt * 16 + 4 * g + e;
      if (r >= p.m) continue;
      if (p.ksplit > 1) {
#pragma unroll
        for (int i = 0; i < NMAT; ++i)
          p.partial[(((size_t)i * p.ksplit + blockIdx.y) * p.m + r) * p.n + col] = acc[i][mt][e];
        continue;
      }
      float v0 = acc[0][mt][e];
      float v1 = NMAT > 1 ? acc[NMAT - 1][mt][e] : 0.f;
      if constexpr (AFP4) {
        const float rs = p.xr[r];
        v0 = v0 * rs;
        v1 = v1 * rs;
      }
      v0 = v0 * p.ts0;
      __bf16 out;
      if constexpr (NMAT > 1) {
        v1 = v1 * p.ts1;
        out = swiglu_bf16(v0, v1);
      } else {
        out = (__bf16)v0;
      }
      ((__bf16 *)p.y)[(size_t)r * p.n + col] = out;
    }
}

// Sums split-K partials in split order and applies the epilogue.
template <int NMAT, bool AFP4>
__global__ __launch_bounds__(256) void k_splitk_reduce(StreamArgs p) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t total = (size_t)p.m * p.n;
  if (idx >= total) return;
  const int r = (int)(idx / p.n);
  float v[NMAT];
#pragma unroll
  for (int i = 0; i < NMAT; ++i) {
    float s = 0.f;
    for (int sp = 0; sp < p.ksplit; ++sp) s += p.partial[((size_t)i * p.ksplit + sp) * total + idx];
    if constexpr (AFP4) s = s * p.xr[r];
    v[i] = s;
  }
  __bf16 out;
  if constexpr (NMAT > 1)
    out = swiglu_bf16(v[0] * p.ts0, v[1] * p.ts1);
  else
    out = (__bf16)(v[0] * p.ts0);
  ((__bf16 *)p.y)[idx] = out;
}

template <int MT, int NMAT, bool AFP4>
hipError_t launch_mt(const StreamArgs &p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((k_stream<MT, NMAT, AFP4>), grid, dim3(kNW * 64), 0, s, p);
  return hipGetLastError();
}

template <int NMAT, bool AFP4>
hipError_t launch_cfg(const StreamArgs &p, int mt, dim3 grid, hipStream_t s) {
  switch (mt) {
    case 1: return launch_mt<1, NMAT, AFP4>(p, grid, s);
    case 2: return launch_mt<2, NMAT, AFP4>(p, grid, s);
    case 3: return launch_mt<3, NMAT, AFP4>(p, grid, s);
    default: return launch_mt<4, NMAT, AFP4>(p, grid, s);
  }
}

}  // namespace

StreamPlan stream_plan(int n, int k) {
  // The split depends on (n, k) only: the same projection shape reduces in
  // the same order at every row count.
  const int tiles = cdiv(n, 16);
  const int nsteps = cdiv(k, 128);
  int ksplit = 1;
  if (tiles < kTargetBlocks) {
    int want = cdiv(kTargetBlocks, tiles);
    int cap = nsteps / (kNW * 2);  // at least two steps per wave
    ksplit = want < cap ? want : cap;
    if (ksplit < 1) ksplit = 1;
  }
  StreamPlan pl;
  pl.steps_per_split = cdiv(nsteps, ksplit);
  pl.ksplit = cdiv(nsteps, pl.steps_per_split);
  return pl;
}

size_t stream_partial_floats(const StreamPlan &pl, int nmat, int m, int n) {
  return pl.ksplit > 1 ? (size_t)nmat * pl.ksplit * m * n : 0;
}

hipError_t launch_stream(const ActRef &a, int m, int k, int n, int nmat,
                         const MatRef *w, void *y, float *partial,
                         const StreamPlan &pl, hipStream_t stream) {
  StreamArgs p{};
  p.x = a.x_bf16;
  p.xc = a.codes;
  p.xs = a.scales;
  p.xr = a.row_scale;
  p.m = m;
  p.k = k;
  p.n = n;
  p.codes0 = w[0].codes;
  p.scales0 = w[0].scales;
  p.ts0 = w[0].ts;
  p.codes1 = nmat > 1 ? w[1].codes : nullptr;
  p.scales1 = nmat > 1 ? w[1].scales : nullptr;
  p.ts1 = nmat > 1 ? w[1].ts : 0.f;
  p.y = y;
  p.partial = partial;
  p.ksplit = pl.ksplit;
  p.steps_per_split = pl.steps_per_split;
  const bool afp4 = a.x_bf16 == nullptr;
  const int mt = m >= 64 ? 4 : cdiv(m, 16);
  dim3 grid(cdiv(n, 16), pl.ksplit, cdiv(m, 64));
  hipError_t e;
  if (nmat == 1)
    e = afp4 ? launch_cfg<1, true>(p, mt, grid, stream) : launch_cfg<1, false>(p, mt, grid, stream);
  else
    e = afp4 ? launch_cfg<2, true>(p, mt, grid, stream) : launch_cfg<2, false>(p, mt, grid, stream);
  if (e != hipSuccess || pl.ksplit == 1) return e;
  const size_t total = (size_t)m * n;
  dim3 rgrid((unsigned)((total + 255) / 256));
  if (nmat == 1) {
    if (afp4)
      hipLaunchKernelGGL((k_splitk_reduce<1, true>), rgrid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((k_splitk_reduce<1, false>), rgrid, dim3(256), 0, stream, p);
  } else {
    if (afp4)
      hipLaunchKernelGGL((k_splitk_reduce<2, true>), rgrid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((k_splitk_reduce<2, false>), rgrid, dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
