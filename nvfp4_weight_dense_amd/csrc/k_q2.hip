// k_q2.hip -- projection on packed-Q2 weights with bf16 activations (gfx950).
//
// Format (page layers/dense_ffn_prefill.rs, `prefill_q2`: Q2_0 weights with
// a group size, dequantized to BF16 for the BF16 GEMM; the code itself is not
// defined on the pages -- the reading taken here):
//   codes  uint8 [n][k/4], element 4j+i in bits 2i..2i+1 of byte j;
//   scales fp16 [n][k/group], group a power of two >= 32 dividing k;
//   W[c][k] = bf16((q - 2) * d[c][k/group]), rounded to nearest even.
// The product (q - 2) * d is exact in fp32 (q - 2 in {-2, -1, 0, 1}, d has
// 11 significant bits), so the kernel's bf16 weights are bit-identical to
// the pages' dequantized BF16 weight; the GEMM then runs on the bf16 matrix
// cores with fp32 sums, and the weights never exist as bf16 in memory.
//
// Serves up to 16 rows, and 17..64 rows when k % 64 != 0 (17..64 rows with
// k % 64 == 0 take k_smallm's packed-Q2 variant).
//
// Work decomposition (the weight-streaming skeleton of the other few-row
// kernels): a workgroup owns CTW tiles of 16 columns of NMAT matrices (2:
// gate and up with the silu epilogue), up to 64 rows and a range of K; its 4
// waves take interleaved 128-element steps.  Lane (c = lane%16, g = lane/16)
// takes the 8 code bytes of column c for K offsets 32g..32g+31 of the step
// (a wave covers 16 rows x 32 contiguous bytes) and that chunk's scale (a
// chunk lies in one group); for up to 16 rows both are loaded in the
// row-contiguous layout (lane s reads row s/4, chunk s%4) and moved to lane
// (c, g) with ds_bpermute, the same bytes as a direct load (measured FFN:
// m=8 48.7 -> 43.1 us; with more rows the activation loads dominate and the
// permute costs more than it saves: m=64 178 -> 196 us, so those load
// directly); it dequantizes them into the
// four B fragments of v_mfma_f32_16x16x32_bf16, and loads the same 32 K of
// each activation row (64 bytes).  K order inside a step is (g, element) on
// both operands.  Waves reduce through LDS in wave order; with ksplit > 1
// the last workgroup of a tile sums the fp32 partials in split order.
#include "launchers.h"
#include "nvfp4_common.h"

namespace nvfp4 {

namespace {

constexpr int kNW = 4;  // waves per workgroup

struct Q2Args {
  const void *x;  // bf16 [m][k]
  int m, k, n, gshift;  // group = 1 << gshift
  const uint8_t *codes0, *codes1;    // [n][k/4]
  const uint16_t *scales0, *scales1;  // fp16 [n][k/group]
  void *y;
  float *partial;      // [tiles * row blocks][NMAT][ksplit][CTW][16*MT][16]
  unsigned *counters;  // [gridDim.z][gridDim.x], zero between calls
  int ksplit, steps_per_split;
};

template <int MT, int NMAT, int CTW>
struct Q2Cfg {
  static constexpr int kRegsPerStep = NMAT * CTW * 3 + MT * 16;
  static constexpr int U =
      kRegsPerStep * 8 <= 128 ? 8 : (kRegsPerStep * 4 <= 128 ? 4 : (kRegsPerStep * 2 < 128 ? 2 : 1));
};

__device__ __forceinline__ uint2 ld8_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kStreamPolicy));
}

// Eight 2-bit codes (16 bits, element e in bits 2e..2e+1) -> the bf16 values
// (q - 2) * d: q*d and 2d are exact in fp32, so the fma is exact and the
// bf16 conversion is the one rounding.
__device__ __forceinline__ bf16x8 dequant_q2x8(uint32_t bits16, float d, float m2d) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float q = (float)((bits16 >> (2 * e)) & 3u);
    r[e] = (__bf16)__builtin_fmaf(q, d, m2d);
  }
  return r;
}

__device__ __forceinline__ float fp16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

template <int MT, int NMAT, int CTW>
__global__ __launch_bounds__(kNW * 64) void k_q2(Q2Args p) {
  constexpr int U = Q2Cfg<MT, NMAT, CTW>::U;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c16 = lane & 15;
  const int g = lane >> 4;
  const int src_addr = load_layout_src_addr(lane);
  constexpr bool kRowLoads = MT == 1;
  // activation rows: row-contiguous loads plus the permute for 17..48 rows
  // (FFN m=32 124 -> 112 us); at one row tile and at four they measured
  // 1.5-2 us slower or even, so those load the operand layout directly
  constexpr bool kRowAct = MT == 2 || MT == 3;
  const uint32_t lrow = kRowLoads ? (uint32_t)(lane >> 2) : (uint32_t)c16;  // weight row loaded
  const uint32_t lpiece = kRowLoads ? (uint32_t)(lane & 3) : (uint32_t)g;   // 32-K chunk loaded
  const int k = p.k;
  const int col0 = blockIdx.x * (16 * CTW);
  const int row0 = blockIdx.z * 64;
  const int nsteps = (k + 127) >> 7;
  const int s_begin = blockIdx.y * p.steps_per_split;
  const int s_end = min(nsteps, s_begin + p.steps_per_split);
  const uint32_t kb4 = (uint32_t)k >> 2;
  const uint32_t ngroups = (uint32_t)k >> p.gshift;

  const int ncols = min(16 * CTW, p.n - col0);
  const int nrows = min(64, p.m - row0);
  __amdgpu_buffer_rsrc_t wc[NMAT], ws[NMAT];
  wc[0] = rsrc(p.codes0 + (size_t)col0 * kb4, (size_t)ncols * kb4);
  ws[0] = rsrc(p.scales0 + (size_t)col0 * ngroups, (size_t)ncols * ngroups * 2);
  if constexpr (NMAT > 1) {
    wc[1] = rsrc(p.codes1 + (size_t)col0 * kb4, (size_t)ncols * kb4);
    ws[1] = rsrc(p.scales1 + (size_t)col0 * ngroups, (size_t)ncols * ngroups * 2);
  }
  const __amdgpu_buffer_rsrc_t ax =
      rsrc((const uint16_t *)p.x + (size_t)row0 * k, (size_t)nrows * k * 2);

  f32x4 acc[NMAT][CTW][MT];
#pragma unroll
  for (int i = 0; i < NMAT; ++i)
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[i][ct][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int base = s_begin + wave; base < s_end; base += kNW * U) {
    uint2 bw[U][NMAT][CTW];
    uint32_t bsc[U][NMAT][CTW];
    uint4 aw[U][MT][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = base + u * kNW;
      const uint32_t kl = (uint32_t)t * 128u + 32u * lpiece;  // K of this lane's weight load
      const bool okl = t < s_end && kl < (uint32_t)k;
      const uint32_t ka = (uint32_t)t * 128u + 32u * (kRowAct ? (uint32_t)(lane & 3) : (uint32_t)g);
      const bool oka = t < s_end && ka < (uint32_t)k;
      const uint32_t arow = kRowAct ? (uint32_t)(lane >> 2) : (uint32_t)c16;
#pragma unroll
      for (int i = 0; i < NMAT; ++i)
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
          const uint32_t row = (uint32_t)(ct * 16) + lrow;
          bw[u][i][ct] = ld8_nt(wc[i], okl ? row * kb4 + (kl >> 2) : kOOB);
          bsc[u][i][ct] = ld2_nt(ws[i], okl ? (row * ngroups + (kl >> p.gshift)) * 2u : kOOB);
        }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint32_t off = oka ? (((uint32_t)(mt * 16) + arow) * (uint32_t)k + ka) * 2u : kOOB;
#pragma unroll
        for (int q = 0; q < 4; ++q) aw[u][mt][q] = ld16(ax, off + 16u * q);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      bf16x8 bf[NMAT][CTW][4];
#pragma unroll
      for (int i = 0; i < NMAT; ++i)
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
          uint32_t sc = bsc[u][i][ct];
          uint2 w = bw[u][i][ct];
          if constexpr (kRowLoads) {
            sc = from_load_layout(sc, src_addr);
            w = uint2{from_load_layout(w.x, src_addr), from_load_layout(w.y, src_addr)};
          }
          const float d = fp16_bits_to_f32(sc);
          const float m2d = -2.0f * d;
          bf[i][ct][0] = dequant_q2x8(w.x & 0xFFFFu, d, m2d);
          bf[i][ct][1] = dequant_q2x8(w.x >> 16, d, m2d);
          bf[i][ct][2] = dequant_q2x8(w.y & 0xFFFFu, d, m2d);
          bf[i][ct][3] = dequant_q2x8(w.y >> 16, d, m2d);
        }
      if constexpr (kRowAct) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int q = 0; q < 4; ++q) aw[u][mt][q] = from_load_layout(aw[u][mt][q], src_addr);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const bf16x8 a = as_bf16x8(aw[u][mt][j]);
#pragma unroll
          for (int i = 0; i < NMAT; ++i)
#pragma unroll
            for (int ct = 0; ct < CTW; ++ct)
              acc[i][ct][mt] =
                  __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bf[i][ct][j], acc[i][ct][mt], 0, 0, 0);
        }
    }
  }

  // fixed-order reduction over the workgroup's waves
  __shared__ float red[kNW - 1][MT][4][64];
#pragma unroll
  for (int i = 0; i < NMAT; ++i)
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct) {
      if (wave > 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int e = 0; e < 4; ++e) red[wave - 1][mt][e][lane] = acc[i][ct][mt][e];
      }
      __syncthreads();
      if (wave == 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float s = acc[i][ct][mt][e];
#pragma unroll
            for (int w = 0; w < kNW - 1; ++w) s += red[w][mt][e][lane];
            acc[i][ct][mt][e] = s;
          }
      }
      __syncthreads();
    }
  if (wave != 0) return;

  if (p.ksplit > 1) {
    constexpr int kTile = 16 * MT * 16;
    const size_t wg = (size_t)blockIdx.z * gridDim.x + blockIdx.x;
    const __amdgpu_buffer_rsrc_t pres = rsrc(p.partial + wg * NMAT * p.ksplit * CTW * kTile,
                                             (size_t)NMAT * p.ksplit * CTW * kTile * 4);
    auto poff = [&](int i, int sp, int ct, int mt, int e) -> uint32_t {
      const uint32_t r = mt * 16 + 4 * g + e;
      return ((((uint32_t)(i * p.ksplit + sp) * CTW + ct) * kTile) + r * 16u + c16) * 4u;
    };
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int i = 0; i < NMAT; ++i)
            st_coherent(pres, poff(i, blockIdx.y, ct, mt, e), acc[i][ct][mt][e]);
    unsigned *cnt = p.counters + wg;
    wait_all_memory();
    unsigned old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __shfl(old, 0);
    if (old != (unsigned)(p.ksplit - 1)) return;
    // last arrival: sum the partials in split order
#pragma unroll
    for (int i = 0; i < NMAT; ++i)
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[i][ct][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < p.ksplit; ++sp) {
      float v[NMAT][CTW][MT][4];
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int i = 0; i < NMAT; ++i) v[i][ct][mt][e] = ld_coherent(pres, poff(i, sp, ct, mt, e));
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int i = 0; i < NMAT; ++i) acc[i][ct][mt][e] += v[i][ct][mt][e];
    }
    if (lane == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // epilogue: output element (row0 + mt*16 + 4g + e, col0 + ct*16 + c16)
#pragma unroll
  for (int ct = 0; ct < CTW; ++ct) {
    const int col = col0 + ct * 16 + c16;
    if (col >= p.n) continue;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = row0 + mt * 16 + 4 * g + e;
        if (r >= p.m) continue;
        __bf16 out;
        if constexpr (NMAT > 1)
          out = swiglu_bf16(acc[0][ct][mt][e], acc[NMAT - 1][ct][mt][e]);
        else
          out = (__bf16)acc[0][ct][mt][e];
        ((__bf16 *)p.y)[(size_t)r * p.n + col] = out;
      }
  }
}

template <int MT, int NMAT, int CTW>
hipError_t launch_one(const Q2Args &p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((k_q2<MT, NMAT, CTW>), grid, dim3(kNW * 64), 0, s, p);
  return hipGetLastError();
}

template <int NMAT, int CTW>
hipError_t launch_mt(const Q2Args &p, int mt, dim3 grid, hipStream_t s) {
  switch (mt) {
    case 1: return launch_one<1, NMAT, CTW>(p, grid, s);
    case 2: return launch_one<2, NMAT, CTW>(p, grid, s);
    case 3: return launch_one<3, NMAT, CTW>(p, grid, s);
    default: return launch_one<4, NMAT, CTW>(p, grid, s);
  }
}

}  // namespace

// Column tiles per workgroup: with more than 16 rows each activation
// fragment (64 bytes per row and step) is shared by several column tiles,
// which divides the activation re-reads from L2 -- two tiles up to 32 rows,
// four above (four tiles of 32 rows need 440 registers per lane, one wave
// per SIMD: FFN on the small-m shape at m=17 and 32 in 107 and 125 us with
// two, 130 and 139 us with four; at m=64 185 against 177 us); with few rows
// the tiles stay narrow so that the weight stream spreads over many
// workgroups.
int q2_ctw(int m, int n) { return m > 32 ? 4 : (m > 16 ? 2 : (n >= 16 * 2 * 512 ? 2 : 1)); }

StreamPlan q2_plan(int m, int n, int k) {
  constexpr int kTarget = 512;  // workgroups before K is split
  const int tiles = cdiv(n, 16 * q2_ctw(m, n));
  const int nsteps = cdiv(k, 128);
  int ksplit = 1;
  if (tiles < kTarget) {
    const int want = cdiv(kTarget, tiles);
    const int cap = nsteps / (kNW * 2);  // at least two steps per wave
    ksplit = want < cap ? want : cap;
    if (ksplit < 1) ksplit = 1;
  }
  StreamPlan pl;
  if (k < splitk_min_k()) ksplit = 1;
  pl.steps_per_split = cdiv(nsteps, ksplit);
  pl.ksplit = cdiv(nsteps, pl.steps_per_split);
  pl.tiles = tiles;
  return pl;
}

size_t q2_partial_floats(const StreamPlan &pl, int nmat, int m, int n) {
  const int mt = m >= 64 ? 4 : cdiv(m, 16);
  return pl.ksplit > 1
             ? (size_t)pl.tiles * cdiv(m, 64) * nmat * pl.ksplit * q2_ctw(m, n) * 16 * mt * 16
             : 0;
}

hipError_t launch_q2(const void *x, int m, int k, int n, int gshift, int nmat, const Q2MatRef *w,
                     void *y, float *partial, unsigned *counters, const StreamPlan &pl,
                     hipStream_t stream) {
  Q2Args p{};
  p.x = x;
  p.m = m;
  p.k = k;
  p.n = n;
  p.gshift = gshift;
  p.codes0 = w[0].codes;
  p.scales0 = w[0].scales;
  p.codes1 = nmat > 1 ? w[1].codes : nullptr;
  p.scales1 = nmat > 1 ? w[1].scales : nullptr;
  p.y = y;
  p.partial = partial;
  p.counters = counters;
  p.ksplit = pl.ksplit;
  p.steps_per_split = pl.steps_per_split;
  const int mt = m >= 64 ? 4 : cdiv(m, 16);
  dim3 grid(pl.tiles, pl.ksplit, cdiv(m, 64));
  switch (q2_ctw(m, n)) {
    case 4: return nmat == 1 ? launch_mt<1, 4>(p, mt, grid, stream) : launch_mt<2, 4>(p, mt, grid, stream);
    case 2: return nmat == 1 ? launch_mt<1, 2>(p, mt, grid, stream) : launch_mt<2, 2>(p, mt, grid, stream);
    default: return nmat == 1 ? launch_mt<1, 1>(p, mt, grid, stream) : launch_mt<2, 1>(p, mt, grid, stream);
  }
}

}  // namespace nvfp4
