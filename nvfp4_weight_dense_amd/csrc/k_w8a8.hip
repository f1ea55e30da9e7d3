// k_w8a8.hip -- the W8A8 fixed-format projection (gfx950): block-scaled FP8
// weights times per-row FP8 activations, exact products on the matrix cores.
//
// Format (page layers/dense_ffn_fixed.rs, `Fixed::W8a8`: per-row FP8
// activations at every row count; page layers/dense_ffn_overlays.rs,
// `set_fp8_weights`: block-scaled FP8 weights with a scale grid):
//   weight  W[c][k] = e4m3(codes[c][k]) * scales[c/128][k/128]   (fp32 grid)
//   activation  x_hat[r][k] = e4m3(xq[r][k]) * s_row[r]
//   y[r][c] = bf16( s_row[r] * sum_b scales[c/128][b] * P_b[r][c] ),
//   P_b = sum over the 128 K of block b of e4m3 * e4m3 (exact products,
//   fp32 sums).
//
// Work decomposition (the same skeleton as the NVFP4 weight-streaming
// kernel, so the K order of every output depends on (n, k) only):
//   * A workgroup owns CTW column tiles of 16 output columns (of NMAT
//     weight matrices: 1, or 2 for gate+up with a fused silu epilogue), up
//     to 64 rows, and a range of K; its 4 waves take interleaved 128-element
//     steps.  A step is one weight block along K, and the 16 columns of a
//     tile lie in one block along N, so a step needs one scale per tile.
//   * Lane (c = lane%16, g = lane/16) holds 32 bytes of weight row c: the
//     16 at K offset 16g of the step and the 16 at 64 + 16g; and the same
//     bytes of each activation row.  Loading the weight bytes that way
//     would give four neighbouring lanes four different rows, and the
//     texture addresser, not HBM, then sets the streaming rate (measured:
//     the m=1 FFN 53.6 us with such loads, 49.5 us with these).  So lane s
//     loads 16 bytes at 16(s%4) (and 64 + 16(s%4)) of row s/4 -- four
//     lanes cover 64 contiguous bytes -- and a ds_bpermute hands lane
//     (c, g) the registers of lane 4c + g.  Activation rows are loaded the
//     same way (loaded in the operand layout they cost 14% at 512 rows:
//     FFN 394 -> 339 us, 93.5 -> 89.7 us at 64 rows).
//     The hardware FP8 -> fp16 conversion
//     (exact: an E4M3 value has 4 significant bits and lies in
//     [2^-9, 448]) turns them into four operand fragments of
//     v_mfma_f32_16x16x32_f16, whose products are exact and whose sums are
//     fp32; P_b is the sum of the four.
//     The FP8 matrix-core forms (v_mfma_scale_f32_16x16x128_f8f6f4,
//     v_mfma_f32_16x16x32_fp8_fp8) take the bytes directly but do not keep
//     every product: measured on this part, inside one group of eight
//     products a term 2^18 or more below the group's largest is dropped
//     (448*448 + 1 gives 448*448, 1 + 2^-18 gives 1), while the fp16 form
//     returns both sums exactly.  So the products here are exact and only
//     the fp32 sums round, as for the NVFP4 paths.
//   * acc = fma(scale_b, P_b, acc) per step, in the wave's step order; waves
//     reduce through LDS in fixed wave order; with ksplit > 1 the last
//     workgroup of a tile to arrive sums the fp32 partials in split order.
//   * Epilogue: times s_row, bf16 (or silu(bf16 g) * bf16 u for NMAT = 2).
// Buffer loads return zero outside a resource's range, so ragged rows,
// columns and K need no branches.
#include "launchers.h"
#include "nvfp4_common.h"

namespace nvfp4 {

namespace {

constexpr int kNW = 4;  // waves per workgroup


struct W8Args {
  const uint8_t *xc;  // E4M3 [m][k]
  const float *xr;    // [m]
  int m, k, n;
  const uint8_t *codes0, *codes1;  // E4M3 [n][k]
  const float *scales0, *scales1;  // [ceil(n/128)][ceil(k/128)]
  void *y;
  float *partial;      // [tiles * row blocks][NMAT][ksplit][CTW][16*MT][16]
  unsigned *counters;  // [row blocks][column blocks], zero between calls
  int ksplit, steps_per_split;
};

template <int MT, int NMAT, int CTW>
struct W8Cfg {
  static constexpr int kRegsPerStep = (NMAT * CTW + MT) * 8;
  // steps whose loads are issued together; the largest tiles take one, which
  // keeps them at two waves per SIMD (measured: m = 64 FFN 127 -> 102 us)
  static constexpr int U = kRegsPerStep * 4 <= 128 ? 4 : (kRegsPerStep * 2 < 128 ? 2 : 1);
};

// the four fragments of a lane's 32 bytes (q0 = K offsets 16g.., q1 =
// 64 + 16g..): fragment j covers bytes 8j..8j+7 of q0 then q1, so MFMA j of
// a step sums the 32 K offsets 16g' + 8j (j < 2) or 64 + 16g' + 8(j-2)
// (j >= 2), plus 0..7, over g' = 0..3
__device__ __forceinline__ void fp8x32_to_f16(const uint4 &q0, const uint4 &q1, f16x8 (&f)[4]) {
  f[0] = fp8x8_to_f16(q0.x, q0.y);
  f[1] = fp8x8_to_f16(q0.z, q0.w);
  f[2] = fp8x8_to_f16(q1.x, q1.y);
  f[3] = fp8x8_to_f16(q1.z, q1.w);
}

template <int MT, int NMAT, int CTW>
__global__ __launch_bounds__(kNW * 64) void k_w8a8(W8Args p) {
  constexpr int U = W8Cfg<MT, NMAT, CTW>::U;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c16 = lane & 15;
  const int g = lane >> 4;
  const int src_addr = load_layout_src_addr(lane);
  const uint32_t wrow = (uint32_t)(lane >> 2);    // weight row this lane loads
  const int k = p.k;
  // One-dimensional grid over (row block, split, column block), row block
  // fastest.  Workgroups go to the eight XCDs in turn (workgroup L to XCD
  // L mod 8); each XCD gets one contiguous range of that order, so the row
  // blocks that read the same weight columns run together behind one L2
  // and the weights leave HBM about once, not once per 64-row block.
  const int nrb = cdiv(p.m, 64);
  const int ncb = cdiv(p.n, 16 * CTW);
  const int q = (int)(gridDim.x >> 3), rem = (int)(gridDim.x & 7), xcd = (int)(blockIdx.x & 7);
  const int u = xcd * q + min(xcd, rem) + (int)(blockIdx.x >> 3);
  const int rb = u % nrb;
  const int split = (u / nrb) % p.ksplit;
  const int cb = u / (nrb * p.ksplit);
  const int col0 = cb * (16 * CTW);
  const int row0 = rb * 64;
  const int nsteps = (k + 127) >> 7;  // = scale blocks along K
  const int s_begin = split * p.steps_per_split;
  const int s_end = min(nsteps, s_begin + p.steps_per_split);
  const int nbn = (p.n + 127) >> 7;   // scale blocks along N

  const int ncols = min(16 * CTW, p.n - col0);
  const int nrows = min(64, p.m - row0);
  __amdgpu_buffer_rsrc_t wc[NMAT];
  const float *wsc[NMAT];
  wc[0] = rsrc(p.codes0 + (size_t)col0 * k, (size_t)ncols * k);
  wsc[0] = p.scales0;
  if constexpr (NMAT > 1) {
    wc[1] = rsrc(p.codes1 + (size_t)col0 * k, (size_t)ncols * k);
    wsc[1] = p.scales1;
  }
  const __amdgpu_buffer_rsrc_t ax = rsrc(p.xc + (size_t)row0 * k, (size_t)nrows * k);

  f32x4 acc[NMAT][CTW][MT];
#pragma unroll
  for (int i = 0; i < NMAT; ++i)
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[i][ct][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  // one step's bytes and block scales
  struct Step {
    uint4 bw[NMAT][CTW][2];
    uint4 aw[MT][2];
    float sc[NMAT][CTW];
  };
  auto load = [&](int t, Step &b) {
    // K offsets of this lane's 16-byte loads (load layout, weights and
    // activations alike); each half is checked on its own (k is only a
    // multiple of 32, so the second 64 bytes of the last step can lie past k)
    const bool in_split = t < s_end;
    const uint32_t kw = (uint32_t)t * 128u + 16u * (uint32_t)(lane & 3);
    const bool okw0 = in_split && kw < (uint32_t)k, okw1 = in_split && kw + 64u < (uint32_t)k;
#pragma unroll
    for (int i = 0; i < NMAT; ++i)
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct) {
        const uint32_t roff = (uint32_t)(ct * 16) + wrow;
        // cached loads: the non-temporal hint let lines go before every
        // lane of a line had read it (FETCH_SIZE of the m=1 gate+up launch
        // 1.35x its algorithmic bytes with the hint, 1.11x without)
        b.bw[i][ct][0] = ld16(wc[i], okw0 ? roff * (uint32_t)k + kw : kOOB);
        b.bw[i][ct][1] = ld16(wc[i], okw1 ? roff * (uint32_t)k + kw + 64u : kOOB);
        // the tile's 16 columns share one scale row (col0 + 16 ct is a
        // multiple of 16, blocks are 128 wide); steps past the end read
        // block 0 and multiply zeros
        const int tb = t < s_end ? t : 0;
        const int cbs = min((col0 + ct * 16) >> 7, nbn - 1);  // a tile past n: any valid row
        b.sc[i][ct] = wsc[i][(size_t)cbs * nsteps + tb];
      }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      // activations in the weights' load layout too (row wrow, K offsets kw)
      const uint32_t roff = (uint32_t)(mt * 16 + (int)wrow) * (uint32_t)k;
      b.aw[mt][0] = ld16(ax, okw0 ? roff + kw : kOOB);
      b.aw[mt][1] = ld16(ax, okw1 ? roff + kw + 64u : kOOB);
    }
  };
  // P_b = the step's four MFMAs from zero, then acc = fma(scale_b, P_b, acc)
  auto compute = [&](const Step &b) {
    f16x8 bf[NMAT][CTW][4];
#pragma unroll
    for (int i = 0; i < NMAT; ++i)
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct)
        fp8x32_to_f16(from_load_layout(b.bw[i][ct][0], src_addr), from_load_layout(b.bw[i][ct][1], src_addr),
                      bf[i][ct]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f16x8 af[4];
      fp8x32_to_f16(from_load_layout(b.aw[mt][0], src_addr), from_load_layout(b.aw[mt][1], src_addr), af);
#pragma unroll
      for (int i = 0; i < NMAT; ++i)
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
          f32x4 pb = zero;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            pb = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[j], bf[i][ct][j], pb, 0, 0, 0);
          const float sv = b.sc[i][ct];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][ct][mt][e] = __builtin_fmaf(sv, pb[e], acc[i][ct][mt][e]);
        }
    }
  };

  for (int base = s_begin + wave; base < s_end; base += kNW * U) {
    Step st[U];
#pragma unroll
    for (int u = 0; u < U; ++u) load(base + u * kNW, st[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) compute(st[u]);
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
    const size_t wg = (size_t)rb * ncb + cb;
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
            st_coherent(pres, poff(i, split, ct, mt, e), acc[i][ct][mt][e]);
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
        const float rs = p.xr[r];
        const float v0 = acc[0][ct][mt][e] * rs;
        __bf16 out;
        if constexpr (NMAT > 1)
          out = swiglu_bf16(v0, acc[NMAT - 1][ct][mt][e] * rs);
        else
          out = (__bf16)v0;
        ((__bf16 *)p.y)[(size_t)r * p.n + col] = out;
      }
  }
}

template <int MT, int NMAT, int CTW>
hipError_t launch_one(const W8Args &p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((k_w8a8<MT, NMAT, CTW>), grid, dim3(kNW * 64), 0, s, p);
  return hipGetLastError();
}

template <int NMAT, int CTW>
hipError_t launch_mt(const W8Args &p, int mt, dim3 grid, hipStream_t s) {
  if constexpr (CTW == 4) return launch_one<4, NMAT, CTW>(p, grid, s);
  switch (mt) {
    case 1: return launch_one<1, NMAT, CTW>(p, grid, s);
    case 2: return launch_one<2, NMAT, CTW>(p, grid, s);
    case 3: return launch_one<3, NMAT, CTW>(p, grid, s);
    default: return launch_one<4, NMAT, CTW>(p, grid, s);
  }
}

}  // namespace

// Column tiles per workgroup: two, so each activation fragment (loaded and
// converted once per step) feeds twice as many MFMAs; a function of n only,
// like the K split, so every row count runs the same K order.
int w8a8_ctw(int n) { return n > 16 ? 2 : 1; }

StreamPlan w8a8_plan(int n, int k) {
  constexpr int kTarget = 256;  // workgroups before K is split (fewer splits: less partial traffic)
  const int tiles = cdiv(n, 16 * w8a8_ctw(n));
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

// Column tiles per launched workgroup: w8a8_ctw(n), or four for a single
// matrix beyond 64 rows (each converted fragment then feeds four MFMAs).
// The K plan stays that of w8a8_ctw(n) column tiles, so the K order of every
// output does not change.
static int w8a8_launch_ctw(int nmat, int m, int n) { return nmat == 1 && m > 64 ? 4 : w8a8_ctw(n); }

size_t w8a8_partial_floats(const StreamPlan &pl, int nmat, int m, int n) {
  // per workgroup: [nmat][ksplit][CTW][16*MT][16], at most nmat*ksplit
  // floats per element of the output padded to whole row and column blocks
  if (pl.ksplit <= 1) return 0;
  const size_t rows = m >= 64 ? (size_t)64 * cdiv(m, 64) : (size_t)16 * cdiv(m, 16);
  const int ctw = w8a8_launch_ctw(nmat, m, n);
  const size_t own = (size_t)nmat * pl.ksplit * rows * 16 * ctw * cdiv(n, 16 * ctw);
  const size_t many = fixed_tall_partial_floats(true, nmat, m, n, pl.ksplit);
  return own > many ? own : many;
}

hipError_t launch_w8a8(const Fp8ActRef &a, int m, int k, int n, int nmat, const Fp8MatRef *w, void *y,
                       float *partial, unsigned *counters, const StreamPlan &pl, hipStream_t stream) {
  W8Args p{};
  p.xc = a.codes;
  p.xr = a.row_scale;
  p.m = m;
  p.k = k;
  p.n = n;
  p.codes0 = w[0].codes;
  p.scales0 = w[0].scales;
  p.codes1 = nmat > 1 ? w[1].codes : nullptr;
  p.scales1 = nmat > 1 ? w[1].scales : nullptr;
  p.y = y;
  p.partial = partial;
  p.counters = counters;
  p.ksplit = pl.ksplit;
  p.steps_per_split = pl.steps_per_split;
  if (fixed_tall_eligible(m) && a.tiles) return launch_fixed_tall_w8a8(a, m, k, n, nmat, w, y, partial, counters, pl, stream);
  const int mt = m >= 64 ? 4 : cdiv(m, 16);
  const int ctw = w8a8_launch_ctw(nmat, m, n);
  dim3 grid(cdiv(n, 16 * ctw) * pl.ksplit * cdiv(m, 64));
  if (ctw == 4)
    return nmat == 1 ? launch_mt<1, 4>(p, mt, grid, stream) : hipErrorInvalidValue;
  if (ctw == 2)
    return nmat == 1 ? launch_mt<1, 2>(p, mt, grid, stream) : launch_mt<2, 2>(p, mt, grid, stream);
  return nmat == 1 ? launch_mt<1, 1>(p, mt, grid, stream) : launch_mt<2, 1>(p, mt, grid, stream);
}

}  // namespace nvfp4
