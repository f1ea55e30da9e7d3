// k_stream.hip -- weight-streaming NVFP4 projection for few rows (gfx950).
//
// Regime: the page layers/dense_ffn_prefill.rs (`w4a16_prefill_gemm`) runs
// a dedicated small-m path for up to 64 rows; with so few rows the FFN is
// bound by streaming the 4.5-bit weights from HBM once.
//
// Work decomposition
//   * A workgroup owns CTW column tiles of 16 output columns (for each of
//     NMAT weight matrices: 1, or 2 for gate+up with a fused silu epilogue)
//     and a range of K; its 4 waves split that range into interleaved
//     128-element steps.
//   * In one step, lane (c = lane%16, g = lane/16) needs 16 bytes of codes
//     (32 K elements of weight row col0+c at K offset 32g) and their 2 scale
//     bytes; per column tile a wave covers 16 rows x 64 contiguous bytes.
//     The loads (one 128-bit, one 16-bit) are issued in the row-contiguous
//     layout -- lane s reads row s/4, piece s%4, so four neighbouring lanes
//     read one 64-byte run -- and ds_bpermute moves each piece to lane
//     (c, g); the bytes a lane ends with are the same.  Buffer loads return
//     zero outside the resource's range, so ragged columns, rows and K need
//     no branches.  The codes are dequantized in registers to four B
//     fragments of v_mfma_f32_16x16x32_bf16 (bf16 activations), or of
//     v_mfma_f32_16x16x32_f16 for W4A4, where both operands are NVFP4 and
//     exact in fp16 (one conversion and one packed multiply per pair instead
//     of four operations); the MFMA's K order inside a step is (g, element),
//     and the activation fragment uses the same order.
//   * The activation fragment of row r is the 32 contiguous K values at the
//     same offset (bf16, 64 bytes), or for W4A4 the row's NVFP4 codes
//     dequantized exactly like the weight (fp16); one fragment feeds
//     CTW*NMAT MFMAs.  Activation rows are loaded in the same row-contiguous
//     layout and permuted the same way.
//   * Waves reduce through LDS in fixed wave order.  With ksplit > 1 each
//     workgroup writes its fp32 partial tile; the last workgroup of a tile to
//     finish (a self-resetting arrival counter) sums the partials in split
//     order and runs the epilogue.  The K order of every output therefore
//     depends only on (n, k), never on m or on arrival order -- the property
//     the W4A4 arm needs.
//   * Up to 64 rows (MT tiles of 16) share each dequantized weight fragment;
//     more rows use more row blocks (grid.z).
//   * NVFP4 activations from 17 rows on take k_stream_tall: the same
//     per-output schedule, fed by a two-stage load pipeline, with two column
//     tiles per workgroup (four for a single matrix beyond 64 rows) and an
//     XCD-aware workgroup order.  Since every output sees the same steps,
//     waves, MFMA sequence and reduction order, the fixed format's rows keep
//     their bits at every row count.
#include <type_traits>

#include "launchers.h"
#include "nvfp4_common.h"

namespace nvfp4 {

namespace {

constexpr int kNW = 4;  // waves per workgroup (K split inside it)
constexpr int kTargetBlocks = 512;
// k_stream_tall: column tiles per workgroup (two; four for one matrix
// beyond 64 rows, so every wave holds 4 x 4 accumulator tiles and each
// dequantized fragment feeds four MFMAs) and row tiles per block beyond 64 rows
constexpr int kTallCtw = 2;
constexpr int kTallCtwWide = 4;
constexpr int kTallRowTiles = 4;
constexpr int kTallMinRows = 17;  // NVFP4 activations with this many rows take k_stream_tall

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
  float *partial;         // per workgroup tile [nmat][ksplit][CTW][16*MT rows][16 columns]
  unsigned *counters;     // [row blocks][column blocks], zero between calls
  int ksplit, steps_per_split;
};


template <int MT, int NMAT, int CTW, bool AFP4>
struct Cfg {
  static constexpr int kRegsPerStep = NMAT * CTW * 5 + MT * (AFP4 ? 5 : 16);
  static constexpr int U = kRegsPerStep * 8 <= 128 ? 8 : (kRegsPerStep * 4 <= 128 ? 4 : 2);
};

// The workgroup's end: reduce the waves' accumulators in wave order, with
// ksplit > 1 hand the tile to the last-arriving split (partials summed in
// split order), then the epilogue.  Shared by both kernels below, so a tile's
// result depends only on its accumulators, never on which kernel made them.
template <int MT, int NMAT, int CTW, bool AFP4>
__device__ __forceinline__ void stream_finish(const StreamArgs &p, f32x4 (&acc)[NMAT][CTW][MT], int lane,
                                              int wave, int col0, int row0, int tile, int split) {
  const int c16 = lane & 15;
  const int g = lane >> 4;
  // fixed-order reduction over the workgroup's waves, one (matrix, tile)
  // pair at a time to bound LDS
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
    // this workgroup's partial tiles: [NMAT][ksplit][CTW][16*MT rows][16 columns]
    constexpr int kTile = 16 * MT * 16;
    const size_t wg = (size_t)tile;
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
    // split order outermost; all of one split's loads are in flight together
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
        float v0 = acc[0][ct][mt][e];
        float v1 = acc[NMAT - 1][ct][mt][e];
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
}

template <int MT, int NMAT, int CTW, bool AFP4>
__global__ __launch_bounds__(kNW * 64) void k_stream(StreamArgs p) {
  constexpr int U = Cfg<MT, NMAT, CTW, AFP4>::U;
  // MFMA operand type: fp16 when both operands are NVFP4 (exact either way,
  // half the conversion work), bf16 for bf16 activations
  using Frag = std::conditional_t<AFP4, f16x8, bf16x8>;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int src_addr = load_layout_src_addr(lane);
  const uint32_t lrow = (uint32_t)(lane >> 2), lpiece = (uint32_t)(lane & 3);  // load layout
  const int k = p.k;
  const int col0 = blockIdx.x * (16 * CTW);
  const int row0 = blockIdx.z * (16 * MT);  // row blocks of 16 MT rows
  const int nsteps = (k + 127) >> 7;
  const int s_begin = blockIdx.y * p.steps_per_split;
  const int s_end = min(nsteps, s_begin + p.steps_per_split);
  const uint32_t kb2 = (uint32_t)k >> 1, kb16 = (uint32_t)k >> 4;

  // resources cover exactly this workgroup's weight rows and activation rows
  const int ncols = min(16 * CTW, p.n - col0);
  const int nrows = min(16 * MT, p.m - row0);
  __amdgpu_buffer_rsrc_t wc[NMAT], ws[NMAT];
  wc[0] = rsrc(p.codes0 + (size_t)col0 * kb2, (size_t)ncols * kb2);
  ws[0] = rsrc(p.scales0 + (size_t)col0 * kb16, (size_t)ncols * kb16);
  if constexpr (NMAT > 1) {
    wc[1] = rsrc(p.codes1 + (size_t)col0 * kb2, (size_t)ncols * kb2);
    ws[1] = rsrc(p.scales1 + (size_t)col0 * kb16, (size_t)ncols * kb16);
  }
  __amdgpu_buffer_rsrc_t ax, axs;
  if constexpr (AFP4) {
    ax = rsrc(p.xc + (size_t)row0 * kb2, (size_t)nrows * kb2);
    axs = rsrc(p.xs + (size_t)row0 * kb16, (size_t)nrows * kb16);
  } else {
    ax = rsrc((const uint16_t *)p.x + (size_t)row0 * k, (size_t)nrows * k * 2);
    axs = ax;
  }

  f32x4 acc[NMAT][CTW][MT];
#pragma unroll
  for (int i = 0; i < NMAT; ++i)
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[i][ct][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int base = s_begin + wave; base < s_end; base += kNW * U) {
    uint4 bw[U][NMAT][CTW];
    uint32_t bsc[U][NMAT][CTW];
    uint4 aw[U][MT][AFP4 ? 1 : 4];
    uint32_t asc[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = base + u * kNW;
      const uint32_t kl = (uint32_t)t * 128u + 32u * lpiece;  // K of this lane's loads
      const bool okl = t < s_end && kl < (uint32_t)k;
#pragma unroll
      for (int i = 0; i < NMAT; ++i)
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
          const uint32_t row = (uint32_t)(ct * 16) + lrow;
          bw[u][i][ct] = ld16(wc[i], okl ? row * kb2 + (kl >> 1) : kOOB);
          bsc[u][i][ct] = ld2(ws[i], okl ? row * kb16 + (kl >> 4) : kOOB);
        }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        // activation rows in the same row-contiguous layout as the weights
        const uint32_t r = (uint32_t)(mt * 16) + lrow;
        if constexpr (AFP4) {
          aw[u][mt][0] = ld16(ax, okl ? r * kb2 + (kl >> 1) : kOOB);
          asc[u][mt] = ld2(axs, okl ? r * kb16 + (kl >> 4) : kOOB);
        } else {
          const uint32_t off = okl ? (r * (uint32_t)k + kl) * 2u : kOOB;
#pragma unroll
          for (int q = 0; q < 4; ++q) aw[u][mt][q] = ld16(ax, off + 16u * q);
          asc[u][mt] = 0;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      Frag bf[NMAT][CTW][4];
#pragma unroll
      for (int i = 0; i < NMAT; ++i)
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
          const uint4 w = from_load_layout(bw[u][i][ct], src_addr);
          const uint32_t sc = from_load_layout(bsc[u][i][ct], src_addr);
          if constexpr (AFP4) {
            const f16x2 s01 = e4m3x2_to_f16x2(sc);
            bf[i][ct][0] = dequant8_f16(w.x, s01[0]);
            bf[i][ct][1] = dequant8_f16(w.y, s01[0]);
            bf[i][ct][2] = dequant8_f16(w.z, s01[1]);
            bf[i][ct][3] = dequant8_f16(w.w, s01[1]);
          } else {
            const float s0 = e4m3_to_f32_sel<0>(sc);
            const float s1 = e4m3_to_f32_sel<1>(sc);
            bf[i][ct][0] = dequant8(w.x, s0);
            bf[i][ct][1] = dequant8(w.y, s0);
            bf[i][ct][2] = dequant8(w.z, s1);
            bf[i][ct][3] = dequant8(w.w, s1);
          }
        }
      // the activations' operand bytes (W4A16 FFN m=16 43.5 -> 39.6 us, W4A4
      // m=16 49.2 -> 47.2 us against loading them in the operand layout)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        asc[u][mt] = AFP4 ? from_load_layout(asc[u][mt], src_addr) : 0u;
#pragma unroll
        for (int q = 0; q < (AFP4 ? 1 : 4); ++q) aw[u][mt][q] = from_load_layout(aw[u][mt][q], src_addr);
      }
      // K sub-step outermost: consecutive MFMAs update different
      // accumulators.  An activation fragment is formed just before its
      // MFMAs (NVFP4 rows dequantized exactly like the weight).
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          Frag af;
          if constexpr (AFP4) {
            const f16x2 sa = e4m3x2_to_f16x2(asc[u][mt]);
            const uint32_t word = j == 0 ? aw[u][mt][0].x : j == 1 ? aw[u][mt][0].y
                                : j == 2 ? aw[u][mt][0].z : aw[u][mt][0].w;
            af = dequant8_f16(word, sa[j >> 1]);
          } else {
            af = as_bf16x8(aw[u][mt][j]);
          }
#pragma unroll
          for (int i = 0; i < NMAT; ++i)
#pragma unroll
            for (int ct = 0; ct < CTW; ++ct) {
              if constexpr (AFP4)
                acc[i][ct][mt] =
                    __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[i][ct][j], acc[i][ct][mt], 0, 0, 0);
              else
                acc[i][ct][mt] =
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[i][ct][j], acc[i][ct][mt], 0, 0, 0);
            }
        }
    }
  }

  stream_finish<MT, NMAT, CTW, AFP4>(p, acc, lane, wave, col0, row0, blockIdx.z * gridDim.x + blockIdx.x,
                                     blockIdx.y);
}

// Row-block variant for NVFP4 activations beyond 16 rows.  The same
// workgroup shape, wave-to-step assignment, MFMA sequence per accumulator
// and tail as k_stream<MT, NMAT, CTW, true>, so every output element gets the
// same bits; what changes is how the steps are fed.  With up to 128 rows per
// block a wave's registers cannot hold several steps in flight, so each wave
// runs a two-stage pipeline: the loads of its next step are issued before the
// current step is dequantized and multiplied, and only one step's raw bytes
// wait in registers.  Activation fragments are formed one (row tile, K
// sub-step) at a time and weight fragments one K sub-step at a time.
template <int MT, int NMAT, int CTW, int NS>
__global__ __launch_bounds__(kNW * 64) void k_stream_tall(StreamArgs p) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int src_addr = load_layout_src_addr(lane);
  const uint32_t lrow = (uint32_t)(lane >> 2), lpiece = (uint32_t)(lane & 3);
  const int k = p.k;
  // One-dimensional grid over (row block, split, column block), row block
  // fastest.  Workgroups go to the eight XCDs in turn (workgroup L to XCD
  // L mod 8); each XCD gets one contiguous range of that order, so the row
  // blocks that share a weight tile run together behind one L2.
  const int nrb = cdiv(p.m, 16 * MT);
  const int q = (int)(gridDim.x >> 3), rem = (int)(gridDim.x & 7), xcd = (int)(blockIdx.x & 7);
  const int u = xcd * q + min(xcd, rem) + (int)(blockIdx.x >> 3);
  const int rb = u % nrb;
  const int split = (u / nrb) % p.ksplit;
  const int cb = u / (nrb * p.ksplit);
  const int col0 = cb * (16 * CTW);
  const int row0 = rb * (16 * MT);
  const int nsteps = (k + 127) >> 7;
  const int s_begin = split * p.steps_per_split;
  const int s_end = min(nsteps, s_begin + p.steps_per_split);
  const uint32_t kb2 = (uint32_t)k >> 1, kb16 = (uint32_t)k >> 4;

  const int ncols = min(16 * CTW, p.n - col0);
  const int nrows = min(16 * MT, p.m - row0);
  __amdgpu_buffer_rsrc_t wc[NMAT], ws[NMAT];
  wc[0] = rsrc(p.codes0 + (size_t)col0 * kb2, (size_t)ncols * kb2);
  ws[0] = rsrc(p.scales0 + (size_t)col0 * kb16, (size_t)ncols * kb16);
  if constexpr (NMAT > 1) {
    wc[1] = rsrc(p.codes1 + (size_t)col0 * kb2, (size_t)ncols * kb2);
    ws[1] = rsrc(p.scales1 + (size_t)col0 * kb16, (size_t)ncols * kb16);
  }
  const __amdgpu_buffer_rsrc_t ax = rsrc(p.xc + (size_t)row0 * kb2, (size_t)nrows * kb2);
  const __amdgpu_buffer_rsrc_t axs = rsrc(p.xs + (size_t)row0 * kb16, (size_t)nrows * kb16);

  // one step's raw bytes, weights and activations both in the row-contiguous
  // load layout (lane s: row s/4, the 16 bytes at K 32 (s%4) of the step);
  // ds_bpermute hands lane (c, g) its operand bytes.  Loading the
  // activations in the operand layout instead (lane (c, g) reading row c
  // directly, four neighbouring lanes on four rows) cost 11% at 512 rows
  // (W4A4 FFN 340 -> 302 us with the permute), as it did for the weights.
  struct Step {
    uint4 bw[NMAT][CTW];
    uint32_t bsc[NMAT][CTW];
    uint4 aw[MT];
    uint32_t asc[MT];
  };
  auto load = [&](int t, Step &b) {
    const uint32_t kl = (uint32_t)t * 128u + 32u * lpiece;
    const bool okl = t < s_end && kl < (uint32_t)k;
#pragma unroll
    for (int i = 0; i < NMAT; ++i)
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct) {
        const uint32_t row = (uint32_t)(ct * 16) + lrow;
        b.bw[i][ct] = ld16(wc[i], okl ? row * kb2 + (kl >> 1) : kOOB);
        b.bsc[i][ct] = ld2(ws[i], okl ? row * kb16 + (kl >> 4) : kOOB);
      }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint32_t r = (uint32_t)(mt * 16) + lrow;
      b.aw[mt] = ld16(ax, okl ? r * kb2 + (kl >> 1) : kOOB);
      b.asc[mt] = ld2(axs, okl ? r * kb16 + (kl >> 4) : kOOB);
    }
  };

  f32x4 acc[NMAT][CTW][MT];
#pragma unroll
  for (int i = 0; i < NMAT; ++i)
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[i][ct][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Step &b) {
    uint4 w[NMAT][CTW];
    f16x2 wsc[NMAT][CTW];
#pragma unroll
    for (int i = 0; i < NMAT; ++i)
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct) {
        w[i][ct] = from_load_layout(b.bw[i][ct], src_addr);
        wsc[i][ct] = e4m3x2_to_f16x2(from_load_layout(b.bsc[i][ct], src_addr));
      }
    f16x2 asc[MT];
    uint4 aw[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      asc[mt] = e4m3x2_to_f16x2(from_load_layout(b.asc[mt], src_addr));
      aw[mt] = from_load_layout(b.aw[mt], src_addr);
    }
    // K sub-step outermost, as in k_stream
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f16x8 bf[NMAT][CTW];
#pragma unroll
      for (int i = 0; i < NMAT; ++i)
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
          const uint32_t word = j == 0 ? w[i][ct].x : j == 1 ? w[i][ct].y : j == 2 ? w[i][ct].z : w[i][ct].w;
          bf[i][ct] = dequant8_f16(word, wsc[i][ct][j >> 1]);
        }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint32_t word = j == 0 ? aw[mt].x : j == 1 ? aw[mt].y : j == 2 ? aw[mt].z : aw[mt].w;
        const f16x8 af = dequant8_f16(word, asc[mt][j >> 1]);
#pragma unroll
        for (int i = 0; i < NMAT; ++i)
#pragma unroll
          for (int ct = 0; ct < CTW; ++ct)
            acc[i][ct][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[i][ct], acc[i][ct][mt], 0, 0, 0);
      }
    }
  };

  // wave w takes steps s_begin + w, s_begin + w + 4, ... in increasing
  // order, NS - 1 of them in flight ahead of the one being computed.  The
  // loop body is one basic block (NS times: the loads of a later step, then
  // the current step's arithmetic), so each step waits only for its own
  // loads; loads past the wave's last step are out of range and fetch
  // nothing.
  const int first = s_begin + wave;
  const int nmine = first < s_end ? (s_end - first + kNW - 1) / kNW : 0;
  Step buf[NS];
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) load(first + s * kNW, buf[s]);
  int i = 0;
  for (int t = first; i + NS <= nmine; i += NS, t += NS * kNW) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      // the barriers keep the scheduler from sinking a step's loads into
      // the arithmetic that they are meant to overlap
      load(t + (s + NS - 1) * kNW, buf[(s + NS - 1) % NS]);
      __builtin_amdgcn_sched_barrier(0);
      compute(buf[s]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // the last nmine - i (< NS) steps are already loaded, in buf[0..]
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < nmine - i) compute(buf[s]);

  stream_finish<MT, NMAT, CTW, true>(p, acc, lane, wave, col0, row0, rb * cdiv(p.n, 16 * CTW) + cb, split);
}

// load stages of k_stream_tall: two.  Three or four stages (the single-matrix
// tiles stay at two waves per SIMD with four) measured no faster at 32, 64 or
// 512 rows; three on the gate+up tiles cost the second wave per SIMD.
template <int MT, int NMAT, int CTW>
constexpr int tall_stages() {
  return 2;
}

template <int MT, int NMAT, int CTW>
hipError_t launch_tall(const StreamArgs &p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((k_stream_tall<MT, NMAT, CTW, tall_stages<MT, NMAT, CTW>()>), grid, dim3(kNW * 64), 0, s,
                     p);
  return hipGetLastError();
}

int tall_ctw(int nmat, int m) { return nmat == 1 && m > 64 ? kTallCtwWide : kTallCtw; }

template <int NMAT>
hipError_t launch_tall_mt(const StreamArgs &p, int mt, int ctw, dim3 grid, hipStream_t s) {
  if (ctw == kTallCtwWide) {
    if constexpr (NMAT == 1) return launch_tall<kTallRowTiles, 1, kTallCtwWide>(p, grid, s);
    return hipErrorInvalidValue;
  }
  switch (mt) {
    case 2: return launch_tall<2, NMAT, kTallCtw>(p, grid, s);
    case 3: return launch_tall<3, NMAT, kTallCtw>(p, grid, s);
    case 4: return launch_tall<4, NMAT, kTallCtw>(p, grid, s);
    default: return launch_tall<kTallRowTiles, NMAT, kTallCtw>(p, grid, s);
  }
}

template <int MT, int NMAT, int CTW, bool AFP4>
hipError_t launch_one(const StreamArgs &p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((k_stream<MT, NMAT, CTW, AFP4>), grid, dim3(kNW * 64), 0, s, p);
  return hipGetLastError();
}

template <int NMAT, int CTW, bool AFP4>
hipError_t launch_mt(const StreamArgs &p, int mt, dim3 grid, hipStream_t s) {
  switch (mt) {
    case 1: return launch_one<1, NMAT, CTW, AFP4>(p, grid, s);
    case 2: return launch_one<2, NMAT, CTW, AFP4>(p, grid, s);
    case 3: return launch_one<3, NMAT, CTW, AFP4>(p, grid, s);
    default: return launch_one<4, NMAT, CTW, AFP4>(p, grid, s);
  }
}

}  // namespace

int stream_ctw(int n) { return n >= 16 * 2 * kTargetBlocks ? 2 : 1; }

StreamPlan stream_plan(int n, int k) {
  // The split depends on (n, k) only: one projection shape reduces in the
  // same order at every row count.
  const int tiles = cdiv(n, 16 * stream_ctw(n));
  const int nsteps = cdiv(k, 128);
  int ksplit = 1;
  if (tiles < kTargetBlocks) {
    const int want = cdiv(kTargetBlocks, tiles);
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

size_t stream_partial_floats(const StreamPlan &pl, int nmat, int m, int n) {
  // per workgroup [nmat][ksplit][CTW][16*MT][16]: nmat*ksplit floats per
  // element of the output padded to whole row blocks (16*MT rows) and whole
  // workgroup columns, for either kernel
  if (pl.ksplit <= 1) return 0;
  const size_t rows_tall = (size_t)16 * kTallRowTiles * cdiv(m, 16 * kTallRowTiles);
  const size_t rows = m <= 64 ? (size_t)16 * cdiv(m, 16)
                              : (rows_tall > (size_t)64 * cdiv(m, 64) ? rows_tall : (size_t)64 * cdiv(m, 64));
  const size_t cols_stream = (size_t)pl.tiles * 16 * stream_ctw(n);
  const size_t cols_tall = (size_t)16 * kTallCtwWide * cdiv(n, 16 * kTallCtwWide);
  const size_t own = (size_t)nmat * pl.ksplit * rows * (cols_stream > cols_tall ? cols_stream : cols_tall);
  const size_t many = fixed_tall_partial_floats(false, nmat, m, n, pl.ksplit);
  return own > many ? own : many;
}

// (also sizes the counters of the FP8 and Q2 streaming kernels; k_stream_tall
// has no more row blocks and no more column blocks than k_stream)
size_t stream_counter_words(const StreamPlan &pl, int m) {
  return pl.ksplit > 1 ? (size_t)pl.tiles * cdiv(m, 64) : 0;
}

hipError_t launch_stream(const ActRef &a, int m, int k, int n, int nmat, const MatRef *w, void *y,
                         float *partial, unsigned *counters, const StreamPlan &pl,
                         hipStream_t stream) {
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
  p.counters = counters;
  p.ksplit = pl.ksplit;
  p.steps_per_split = pl.steps_per_split;
  const bool afp4 = a.x_bf16 == nullptr;
  if (afp4 && fixed_tall_eligible(m) && a.tiles)
    return launch_fixed_tall_w4a4(a, m, k, n, nmat, w, y, partial, counters, pl, stream);
  if (afp4 && m >= kTallMinRows) {
    const int mt = m > 64 ? kTallRowTiles : cdiv(m, 16);
    const int ctw = tall_ctw(nmat, m);
    dim3 grid(cdiv(n, 16 * ctw) * pl.ksplit * cdiv(m, 16 * mt));
    return nmat == 1 ? launch_tall_mt<1>(p, mt, ctw, grid, stream) : launch_tall_mt<2>(p, mt, ctw, grid, stream);
  }
  const int mt = m >= 64 ? 4 : cdiv(m, 16);
  const int ctw = stream_ctw(n);
  dim3 grid(pl.tiles, pl.ksplit, cdiv(m, 64));
  if (ctw == 2) {
    if (nmat == 1)
      return afp4 ? launch_mt<1, 2, true>(p, mt, grid, stream) : launch_mt<1, 2, false>(p, mt, grid, stream);
    return afp4 ? launch_mt<2, 2, true>(p, mt, grid, stream) : launch_mt<2, 2, false>(p, mt, grid, stream);
  }
  if (nmat == 1)
    return afp4 ? launch_mt<1, 1, true>(p, mt, grid, stream) : launch_mt<1, 1, false>(p, mt, grid, stream);
  return afp4 ? launch_mt<2, 1, true>(p, mt, grid, stream) : launch_mt<2, 1, false>(p, mt, grid, stream);
}

}  // namespace nvfp4
