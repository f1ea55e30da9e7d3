// k_fixed_tall.hip -- many-row fixed-format projections (W4A4 and W8A8) on
// gfx950, with the per-output K order of the streaming kernels.
//
// Regime: page layers/dense_ffn_fixed.rs (module doc; `Fixed::W4a4`,
// `Fixed::W8a8`) runs one activation format at every row count, so a row's
// result must not depend on how many rows share the call.  The streaming
// kernels (k_stream, k_stream_tall, k_w8a8) fix that order by (n, k) alone:
//   * K is cut into 128-element steps, the steps into `ksplit` contiguous
//     splits (the plans of stream_plan / w8a8_plan);
//   * inside a split the steps are dealt to four classes in turn (step
//     s_begin + c, s_begin + c + 4, ... to class c, one class per wave);
//   * a class sums its steps in increasing order from zero: W4A4 as four
//     v_mfma_f32_16x16x32_f16 per step straight into the class sum, W8A8 as
//     a block product of four MFMAs from zero folded in by one fma with the
//     block scale;
//   * the classes are added ((c0 + c1) + c2) + c3, the splits in split
//     order from zero, and the epilogue scales, rounds and (gate+up) applies
//     silu.
// Each MFMA takes the same K slots as there: lane (c, g) of the 16x16x32
// operand holds K offsets 32 g + 8 j .. + 7 of the step for sub-step j
// (W4A4), or 16 g + 8 j (j < 2) and 64 + 16 g + 8 (j - 2) (j >= 2) (W8A8),
// and row r / column n sits at position r % 16 / n % 16 of its tile.
//
// What changes is who does the work.  The streaming kernels give every
// wave its own class, so no operand fragment is shared: each wave decodes
// the activations of its steps for its 64 rows and its weights for its
// columns.  Here a workgroup of eight waves (two per SIMD) owns 64 or 128
// rows and 128 (gate+up) or 256 columns, and walks the classes one after
// another: class 0's steps, then class 1's, and so on.  Each wave keeps two
// accumulator sets -- the running sum of finished classes and the class in
// progress -- which is all the fixed order needs.  Per step:
//   * activations arrive already decoded: the row quantizer writes them as
//     fp16 operand tiles (exact values; layout in launchers.h), and LDS-DMA
//     copies the step's 1 KB fragments into LDS, where every wave of the
//     workgroup reads them with one linear ds_read_b128 per lane;
//   * each wave copies the raw codes of its two 16-column weight tiles into
//     LDS the same way, already in operand order (lane (c, g) of a copy
//     loads row c, 16-byte piece g (FP8: 4 h + g for half h), so each lane
//     reads its bytes back at position 16 lane), and loads their block
//     scales into registers; it decodes each weight fragment once and feeds
//     it to its 4 or 8 row tiles;
//   * three LDS stages: the copies of step i + 2 are issued before step i's
//     MFMAs, and each step ends with a wait for the copies of step i + 1 and
//     one barrier;
//   * the next sub-step's LDS reads and weight decode are interleaved with
//     the current sub-step's MFMAs.
// Buffer loads return zero outside a resource's range, so ragged rows,
// columns and K need no branches.
#include <climits>
#include <type_traits>

#include "launchers.h"
#include "nvfp4_common.h"

namespace nvfp4 {

namespace {

constexpr int kNW = 8;             // waves per workgroup (two per SIMD)
constexpr int kNC = 2;             // 16-column weight tiles per wave
constexpr int kTiles = kNW * kNC;  // weight tiles per workgroup
constexpr int kThreads = kNW * 64;
constexpr int kStages = 3;         // LDS stages

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct TallArgs {
  const uint16_t *xt;  // fp16 operand tiles of the activations
  const float *xr;     // per-row scale [m]
  int m, k, n;
  const uint8_t *codes0, *codes1;    // weight codes: NVFP4 [n][k/2] or E4M3 [n][k]
  const uint8_t *scales0, *scales1;  // NVFP4 block scales [n][k/16] (W4A4)
  const float *fscales0, *fscales1;  // FP8 block scales [ceil(n/128)][ceil(k/128)] (W8A8)
  float ts0, ts1;                    // NVFP4 tensor scales (W4A4)
  void *y;
  float *partial;      // [row block][column block][ksplit][wave][MT][kNC][64 lanes][4]
  unsigned *counters;  // [row block][column block], zero between calls
  int ksplit, steps_per_split;
};

__device__ __forceinline__ void st16_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kCoherent);
}
__device__ __forceinline__ f32x4 ld16_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherent));
}

// One 16-byte LDS read as a single vector load (a uint4 struct is read as
// four dwords that are merged late, and the merged access no longer tells
// the compiler which LDS stage it reads, so it waits for every copy in
// flight before it).
__device__ __forceinline__ uint4 lds16(const uint8_t *p) {
  const u32x4 v = *(const u32x4 *)p;
  return uint4{v.x, v.y, v.z, v.w};
}

__device__ __forceinline__ uint32_t word_of(const uint4 &v, int j) {
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// s_waitcnt with at most n vector-memory requests of this wave in flight
// (the other counters unconstrained)
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <bool FP8, int NMAT, int MT>
__global__ __launch_bounds__(kThreads) void k_fixed_tall(TallArgs p) {
  constexpr int kRows = 16 * MT;
  constexpr int kWgCols = NMAT == 2 ? 16 * kNW : 16 * kTiles;  // output columns per workgroup
  constexpr int kABytes = MT * 4 * 1024;                       // activation fragments per step
  constexpr int kBTile = FP8 ? 2048 : 1024;                    // codes of a weight tile per step
  constexpr int kWBytes = kTiles * kBTile;                     // weight codes per step
  constexpr int kADma = MT / 2;                                // 1 KB activation blocks per wave
  constexpr int kReqs = kADma + (kBTile / 1024 + 1) * kNC;     // vector-memory requests per wave and step
  static_assert(MT % 2 == 0 && (MT * 4) % kNW == 0, "activation blocks per wave");

  // activation fragments: three stages (shared by all waves); weight codes:
  // two stages (each wave reads only its own tiles, at the start of a step,
  // so the copy two steps ahead may overwrite them right after)
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[kABytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[kABytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[kABytes];
  __shared__ __attribute__((aligned(1024))) uint8_t ldsw[2][kWBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, gq = lane >> 4;
  const int k = p.k;

  // One-dimensional grid over (row block, split, column block), row block
  // fastest.  Workgroup L runs on XCD L mod 8; each XCD gets one contiguous
  // range of that order, so the row blocks that read the same weight
  // columns run together behind one L2.
  const int nrb = cdiv(p.m, kRows);
  const int ncb = cdiv(p.n, kWgCols);
  const int q = (int)(gridDim.x >> 3), rem = (int)(gridDim.x & 7), xcd = (int)(blockIdx.x & 7);
  const int u = xcd * q + min(xcd, rem) + (int)(blockIdx.x >> 3);
  const int rb = u % nrb;
  const int split = (u / nrb) % p.ksplit;
  const int cb = u / (nrb * p.ksplit);
  const int row0 = rb * kRows, col0 = cb * kWgCols;
  const int nsteps = (k + 127) >> 7;
  const int s_begin = split * p.steps_per_split;
  const int s_end = min(nsteps, s_begin + p.steps_per_split);
  const int S = s_end - s_begin;  // >= 1: no split is empty

  // steps of class c, and the step at position i of the class-by-class
  // sequence (positions past the split give a step >= s_end)
  auto class_count = [&](int c) __attribute__((always_inline)) { return S > c ? (S - c + 3) >> 2 : 0; };
  auto step_at = [&](int i) __attribute__((always_inline)) {
    int c = 0, base = 0;
    for (; c < 3; ++c) {
      const int nc = class_count(c);
      if (i < base + nc) break;
      base += nc;
    }
    return s_begin + c + 4 * (i - base);
  };

  const uint32_t kb2 = (uint32_t)k >> 1, kb16 = (uint32_t)k >> 4;
  const uint32_t wrow_bytes = FP8 ? (uint32_t)k : kb2;  // code bytes per weight row
  // this row block's operand tiles: 4 KB per (row tile, step)
  const int rtiles = min(MT, cdiv(p.m, 16) - (row0 >> 4));
  const __amdgpu_buffer_rsrc_t xtr =
      rsrc_uniform(p.xt + (size_t)(row0 >> 4) * nsteps * 2048, (size_t)rtiles * nsteps * 4096);
  __amdgpu_buffer_rsrc_t wc[NMAT], wsr[NMAT];
  const int nbn = (p.n + 127) >> 7;
  wc[0] = rsrc_uniform(p.codes0, (size_t)p.n * wrow_bytes);
  wsr[0] = FP8 ? rsrc_uniform(p.fscales0, (size_t)nbn * nsteps * 4) : rsrc_uniform(p.scales0, (size_t)p.n * kb16);
  if constexpr (NMAT == 2) {
    wc[1] = rsrc_uniform(p.codes1, (size_t)p.n * wrow_bytes);
    wsr[1] = FP8 ? rsrc_uniform(p.fscales1, (size_t)nbn * nsteps * 4) : rsrc_uniform(p.scales1, (size_t)p.n * kb16);
  }
  // weight tile ct of this wave: matrix and first column
  auto tile_mat = [&](int ct) __attribute__((always_inline)) { return NMAT == 2 ? ct : 0; };
  auto tile_col = [&](int ct) __attribute__((always_inline)) {
    return col0 + (NMAT == 2 ? 16 * wave : 32 * wave + 16 * ct);
  };
  auto stage = [&](int s) __attribute__((always_inline)) { return s == 0 ? lds0 : s == 1 ? lds1 : lds2; };

  // block scales of the wave's tiles, per LDS stage: NVFP4 the lane's scale
  // pair (row c, K 32 g of the step), FP8 the tile's block scale
  uint32_t scs[kStages][kNC];

  // ---- copies of step i: activations into stage s, weights into weight
  // stage ws (scales into register slot s) ----
  auto issue = [&](int i, int s, int ws) __attribute__((always_inline)) {
    const int t = step_at(i);
    const bool live = t < s_end;
    uint8_t *st = stage(s);
#pragma unroll
    for (int qq = 0; qq < kADma; ++qq) {
      const int b = wave * kADma + qq;  // block (row tile b / 4, sub-step b % 4)
      const uint32_t off = ((uint32_t)((b >> 2) * nsteps + t) * 4u + (uint32_t)(b & 3)) * 1024u + lane * 16u;
      dma16(xtr, st + b * 1024, live ? off : kOOB);
    }
#pragma unroll
    for (int ct = 0; ct < kNC; ++ct) {
      const int mat = tile_mat(ct);
      uint8_t *bt = ldsw[ws] + (kNC * wave + ct) * kBTile;
      if constexpr (FP8) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          // row-contiguous copy of rows 8 h .. 8 h + 7: lane l loads row
          // 8 h + l / 8, piece (l % 8) ^ (l / 8) (K 16 piece), landing at
          // 16 l of the half's 1 KB; the XOR spreads a read phase over the banks
          const uint32_t rr = (uint32_t)lane >> 3;
          const uint32_t piece = ((uint32_t)lane & 7u) ^ rr;
          const uint32_t kw = (uint32_t)t * 128u + 16u * piece;
          const bool ok = live && kw < (uint32_t)k;
          dma16(wc[mat], bt + h * 1024, ok ? (uint32_t)(tile_col(ct) + 8 * h + (int)rr) * wrow_bytes + kw : kOOB);
        }
        const int cbs = min(tile_col(ct) >> 7, nbn - 1);
        scs[s][ct] = ld4(wsr[mat], (uint32_t)(cbs * nsteps + (live ? t : 0)) * 4u);
      } else {
        // row-contiguous copy: lane l loads row l / 4, piece l % 4 (K 32 (l % 4)),
        // landing at 16 l of the tile's 1 KB region
        const uint32_t row = (uint32_t)lane >> 2;
        const uint32_t piece = (uint32_t)lane & 3u;
        const uint32_t kl = (uint32_t)t * 128u + 32u * piece;
        const bool ok = live && kl < (uint32_t)k;
        dma16(wc[mat], bt, ok ? (uint32_t)(tile_col(ct) + row) * wrow_bytes + (kl >> 1) : kOOB);
        const uint32_t ks = (uint32_t)t * 128u + 32u * gq;
        scs[s][ct] = ld2(wsr[mat], live && ks < (uint32_t)k ? (uint32_t)(tile_col(ct) + c16) * kb16 + (ks >> 4) : kOOB);
      }
    }
  };

  // ---- accumulators: finished classes (tot) and the class in progress (cur) ----
  f32x4 tot[MT][kNC], cur[MT][kNC];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ct = 0; ct < kNC; ++ct) {
      tot[mt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      cur[mt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  // the wave's weight operands of stage s, read before the copies of a later
  // step are issued (the compiler's wait for pending copies then covers
  // only the copies issued a step earlier, which have had a step to land):
  // NVFP4 lane (c, g) reads row c, piece g (position 4 c + g) of each tile
  // and its scale pair; FP8 lane (c, g) reads pieces g and 4 + g of row c
  struct WOps {
    uint4 w[kNC][FP8 ? 2 : 1];
    uint32_t sc[kNC];
  };
  auto read_w = [&](int s, int ws, WOps &wo) __attribute__((always_inline)) {
    const uint8_t *sbw = ldsw[ws] + kNC * wave * kBTile;
#pragma unroll
    for (int ct = 0; ct < kNC; ++ct) {
      if constexpr (FP8) {
        const int r7 = c16 & 7;
        const uint8_t *half = sbw + ct * kBTile + (c16 >> 3) * 1024 + 128 * r7;
        wo.w[ct][0] = lds16(half + 16 * (gq ^ r7));
        wo.w[ct][1] = lds16(half + 16 * ((4 + gq) ^ r7));
      } else {
        wo.w[ct][0] = lds16(sbw + ct * kBTile + 16 * (4 * c16 + gq));
      }
      wo.sc[ct] = scs[s][ct];
    }
  };

  auto compute = [&](int s, const WOps &wo) __attribute__((always_inline)) {
    const uint8_t *sa = stage(s);
    auto aread = [&](int j, f16x8 (&a)[MT]) __attribute__((always_inline)) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) a[mt] = *(const f16x8 *)(sa + (mt * 4 + j) * 1024 + lane * 16);
    };
    f16x8 af[2][MT];
    if constexpr (FP8) {
      // fragment j of the lane's weight bytes: q0 bytes 8 j.. (j < 2), q1
      // bytes 8 (j - 2).. (j >= 2)
      auto bdec8 = [&](int j, f16x8 (&b)[kNC]) __attribute__((always_inline)) {
#pragma unroll
        for (int ct = 0; ct < kNC; ++ct) {
          const uint4 &q = wo.w[ct][j >> 1];
          b[ct] = (j & 1) ? fp8x8_to_f16(q.z, q.w) : fp8x8_to_f16(q.x, q.y);
        }
      };
      float sv[kNC];
#pragma unroll
      for (int ct = 0; ct < kNC; ++ct) sv[ct] = __uint_as_float(wo.sc[ct]);
      // block products of up to four row tiles at a time (eight independent
      // MFMA chains), then cur = fma(scale, block product, cur)
      constexpr int kH = MT < 4 ? MT : 4;
#pragma unroll
      for (int m0 = 0; m0 < MT; m0 += kH) {
        f32x4 pb[kH][kNC];
#pragma unroll
        for (int mt = 0; mt < kH; ++mt)
#pragma unroll
          for (int ct = 0; ct < kNC; ++ct) pb[mt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        f16x8 ah[2][kH], bf[2][kNC];
#pragma unroll
        for (int mt = 0; mt < kH; ++mt) ah[0][mt] = *(const f16x8 *)(sa + ((m0 + mt) * 4) * 1024 + lane * 16);
        bdec8(0, bf[0]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (j < 3) {
#pragma unroll
            for (int mt = 0; mt < kH; ++mt)
              ah[(j + 1) & 1][mt] = *(const f16x8 *)(sa + ((m0 + mt) * 4 + j + 1) * 1024 + lane * 16);
            bdec8(j + 1, bf[(j + 1) & 1]);
          }
#pragma unroll
          for (int mt = 0; mt < kH; ++mt)
#pragma unroll
            for (int ct = 0; ct < kNC; ++ct)
              pb[mt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[j & 1][mt], bf[j & 1][ct], pb[mt][ct], 0, 0, 0);
          if (j < 3) __builtin_amdgcn_sched_group_barrier(0x100, kH, 0);
#pragma unroll
          for (int qq = 0; qq < kH * kNC; ++qq) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
          }
        }
#pragma unroll
        for (int mt = 0; mt < kH; ++mt)
#pragma unroll
          for (int ct = 0; ct < kNC; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              cur[m0 + mt][ct][e] = __builtin_fmaf(sv[ct], pb[mt][ct][e], cur[m0 + mt][ct][e]);
      }
    } else {
      f16x2 s01[kNC];
#pragma unroll
      for (int ct = 0; ct < kNC; ++ct) s01[ct] = e4m3x2_to_f16x2(wo.sc[ct]);
      f16x8 bf[2][kNC];
      auto bdec = [&](int j, f16x8 (&b)[kNC]) __attribute__((always_inline)) {
#pragma unroll
        for (int ct = 0; ct < kNC; ++ct) b[ct] = dequant8_f16(word_of(wo.w[ct][0], j), s01[ct][j >> 1]);
      };
      aread(0, af[0]);
      bdec(0, bf[0]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j < 3) {
          aread(j + 1, af[(j + 1) & 1]);
          bdec(j + 1, bf[(j + 1) & 1]);
        }
        // sub-step outermost: consecutive MFMAs update different accumulators
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int ct = 0; ct < kNC; ++ct)
            cur[mt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[j & 1][mt], bf[j & 1][ct], cur[mt][ct], 0, 0, 0);
        // issue order: the next sub-step's LDS reads, then each MFMA
        // followed by one VALU instruction of the next decode
        if (j < 3) __builtin_amdgcn_sched_group_barrier(0x100, MT, 0);
#pragma unroll
        for (int qq = 0; qq < MT * kNC; ++qq) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
        }
      }
    }
  };

  // close the class in progress: the first is the running sum, later ones
  // are added to it (the streaming kernels' wave-order reduction)
  auto close_class = [&](bool first) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ct = 0; ct < kNC; ++ct) {
        tot[mt][ct] = first ? cur[mt][ct] : tot[mt][ct] + cur[mt][ct];
        cur[mt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
  };

  // ---- main loop over the class-by-class step sequence ----
  issue(0, 0, 0);
  issue(1, 1, 1);
  wait_vm<kReqs>();
  lds_barrier();

  int cls = 0;                   // class in progress
  int cls_end = class_count(0);  // sequence position where it ends
  // One sequence position: read this wave's weight bytes of step i (weight
  // stage i % 2), copy step i + 2 into the activation stage step i - 1
  // used (free since the last barrier) and into the weight stage just
  // read, multiply step i (activation stage i % 3), wait for step i + 1's
  // copies, barrier: every copy has two steps' MFMAs to land.  Every
  // position issues the same requests and barrier whether or not it
  // computes (the last group may run past the split), so the compiler's
  // wait counts see one request sequence.
  auto unit = [&](int i, auto phase) __attribute__((always_inline)) {
    constexpr int PH = decltype(phase)::value;  // i % 3
    const int ws = i & 1;                       // weight stage (wave-uniform)
    WOps wo;
    read_w(PH, ws, wo);
    // the reads are complete before the copy into the same weight stage
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_sched_barrier(0);
    issue(i + 2, (PH + 2) % 3, ws);
    __builtin_amdgcn_sched_barrier(0);
    if (i < S) compute(PH, wo);
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<kReqs>();
    lds_barrier();
    if (i + 1 == cls_end) {
      close_class(cls == 0);
      ++cls;
      cls_end = cls < 4 ? cls_end + class_count(cls) : INT_MAX;
    }
  };
  for (int i0 = 0; i0 < S; i0 += 3) {
    unit(i0, std::integral_constant<int, 0>{});
    unit(i0 + 1, std::integral_constant<int, 1>{});
    unit(i0 + 2, std::integral_constant<int, 2>{});
  }
  // classes with no step (a split of fewer than four steps) still add
  // their zero sum, as an idle wave does in the streaming kernels
  for (; cls < 4; ++cls) close_class(false);
  // requests past the split fetch nothing, but must land before the end
  wait_all_memory();

  // ---- split hand-off: the last split of a tile to arrive sums the
  // partials in split order from zero ----
  const int tile = rb * ncb + cb;
  if (p.ksplit > 1) {
    constexpr uint32_t kWaveFloats = MT * kNC * 256;
    auto part_rsrc = [&](int sp) __attribute__((always_inline)) {
      const size_t off = (((size_t)tile * p.ksplit + sp) * kNW + wave) * kWaveFloats;
      return rsrc_uniform(p.partial + off, (size_t)kWaveFloats * 4);
    };
    {
      const __amdgpu_buffer_rsrc_t pr = part_rsrc(split);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ct = 0; ct < kNC; ++ct)
          st16_coherent(pr, (uint32_t)((mt * kNC + ct) * 1024 + lane * 16), tot[mt][ct]);
    }
    wait_all_memory();
    __syncthreads();
    // (the weight stages are free: every wave has passed its loop and its
    // final wait for all requests)
    unsigned *last_flag = (unsigned *)ldsw[0];
    if (tid == 0) {
      const unsigned old = __hip_atomic_fetch_add(&p.counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *last_flag = old == (unsigned)(p.ksplit - 1);
    }
    __syncthreads();
    if (!*last_flag) return;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ct = 0; ct < kNC; ++ct) tot[mt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < p.ksplit; ++sp) {
      const __amdgpu_buffer_rsrc_t pr = part_rsrc(sp);
      f32x4 v[MT][kNC];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ct = 0; ct < kNC; ++ct) v[mt][ct] = ld16_coherent(pr, (uint32_t)((mt * kNC + ct) * 1024 + lane * 16));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int ct = 0; ct < kNC; ++ct) tot[mt][ct] += v[mt][ct];
    }
    if (tid == 0) __hip_atomic_store(&p.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- epilogue: element e of row tile mt, column tile ct is output
  // (row0 + 16 mt + 4 g + e, column of the tile + c) ----
#pragma unroll
  for (int ct = 0; ct < (NMAT == 2 ? 1 : kNC); ++ct) {
    const int col = tile_col(ct) + c16;
    if (col >= p.n) continue;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = row0 + mt * 16 + 4 * gq + e;
        if (r >= p.m) continue;
        const float rs = p.xr[r];
        __bf16 out;
        if constexpr (FP8) {
          const float v0 = tot[mt][ct][e] * rs;
          if constexpr (NMAT == 2)
            out = swiglu_bf16(v0, tot[mt][1][e] * rs);
          else
            out = (__bf16)v0;
        } else {
          float v0 = tot[mt][ct][e];
          float v1 = tot[mt][NMAT == 2 ? 1 : ct][e];
          v0 = v0 * rs;
          v1 = v1 * rs;
          v0 = v0 * p.ts0;
          if constexpr (NMAT == 2) {
            v1 = v1 * p.ts1;
            out = swiglu_bf16(v0, v1);
          } else {
            out = (__bf16)v0;
          }
        }
        ((__bf16 *)p.y)[(size_t)r * p.n + col] = out;
      }
  }
}

constexpr int kTargetWG = 256;  // one workgroup per CU

// Row tiles per workgroup: eight (each decoded weight fragment feeds eight
// MFMAs, and every weight byte is copied half as often) when that still
// gives every CU a workgroup, else four.
template <bool FP8, int NMAT>
int tall_mt(int m, int n, int ksplit) {
  constexpr int wg_cols = NMAT == 2 ? 16 * kNW : 16 * kTiles;
  return cdiv(m, 128) * ksplit * cdiv(n, wg_cols) >= kTargetWG ? 8 : 4;
}

template <bool FP8, int NMAT>
hipError_t launch_tall(const TallArgs &p, int mt, hipStream_t s) {
  constexpr int wg_cols = NMAT == 2 ? 16 * kNW : 16 * kTiles;
  const dim3 grid(cdiv(p.m, 16 * mt) * p.ksplit * cdiv(p.n, wg_cols));
  if (mt == 8)
    hipLaunchKernelGGL((k_fixed_tall<FP8, NMAT, 8>), grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((k_fixed_tall<FP8, NMAT, 4>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <bool FP8>
int tall_mt_any(int nmat, int m, int n, int ksplit) {
  return nmat == 2 ? tall_mt<FP8, 2>(m, n, ksplit) : tall_mt<FP8, 1>(m, n, ksplit);
}

size_t tall_partial(int nmat, int m, int n, int ksplit, int mt) {
  if (ksplit <= 1) return 0;
  const int wg_cols = nmat == 2 ? 16 * kNW : 16 * kTiles;
  return (size_t)cdiv(m, 16 * mt) * cdiv(n, wg_cols) * ksplit * kNW * mt * kNC * 256;
}

}  // namespace

bool fixed_tall_eligible(int m) { return m >= kFixedTallMinRows; }

size_t fixed_tall_partial_floats(bool fp8, int nmat, int m, int n, int ksplit) {
  if (!fixed_tall_eligible(m)) return 0;
  const int mt = fp8 ? tall_mt_any<true>(nmat, m, n, ksplit) : tall_mt_any<false>(nmat, m, n, ksplit);
  return tall_partial(nmat, m, n, ksplit, mt);
}

hipError_t launch_fixed_tall_w4a4(const ActRef &a, int m, int k, int n, int nmat, const MatRef *w, void *y,
                                  float *partial, unsigned *counters, const StreamPlan &pl,
                                  hipStream_t stream) {
  TallArgs p{};
  p.xt = a.tiles;
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
  const int mt = tall_mt_any<false>(nmat, m, n, pl.ksplit);
  return nmat == 2 ? launch_tall<false, 2>(p, mt, stream) : launch_tall<false, 1>(p, mt, stream);
}

hipError_t launch_fixed_tall_w8a8(const Fp8ActRef &a, int m, int k, int n, int nmat, const Fp8MatRef *w,
                                  void *y, float *partial, unsigned *counters, const StreamPlan &pl,
                                  hipStream_t stream) {
  TallArgs p{};
  p.xt = a.tiles;
  p.xr = a.row_scale;
  p.m = m;
  p.k = k;
  p.n = n;
  p.codes0 = w[0].codes;
  p.fscales0 = w[0].scales;
  p.codes1 = nmat > 1 ? w[1].codes : nullptr;
  p.fscales1 = nmat > 1 ? w[1].scales : w[0].scales;
  p.ts0 = 1.f;
  p.ts1 = 1.f;
  p.y = y;
  p.partial = partial;
  p.counters = counters;
  p.ksplit = pl.ksplit;
  p.steps_per_split = pl.steps_per_split;
  const int mt = tall_mt_any<true>(nmat, m, n, pl.ksplit);
  return nmat == 2 ? launch_tall<true, 2>(p, mt, stream) : launch_tall<true, 1>(p, mt, stream);
}

}  // namespace nvfp4
