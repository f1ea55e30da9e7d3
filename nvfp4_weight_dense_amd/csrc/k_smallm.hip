// k_smallm.hip -- weight-streaming NVFP4 projection for 17..64 rows (gfx950).
//
// Regime: the pages' small-m edge (page layers/dense_ffn_prefill.rs,
// `w4a16_prefill_gemm`: m <= 64 takes the small-m kernels).  With tens of
// rows the weights are still the whole HBM stream and every weight is
// dequantized exactly once, so the VALU work of the dequantization is as
// large as the matrix-core work: one 8-weight fragment per lane (16 VALU
// instructions) feeds MT 16x16x32 MFMAs.  Both pipes only stay busy when
// every SIMD holds two waves with the same amount of work, so the kernel is
// built around an even split:
//
//   * one workgroup of eight waves per CU (about 100 KB of LDS keeps it to
//     one), at most 256 workgroups.  Output columns come in column groups
//     (64 gate columns and the same 64 up columns, or 128 columns of one
//     matrix) and K in units of 256; the (group, unit) pairs, group-major,
//     are cut into equal contiguous ranges, one per workgroup (stream-K).
//     A range is walked in segments, one per column group it touches.
//   * wave w owns column slot w % 4 -- 16 gate and 16 up columns (fused
//     silu epilogue), or 32 columns of one matrix -- for all rows, and K
//     half w / 4 of every unit, so the two waves on a SIMD do the same
//     work.  Within its 128 K of a unit, lane group g = lane / 16 of a wave
//     takes K 32g .. 32g + 31 and MFMA step s sums K {32g + 8s .. + 7 : g};
//     the activation fragments are read at the same K, so each step is an
//     ordinary 16x16x32 product over a permuted K.
//   * weights move as whole 128-byte lines (eight lanes per line) and the
//     activations of a unit (rows x 256 K, bf16) as whole rows; both are
//     requested three units ahead and written to a two-unit LDS ring one
//     unit ahead, in the order the MFMA operands are read back (one 16-byte
//     read per lane and fragment, bank-conflict free); the unit barrier
//     waits for LDS operations only.
//   * at the end of a segment the two K halves are summed through LDS.  A
//     segment that covers its whole column group is finished at once; a
//     partial one is stored as an fp32 piece, and the last of a group's
//     pieces to arrive sums them in K order and finishes the group.
//
// Requires k % 64 == 0 (K pieces of 32 are whole or absent); K beyond k,
// rows beyond m and columns beyond n read as zero and are not stored.
#include <algorithm>
#include <type_traits>

#include "launchers.h"
#include "nvfp4_common.h"

namespace nvfp4 {

namespace {

constexpr int kNW = 8;                    // waves per workgroup
constexpr int kColSlots = 4;              // column slots per workgroup
constexpr int kUnitK = 256;               // K per unit (two halves of 128)
constexpr int kMaxWG = 256;               // workgroups: one per CU
constexpr int kNS = 4;                    // weight stages: three units in flight
static_assert(kNS == 4, "the unit loop is written out for four stages");

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct SmallArgs {
  const void *x;  // bf16 [m][k]
  int m, k, n;
  const uint8_t *codes0, *scales0;  // gate (two matrices) or the matrix
  const uint8_t *codes1, *scales1;  // up (two matrices) or unused
  float ts0, ts1;
  void *y;
  float *partial;      // [nwg][2][kColSlots][2 MT][64 lanes][4]
  unsigned *counters;  // [groups], zero between calls
  int kunits, units, nwg;
  int gshift;  // packed-Q2 weights: fp16 scale per 1 << gshift of K
};

__device__ __forceinline__ void st16_coherent(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                              f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff, soff, kCoherent);
}
__device__ __forceinline__ f32x4 ld16_coherent(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kCoherent));
}

// first unit of workgroup w's range (range w is [begin(w), begin(w + 1)))
__host__ __device__ __forceinline__ int range_begin(int units, int nwg, int w) {
  return (int)(((int64_t)units * w) / nwg);
}
// the workgroup whose range holds unit u: the w with begin(w) <= u < begin(w + 1)
__host__ __device__ __forceinline__ int range_owner(int units, int nwg, int u) {
  return (int)((((int64_t)u + 1) * nwg + units - 1) / units) - 1;
}

// Q2: packed-Q2 weights (2-bit codes, fp16 scale per group of K; the
// values bf16((q - 2) d) come from q2_table / q2_dequant8) instead of NVFP4.
template <int MT, int NMAT, bool Q2>
__global__ __launch_bounds__(kNW * 64) void k_smallm(SmallArgs p) {
  constexpr int kRows = 16 * MT;
  constexpr int kQ = 2 * MT;  // accumulator tiles per wave: two column tiles x MT row tiles
  constexpr int kGroupCols = NMAT == 2 ? 64 : 128;
  constexpr int kXPieces = kRows * (kUnitK * 2 / 16) / (kNW * 64);  // 16-byte pieces per thread
  __shared__ uint4 xs[2][8 * MT][64];                             // activations, two units
  __shared__ uint4 wsm[2][kColSlots][2][2][Q2 ? 1 : 64];          // NVFP4 codes, two units
  __shared__ uint16_t ssm[2][kColSlots][2][2][Q2 ? 1 : 64];       // NVFP4 scales, two units
  __shared__ uint2 wsq[2][kColSlots][2][2][Q2 ? 64 : 1];          // packed-Q2 codes, two units
  __shared__ f32x4 red[kColSlots][kQ][64];
  __shared__ unsigned last_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = wave & 3, kh = wave >> 2;
  const int c16 = lane & 15, gq = lane >> 4;
  const int k = p.k;
  // bytes per weight row: codes, and scales (E4M3 per 16 K; fp16 per group)
  const uint32_t kb2 = Q2 ? (uint32_t)k >> 2 : (uint32_t)k >> 1;
  const uint32_t kb16 = Q2 ? ((uint32_t)k >> p.gshift) * 2u : (uint32_t)k >> 4;
  const int KU = p.kunits;
  const int w = (int)blockIdx.x;
  const int ub = range_begin(p.units, p.nwg, w);
  const int nloc = range_begin(p.units, p.nwg, w + 1) - ub;

  // first column of this wave's column tile j in group g
  auto tile_col = [&](int g, int j) __attribute__((always_inline)) {
    return g * kGroupCols + (NMAT == 2 ? 16 * slot : 32 * slot + 16 * j);
  };

  // ---- weights: per unit and column tile the two waves of a slot load the
  // tile's 16 rows as whole 128-byte lines (wave kh rows 8 kh .. 8 kh + 7;
  // lane s: row s / 8, 16-byte piece s % 8 = K 32 (s % 8) of the unit) and
  // their scale bytes (two per lane, the same K), two units ahead; one unit
  // ahead they are written to LDS in operand order, so each lane reads its
  // 16 code bytes and 2 scale bytes back with one instruction apiece
  struct WStage {
    uint4 c[2];
    uint32_t s[2];
  };
  const uint32_t wrow = 8u * (uint32_t)kh + ((uint32_t)lane >> 3), wpiece = (uint32_t)lane & 7;
  // (units past the range get a K start beyond every k: their requests are
  // out of range and fetch nothing, with no branch)
  auto load_w = [&](int i, WStage &b) __attribute__((always_inline)) {
    const bool live = i < nloc;
    const int u = ub + (live ? i : 0);
    const int g = u / KU;
    const uint32_t k0 = live ? (uint32_t)(u - g * KU) * kUnitK : 0x40000000u;
    if constexpr (Q2) {
      // codes of tile kh: 16 rows x 64 bytes (lane s: row s / 4, 16 bytes
      // = K 64 (s % 4) of the unit); fp16 scales of both tiles for this
      // lane's operand K range (row c, K 128 kh + 32 g, one group)
      const uint32_t lr = (uint32_t)lane >> 2, lp = (uint32_t)lane & 3;
      const uint32_t kp = k0 + 64u * lp;
      const uint32_t ks = k0 + 128u * (uint32_t)kh + 32u * (uint32_t)gq;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = tile_col(g, j);
        const bool second = NMAT == 2 && j == 1;
        const uint8_t *cb = second ? p.codes1 : p.codes0;
        const uint8_t *sb = second ? p.scales1 : p.scales0;
        const int nc = max(0, min(16, p.n - col));
        const size_t base = (size_t)min(col, p.n);
        if (j == kh) {
          const __amdgpu_buffer_rsrc_t rc = rsrc_uniform(cb + base * kb2, (size_t)nc * kb2);
          b.c[0] = ld16(rc, kp < (uint32_t)k ? lr * kb2 + (kp >> 2) : kOOB);
        }
        const __amdgpu_buffer_rsrc_t rs = rsrc_uniform(sb + base * kb16, (size_t)nc * kb16);
        b.s[j] = ld2(rs, ks < (uint32_t)k ? (uint32_t)c16 * kb16 + ((ks >> p.gshift) << 1) : kOOB);
      }
      return;
    }
    const uint32_t kp = k0 + 32u * wpiece;
    const bool ok = kp < (uint32_t)k;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = tile_col(g, j);
      const bool second = NMAT == 2 && j == 1;
      const uint8_t *cb = second ? p.codes1 : p.codes0;
      const uint8_t *sb = second ? p.scales1 : p.scales0;
      const int nc = max(0, min(16, p.n - col));
      const size_t base = (size_t)min(col, p.n);
      const __amdgpu_buffer_rsrc_t rc = rsrc_uniform(cb + base * kb2, (size_t)nc * kb2);
      const __amdgpu_buffer_rsrc_t rs = rsrc_uniform(sb + base * kb16, (size_t)nc * kb16);
      b.c[j] = ld16(rc, ok ? wrow * kb2 + (kp >> 1) : kOOB);
      b.s[j] = ld2(rs, ok ? wrow * kb16 + (kp >> 4) : kOOB);
    }
  };
  // LDS image of a unit's weights: per (slot, tile, K half) 64 lanes x 16
  // code bytes and 64 x 2 scale bytes; lane (c, g) of K half h holds row c,
  // piece 4 h + g, at code position 16 g + (c ^ 2 (g + 4 h)) (the XOR keeps
  // the 16 lanes of a write or read phase on distinct banks) and scale
  // position 16 g + c
  // packed Q2: per (slot, tile, K half) 64 lanes x 8 code bytes; lane (c, g)
  // of K half h holds row c, K 128 h + 32 g .. + 31, at position 16 g + c
  auto store_w = [&](int buf, const WStage &b) __attribute__((always_inline)) {
    if constexpr (Q2) {
      const uint32_t lr = (uint32_t)lane >> 2, lp = (uint32_t)lane & 3;
      const uint32_t h = lp >> 1, g4 = 2u * (lp & 1u);
      wsq[buf][slot][kh][h][16u * g4 + lr] = uint2{b.c[0].x, b.c[0].y};
      wsq[buf][slot][kh][h][16u * (g4 + 1u) + lr] = uint2{b.c[0].z, b.c[0].w};
      return;
    }
    const uint32_t h = wpiece >> 2, g4 = wpiece & 3;
    const uint32_t cpos = 16u * g4 + (wrow ^ (2u * (g4 + 4u * h)));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      wsm[buf][slot][j][h][cpos] = b.c[j];
      ssm[buf][slot][j][h][16u * g4 + wrow] = (uint16_t)b.s[j];
    }
  };
  const int wpos = 16 * gq + (c16 ^ (2 * (gq + 4 * kh)));

  // ---- activations: a unit's rows x 256 K; thread tid moves 16-byte
  // pieces tid + 512 q (row piece / 32, K 8 (piece % 32) of the unit).  In
  // LDS each MFMA fragment is one 1 KB block -- block (4 kh + s) MT + mt of
  // a buffer holds row tile mt at K 128 kh + 32 g + 8 s -- with lane (c, g)
  // at position 16 g + (c ^ (4 g + s)).
  const __amdgpu_buffer_rsrc_t xres = rsrc_uniform(p.x, (size_t)min(kRows, p.m) * (size_t)k * 2);
  uint4 xr[2][kXPieces];
  auto load_x = [&](int i, uint4 (&xv)[kXPieces]) __attribute__((always_inline)) {
    const uint32_t k0 = i < nloc ? (uint32_t)((ub + i) % KU) * kUnitK : 0x40000000u;
#pragma unroll
    for (int q = 0; q < kXPieces; ++q) {
      const int piece = tid + kNW * 64 * q;
      const uint32_t kk = k0 + 8u * (uint32_t)(piece & 31);
      xv[q] = ld16(xres, kk < (uint32_t)k ? ((uint32_t)(piece >> 5) * (uint32_t)k + kk) * 2u : kOOB);
    }
  };
  auto store_x = [&](int buf, const uint4 (&xv)[kXPieces]) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < kXPieces; ++q) {
      const int piece = tid + kNW * 64 * q;
      const int r = piece >> 5, ch = piece & 31;
      const int h = ch >> 4, g4 = (ch >> 2) & 3, st = ch & 3;
      xs[buf][(4 * h + st) * MT + (r >> 4)][16 * g4 + ((r & 15) ^ (4 * g4 + st))] = xv[q];
    }
  };
  auto read_a = [&](int buf, int s, bf16x8 (&a)[MT]) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      a[mt] = as_bf16x8(xs[buf][(4 * kh + s) * MT + mt][16 * gq + (c16 ^ (4 * gq + s))]);
  };

  f32x4 acc[2][MT];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[j][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  zero_acc();

  // (b: the unit's register stage, for the packed-Q2 scales)
  auto compute = [&](int buf, const WStage &b) __attribute__((always_inline)) {
    uint4 wc[2];
    float sc[2][2];
    uint32_t lo[2], hi[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if constexpr (Q2) {
        const uint2 v = wsq[buf][slot][j][kh][16 * gq + c16];
        wc[j] = uint4{v.x, v.y, 0u, 0u};
        q2_table(b.s[j], lo[j], hi[j]);
      } else {
        wc[j] = wsm[buf][slot][j][kh][wpos];
        const uint32_t sv = ssm[buf][slot][j][kh][16 * gq + c16];
        sc[j][0] = e4m3_to_f32_sel<0>(sv);  // block 2g: steps 0, 1
        sc[j][1] = e4m3_to_f32_sel<1>(sv);  // block 2g + 1: steps 2, 3
      }
    }
    bf16x8 a[2][MT];
    bf16x8 bb[2][2];
    auto dq = [&](int s, bf16x8 (&out)[2]) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if constexpr (Q2) {
          // step s: the 8 codes at bits 16 s of the lane's 64 bits
          const uint32_t word = s < 2 ? wc[j].x : wc[j].y;
          out[j] = q2_dequant8((s & 1) ? word >> 16 : word & 0xFFFFu, lo[j], hi[j]);
        } else {
          const uint32_t word = s == 0 ? wc[j].x : s == 1 ? wc[j].y : s == 2 ? wc[j].z : wc[j].w;
          out[j] = dequant8(word, sc[j][s >> 1]);
        }
      }
    };
    read_a(buf, 0, a[0]);
    dq(0, bb[0]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) {
        read_a(buf, s + 1, a[(s + 1) & 1]);
        dq(s + 1, bb[(s + 1) & 1]);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s & 1][mt], bb[s & 1][j], acc[j][mt], 0, 0, 0);
    }
  };

  // element i of row tile mt, column tile j: row 16 mt + 4 g + i, column
  // tile_col(g, j) + c; rows past m fall outside the output resource
  const __amdgpu_buffer_rsrc_t yres = rsrc_uniform(p.y, (size_t)min(kRows, p.m) * (size_t)p.n * 2);
  const uint32_t n2 = (uint32_t)p.n * 2u;
  auto epilogue = [&](int g) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < (NMAT == 2 ? 1 : 2); ++j) {
      const int col = tile_col(g, j) + c16;
      const uint32_t vo = col < p.n ? (uint32_t)(4 * gq) * n2 + (uint32_t)col * 2u : kOOB;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const __bf16 out = NMAT == 2 ? swiglu_bf16(acc[0][mt][e] * p.ts0, acc[1][mt][e] * p.ts1)
                                       : (__bf16)(acc[j][mt][e] * p.ts0);
          st2s(yres, vo, (uint32_t)(mt * 16 + e) * n2, out);
        }
    }
  };

  // piece of workgroup v for the group starting at or before its range:
  // slot 0 holds the segment of its first group, slot 1 that of its last
  auto piece_rsrc = [&](int v, int pslot) __attribute__((always_inline)) {
    return rsrc_uniform(p.partial + ((size_t)(v * 2 + pslot) * kColSlots + slot) * (kQ * 256),
                        (size_t)kQ * 256 * 4);
  };

  // the last of a split group's pieces to arrive finishes the group: every
  // wave sums column tile kh of its slot over the pieces in K (workgroup)
  // order, four pieces' loads in flight together
  auto finish_split = [&](int g) __attribute__((always_inline)) {
    const int v0 = range_owner(p.units, p.nwg, g * KU);
    const int v1 = range_owner(p.units, p.nwg, g * KU + KU - 1);
    f32x4 sum[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) sum[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int v = v0; v <= v1; v += 4) {
      f32x4 t[4][MT];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int vv = min(v + d, v1);
        const int ps = g == range_begin(p.units, p.nwg, vv) / KU ? 0 : 1;
        const __amdgpu_buffer_rsrc_t pr = piece_rsrc(vv, ps);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          t[d][mt] = ld16_coherent(pr, (uint32_t)lane * 16u, (uint32_t)(kh * MT + mt) * 1024u);
      }
#pragma unroll
      for (int d = 0; d < 4; ++d)
        if (v + d <= v1) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) sum[mt] += t[d][mt];
        }
    }
    // column tile 1 goes to the K-half-0 wave of the slot
    if (kh == 1) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) red[slot][mt][lane] = sum[mt];
    }
    lds_barrier();
    if (kh == 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc[0][mt] = sum[mt];
        acc[1][mt] = red[slot][mt][lane];
      }
      epilogue(g);
    }
    if (tid == 0) __hip_atomic_store(&p.counters[g], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  // end of a segment of group g: sum the K halves through LDS; finish a
  // whole group at once, or store this workgroup's piece of a split one and
  // count its arrival (the last piece to arrive finishes the group).
  // Counting every arrival after the whole range instead, so that the
  // stores need no wait mid-stream, measured slower: the finishing work
  // then all lands at the end of the launch.
  auto flush = [&](int g, bool whole, int pslot) __attribute__((always_inline)) {
    if (kh == 1) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) red[slot][j * MT + mt][lane] = acc[j][mt];
    }
    lds_barrier();
    if (kh == 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[j][mt] += red[slot][j * MT + mt][lane];
      if (whole) {
        epilogue(g);
      } else {
        const __amdgpu_buffer_rsrc_t pr = piece_rsrc(w, pslot);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            st16_coherent(pr, (uint32_t)lane * 16u, (uint32_t)(j * MT + mt) * 1024u, acc[j][mt]);
      }
    }
    if (!whole) {
      const int v0 = range_owner(p.units, p.nwg, g * KU);
      const int v1 = range_owner(p.units, p.nwg, g * KU + KU - 1);
      wait_all_memory();
      __syncthreads();
      if (tid == 0) {
        const unsigned old =
            __hip_atomic_fetch_add(&p.counters[g], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_flag = old == (unsigned)(v1 - v0);
      }
      __syncthreads();
      if (last_flag) finish_split(g);
    }
    zero_acc();
    // every request of this path is complete again when the unit loop
    // resumes (its wait-count bookkeeping then matches the other path's);
    // red is rewritten only after the next unit's barrier
    wait_all_memory();
  };

  // ---- main loop: units in order.  Each unit first writes the activations
  // and weights of the next unit into LDS (loaded two units earlier, into
  // two and four register sets), then requests those of the unit three
  // ahead.  Vector-memory loads complete in issue order as far as the wait
  // counter goes, so the wait before a write to LDS also covers every
  // older request -- all of them for units already due.
  WStage wb[kNS];
  load_x(0, xr[0]);
  load_w(0, wb[0]);
  load_x(1, xr[1]);
  load_w(1, wb[1]);
  store_x(0, xr[0]);
  store_w(0, wb[0]);
  load_x(2, xr[0]);
  load_w(2, wb[2]);
  lds_barrier();

  // Segment bookkeeping (all wave-uniform): the current segment covers
  // local units [seg_first, seg_end) of column group g.
  int g = ub / KU;
  int seg_first = 0;
  int seg_end = min(nloc, (g + 1) * KU - ub);

  // One unit.  Every unit issues the same requests and barrier whether or
  // not it computes (the last block of four may run past the range), so
  // the compiler's wait-count bookkeeping sees the same request sequence
  // on every path and waits for each unit's own requests only.
  auto unit = [&](int i, auto phase) __attribute__((always_inline)) {
    constexpr int S = decltype(phase)::value;  // i % kNS (kNS even: also the LDS slot parity)
    store_x((S + 1) & 1, xr[(S + 1) & 1]);
    store_w((S + 1) & 1, wb[(S + 1) % kNS]);
    load_x(i + 3, xr[(S + 1) & 1]);
    load_w(i + 3, wb[(S + 3) % kNS]);
    __builtin_amdgcn_sched_barrier(0);
    if (i < nloc) compute(S & 1, wb[S]);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    if (i + 1 == seg_end) {
      const bool whole = ub + seg_first == g * KU && (g + 1) * KU - ub <= nloc;
      flush(g, whole, seg_first == 0 ? 0 : 1);
      seg_first = seg_end;
      ++g;
      seg_end = min(nloc, (g + 1) * KU - ub);
    }
  };

  for (int i0 = 0; i0 < nloc; i0 += kNS) {
    unit(i0, std::integral_constant<int, 0>{});
    unit(i0 + 1, std::integral_constant<int, 1>{});
    unit(i0 + 2, std::integral_constant<int, 2>{});
    unit(i0 + 3, std::integral_constant<int, 3>{});
  }
  // weight and activation requests past the range fetch nothing, but any
  // still in flight must land before the workgroup ends
  wait_all_memory();
}

}  // namespace

bool smallm_eligible(int m, int k) { return m >= 17 && m <= 64 && k % 64 == 0; }

SmallPlan smallm_plan(int m, int n, int k, int nmat) {
  SmallPlan pl;
  pl.mt = m <= 32 ? 2 : 4;
  pl.groups = cdiv(n, nmat == 2 ? 64 : 128);
  pl.kunits = cdiv(k, kUnitK);
  pl.units = pl.groups * pl.kunits;
  pl.nwg = std::min(kMaxWG, pl.units);
  // with at most half as many column groups as workgroups, a whole number
  // of workgroups per group: every range then lies in one group, so no
  // workgroup holds two pieces (down projection at m=64: 33.2 -> 31.9 us)
  if (pl.groups * 2 <= kMaxWG && pl.units >= kMaxWG) pl.nwg = (kMaxWG / pl.groups) * pl.groups;
  return pl;
}

size_t smallm_partial_floats(const SmallPlan &pl) {
  return (size_t)pl.nwg * 2 * kColSlots * (2 * pl.mt) * 256;
}

size_t smallm_counter_words(const SmallPlan &pl) { return (size_t)pl.groups; }

namespace {
// One workgroup per CU: the static LDS (84 to 132 KB) keeps it so, except
// for packed Q2 with two row tiles (64 KB), which takes 20 KB more.
template <bool Q2>
hipError_t launch_kernel(const SmallArgs &p, int nmat, const SmallPlan &pl, hipStream_t stream) {
  const dim3 grid(pl.nwg), block(kNW * 64);
  const unsigned pad = Q2 && pl.mt == 2 ? 20480u : 0u;
  if (nmat == 2) {
    if (pl.mt == 2) hipLaunchKernelGGL((k_smallm<2, 2, Q2>), grid, block, pad, stream, p);
    else hipLaunchKernelGGL((k_smallm<4, 2, Q2>), grid, block, pad, stream, p);
  } else {
    if (pl.mt == 2) hipLaunchKernelGGL((k_smallm<2, 1, Q2>), grid, block, pad, stream, p);
    else hipLaunchKernelGGL((k_smallm<4, 1, Q2>), grid, block, pad, stream, p);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_smallm(const void *x, int m, int k, int n, int nmat, const MatRef *w, void *y,
                         float *partial, unsigned *counters, const SmallPlan &pl,
                         hipStream_t stream) {
  SmallArgs p{};
  p.x = x;
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
  p.kunits = pl.kunits;
  p.units = pl.units;
  p.nwg = pl.nwg;
  return launch_kernel<false>(p, nmat, pl, stream);
}

hipError_t launch_smallm_q2(const void *x, int m, int k, int n, int gshift, int nmat, const Q2MatRef *w,
                            void *y, float *partial, unsigned *counters, const SmallPlan &pl,
                            hipStream_t stream) {
  SmallArgs p{};
  p.x = x;
  p.m = m;
  p.k = k;
  p.n = n;
  p.codes0 = w[0].codes;
  p.scales0 = (const uint8_t *)w[0].scales;
  p.ts0 = 1.0f;
  p.codes1 = nmat > 1 ? w[1].codes : nullptr;
  p.scales1 = nmat > 1 ? (const uint8_t *)w[1].scales : nullptr;
  p.ts1 = 1.0f;
  p.y = y;
  p.partial = partial;
  p.counters = counters;
  p.kunits = pl.kunits;
  p.units = pl.units;
  p.nwg = pl.nwg;
  p.gshift = gshift;
  return launch_kernel<true>(p, nmat, pl, stream);
}

}  // namespace nvfp4
