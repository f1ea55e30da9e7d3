// k_stream_lds.hip -- weight-streaming NVFP4 projection for 17..64 rows with
// the activations shared through LDS (gfx950).
//
// With tens of rows both the MFMA work and the activation traffic matter:
//   * MFMA: v_mfma_f32_32x32x16_bf16 (32x32 outputs per instruction); on
//     gfx950 it sustains about twice the bf16 rate of the 16x16x32 form.
//   * activations: per 64-element K step a 32-column weight tile is 1 KB of
//     codes, while 64 activation rows are 8 KB of bf16.  The four waves of a
//     workgroup own different column tiles and consume the same K step, so
//     each activation chunk is fetched from L2 once per workgroup and read
//     by every wave from LDS; one activation fragment feeds NMAT MFMAs.
//
//   * step t (64 K): rows [0, 32*MT) x K [64t, 64t+64) of the activations sit
//     in one of three LDS slots (rows padded by 16 bytes); the workgroup
//     loads them two steps ahead, and each lane prefetches its weight
//     codes/scales six steps ahead.
//   * lane (c = lane%32, h = lane/32) holds, for weight row col0+c, the 32
//     codes at K offset 32h of the step: four bf16 B fragments after
//     in-register dequantization; MFMA j of the step sums K offsets
//     {8j..8j+7} U {32+8j..32+8j+7}, and the A fragment of row tile rt is
//     read from LDS at row 32rt+c, the same offsets.
//   * split-K over workgroups with the fixed-order, last-arrival fixup of
//     the streaming kernel (partials summed in split order).
//   * Workgroups that run together start their K range at different steps
//     (a rotation by the column-group index), so they do not all read the
//     same activation chunk at the same moment.
#include <cmath>
#include <type_traits>

#include "launchers.h"
#include "nvfp4_common.h"

namespace nvfp4 {

namespace {

constexpr int kWaves = 4;
constexpr int kStep = 64;                  // K elements per step
constexpr int kRowBytes = kStep * 2 + 16;  // LDS row pitch (bf16 + pad)

struct LdsArgs {
  const void *x;  // bf16 [m][k]
  int m, k, n;
  const uint8_t *codes0, *scales0;
  const uint8_t *codes1, *scales1;
  float ts0, ts1;
  void *y;
  float *partial;       // [nmat][ksplit][m][n]
  unsigned *counters;   // [gridDim.x], zero between calls
  int ksplit, steps_per_split;
  int row_blocks;       // 32*MT-row blocks along m
  int rotate;           // stagger the K start of column groups
};

template <int MT, int NMAT>
__global__ __launch_bounds__(kWaves * 64)
void k_stream_lds(LdsArgs p) {
  constexpr int kRows = 32 * MT;
  __shared__ __attribute__((aligned(16))) uint8_t abuf[3][kRows * kRowBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform, so the weight resources live in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31;
  const int h = lane >> 5;
  const int k = p.k;
  const uint32_t kb2 = (uint32_t)k >> 1, kb16 = (uint32_t)k >> 4;
  const int nsteps = (k + kStep - 1) / kStep;
  const int s_begin = blockIdx.y * p.steps_per_split;
  const int s_end = min(nsteps, s_begin + p.steps_per_split);
  const int len = s_end - s_begin;
  // blockIdx.x = row block + row_blocks * column group: consecutive
  // workgroups (dealt round-robin to the XCDs) take different row blocks
  // of the same columns, so with 8 row blocks each XCD's L2 keeps one
  // activation row block for the whole launch.
  const int rb = (int)(blockIdx.x % (unsigned)p.row_blocks);
  const int cg = (int)(blockIdx.x / (unsigned)p.row_blocks);
  const int row0 = rb * kRows;
  const int rows = min(kRows, p.m - row0);
  const int rot = (p.rotate && len > 0) ? cg % len : 0;
  auto kstep = [&](int tl) { int q = tl + rot; return s_begin + (q >= len ? q - len : q); };
  const int col0 = (cg * kWaves + wave) * 32;  // this wave's columns

  const int ncols = max(0, min(32, p.n - col0));
  const size_t cbase = (size_t)min(col0, p.n);
  __amdgpu_buffer_rsrc_t wc[NMAT], ws[NMAT];
  wc[0] = rsrc(p.codes0 + cbase * kb2, (size_t)ncols * kb2);
  ws[0] = rsrc(p.scales0 + cbase * kb16, (size_t)ncols * kb16);
  if constexpr (NMAT > 1) {
    wc[1] = rsrc(p.codes1 + cbase * kb2, (size_t)ncols * kb2);
    ws[1] = rsrc(p.scales1 + cbase * kb16, (size_t)ncols * kb16);
  }
  const __amdgpu_buffer_rsrc_t xres =
      rsrc((const uint8_t *)p.x + (size_t)row0 * k * 2, (size_t)rows * k * 2);

  // cooperative activation chunk: 16-byte pieces (row = piece / 8, byte
  // offset 16 * (piece % 8)); thread tid moves pieces tid + 256 i
  constexpr int kPieces = kRows * (kStep * 2 / 16);
  constexpr int kPerThread = kPieces / (kWaves * 64);
  static_assert(kPerThread * kWaves * 64 == kPieces, "chunk split");
  uint4 areg[2][kPerThread];
  auto load_a = [&](int tl, uint4 (&a)[kPerThread]) {
    const int t = kstep(tl);
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int piece = tid + kWaves * 64 * i;
      const uint32_t r = (uint32_t)(piece >> 3);
      const uint32_t kk = (uint32_t)t * kStep + 8u * (uint32_t)(piece & 7);
      const bool ok = tl < len && kk < (uint32_t)k && r < (uint32_t)rows;
      a[i] = ld16(xres, ok ? (r * (uint32_t)k + kk) * 2u : kOOB);
    }
  };
  auto store_a = [&](int buf, const uint4 (&a)[kPerThread]) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int piece = tid + kWaves * 64 * i;
      *(uint4 *)&abuf[buf][(piece >> 3) * kRowBytes + 16 * (piece & 7)] = a[i];
    }
  };
  auto load_b = [&](int tl, uint4 (&w)[NMAT], uint32_t (&s)[NMAT]) {
    const int t = kstep(tl);
    const uint32_t kk = (uint32_t)t * kStep + 32u * (uint32_t)h;
    const bool ok = tl < len && kk < (uint32_t)k;
#pragma unroll
    for (int i = 0; i < NMAT; ++i) {
      w[i] = ld16(wc[i], ok ? (uint32_t)c32 * kb2 + (kk >> 1) : kOOB);
      s[i] = ld2(ws[i], ok ? (uint32_t)c32 * kb16 + (kk >> 4) : kOOB);
    }
  };

  f32x16 acc[NMAT][MT];
#pragma unroll
  for (int i = 0; i < NMAT; ++i)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][mt][e] = 0.f;

  // Pipeline: weight codes are prefetched kDB steps ahead into a register
  // ring, activation chunks two steps ahead into registers and then into a
  // three-slot LDS ring.  All slot indices are compile-time (the loop is
  // unrolled by six), so the compiler's own load waits do the pipelining.
  // (six steps cover HBM latency for few rows; with many rows a step is long
  // and the weights mostly come from L2, so three are enough)
  constexpr int kDB = MT >= 4 ? 3 : 6;
  static_assert(6 % kDB == 0, "ring slots must divide the unroll");
  uint4 bw[kDB][NMAT];
  uint32_t bs[kDB][NMAT];
#pragma unroll
  for (int d = 0; d < kDB; ++d) load_b(d, bw[d], bs[d]);
  load_a(0, areg[0]);
  load_a(1, areg[1]);
  store_a(0, areg[0]);
  lds_barrier();

  auto step = [&](int tl, auto slot_c) {
    constexpr int s6 = decltype(slot_c)::value;  // tl % 6
    constexpr int sb = s6 % kDB, sa = s6 % 2, sl = s6 % 3;
    bf16x8 bf[NMAT][4];
#pragma unroll
    for (int i = 0; i < NMAT; ++i) {
      const float s0 = e4m3_to_f32_sel<0>(bs[sb][i]);
      const float s1 = e4m3_to_f32_sel<1>(bs[sb][i]);
      bf[i][0] = dequant8(bw[sb][i].x, s0);
      bf[i][1] = dequant8(bw[sb][i].y, s0);
      bf[i][2] = dequant8(bw[sb][i].z, s1);
      bf[i][3] = dequant8(bw[sb][i].w, s1);
    }
    load_b(tl + kDB, bw[sb], bs[sb]);
    load_a(tl + 2, areg[sa]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 af = as_bf16x8(
            *(const uint4 *)&abuf[sl][(mt * 32 + c32) * kRowBytes + 2 * (32 * h + 8 * j)]);
#pragma unroll
        for (int i = 0; i < NMAT; ++i)
          acc[i][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf[i][j], acc[i][mt], 0, 0, 0);
      }
    }
    if (tl + 1 < len) store_a((sl + 1) % 3, areg[sa ^ 1]);
    // LDS hand-off only: the weight prefetch ring stays in flight
    lds_barrier();
  };
  for (int tl = 0; tl < len; tl += 6) {
    step(tl, std::integral_constant<int, 0>{});
    if (tl + 1 < len) step(tl + 1, std::integral_constant<int, 1>{});
    if (tl + 2 < len) step(tl + 2, std::integral_constant<int, 2>{});
    if (tl + 3 < len) step(tl + 3, std::integral_constant<int, 3>{});
    if (tl + 4 < len) step(tl + 4, std::integral_constant<int, 4>{});
    if (tl + 5 < len) step(tl + 5, std::integral_constant<int, 5>{});
  }

  // output element of lane, register e, row tile mt:
  //   row 32mt + 8(e/4) + 4h + e%4, column col0 + c32
  const int col = col0 + c32;
  if (p.ksplit > 1) {
    // this wave's partial tiles: [NMAT][ksplit][32*MT rows][32 columns]
    constexpr int kTile = 32 * MT * 32;
    const size_t wtile = (size_t)blockIdx.x * kWaves + wave;
    const __amdgpu_buffer_rsrc_t pres =
        rsrc(p.partial + wtile * NMAT * p.ksplit * kTile, (size_t)NMAT * p.ksplit * kTile * 4);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t r = mt * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
#pragma unroll
        for (int i = 0; i < NMAT; ++i)
          st_coherent(pres, (((uint32_t)(i * p.ksplit + blockIdx.y) * kTile) + r * 32u + c32) * 4u,
                      acc[i][mt][e]);
      }
    __shared__ unsigned last;
    wait_all_memory();
    __syncthreads();
    if (tid == 0) {
      const unsigned old =
          __hip_atomic_fetch_add(&p.counters[blockIdx.x], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last = old == (unsigned)(p.ksplit - 1);
    }
    __syncthreads();
    if (!last) return;
    // split order outermost; all of one split's loads are in flight together
#pragma unroll
    for (int i = 0; i < NMAT; ++i)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][mt][e] = 0.f;
    // the loads of one split (up to four tiles at a time) are in flight together
    constexpr int kChunk = NMAT * MT <= 4 ? NMAT * MT : 4;
    for (int sp = 0; sp < p.ksplit; ++sp) {
#pragma unroll
      for (int c0 = 0; c0 < NMAT * MT; c0 += kChunk) {
        float v[kChunk][16];
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
          const int i = (c0 + c) / MT, mt = (c0 + c) % MT;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const uint32_t r = mt * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
            v[c][e] = ld_coherent(pres, (((uint32_t)(i * p.ksplit + sp) * kTile) + r * 32u + c32) * 4u);
          }
        }
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
          const int i = (c0 + c) / MT, mt = (c0 + c) % MT;
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[i][mt][e] += v[c][e];
        }
      }
    }
    if (tid == 0) __hip_atomic_store(&p.counters[blockIdx.x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  if (col >= p.n) return;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = mt * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
      if (r >= rows) continue;
      __bf16 out;
      if constexpr (NMAT > 1)
        out = swiglu_bf16(acc[0][mt][e] * p.ts0, acc[1][mt][e] * p.ts1);
      else
        out = (__bf16)(acc[0][mt][e] * p.ts0);
      ((__bf16 *)p.y)[(size_t)(row0 + r) * p.n + col] = out;
    }
}

template <int MT, int NMAT>
hipError_t launch2(const LdsArgs &p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((k_stream_lds<MT, NMAT>), grid, dim3(kWaves * 64), 0, s, p);
  return hipGetLastError();
}

}  // namespace

int lds_row_tiles(int m) { return m <= 32 ? 1 : m <= 64 ? 2 : 8; }

LdsPlan stream_lds_plan(int m, int n, int k, int nmat) {
  LdsPlan pl;
  pl.mt = lds_row_tiles(m);
  pl.row_blocks = cdiv(m, 32 * pl.mt);
  pl.groups = cdiv(n, kWaves * 32);
  const int nsteps = cdiv(k, kStep);
  const int tiles = pl.groups * pl.row_blocks;
  int ksplit = 1;
  if (pl.row_blocks == 1) {
    // few rows: up to two workgroups per CU (the resident limit of the 17..64
    // row shapes), never more, so no second round; the split then depends
    // on (n, k) only
    ksplit = 512 / pl.groups;
  } else if (nmat == 1) {
    // many rows: one workgroup per CU; split K only to even out the last
    // round (partials cost 4 bytes per output and split)
    const int slots = 256;
    double best = 0;
    for (int ks = 1; ks <= 4; ++ks) {
      const double rounds = (double)tiles * ks / slots;
      const double eff = rounds / std::ceil(rounds);
      if (eff > best + 0.05) { best = eff; ksplit = ks; }
    }
  }
  const int cap = nsteps / 4 > 0 ? nsteps / 4 : 1;  // at least four steps per split
  if (ksplit > cap) ksplit = cap;
  if (ksplit < 1) ksplit = 1;
  if (k < splitk_min_k()) ksplit = 1;
  pl.steps_per_split = cdiv(nsteps, ksplit);
  pl.ksplit = cdiv(nsteps, pl.steps_per_split);
  pl.rotate = pl.row_blocks == 1;
  return pl;
}

size_t stream_lds_partial_floats(const LdsPlan &pl, int nmat, int m, int n) {
  // per wave: [nmat][ksplit][32*mt][32]
  (void)m;
  (void)n;
  return pl.ksplit > 1
             ? (size_t)pl.groups * pl.row_blocks * kWaves * nmat * pl.ksplit * 32 * pl.mt * 32
             : 0;
}

size_t stream_lds_counter_words(const LdsPlan &pl) { return (size_t)pl.groups * pl.row_blocks; }

hipError_t launch_stream_lds(const void *x, int m, int k, int n, int nmat, const MatRef *w,
                             void *y, float *partial, unsigned *counters, const LdsPlan &pl,
                             hipStream_t stream) {
  LdsArgs p{};
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
  p.ksplit = pl.ksplit;
  p.steps_per_split = pl.steps_per_split;
  p.row_blocks = pl.row_blocks;
  p.rotate = pl.rotate;
  dim3 grid(pl.groups * pl.row_blocks, pl.ksplit);
  if (nmat == 2) {
    switch (pl.mt) {
      case 1: return launch2<1, 2>(p, grid, stream);
      case 2: return launch2<2, 2>(p, grid, stream);
      default: return launch2<8, 2>(p, grid, stream);
    }
  }
  switch (pl.mt) {
    case 1: return launch2<1, 1>(p, grid, stream);
    case 2: return launch2<2, 1>(p, grid, stream);
    default: return launch2<8, 1>(p, grid, stream);
  }
}

}  // namespace nvfp4
