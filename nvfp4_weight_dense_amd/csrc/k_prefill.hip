// k_prefill.hip -- NVFP4 projection for many rows (gfx950), bound by bf16
// MFMA throughput.
//
// Regime: above the small-m edge the pages' prefill GEMM switches to tiles
// of 128 rows (page layers/dense_ffn_prefill.rs, `w4a16_prefill_gemm`); with
// thousands of rows every weight element meets many activation rows, so the
// cost that matters besides the MFMAs is the in-register dequantization
// (about two VALU instructions per weight element).
//
// Workgroup: four waves, 256 rows.  Each wave owns 256 rows x two 32-column
// B tiles -- gate and up at the same columns (SWIGLU), or two adjacent
// column tiles of one matrix -- so a dequantized B fragment feeds eight
// v_mfma_f32_32x32x16_bf16 and an activation fragment read from LDS feeds
// two.  Accumulators: 2 x 8 x 16 fp32 per lane (the AGPR file).
//
// Step (64 K): rows x 64 K of bf16 activations sit in one of two LDS slots
// (row pitch 144 bytes: conflict-free 16-byte fragment reads).  Software
// pipeline, per step t:
//   * MFMA group j (0..3) of step t consumes A fragments of LDS slot t%2
//     and B fragments dequantized from a three-deep register ring of codes
//     (loaded three steps ahead); the fragments of group j+1 are read and
//     dequantized while group j runs;
//   * the activation chunk of step t+1 (loaded into registers during step
//     t) is written to the other LDS slot, then the chunk of step t+2 is
//     requested; one barrier closes the step.
// Lane (c = lane%32, h = lane/32) holds for weight row col+c the 32 codes at
// K offset 32h of the step; MFMA j sums K offsets {8j..8j+7} U
// {32+8j..32+8j+7}, and the A fragment of row tile mt is read at LDS row
// 32mt+c at the same offsets.
//
// Grid: blockIdx.x = row block + row_blocks * column group (consecutive
// workgroups, dealt round-robin to the eight XCDs, take different row blocks
// of the same columns; with eight row blocks each XCD's L2 keeps one
// activation block), blockIdx.y = K split.  With ksplit > 1 each wave writes
// fp32 partial tiles and the last-arriving workgroup of a tile sums them in
// split order (deterministic) before the epilogue.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <type_traits>

#include "launchers.h"
#include "nvfp4_common.h"

namespace nvfp4 {

namespace {

constexpr int kWaves = 4;
constexpr int kStep = 64;                  // K elements per step
constexpr int kRowBytes = kStep * 2 + 16;  // LDS row pitch

struct PrefillArgs {
  const void *x;  // bf16 [m][k]
  int m, k, n;
  const uint8_t *codes0, *scales0;  // gate (SWIGLU) or the matrix
  const uint8_t *codes1, *scales1;  // up (SWIGLU) or unused
  float ts0, ts1;
  void *y;
  float *partial;      // per wave: [NB][ksplit][32*MT][32]
  unsigned *counters;  // [gridDim.x], zero between calls
  int ksplit, steps_per_split;
  int row_blocks;
};

// MT: 32-row tiles per workgroup; NBC: 32-column tiles per wave and matrix
// (gate and up each with SWIGLU); NB = B tiles per wave.
template <int MT, int NBC, bool SWIGLU>
__global__ __launch_bounds__(kWaves * 64) void k_prefill(PrefillArgs p) {
  constexpr int kMT = MT;
  constexpr int kRows = 32 * MT;
  constexpr int kNB = SWIGLU ? 2 * NBC : NBC;
  __shared__ __attribute__((aligned(16))) uint8_t lds0[kRows * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[kRows * kRowBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31;
  const int h = lane >> 5;
  const int k = p.k;
  const uint32_t kb2 = (uint32_t)k >> 1, kb16 = (uint32_t)k >> 4;
  const int nsteps = (k + kStep - 1) / kStep;
  const int s_begin = blockIdx.y * p.steps_per_split;
  const int len = max(0, min(nsteps, s_begin + p.steps_per_split) - s_begin);

  const int rb = (int)(blockIdx.x % (unsigned)p.row_blocks);
  const int cg = (int)(blockIdx.x / (unsigned)p.row_blocks);
  const int row0 = rb * kRows;
  const int rows = min(kRows, p.m - row0);

  // this wave's B tiles: columns col[i] .. col[i]+31
  int col[kNB];
  __amdgpu_buffer_rsrc_t wc[kNB], ws[kNB];
#pragma unroll
  for (int i = 0; i < kNB; ++i) {
    // tile i: column tile i % NBC of the wave; with SWIGLU tiles NBC.. are up
    col[i] = (cg * kWaves + wave) * (32 * NBC) + 32 * (i % NBC);
    const bool up = SWIGLU && i >= NBC;
    const uint8_t *cb = up ? p.codes1 : p.codes0;
    const uint8_t *sb = up ? p.scales1 : p.scales0;
    const int nc = max(0, min(32, p.n - col[i]));
    const size_t base = (size_t)min(col[i], p.n);
    wc[i] = rsrc(cb + base * kb2, (size_t)nc * kb2);
    ws[i] = rsrc(sb + base * kb16, (size_t)nc * kb16);
  }
  const __amdgpu_buffer_rsrc_t xres =
      rsrc((const uint8_t *)p.x + (size_t)row0 * k * 2, (size_t)max(rows, 0) * k * 2);

  // activation chunk: 16-byte pieces, row = piece / 8, byte 16 * (piece % 8);
  // thread tid moves pieces tid + 256 i
  constexpr int kPerThread = kRows * 8 / (kWaves * 64);
  // (a piece's K offset within the step, 8 * (tid % 8), is the same for all i)
  const uint32_t kin = 8u * (uint32_t)(tid & 7);
  uint32_t aoff[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int r = (tid + kWaves * 64 * i) >> 3;
    aoff[i] = r < rows ? ((uint32_t)r * (uint32_t)k + kin) * 2u : kOOB;
  }
  uint4 areg[kPerThread];
  auto load_a = [&](int tl) {
    const uint32_t kk = (uint32_t)(s_begin + tl) * kStep;
    const bool ok = tl < len && kk + kin < (uint32_t)k;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i)
      areg[i] = ld16(xres, (ok && aoff[i] != kOOB) ? aoff[i] + kk * 2u : kOOB);
  };
  auto store_a = [&](uint8_t *slot) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int piece = tid + kWaves * 64 * i;
      *(uint4 *)&slot[(piece >> 3) * kRowBytes + 16 * (piece & 7)] = areg[i];
    }
  };

  // weight codes / scales of one step: a three-deep register ring
  uint4 bw[3][kNB];
  uint32_t bs[3][kNB];
  auto load_b = [&](int tl, uint4 (&w)[kNB], uint32_t (&s)[kNB]) {
    const uint32_t kk = (uint32_t)(s_begin + tl) * kStep + 32u * (uint32_t)h;
    const bool ok = tl < len && kk < (uint32_t)k;
#pragma unroll
    for (int i = 0; i < kNB; ++i) {
      w[i] = ld16(wc[i], ok ? (uint32_t)c32 * kb2 + (kk >> 1) : kOOB);
      s[i] = ld2(ws[i], ok ? (uint32_t)c32 * kb16 + (kk >> 4) : kOOB);
    }
  };
  auto dequant_j = [&](const uint4 (&w)[kNB], const uint32_t (&s)[kNB], int j, bf16x8 (&out)[kNB]) {
#pragma unroll
    for (int i = 0; i < kNB; ++i) {
      const float sc = j < 2 ? e4m3_to_f32_sel<0>(s[i]) : e4m3_to_f32_sel<1>(s[i]);
      const uint32_t word = j == 0 ? w[i].x : j == 1 ? w[i].y : j == 2 ? w[i].z : w[i].w;
      out[i] = dequant8(word, sc);
    }
  };

  f32x16 acc[kNB][kMT];
#pragma unroll
  for (int i = 0; i < kNB; ++i)
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][mt][e] = 0.f;

  // prologue: B codes of steps 0..2, A chunk 0 in LDS, chunk 1 in flight
  load_b(0, bw[0], bs[0]);
  load_b(1, bw[1], bs[1]);
  load_b(2, bw[2], bs[2]);
  load_a(0);
  store_a(lds0);
  load_a(1);
  __syncthreads();

  auto read_a = [&](const uint8_t *slot, int j, bf16x8 (&af)[kMT]) {
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
      af[mt] = as_bf16x8(*(const uint4 *)&slot[(mt * 32 + c32) * kRowBytes + 2 * (32 * h + 8 * j)]);
  };

  // one step; slot_c = t % 6 picks the LDS slot (t % 2) and the ring slot
  // of step t (t % 3) at compile time.  Fragments of MFMA group j+1 (A from
  // LDS, B dequantized from the ring) are prepared while group j runs.
  auto step = [&](int tl, auto slot_c) {
    constexpr int s6 = decltype(slot_c)::value;
    const uint8_t *cur = (s6 % 2) ? lds1 : lds0;
    uint8_t *nxt = (s6 % 2) ? lds0 : lds1;
    constexpr int rs = s6 % 3;  // ring slot of step t, refilled with step t+3
    bf16x8 af[2][kMT];
    bf16x8 bf[2][kNB];
    read_a(cur, 0, af[0]);
    dequant_j(bw[rs], bs[rs], 0, bf[0]);
    // (scheduling groups are filled in order by instruction kind: this
    // first group takes the reads of group 0)
    __builtin_amdgcn_sched_group_barrier(0x100, kMT, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j < 3) {
        read_a(cur, j + 1, af[(j + 1) & 1]);
        dequant_j(bw[rs], bs[rs], j + 1, bf[(j + 1) & 1]);
      }
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int i = 0; i < kNB; ++i)
          acc[i][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[j & 1][mt], bf[j & 1][i], acc[i][mt], 0, 0, 0);
      // issue order of the group: the next group's LDS reads first, then
      // each MFMA followed by up to four VALU instructions (the next
      // dequant), which run while the MFMA occupies the matrix pipe
      if (j < 3) __builtin_amdgcn_sched_group_barrier(0x100, kMT, 0);
#pragma unroll
      for (int q = 0; q < kMT * kNB; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
    }
    load_b(tl + 3, bw[rs], bs[rs]);
    // (unconditional, so the step stays one basic block: after the last
    // step the other slot is not read again)
    store_a(nxt);
    load_a(tl + 2);
    // the chunk's LDS writes after all MFMAs, so its loads (issued a step
    // earlier) have had the whole step to arrive
    __builtin_amdgcn_sched_group_barrier(0x200, kPerThread, 0);
    __syncthreads();
  };
  for (int tl = 0; tl < len; tl += 6) {
    step(tl, std::integral_constant<int, 0>{});
    if (tl + 1 < len) step(tl + 1, std::integral_constant<int, 1>{});
    if (tl + 2 < len) step(tl + 2, std::integral_constant<int, 2>{});
    if (tl + 3 < len) step(tl + 3, std::integral_constant<int, 3>{});
    if (tl + 4 < len) step(tl + 4, std::integral_constant<int, 4>{});
    if (tl + 5 < len) step(tl + 5, std::integral_constant<int, 5>{});
  }

  // lane's element e of row tile mt: row 32mt + 8(e/4) + 4h + e%4, column col[i] + c32
  if (p.ksplit > 1) {
    constexpr int kTile = kRows * 32;
    const size_t wtile = (size_t)blockIdx.x * kWaves + wave;
    const __amdgpu_buffer_rsrc_t pres =
        rsrc(p.partial + wtile * kNB * p.ksplit * kTile, (size_t)kNB * p.ksplit * kTile * 4);
#pragma unroll
    for (int i = 0; i < kNB; ++i)
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const uint32_t r = mt * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
          st_coherent(pres, (((uint32_t)(i * p.ksplit + blockIdx.y) * kTile) + r * 32u + c32) * 4u,
                      acc[i][mt][e]);
        }
    __shared__ unsigned last;
    wait_all_memory();
    __syncthreads();
    if (tid == 0) {
      const unsigned old = __hip_atomic_fetch_add(&p.counters[blockIdx.x], 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      last = old == (unsigned)(p.ksplit - 1);
    }
    __syncthreads();
    if (!last) return;
#pragma unroll
    for (int i = 0; i < kNB; ++i)
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][mt][e] = 0.f;
    // split order outermost; four tiles' loads in flight at a time
    for (int sp = 0; sp < p.ksplit; ++sp) {
#pragma unroll
      for (int c0 = 0; c0 < kNB * kMT; c0 += 4) {
        float v[4][16];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int i = (c0 + c) / kMT, mt = (c0 + c) % kMT;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const uint32_t r = mt * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
            v[c][e] = ld_coherent(pres, (((uint32_t)(i * p.ksplit + sp) * kTile) + r * 32u + c32) * 4u);
          }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int i = (c0 + c) / kMT, mt = (c0 + c) % kMT;
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[i][mt][e] += v[c][e];
        }
      }
    }
    if (tid == 0)
      __hip_atomic_store(&p.counters[blockIdx.x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // rows past m fall outside the output resource and are dropped
  const __amdgpu_buffer_rsrc_t yres =
      rsrc((uint8_t *)p.y + (size_t)row0 * p.n * 2, (size_t)max(rows, 0) * p.n * 2);
  if constexpr (SWIGLU) {
#pragma unroll
    for (int i = 0; i < NBC; ++i) {
      const int c = col[i] + c32;
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const uint32_t r = mt * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
          st2(yres, c < p.n ? (r * (uint32_t)p.n + c) * 2u : kOOB,
              swiglu_bf16(acc[i][mt][e] * p.ts0, acc[NBC + i][mt][e] * p.ts1));
        }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kNB; ++i) {
      const int c = col[i] + c32;
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const uint32_t r = mt * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
          st2(yres, c < p.n ? (r * (uint32_t)p.n + c) * 2u : kOOB, (__bf16)(acc[i][mt][e] * p.ts0));
        }
    }
  }
}

}  // namespace

// Tile shape: 256 rows x one tile per matrix (gate+up) or two (one matrix)
// per wave, or 128 rows x twice as many column tiles (half the LDS reads per
// MFMA, twice the dequantization).  NVFP4_PREFILL_SHAPE=<mt>x<nbc> selects
// one of the built shapes for measurements.
static void prefill_shape(int nmat, int *mt, int *nbc) {
  *mt = 8;
  *nbc = nmat == 2 ? 1 : 2;
  if (const char *v = getenv("NVFP4_PREFILL_SHAPE")) {
    int a = 0, b = 0;
    if (sscanf(v, "%dx%d", &a, &b) == 2 &&
        ((a == 8 && b == 3 - nmat) || (a == 4 && b == 2 * (3 - nmat)))) {
      *mt = a;
      *nbc = b;
    }
  }
}

PrefillPlan prefill_plan(int m, int n, int k, int nmat) {
  PrefillPlan pl;
  prefill_shape(nmat, &pl.mt, &pl.nbc);
  pl.row_blocks = cdiv(m, 32 * pl.mt);
  pl.groups = cdiv(n, kWaves * 32 * pl.nbc);
  const int nsteps = cdiv(k, kStep);
  const int tiles = pl.groups * pl.row_blocks;
  // One workgroup per CU.  Split K when the tiles leave CUs idle: time is
  // proportional to rounds / ksplit, plus the fp32 partial tiles (256 KB per
  // workgroup and split, written and read back) weighed against the
  // workgroup's MFMA work, which shrinks with K / ksplit (measured: about 4%
  // per split at K = 17408).
  const int slots = 256;
  int best_ks = 1;
  double best = 1e30;
  for (int ks = 1; ks <= 8; ++ks) {
    if (nsteps / ks < 8) break;  // keep at least eight steps per split
    const double rounds = std::ceil((double)tiles * ks / slots);
    double t = rounds / ks;
    if (ks > 1) t *= 1.0 + 0.04 * ks * 17408.0 / k;
    if (t < best - 1e-9) {
      best = t;
      best_ks = ks;
    }
  }
  pl.steps_per_split = cdiv(nsteps, best_ks);
  pl.ksplit = cdiv(nsteps, pl.steps_per_split);
  return pl;
}

size_t prefill_partial_floats(const PrefillPlan &pl) {
  // per wave: [NB][ksplit][32*mt][32], NB * mt = 16 for every built shape
  return pl.ksplit > 1 ? (size_t)pl.groups * pl.row_blocks * kWaves * 16 * pl.ksplit * 32 * 32 : 0;
}

size_t prefill_counter_words(const PrefillPlan &pl) { return (size_t)pl.groups * pl.row_blocks; }

hipError_t launch_prefill(const void *x, int m, int k, int n, int nmat, const MatRef *w, void *y,
                          float *partial, unsigned *counters, const PrefillPlan &pl,
                          hipStream_t stream) {
  PrefillArgs p{};
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
  dim3 grid(pl.groups * pl.row_blocks, pl.ksplit), block(kWaves * 64);
  if (nmat == 2) {
    if (pl.mt == 4) hipLaunchKernelGGL((k_prefill<4, 2, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((k_prefill<8, 1, true>), grid, block, 0, stream, p);
  } else {
    if (pl.mt == 4) hipLaunchKernelGGL((k_prefill<4, 4, false>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((k_prefill<8, 2, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
