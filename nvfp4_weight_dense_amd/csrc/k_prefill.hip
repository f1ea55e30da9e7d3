// k_prefill.hip -- NVFP4 projection for many rows (gfx950), bound by bf16
// MFMA throughput.
//
// Regime: above the small-m edge the pages' prefill GEMM switches to tiles
// of 128 rows (page layers/dense_ffn_prefill.rs, `w4a16_prefill_gemm`); with
// thousands of rows every weight element meets many activation rows, so the
// cost that matters besides the MFMAs is the in-register dequantization
// (about two VALU instructions per weight element).
//
// Workgroup: four waves, 32*MT rows (MT = 8, 6, 5 or 4, chosen per shape so
// that the tiles fill the CUs' rounds best).  Each wave owns those rows x
// two 32-column B tiles -- gate and up at the same columns (SWIGLU), or two
// adjacent column tiles of one matrix -- so a dequantized B fragment feeds
// MT v_mfma_f32_32x32x16_bf16 and an activation fragment read from LDS
// feeds two.  Accumulators: 2 x MT x 16 fp32 per lane (the AGPR file).
//
// Step (64 K): rows x 64 K of bf16 activations sit in one of two LDS slots
// (row pitch 144 bytes: conflict-free 16-byte fragment reads); the chunk of
// step t+1 goes global -> registers during step t and into the other slot
// at its end.  MFMA group j (0..3) of a step consumes A fragments read one
// group ahead and B fragments dequantized one group ahead.
//
// Weights move in groups of four steps -- 128 code bytes, one cache line,
// of each weight row -- straight from memory into a two-slot LDS ring with
// 16-byte LDS-DMA loads (buffer_load ... lds): one instruction moves eight
// rows x 128 bytes (eight full lines), so a group of a 32-row tile costs
// four instructions.  Each wave owns its slot region, so the ring needs no
// barrier, only the wave's own load counter, and a group is requested three
// steps before use.  Within a row the eight 16-byte chunks are
// stored XOR-swizzled by row, which keeps the per-lane 16-byte reads
// (lane c, half h: row c, chunk 2q+h of step q) free of bank conflicts.  The
// E4M3 scales of a group (16 bytes per row) come in one register load.
// The step barrier waits for LDS operations only, so the weight and
// activation loads stay in flight across it.
//
// Lane (c = lane%32, h = lane/32) holds for weight row col+c the 32 codes at
// K offset 32h of the step; MFMA j sums K offsets {8j..8j+7} U
// {32+8j..32+8j+7}, and the A fragment of row tile mt is read at LDS row
// 32mt+c at the same offsets.
//
// Schedule: one persistent workgroup per CU walks tiles (row block
// fastest) round-robin.  Workgroups are dealt round-robin to the eight XCDs,
// so with eight row blocks each XCD works on one activation block, which
// stays in its L2, and the eight workgroups that share a column group's
// weights run at the same time.  (Splitting tiles over workgroups by K, with
// fp32 partials handed over through memory, was measured slower on every
// shape tried: the split parts lose the L2 sharing and the hand-off reads
// wait on memory latency.)
//
// Requires k % 64 == 0 (whole steps).  When k % 256 != 0 the last weight
// group is partial: the steps it lacks are never run, so the code bytes its
// requests bring from beyond each row's end are never read, and its scales
// come a dword (one step) at a time -- for every group, since the scale
// rows are then only 4-byte aligned -- so that no scale load reaches past
// the last row's end, where a 16-byte load would straddle the resource
// bound.
#include <algorithm>
#include <cstdint>
#include <initializer_list>
#include <cmath>
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
  int gshift;              // packed-Q2 weights: scale group = 1 << gshift
  void *y;
  int ldy;                 // row stride of y in elements (>= n)
  int row_blocks, groups;  // tile = column group * row_blocks + row block
  int nwg;                 // persistent workgroups (gridDim.x)
};

// MT: 32-row tiles per workgroup; NBC: 32-column tiles per wave and matrix
// (gate and up each with SWIGLU); NB = B tiles per wave.  Q2: packed-Q2
// weights instead of NVFP4 (q2_table in nvfp4_common.h).
template <int MT, int NBC, bool SWIGLU, bool Q2>
__global__ __launch_bounds__(kWaves * 64) void k_prefill(PrefillArgs p) {
  constexpr int kMT = MT;
  constexpr int kRows = 32 * MT;
  constexpr int kNB = SWIGLU ? 2 * NBC : NBC;
  // steps per weight group: a group is 128 code bytes of a row either way
  // (4 steps of NVFP4 at 32 bytes, 8 steps of packed Q2 at 16 bytes)
  constexpr int kGroup = Q2 ? 8 : 4;
  constexpr uint32_t kStepBytes = Q2 ? 16u : 32u;  // code bytes of a row per step
  __shared__ __attribute__((aligned(16))) uint8_t lds0[kRows * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[kRows * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t wb0[kWaves * kNB * 32 * 32 * 4];
  __shared__ __attribute__((aligned(16))) uint8_t wb1[kWaves * kNB * 32 * 32 * 4];

  const int nsteps = (p.k + kStep - 1) / kStep;
  const int tiles = p.row_blocks * p.groups;

  // one segment: steps [s_begin, s_begin + len) of tile `tile` (the same in
  // every lane; readfirstlane lets the compiler know, so per-step
  // conditions stay scalar branches)
  auto segment = [&](int tile_, int s_begin_, int len_) __attribute__((always_inline)) {
  const int tile = __builtin_amdgcn_readfirstlane(tile_);
  const int s_begin = __builtin_amdgcn_readfirstlane(s_begin_);
  const int len = __builtin_amdgcn_readfirstlane(len_);
  // Lane indices and shape values are re-derived here, through empty asm,
  // for every segment: otherwise the compiler hoists everything computed
  // from them (hundreds of per-lane offsets) out of the segment loop and
  // spills it, since the step loop leaves no registers free.
  int tid_v = (int)threadIdx.x, k_v = p.k;
  asm volatile("" : "+v"(tid_v));
  asm volatile("" : "+s"(k_v));
  const int tid = tid_v;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31;
  const int h = lane >> 5;
  const int k = k_v;
  // bytes per weight row: codes, and scales (E4M3 per 16 K; fp16 per group)
  const uint32_t kb2 = Q2 ? (uint32_t)k >> 2 : (uint32_t)k >> 1;
  const uint32_t kb16 = Q2 ? ((uint32_t)k >> p.gshift) * 2u : (uint32_t)k >> 4;
  const int cg = tile / p.row_blocks;
  const int rb = tile - cg * p.row_blocks;
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
    wc[i] = rsrc_uniform(cb + base * kb2, (size_t)nc * kb2);
    ws[i] = rsrc_uniform(sb + base * kb16, (size_t)nc * kb16);
  }
  const __amdgpu_buffer_rsrc_t xres =
      rsrc_uniform((const uint8_t *)p.x + (size_t)row0 * k * 2, (size_t)max(rows, 0) * k * 2);

  // activation chunk: 16-byte pieces, row = piece / 8, byte 16 * (piece % 8);
  // thread tid moves pieces tid + 256 i, i.e. row tid/8 + 32 i at K offset
  // 8 (tid % 8) of the step (MT pieces per thread).  The per-lane part of
  // the address is one VGPR, the 32 i rows go in the scalar offset; rows
  // past m fall outside xres.
  constexpr int kPerThread = kRows * 8 / (kWaves * 64);
  static_assert(kPerThread * kWaves * 64 == kRows * 8, "activation pieces per thread");
  const uint32_t kin = 8u * (uint32_t)(tid & 7);
  const uint32_t avoff = ((uint32_t)(tid >> 3) * (uint32_t)k + kin) * 2u;
  uint4 areg[kPerThread];
  auto load_a = [&](int tl) {
    const uint32_t kk = (uint32_t)(s_begin + tl) * kStep;
    const uint32_t vo = tl < len ? avoff + kk * 2u : kOOB;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) areg[i] = ld16s(xres, vo, (uint32_t)(32 * i) * (uint32_t)k * 2u);
  };
  auto store_a = [&](uint8_t *slot) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int piece = tid + kWaves * 64 * i;
      *(uint4 *)&slot[(piece >> 3) * kRowBytes + 16 * (piece & 7)] = areg[i];
    }
  };

  // weight groups: codes through the LDS ring, scales through registers
  // DMA lane mapping: instruction g moves rows 8g..8g+7; lane l loads row
  // 8g + l/8, chunk (l%8) ^ (l/8), and lands at 16 l
  const uint32_t drow = (uint32_t)lane >> 3, dchunk = ((uint32_t)lane & 7) ^ drow;
  // read side: row c32 = 8g + a sits in instruction g, lane 8a + (x ^ a);
  // step q of the group is chunk x = 2q + h (NVFP4: 16 bytes per lane) or
  // chunk q, bytes 8h.. (packed Q2: 8 bytes per lane)
  const uint32_t ra = (uint32_t)c32 & 7;
  uint32_t coff[kGroup];
#pragma unroll
  for (int q = 0; q < kGroup; ++q)
    coff[q] = (uint32_t)(wave * kNB * 4 + (c32 >> 3)) * 1024u +
              (Q2 ? 16u * (8u * ra + ((uint32_t)q ^ ra)) + 8u * (uint32_t)h
                  : 16u * (8u * ra + ((2u * q + h) ^ ra)));
  auto load_group = [&](int G, uint8_t *slot) {
    const uint32_t goff = (uint32_t)(s_begin + kGroup * G) * kStepBytes;
    const bool ok = kGroup * G < len;
#pragma unroll
    for (int i = 0; i < kNB; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        dma16(wc[i], slot + ((wave * kNB + i) * 4 + g) * 1024,
              ok ? (8u * g + drow) * kb2 + goff + 16u * dchunk : kOOB);
  };
  // packed Q2: lane (c32, h) needs one fp16 scale per step, that of K
  // 64 t + 32 h (a lane's 32 K values lie in one group, group >= 32); step t's
  // scales are loaded two steps ahead into slot t % 4
  uint32_t qs[4][kNB];
  auto load_q2_scales = [&](int tl, uint32_t (&sv)[kNB]) {
    const uint32_t kk = (uint32_t)(s_begin + tl) * 64u + 32u * (uint32_t)h;
    const uint32_t o = tl < len ? (uint32_t)c32 * kb16 + (kk >> p.gshift) * 2u : kOOB;
#pragma unroll
    for (int i = 0; i < kNB; ++i) sv[i] = ld2(ws[i], o);
  };
  uint4 sc[2][kNB];
  auto load_scales = [&](int G, uint4 (&sv)[kNB]) {
    if constexpr (Q2) return;
    const uint32_t goff = (uint32_t)(s_begin + kGroup * G) * 4u;
    const int nst = len - kGroup * G;  // steps of this group that run (uniform)
    if (nst >= kGroup && (kb16 & 15u) == 0) {
#pragma unroll
      for (int i = 0; i < kNB; ++i) sv[i] = ld16(ws[i], (uint32_t)c32 * kb16 + goff);
    } else {
      // k % 256 != 0 (scale rows only 4-byte aligned; the last group
      // partial) or past the end: one dword per step that runs
      const uint32_t o = (uint32_t)c32 * kb16 + goff;
#pragma unroll
      for (int i = 0; i < kNB; ++i)
        sv[i] = uint4{ld4(ws[i], nst > 0 ? o : kOOB), ld4(ws[i], nst > 1 ? o + 4u : kOOB),
                      ld4(ws[i], nst > 2 ? o + 8u : kOOB), ld4(ws[i], nst > 3 ? o + 12u : kOOB)};
    }
  };
  // NVFP4: w holds the step's 32 codes of the lane, s its two scale bytes.
  // Packed Q2: w.xy holds the 32 two-bit codes, s the two table dwords.
  auto dequant_j = [&](const uint4 (&w)[kNB], const uint32_t (&s)[kNB][2], int j, bf16x8 (&out)[kNB]) {
#pragma unroll
    for (int i = 0; i < kNB; ++i) {
      if constexpr (Q2) {
        const uint32_t word = j < 2 ? w[i].x : w[i].y;
        out[i] = q2_dequant8((j & 1) ? word >> 16 : word & 0xFFFFu, s[i][0], s[i][1]);
      } else {
        const float sc_ = j < 2 ? e4m3_to_f32_sel<0>(s[i][0]) : e4m3_to_f32_sel<1>(s[i][0]);
        const uint32_t word = j == 0 ? w[i].x : j == 1 ? w[i].y : j == 2 ? w[i].z : w[i].w;
        out[i] = dequant8(word, sc_);
      }
    }
  };

  f32x16 acc[kNB][kMT];
#pragma unroll
  for (int i = 0; i < kNB; ++i)
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][mt][e] = 0.f;

  // prologue: weight group 0, A chunk 0 in LDS, chunk 1 in flight (every
  // wave has finished with the LDS of the previous segment)
  lds_barrier();
  load_group(0, wb0);
  load_scales(0, sc[0]);
  if constexpr (Q2) {
    load_q2_scales(0, qs[0]);
    load_q2_scales(1, qs[1]);
  }
  load_a(0);
  store_a(lds0);
  load_a(1);
  lds_barrier();

  auto read_a = [&](const uint8_t *slot, int j, bf16x8 (&af)[kMT]) {
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
      af[mt] = as_bf16x8(*(const uint4 *)&slot[(mt * 32 + c32) * kRowBytes + 2 * (32 * h + 8 * j)]);
  };

  // one step; slot_c = t % (2 kGroup) fixes at compile time the A slot
  // (t % 2), the weight-ring slot (t / kGroup % 2), the step within its
  // group (t % kGroup) and, for packed Q2, the scale slot (t % 4)
  auto step = [&](int tl, auto slot_c) {
    constexpr int s8 = decltype(slot_c)::value;
    constexpr int q = s8 % kGroup, bsl = (s8 / kGroup) % 2;
    const uint8_t *cur = (s8 % 2) ? lds1 : lds0;
    uint8_t *nxt = (s8 % 2) ? lds0 : lds1;
    const uint8_t *bcur = bsl ? wb1 : wb0;
    uint4 w[kNB];
    uint32_t sw[kNB][2];
#pragma unroll
    for (int i = 0; i < kNB; ++i) {
      if constexpr (Q2) {
        const uint2 c2 = *(const uint2 *)&bcur[coff[q] + i * 4 * 1024];
        w[i] = uint4{c2.x, c2.y, 0u, 0u};
        q2_table(qs[s8 % 4][i], sw[i][0], sw[i][1]);
      } else {
        w[i] = *(const uint4 *)&bcur[coff[q] + i * 4 * 1024];
        const uint32_t d = q == 0 ? sc[bsl][i].x : q == 1 ? sc[bsl][i].y : q == 2 ? sc[bsl][i].z : sc[bsl][i].w;
        sw[i][0] = d >> (16u * h);
      }
    }
    if constexpr (Q2) load_q2_scales(tl + 2, qs[(s8 + 2) % 4]);
    if constexpr (q == 1) {
      // second step of a group: request the next group into the other slot
      // (last read before the previous barrier), three steps ahead of use.
      // Pinned after this step's code reads: the load-counter wait the
      // compiler places before a ring read then covers only older requests.
      __builtin_amdgcn_sched_barrier(0);
      load_group(tl / kGroup + 1, bsl ? wb0 : wb1);
      load_scales(tl / kGroup + 1, sc[bsl ^ 1]);
    }
    bf16x8 af[2][kMT];
    bf16x8 bf[2][kNB];
    read_a(cur, 0, af[0]);
    dequant_j(w, sw, 0, bf[0]);
    // (scheduling groups are filled in order by instruction kind: this
    // first group takes the reads of group 0)
    __builtin_amdgcn_sched_group_barrier(0x100, kMT, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j < 3) {
        read_a(cur, j + 1, af[(j + 1) & 1]);
        dequant_j(w, sw, j + 1, bf[(j + 1) & 1]);
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
      for (int qq = 0; qq < kMT * kNB; ++qq) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
    }
    // (unconditional, so the step stays one basic block: after the last
    // step the other slot is not read again)
    store_a(nxt);
    load_a(tl + 2);
    // the chunk's LDS writes after all MFMAs, so its loads (issued a step
    // earlier) have had the whole step to arrive
    __builtin_amdgcn_sched_group_barrier(0x200, kPerThread, 0);
    lds_barrier();
  };
  for (int tl = 0; tl < len; tl += 2 * kGroup) {
    step(tl, std::integral_constant<int, 0>{});
    if (tl + 1 < len) step(tl + 1, std::integral_constant<int, 1>{});
    if (tl + 2 < len) step(tl + 2, std::integral_constant<int, 2>{});
    if (tl + 3 < len) step(tl + 3, std::integral_constant<int, 3>{});
    if (tl + 4 < len) step(tl + 4, std::integral_constant<int, 4>{});
    if (tl + 5 < len) step(tl + 5, std::integral_constant<int, 5>{});
    if (tl + 6 < len) step(tl + 6, std::integral_constant<int, 6>{});
    if (tl + 7 < len) step(tl + 7, std::integral_constant<int, 7>{});
    if constexpr (Q2) {
      if (tl + 8 < len) step(tl + 8, std::integral_constant<int, 8>{});
      if (tl + 9 < len) step(tl + 9, std::integral_constant<int, 9>{});
      if (tl + 10 < len) step(tl + 10, std::integral_constant<int, 10>{});
      if (tl + 11 < len) step(tl + 11, std::integral_constant<int, 11>{});
      if (tl + 12 < len) step(tl + 12, std::integral_constant<int, 12>{});
      if (tl + 13 < len) step(tl + 13, std::integral_constant<int, 13>{});
      if (tl + 14 < len) step(tl + 14, std::integral_constant<int, 14>{});
      if (tl + 15 < len) step(tl + 15, std::integral_constant<int, 15>{});
    }
  }
  // the last group request may still be in flight; the LDS it targets is not
  // read again, but it must land before the workgroup's LDS is released
  wait_all_memory();

  // lane's element e of row tile mt: row 32mt + 8(e/4) + 4h + e%4, column col[i] + c32
  // rows past m fall outside the output resource and are dropped
  const __amdgpu_buffer_rsrc_t yres =
      rsrc_uniform((uint8_t *)p.y + (size_t)row0 * p.ldy * 2, (size_t)max(rows, 0) * p.ldy * 2);
  // element (mt, e): row 32mt + 8(e/4) + 4h + e%4 -- the 4h row and the
  // column are the per-lane part, the rest is uniform (scalar offset)
  const uint32_t n2 = (uint32_t)p.ldy * 2u;
  if constexpr (SWIGLU) {
#pragma unroll
    for (int i = 0; i < NBC; ++i) {
      const int c = col[i] + c32;
      const uint32_t vo = c < p.n ? (uint32_t)(4 * h) * n2 + (uint32_t)c * 2u : kOOB;
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          st2s(yres, vo, (uint32_t)(mt * 32 + 8 * (e >> 2) + (e & 3)) * n2,
               swiglu_bf16(acc[i][mt][e] * p.ts0, acc[NBC + i][mt][e] * p.ts1));
    }
  } else {
#pragma unroll
    for (int i = 0; i < kNB; ++i) {
      const int c = col[i] + c32;
      const uint32_t vo = c < p.n ? (uint32_t)(4 * h) * n2 + (uint32_t)c * 2u : kOOB;
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          st2s(yres, vo, (uint32_t)(mt * 32 + 8 * (e >> 2) + (e & 3)) * n2,
               (__bf16)(acc[i][mt][e] * p.ts0));
    }
  }
  };  // segment

  // this workgroup's tiles, round-robin (one call site, so the tile body is
  // inlined)
  for (int t = (int)blockIdx.x; t < tiles; t += p.nwg) segment(t, 0, nsteps);
}

}  // namespace

// compute units of the current device (one persistent workgroup each)
static int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

namespace {

struct PartCost {
  int mt, row_blocks, groups;
  long cost;
};

// tile height for a column range of `cols` columns, charged rounds x (6 + MT)
PartCost best_part(int m, int cols, int cw, int cus, std::initializer_list<int> mts) {
  PartCost best{0, 0, 0, -1};
  for (int mt : mts) {
    const int rb = cdiv(m, 32 * mt), g = cdiv(cols, cw);
    const long cost = (long)cdiv(rb * g, cus) * (6 + mt);
    if (best.cost < 0 || cost < best.cost) best = {mt, rb, g, cost};
  }
  return best;
}

}  // namespace

PrefillPlan prefill_plan(int m, int n, int k, int nmat) {
  (void)k;
  // Tile height: 32 * MT rows.  A workgroup's time per K step grows with MT
  // plus a part that does not (weight groups, B dequantization, the step
  // barrier): measured about 6 MT-units of fixed cost per step.  Persistent
  // workgroups walk the tiles in rounds of one per CU, so a column range is
  // charged rounds x (6 + MT) and the cheapest height wins (ties to the
  // taller tile, which reuses each weight fragment most).  When the tiles
  // overflow their last round, the columns may instead be split: a first
  // launch over whole rounds of tall tiles, a second over the remaining
  // column groups with short tiles that fill one round.
  const int cus = device_cus();
  const int nbc = nmat == 2 ? 1 : 2;
  const int cw = kWaves * 32 * nbc;  // columns per column group
  PrefillPlan pl{};
  pl.nbc = nbc;
  const PartCost one = best_part(m, n, cw, cus, {8, 6, 5, 4, 2});
  pl.mt = one.mt;
  pl.row_blocks = one.row_blocks;
  pl.groups = one.groups;
  pl.n_bulk = n;
  long best_cost = one.cost;
  for (int mt : {8, 6, 5, 4}) {
    const int rb = cdiv(m, 32 * mt), g = cdiv(n, cw);
    const long tiles = (long)rb * g;
    if (tiles <= cus) continue;
    const int gb = (int)((tiles / cus) * cus / rb);  // column groups in whole rounds
    if (gb <= 0 || gb >= g) continue;
    const PartCost rest = best_part(m, n - gb * cw, cw, cus, {8, 6, 5, 4, 2});
    const long cost = (long)cdiv(gb * rb, cus) * (6 + mt) + rest.cost;
    if (cost < best_cost) {
      best_cost = cost;
      pl.mt = mt;
      pl.row_blocks = rb;
      pl.groups = gb;
      pl.n_bulk = gb * cw;
      pl.mt2 = rest.mt;
      pl.row_blocks2 = rest.row_blocks;
      pl.groups2 = rest.groups;
    }
  }
  pl.nwg = std::max(1, std::min(cus, pl.row_blocks * pl.groups));
  pl.nwg2 = pl.n_bulk < n ? std::max(1, std::min(cus, pl.row_blocks2 * pl.groups2)) : 0;
  return pl;
}

namespace {

template <bool Q2>
hipError_t launch_part(PrefillArgs p, int nmat, int mt, hipStream_t stream) {
  dim3 grid(p.nwg), block(kWaves * 64);
  switch ((nmat == 2 ? 100 : 0) + mt) {
    case 108: hipLaunchKernelGGL((k_prefill<8, 1, true, Q2>), grid, block, 0, stream, p); break;
    case 106: hipLaunchKernelGGL((k_prefill<6, 1, true, Q2>), grid, block, 0, stream, p); break;
    case 105: hipLaunchKernelGGL((k_prefill<5, 1, true, Q2>), grid, block, 0, stream, p); break;
    case 104: hipLaunchKernelGGL((k_prefill<4, 1, true, Q2>), grid, block, 0, stream, p); break;
    case 102: hipLaunchKernelGGL((k_prefill<2, 1, true, Q2>), grid, block, 0, stream, p); break;
    case 8: hipLaunchKernelGGL((k_prefill<8, 2, false, Q2>), grid, block, 0, stream, p); break;
    case 6: hipLaunchKernelGGL((k_prefill<6, 2, false, Q2>), grid, block, 0, stream, p); break;
    case 5: hipLaunchKernelGGL((k_prefill<5, 2, false, Q2>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((k_prefill<4, 2, false, Q2>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((k_prefill<2, 2, false, Q2>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Both launches of a plan; codes/scales of matrix i start at w_codes[i] /
// w_scales[i], with code and scale bytes per weight row cb and sb.
template <bool Q2>
hipError_t launch_plan(PrefillArgs p, int n, int nmat, const uint8_t *const *w_codes,
                       const uint8_t *const *w_scales, size_t cb, size_t sb, void *y,
                       const PrefillPlan &pl, hipStream_t stream) {
  // columns [c0, c0 + cols) of every matrix and of y
  auto part = [&](int c0, int cols, int mt, int rb, int groups, int nwg) {
    p.n = cols;
    p.codes0 = w_codes[0] + (size_t)c0 * cb;
    p.scales0 = w_scales[0] + (size_t)c0 * sb;
    p.codes1 = nmat > 1 ? w_codes[1] + (size_t)c0 * cb : nullptr;
    p.scales1 = nmat > 1 ? w_scales[1] + (size_t)c0 * sb : nullptr;
    p.y = (uint8_t *)y + (size_t)c0 * 2;
    p.row_blocks = rb;
    p.groups = groups;
    p.nwg = nwg;
    return launch_part<Q2>(p, nmat, mt, stream);
  };
  hipError_t e = part(0, pl.n_bulk, pl.mt, pl.row_blocks, pl.groups, pl.nwg);
  if (e != hipSuccess || pl.n_bulk >= n) return e;
  return part(pl.n_bulk, n - pl.n_bulk, pl.mt2, pl.row_blocks2, pl.groups2, pl.nwg2);
}

}  // namespace

hipError_t launch_prefill(const void *x, int m, int k, int n, int nmat, const MatRef *w, void *y,
                          const PrefillPlan &pl, hipStream_t stream) {
  PrefillArgs p{};
  p.x = x;
  p.m = m;
  p.k = k;
  p.ldy = n;
  p.ts0 = w[0].ts;
  p.ts1 = nmat > 1 ? w[1].ts : 0.f;
  const uint8_t *codes[2] = {w[0].codes, nmat > 1 ? w[1].codes : nullptr};
  const uint8_t *scales[2] = {w[0].scales, nmat > 1 ? w[1].scales : nullptr};
  return launch_plan<false>(p, n, nmat, codes, scales, (size_t)(k / 2), (size_t)(k / 16), y, pl, stream);
}

hipError_t launch_prefill_q2(const void *x, int m, int k, int n, int gshift, int nmat, const Q2MatRef *w,
                             void *y, const PrefillPlan &pl, hipStream_t stream) {
  PrefillArgs p{};
  p.x = x;
  p.m = m;
  p.k = k;
  p.ldy = n;
  p.ts0 = 1.0f;
  p.ts1 = 1.0f;
  p.gshift = gshift;
  const uint8_t *codes[2] = {w[0].codes, nmat > 1 ? w[1].codes : nullptr};
  const uint8_t *scales[2] = {(const uint8_t *)w[0].scales, nmat > 1 ? (const uint8_t *)w[1].scales : nullptr};
  return launch_plan<true>(p, n, nmat, codes, scales, (size_t)(k / 4), (size_t)(k >> gshift) * 2, y, pl,
                           stream);
}

}  // namespace nvfp4
