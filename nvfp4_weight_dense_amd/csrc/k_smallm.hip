// k_smallm.hip -- weight-streaming NVFP4 projection for 17..64 rows (gfx950).
//
// Regime: the pages' small-m edge (page layers/dense_ffn_prefill.rs,
// `w4a16_prefill_gemm`: m <= 64 takes the small-m kernels).  With tens of
// rows the weights are still the whole HBM stream, so the kernel is built
// around moving them at full bandwidth:
//
//   * weights move in groups of four 64-K steps -- 128 code bytes, one cache
//     line, of each weight row -- straight into LDS with 16-byte LDS-DMA
//     loads (buffer_load ... lds; one instruction moves eight whole lines).
//     Each wave owns its region of a two-slot ring and requests a group
//     three steps before use.
//     Within a row the eight 16-byte chunks are XOR-swizzled by row, which
//     keeps the per-lane 16-byte reads in MFMA operand order free of bank
//     conflicts.  A group's E4M3 scales (16 bytes per row) come in one
//     register load.
//   * a workgroup is two waves; each wave owns 32 columns of gate and of up
//     (fused silu epilogue), or 64 columns of one matrix, for all 32 or 64
//     rows (v_mfma_f32_32x32x16_bf16); three workgroups share a CU, and K
//     is split until every SIMD has a wave.
//   * the activation chunk of a step (rows x 64 K, bf16) is loaded into
//     registers two steps ahead and written into a two-slot LDS ring one
//     step ahead; the step barrier waits for LDS operations only, so weight
//     and activation requests stay in flight.
//   * deep K is split over workgroups (blockIdx.y) by whole weight groups;
//     each split writes fp32 partial tiles.  For gate+up (two splits at
//     most on these shapes) the last split to arrive sums them in split
//     order and runs the silu epilogue; for one matrix a second launch sums
//     them in split order over the whole output in parallel.
//
// Lane (c = lane%32, h = lane/32) holds for weight row col+c the 32 codes at
// K offset 32h of a step; MFMA j sums K offsets {8j..8j+7} U
// {32+8j..32+8j+7}, and the A fragment of row tile mt is read at LDS row
// 32mt+c at the same offsets.  Requires k % 64 == 0 (whole steps).  When
// k % 256 != 0 the last weight group of the last split is partial: the
// steps it lacks are never run (the code bytes its requests bring from
// beyond each row's end are never read), and the scales come a dword (one
// step) at a time, since the scale rows are then only 4-byte aligned and a
// 16-byte load could straddle the end of the last row.
#include <algorithm>
#include <type_traits>

#include "launchers.h"
#include "nvfp4_common.h"

namespace nvfp4 {

namespace {

constexpr int kNW = 2;                     // waves per workgroup
constexpr int kStep = 64;                  // K elements per step
constexpr int kGroup = 4;                  // steps per weight group
constexpr int kRing = 2;                   // weight groups in the LDS ring
constexpr int kRowBytes = kStep * 2 + 16;  // LDS row pitch of the activation chunk
constexpr int kNB = 2;                     // B tiles per wave
constexpr int kTileBytes = 32 * 32 * kGroup;  // one B tile's group: 32 rows x 128 B

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct SmallArgs {
  const void *x;  // bf16 [m][k]
  int m, k, n;
  const uint8_t *codes0, *scales0;  // gate (SWIGLU) or the matrix
  const uint8_t *codes1, *scales1;  // up (SWIGLU) or unused
  float ts0, ts1;
  void *y;
  float *partial;      // [tiles][ksplit][kNW][kNB * 32MT * 32]
  unsigned *counters;  // [tiles], zero between calls
  int ksplit, steps_per_split;
};

__device__ __forceinline__ void st16_coherent(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                              f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff, soff, kCoherent);
}
__device__ __forceinline__ f32x4 ld16_coherent(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kCoherent));
}

template <int MT, bool SWIGLU>
__global__ __launch_bounds__(kNW * 64) void k_smallm(SmallArgs p) {
  constexpr int kRows = 32 * MT;
  constexpr int NBC = SWIGLU ? 1 : 2;  // column tiles per wave and matrix
  __shared__ __attribute__((aligned(16))) uint8_t lds0[kRows * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[kRows * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t wb0[kNW * kNB * kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t wb1[kNW * kNB * kTileBytes];
  __shared__ unsigned last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c32 = lane & 31;
  const int h = lane >> 5;
  const int k = p.k;
  const uint32_t kb2 = (uint32_t)k >> 1, kb16 = (uint32_t)k >> 4;
  const int nsteps = k / kStep;
  const int tile = (int)blockIdx.x;
  const int split = (int)blockIdx.y;
  const int s_begin = split * p.steps_per_split;
  const int len = max(0, min(nsteps, s_begin + p.steps_per_split) - s_begin);
  const int rows = min(kRows, p.m);

  // this wave's B tiles: columns col[i] .. col[i]+31
  int col[kNB];
  __amdgpu_buffer_rsrc_t wc[kNB], ws[kNB];
#pragma unroll
  for (int i = 0; i < kNB; ++i) {
    col[i] = (tile * kNW + wave) * (32 * NBC) + 32 * (i % NBC);
    const bool up = SWIGLU && i >= NBC;
    const uint8_t *cb = up ? p.codes1 : p.codes0;
    const uint8_t *sb = up ? p.scales1 : p.scales0;
    const int nc = max(0, min(32, p.n - col[i]));
    const size_t base = (size_t)min(col[i], p.n);
    wc[i] = rsrc_uniform(cb + base * kb2, (size_t)nc * kb2);
    ws[i] = rsrc_uniform(sb + base * kb16, (size_t)nc * kb16);
  }
  const __amdgpu_buffer_rsrc_t xres = rsrc_uniform(p.x, (size_t)rows * k * 2);

  // activation chunk: 16-byte pieces, row = piece / 8, byte 16 * (piece % 8);
  // thread tid moves pieces tid + 128 i (row tid/8 + 16 i); rows past m fall
  // outside xres and read as zero
  constexpr int kPerThread = kRows * 8 / (kNW * 64);
  const uint32_t kin = 8u * (uint32_t)(tid & 7);
  const uint32_t avoff = ((uint32_t)(tid >> 3) * (uint32_t)k + kin) * 2u;
  uint4 areg[2][kPerThread];
  auto load_a = [&](int tl, uint4 (&a)[kPerThread]) {
    const uint32_t kk = (uint32_t)(s_begin + tl) * kStep;
    const uint32_t vo = tl < len ? avoff + kk * 2u : kOOB;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) a[i] = ld16s(xres, vo, (uint32_t)(16 * i) * (uint32_t)k * 2u);
  };
  auto store_a = [&](uint8_t *slot, const uint4 (&a)[kPerThread]) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int piece = tid + kNW * 64 * i;
      *(uint4 *)&slot[(piece >> 3) * kRowBytes + 16 * (piece & 7)] = a[i];
    }
  };

  // weight groups: DMA lane l moves row 8g + l/8, chunk (l%8) ^ (l/8) of
  // instruction g and lands at 16 l; row c32 = 8g + a is read back from
  // instruction g, lane 8a + (x ^ a) for chunk x = 2q + h of step q
  const uint32_t drow = (uint32_t)lane >> 3, dchunk = ((uint32_t)lane & 7) ^ drow;
  const uint32_t ra = (uint32_t)c32 & 7;
  uint32_t coff[kGroup];
#pragma unroll
  for (int q = 0; q < kGroup; ++q)
    coff[q] = (uint32_t)(wave * kNB * 4 + (c32 >> 3)) * 1024u + 16u * (8u * ra + ((2u * q + h) ^ ra));
  auto load_group = [&](int G, uint8_t *slot) {
    const uint32_t goff = (uint32_t)(s_begin + kGroup * G) * 32u;
    const bool ok = kGroup * G < len;
#pragma unroll
    for (int i = 0; i < kNB; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        dma16(wc[i], slot + ((wave * kNB + i) * 4 + g) * 1024,
              ok ? (8u * g + drow) * kb2 + goff + 16u * dchunk : kOOB);
  };
  uint4 sc[kRing][kNB];
  auto load_scales = [&](int G, uint4 (&sv)[kNB]) {
    const uint32_t goff = (uint32_t)(s_begin + kGroup * G) * 4u;
    const int nst = len - kGroup * G;  // steps of this group that run (uniform)
    if (nst >= kGroup && (kb16 & 15u) == 0) {
#pragma unroll
      for (int i = 0; i < kNB; ++i) sv[i] = ld16(ws[i], (uint32_t)c32 * kb16 + goff);
    } else {
      const uint32_t o = (uint32_t)c32 * kb16 + goff;
#pragma unroll
      for (int i = 0; i < kNB; ++i)
        sv[i] = uint4{ld4(ws[i], nst > 0 ? o : kOOB), ld4(ws[i], nst > 1 ? o + 4u : kOOB),
                      ld4(ws[i], nst > 2 ? o + 8u : kOOB), ld4(ws[i], nst > 3 ? o + 12u : kOOB)};
    }
  };
  auto dequant_j = [&](const uint4 (&w)[kNB], const uint32_t (&s)[kNB], int j, bf16x8 (&out)[kNB]) {
#pragma unroll
    for (int i = 0; i < kNB; ++i) {
      const float sc_ = j < 2 ? e4m3_to_f32_sel<0>(s[i]) : e4m3_to_f32_sel<1>(s[i]);
      const uint32_t word = j == 0 ? w[i].x : j == 1 ? w[i].y : j == 2 ? w[i].z : w[i].w;
      out[i] = dequant8(word, sc_);
    }
  };
  auto read_a = [&](const uint8_t *slot, int j, bf16x8 (&af)[MT]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      af[mt] = as_bf16x8(*(const uint4 *)&slot[(mt * 32 + c32) * kRowBytes + 2 * (32 * h + 8 * j)]);
  };

  f32x16 acc[kNB][MT];
#pragma unroll
  for (int i = 0; i < kNB; ++i)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][mt][e] = 0.f;

  // prologue: weight group 0 requested, A chunk 0 in LDS, chunk 1 in
  // registers
  load_group(0, wb0);
  load_scales(0, sc[0]);
  load_a(0, areg[0]);
  load_a(1, areg[1]);
  store_a(lds0, areg[0]);
  lds_barrier();

  // one step; slot_c = t % 8 fixes at compile time the A slot and register
  // set (t % 2), the ring slot of the step's group (t / 4 % 2) and the step
  // within it (t % 4).  Activation chunks are loaded two steps ahead and
  // written to LDS one step ahead (into the slot read two steps ago).
  auto step = [&](int tl, auto slot_c) {
    constexpr int s8 = decltype(slot_c)::value;
    constexpr int q = s8 % kGroup, bsl = (s8 / kGroup) % kRing, sa = s8 % 2;
    const uint8_t *cur = sa ? lds1 : lds0;
    uint8_t *nxt = sa ? lds0 : lds1;
    const uint8_t *bcur = bsl ? wb1 : wb0;
    uint4 w[kNB];
    uint32_t sw[kNB];
#pragma unroll
    for (int i = 0; i < kNB; ++i) {
      w[i] = *(const uint4 *)&bcur[coff[q] + i * 4 * 1024];
      const uint32_t d = q == 0 ? sc[bsl][i].x : q == 1 ? sc[bsl][i].y : q == 2 ? sc[bsl][i].z : sc[bsl][i].w;
      sw[i] = d >> (16u * h);
    }
    if constexpr (q == 1) {
      // request the next group into the other slot (read during the previous
      // group, finished before the last barrier), three steps ahead of use;
      // pinned after this step's reads so the load-counter wait before a
      // ring read covers only older requests
      __builtin_amdgcn_sched_barrier(0);
      load_group(tl / kGroup + 1, bsl ? wb0 : wb1);
      load_scales(tl / kGroup + 1, sc[bsl ^ 1]);
    }
    bf16x8 af[2][MT];
    bf16x8 bf[2][kNB];
    read_a(cur, 0, af[0]);
    dequant_j(w, sw, 0, bf[0]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j < 3) {
        read_a(cur, j + 1, af[(j + 1) & 1]);
        dequant_j(w, sw, j + 1, bf[(j + 1) & 1]);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < kNB; ++i)
          acc[i][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[j & 1][mt], bf[j & 1][i], acc[i][mt], 0, 0, 0);
    }
    // (unconditional, so the step stays one basic block: after the last
    // step the slot is not read again)
    store_a(nxt, areg[sa ^ 1]);
    load_a(tl + 2, areg[sa]);
    lds_barrier();
  };
  for (int tl = 0; tl < len; tl += 8) {
    step(tl, std::integral_constant<int, 0>{});
    if (tl + 1 < len) step(tl + 1, std::integral_constant<int, 1>{});
    if (tl + 2 < len) step(tl + 2, std::integral_constant<int, 2>{});
    if (tl + 3 < len) step(tl + 3, std::integral_constant<int, 3>{});
    if (tl + 4 < len) step(tl + 4, std::integral_constant<int, 4>{});
    if (tl + 5 < len) step(tl + 5, std::integral_constant<int, 5>{});
    if (tl + 6 < len) step(tl + 6, std::integral_constant<int, 6>{});
    if (tl + 7 < len) step(tl + 7, std::integral_constant<int, 7>{});
  }
  // group requests past the split may still be in flight; they must land
  // before the workgroup's LDS is released
  wait_all_memory();

  if (p.ksplit > 1) {
    // per wave: [q = (i*MT + mt)*4 + e/4][lane][e%4], 16 contiguous bytes
    // per lane and 1 KB per instruction
    constexpr int kWaveFloats = kNB * kRows * 32;
    const uint32_t pvoff = (uint32_t)lane * 16u;
    auto pres_of = [&](int sp) {
      return rsrc_uniform(p.partial + (((size_t)tile * p.ksplit + sp) * kNW + wave) * kWaveFloats,
                          (size_t)kWaveFloats * 4);
    };
    {
      const __amdgpu_buffer_rsrc_t pres = pres_of(split);
#pragma unroll
      for (int i = 0; i < kNB; ++i)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            const f32x4 v = {acc[i][mt][4 * e4], acc[i][mt][4 * e4 + 1], acc[i][mt][4 * e4 + 2],
                             acc[i][mt][4 * e4 + 3]};
            st16_coherent(pres, pvoff, (uint32_t)((i * MT + mt) * 4 + e4) * 1024u, v);
          }
    }
    if (!SWIGLU) return;  // k_smallm_reduce sums the splits
    wait_all_memory();
    __syncthreads();
    if (tid == 0) {
      const unsigned old =
          __hip_atomic_fetch_add(&p.counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last = old == (unsigned)(p.ksplit - 1);
    }
    __syncthreads();
    if (!last) return;
#pragma unroll
    for (int i = 0; i < kNB; ++i)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][mt][e] = 0.f;
    // split order outermost; all of one split's loads in flight together
    for (int sp = 0; sp < p.ksplit; ++sp) {
      const __amdgpu_buffer_rsrc_t pres = pres_of(sp);
      f32x4 v[kNB * MT * 4];
#pragma unroll
      for (int q = 0; q < kNB * MT * 4; ++q) v[q] = ld16_coherent(pres, pvoff, (uint32_t)q * 1024u);
#pragma unroll
      for (int q = 0; q < kNB * MT * 4; ++q) {
        const int i = q / (4 * MT), mt = (q / 4) % MT, e4 = q % 4;
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[i][mt][4 * e4 + t] += v[q][t];
      }
    }
    if (tid == 0)
      __hip_atomic_store(&p.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // element (mt, e): row 32mt + 8(e/4) + 4h + e%4; the 4h row and the column
  // are the per-lane part of the offset, the rest is uniform; rows past m
  // fall outside the output resource and are dropped
  const __amdgpu_buffer_rsrc_t yres = rsrc_uniform(p.y, (size_t)rows * p.n * 2);
  const uint32_t n2 = (uint32_t)p.n * 2u;
#pragma unroll
  for (int i = 0; i < (SWIGLU ? 1 : kNB); ++i) {
    const int c = col[i] + c32;
    const uint32_t vo = c < p.n ? (uint32_t)(4 * h) * n2 + (uint32_t)c * 2u : kOOB;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const __bf16 out = SWIGLU ? swiglu_bf16(acc[0][mt][e] * p.ts0, acc[1][mt][e] * p.ts1)
                                  : (__bf16)(acc[i][mt][e] * p.ts0);
        st2s(yres, vo, (uint32_t)(mt * 32 + 8 * (e >> 2) + (e & 3)) * n2, out);
      }
  }
}

// The split sum of a one-matrix launch, in parallel over the whole output:
// one thread per 16-byte partial chunk (four rows of one column), summing
// the splits in split order -- the order the in-kernel sum of the fused
// gate+up launch uses -- then the epilogue.  With one workgroup per tile
// doing the sum, a deep K split left one CU per tile reading every split's
// partials at the end of the launch.
template <int MT>
__global__ __launch_bounds__(256) void k_smallm_reduce(const float *__restrict__ partial, int tiles,
                                                       int ksplit, int m, int n, float ts, void *y) {
  constexpr int kRows = 32 * MT;
  constexpr int kWaveFloats = kNB * kRows * 32;
  constexpr int kChunks = kNB * MT * 4 * 64;  // 16-byte chunks per wave
  const int gid = (int)(blockIdx.x * 256 + threadIdx.x);
  if (gid >= tiles * kNW * kChunks) return;
  const int tile = gid / (kNW * kChunks);
  const int rem = gid - tile * (kNW * kChunks);
  const int wave = rem / kChunks;
  const int q = (rem - wave * kChunks) >> 6, lane = rem & 63;
  const int i = q / (4 * MT), mt = (q >> 2) % MT, e4 = q & 3;
  const float4 *src = (const float4 *)(partial + ((size_t)tile * ksplit * kNW + wave) * kWaveFloats) +
                      (size_t)q * 64 + lane;
  const size_t split_stride = (size_t)kNW * kWaveFloats / 4;  // in float4
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < ksplit; ++sp) {
    const float4 v = src[sp * split_stride];
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  const int col = (tile * kNW + wave) * 64 + 32 * i + (lane & 31);
  if (col >= n) return;
  const int row0 = 32 * mt + 8 * e4 + 4 * (lane >> 5);
  const float v[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
  for (int t = 0; t < 4; ++t)
    if (row0 + t < m) ((__bf16 *)y)[(size_t)(row0 + t) * n + col] = (__bf16)(v[t] * ts);
}

}  // namespace

bool smallm_eligible(int m, int k) { return m >= 17 && m <= 64 && k % 64 == 0; }

SmallPlan smallm_plan(int m, int n, int k, int nmat) {
  SmallPlan pl;
  pl.mt = m <= 32 ? 1 : 2;
  pl.tiles = cdiv(n, kNW * 32 * (nmat == 2 ? 1 : 2));
  const int nsteps = k / kStep;
  // Three workgroups per CU are resident (about 50 KB of LDS each); split K
  // as far as every split workgroup still fits in one round, by whole
  // weight groups and with at least eight steps per split, so that all
  // SIMDs get a wave.  The split depends on (n, k) only.
  const int slots = 3 * 256;
  int ksplit = std::max(1, slots / pl.tiles);
  ksplit = std::min(ksplit, std::max(1, nsteps / 8));
  if (k < splitk_min_k()) ksplit = 1;
  pl.steps_per_split = cdiv(cdiv(nsteps, ksplit), kGroup) * kGroup;
  pl.ksplit = cdiv(nsteps, pl.steps_per_split);
  (void)m;
  return pl;
}

size_t smallm_partial_floats(const SmallPlan &pl) {
  return pl.ksplit > 1 ? (size_t)pl.tiles * pl.ksplit * kNW * kNB * 32 * pl.mt * 32 : 0;
}

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
  p.ksplit = pl.ksplit;
  p.steps_per_split = pl.steps_per_split;
  dim3 grid(pl.tiles, pl.ksplit), block(kNW * 64);
  if (nmat == 2) {
    if (pl.mt == 1) hipLaunchKernelGGL((k_smallm<1, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((k_smallm<2, true>), grid, block, 0, stream, p);
    return hipGetLastError();
  }
  if (pl.mt == 1) hipLaunchKernelGGL((k_smallm<1, false>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((k_smallm<2, false>), grid, block, 0, stream, p);
  if (pl.ksplit > 1) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int threads = pl.tiles * kNW * kNB * pl.mt * 4 * 64;
    const dim3 rgrid((threads + 255) / 256);
    if (pl.mt == 1)
      hipLaunchKernelGGL((k_smallm_reduce<1>), rgrid, dim3(256), 0, stream, partial, pl.tiles, pl.ksplit, m,
                         n, p.ts0, y);
    else
      hipLaunchKernelGGL((k_smallm_reduce<2>), rgrid, dim3(256), 0, stream, partial, pl.tiles, pl.ksplit, m,
                         n, p.ts0, y);
  }
  return hipGetLastError();
}

}  // namespace nvfp4
