// k_gemv.hip -- NVFP4 projection for 1..4 rows on the vector ALUs (gfx950).
//
// Regime: single-row decode (page layers/dense_ffn_overlays.rs,
// `set_lora_weights`: the split-SiLU decode path is a W4A16 GEMV followed by
// the activation).  At one to four rows a 16x16 MFMA would waste most of
// its rows, and the weight stream from HBM is the whole cost, so the
// dequantize+multiply work per weight must stay far below the bandwidth
// budget (about 2.8 vector ops per weight at 8 TB/s).
//
// Per weight: the hardware fp4 conversion turns a code byte into an exact
// bf16 pair (scale operand 1.0), one v_dot2_f32_bf16 multiplies the pair
// with a register-resident activation pair and accumulates in fp32; each
// 16-element block sum is then multiplied by its E4M3 scale (one fma per
// block and row).  About 1.1 vector ops per weight at one row.
//
// Layout of the work:
//   * A workgroup of KW waves splits K into KW contiguous chunks; lane l of
//     wave w owns the 32-element K granules w*64*G + g*64 + l (g < G), so one
//     128-bit load of a weight row covers 64 consecutive granules (1 KB,
//     fully coalesced).  The lane keeps x for its granules in registers for
//     the whole kernel.
//   * The workgroup walks batches of 8 weight rows (8 columns, or 4 gate +
//     4 up columns for the fused gate+up+silu).  Each lane produces 8 partial
//     sums; a butterfly that halves the list at each exchange leaves lane
//     group l>>3 with column l>>3 summed over all 64 lanes (17 shuffles per
//     batch), then the waves add their chunk sums in fixed wave order.
#include <cstdlib>

#include "launchers.h"
#include "nvfp4_common.h"

namespace nvfp4 {

namespace {

constexpr int kCB = 8;      // weight rows per batch
constexpr int kMaxKW = 8;   // waves per workgroup

struct GemvArgs {
  const void *x;          // bf16 [m][k]
  int m, k, n;
  const uint8_t *codes0, *scales0;
  const uint8_t *codes1, *scales1;
  float ts0, ts1;
  void *y;                // bf16 [m][n]
  int nbatch;
  // LoRA epilogue (lora_xa non-null; see GemvLora)
  const float *lora_xa;
  int lora_nkc, lora_rmax;
  const uint16_t *lora_b[2];
  int lora_r[2];
  float lora_scale[2];
};

// The LoRA epilogue's xa into LDS, once per workgroup: xs[row][i][j] is the
// sum of pair i's chunk partials in chunk order (loads issued four at a
// time, added in order).
template <int M>
__device__ void lora_gather(const GemvArgs &p, float (&xs)[M][2][kMaxRank]) {
  const int rmax = p.lora_rmax, nkc = p.lora_nkc;
  const size_t cstride = (size_t)p.m * rmax;
  for (int idx = threadIdx.x; idx < M * 2 * rmax; idx += blockDim.x) {
    const int j = idx % rmax, i = (idx / rmax) % 2, row = idx / (2 * rmax);
    float v = 0.f;
    if (row < p.m && j < p.lora_r[i]) {
      const float *part = p.lora_xa + (size_t)i * nkc * cstride + (size_t)row * rmax + j;
      int kc = 0;
      for (; kc + 4 <= nkc; kc += 4) {
        const float a0 = part[kc * cstride], a1 = part[(kc + 1) * cstride];
        const float a2 = part[(kc + 2) * cstride], a3 = part[(kc + 3) * cstride];
        v += a0;
        v += a1;
        v += a2;
        v += a3;
      }
      for (; kc < nkc; ++kc) v += part[kc * cstride];
    }
    xs[row][i][j] = v;
  }
}

// v + scale * xa . B[col] for pair i of the LoRA epilogue, rounded to bf16:
// the dot runs in j order with fma -- the arithmetic of the separate LoRA
// passes.  Ranks up to kLoraPre take B[col] from pre (loaded with the
// batch's weights), larger ranks load it here.
constexpr int kLoraPre = 16;
__device__ float lora_apply(const GemvArgs &p, const float *xs, int i, int col, float v, const uint4 (&pre)[2]) {
  const int r = p.lora_r[i];
  if (r == 0) return v;
  auto xa = [&](int j) { return xs[j]; };
  const uint4 *bc = (const uint4 *)(p.lora_b[i] + (size_t)col * r);
  float d = 0.f;
  for (int j8 = 0; j8 < (r >> 3); ++j8) {
    const uint4 bv = r <= kLoraPre ? (j8 == 0 ? pre[0] : pre[1]) : bc[j8];
    const uint32_t bw[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      d = fmaf(xa(8 * j8 + 2 * q), __builtin_bit_cast(float, bw[q] << 16), d);
      d = fmaf(xa(8 * j8 + 2 * q + 1), __builtin_bit_cast(float, bw[q] & 0xFFFF0000u), d);
    }
  }
  return (float)(__bf16)(v + p.lora_scale[i] * d);
}

__device__ __forceinline__ bf16x2 u32_as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

// value of lane (lane ^ O): ds_swizzle's xor mode within 32 lanes, a
// bpermute across the halves
template <int O>
__device__ __forceinline__ float xor_shfl(float v) {
  if constexpr (O >= 32) {
    return __shfl_xor(v, O);
  } else {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                                (O << 10) | 0x1F));
  }
}

// One exchange of the halving butterfly over a list of 2H partial sums: a
// lane keeps the half selected by its lane bit O and adds the partner's
// copy of that half.  Afterwards entry i stands for entry i + H*(bit O).
template <int H, int O>
__device__ __forceinline__ void halve(float *a, int lane) {
  const bool up = (lane & O) != 0;
#pragma unroll
  for (int i = 0; i < H; ++i) {
    const float lo = a[i], hi = a[i + H];
    const float send = up ? lo : hi;
    const float keep = up ? hi : lo;
    a[i] = keep + xor_shfl<O>(send);
  }
}

// LORA: the LoRA epilogue (see GemvLora).  A template argument of the
// kernel itself: the same body behind a device-function wrapper measured
// 0.5 us slower per decode FFN even without the epilogue.
template <int M, int NMAT, int G, bool LORA>
__global__ __launch_bounds__(kMaxKW * 64) void k_gemv(GemvArgs p) {
  static_assert(G <= 3, "granules per lane");
  constexpr int NC = kCB / NMAT;  // output columns per batch
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kw = blockDim.x >> 6;
  const int k = p.k;
  const uint32_t kb2 = (uint32_t)k >> 1, kb16 = (uint32_t)k >> 4;
  const uint32_t gran = (uint32_t)k >> 5;

  uint32_t jg[G];
  bool jok[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    jg[g] = (uint32_t)(wave * 64 * G + g * 64 + lane);
    jok[g] = jg[g] < gran;
  }

  // activations of this lane's granules, as bf16 pairs
  uint32_t xr[M][G][16];
  {
    const __amdgpu_buffer_rsrc_t xres = rsrc(p.x, (size_t)p.m * k * 2);
#pragma unroll
    for (int r = 0; r < M; ++r)
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint32_t off = (jok[g] && r < p.m) ? ((uint32_t)r * (uint32_t)k + jg[g] * 32u) * 2u : kOOB;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 v = ld16(xres, off + 16u * q);
          xr[r][g][4 * q + 0] = v.x;
          xr[r][g][4 * q + 1] = v.y;
          xr[r][g][4 * q + 2] = v.z;
          xr[r][g][4 * q + 3] = v.w;
        }
      }
  }

  __shared__ float red[kMaxKW][kCB][M];
  __shared__ float lxs[LORA ? M : 1][2][LORA ? kMaxRank : 1];  // LoRA epilogue: xa per row and pair

  // weight rows of batch b: 8 code granules and their scale pairs per lane
  // LORA: the B rows of this lane's epilogue column (ranks up to kLoraPre),
  // loaded with the batch's weights so that the epilogue waits on nothing
  // issued after them (loads complete in order)
  auto load_batch = [&](int b, uint4 (&cw)[kCB][G], uint32_t (&sw)[kCB][G], uint4 (&lb)[2][2]) {
    const int c0 = b * NC;
    const int ncols = b < p.nbatch ? min(NC, p.n - c0) : 0;
    __amdgpu_buffer_rsrc_t wres[NMAT], sres[NMAT];
    wres[0] = rsrc(p.codes0 + (size_t)c0 * kb2, (size_t)ncols * kb2);
    sres[0] = rsrc(p.scales0 + (size_t)c0 * kb16, (size_t)ncols * kb16);
    if constexpr (NMAT > 1) {
      wres[1] = rsrc(p.codes1 + (size_t)c0 * kb2, (size_t)ncols * kb2);
      sres[1] = rsrc(p.scales1 + (size_t)c0 * kb16, (size_t)ncols * kb16);
    }
#pragma unroll
    for (int i = 0; i < kCB; ++i) {
      const int mat = i % NMAT;
      const uint32_t col = (uint32_t)(i / NMAT);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        cw[i][g] = ld16_nt(wres[mat], jok[g] ? col * kb2 + jg[g] * 16u : kOOB);
        sw[i][g] = ld2_nt(sres[mat], jok[g] ? col * kb16 + jg[g] * 2u : kOOB);
      }
    }
    if constexpr (LORA) {
      // the epilogue lane of column c of the batch (see compute_batch)
      const int c = NMAT == 2 ? (lane >> 4) : (lane >> 3);
      const bool epi = NMAT == 2 ? (lane & 15) == 0 : (lane & 7) == 0;
#pragma unroll
      for (int i = 0; i < NMAT; ++i) {
        const int r = p.lora_r[i];
        const bool pre = epi && r > 0 && r <= kLoraPre;
        const __amdgpu_buffer_rsrc_t bres = rsrc(p.lora_b[i] + (size_t)c0 * r, (size_t)ncols * r * 2);
#pragma unroll
        for (int h = 0; h < 2; ++h)
          lb[i][h] = ld16(bres, (pre && 8 * h < r) ? (uint32_t)(c * r * 2 + 16 * h) : kOOB);
      }
    }
  };

  auto compute_batch = [&](int b, const uint4 (&cw)[kCB][G], const uint32_t (&sw)[kCB][G],
                           const uint4 (&lb)[2][2]) {
    const int c0 = b * NC;
    const int ncols = min(NC, p.n - c0);
    float v[kCB][M];
#pragma unroll
    for (int i = 0; i < kCB; ++i) {
#pragma unroll
      for (int r = 0; r < M; ++r) v[i][r] = 0.f;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float s[2] = {e4m3_to_f32_sel<0>(sw[i][g]), e4m3_to_f32_sel<1>(sw[i][g])};
        const uint32_t words[4] = {cw[i][g].x, cw[i][g].y, cw[i][g].z, cw[i][g].w};
#pragma unroll
        for (int h = 0; h < 2; ++h) {  // the two 16-element scale blocks
          float blk[M];
#pragma unroll
          for (int r = 0; r < M; ++r) blk[r] = 0.f;
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const uint32_t w = words[2 * h + q];
            bf16x2 c2[4];
            c2[0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
            c2[1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
            c2[2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
            c2[3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
              for (int r = 0; r < M; ++r)
                blk[r] = __builtin_amdgcn_fdot2_f32_bf16(
                    c2[e], u32_as_bf16x2(xr[r][g][(2 * h + q) * 4 + e]), blk[r], false);
          }
#pragma unroll
          for (int r = 0; r < M; ++r) v[i][r] = fmaf(blk[r], s[h], v[i][r]);
        }
      }
    }

    // butterfly: after the exchanges at 32, 16, 8 lane l holds list entry
    // (l >> 3) summed over 8 lanes; then a full sum over the remaining bits
    float tot[M];
#pragma unroll
    for (int r = 0; r < M; ++r) {
      float a[kCB];
#pragma unroll
      for (int i = 0; i < kCB; ++i) a[i] = v[i][r];
      static_assert(kCB == 8, "butterfly written for 8 entries");
      halve<4, 32>(a, lane);
      halve<2, 16>(a, lane);
      halve<1, 8>(a, lane);
      float t = a[0];
      t += xor_shfl<4>(t);
      t += xor_shfl<2>(t);
      t += xor_shfl<1>(t);
      tot[r] = t;
    }

    if (kw > 1) {
      if ((lane & 7) == 0) {
#pragma unroll
        for (int r = 0; r < M; ++r) red[wave][lane >> 3][r] = tot[r];
      }
      __syncthreads();
      if (wave == 0) {
#pragma unroll
        for (int r = 0; r < M; ++r) {
          float t = red[0][lane >> 3][r];
          for (int w = 1; w < kw; ++w) t += red[w][lane >> 3][r];
          tot[r] = t;
        }
      }
      __syncthreads();
    }
    if (wave != 0) return;

#pragma unroll
    for (int r = 0; r < M; ++r) {
      if (r >= p.m) break;
      if constexpr (NMAT == 1) {
        const int c = lane >> 3;
        if ((lane & 7) == 0 && c < ncols) {
          __bf16 o = (__bf16)(tot[r] * p.ts0);
          if constexpr (LORA) o = (__bf16)lora_apply(p, lxs[r][0], 0, c0 + c, (float)o, lb[0]);
          ((__bf16 *)p.y)[(size_t)r * p.n + c0 + c] = o;
        }
      } else {
        const float up = xor_shfl<8>(tot[r]);  // entry 2c+1 (up) next to 2c (gate)
        const int c = lane >> 4;
        if ((lane & 15) == 0 && c < ncols) {
          const size_t o = (size_t)r * p.n + c0 + c;
          if constexpr (LORA) {  // deltas on the bf16 gate and up, then silu_mul
            const float gb = lora_apply(p, lxs[r][0], 0, c0 + c, (float)(__bf16)(tot[r] * p.ts0), lb[0]);
            const float ub = lora_apply(p, lxs[r][1], 1, c0 + c, (float)(__bf16)(up * p.ts1), lb[1]);
            ((__bf16 *)p.y)[o] = (__bf16)(silu_f32(gb) * ub);
          } else {
            ((__bf16 *)p.y)[o] = swiglu_bf16(tot[r] * p.ts0, up * p.ts1);
          }
        }
      }
    }
  };

  // two register sets: the loads of the next batch are in flight while the
  // current one is computed
  uint4 cwA[kCB][G], cwB[kCB][G];
  uint32_t swA[kCB][G], swB[kCB][G];
  int b = blockIdx.x;
  uint4 lbA[2][2] = {}, lbB[2][2] = {};
  load_batch(b, cwA, swA, lbA);
  if constexpr (LORA) {  // while the first batch's weights are in flight
    lora_gather<M>(p, lxs);
    __syncthreads();
  }
  for (; b < p.nbatch; b += 2 * gridDim.x) {
    const int b1 = b + gridDim.x;
    load_batch(b1, cwB, swB, lbB);
    compute_batch(b, cwA, swA, lbA);
    if (b1 >= p.nbatch) break;
    const int b2 = b1 + gridDim.x;
    load_batch(b2, cwA, swA, lbA);
    compute_batch(b1, cwB, swB, lbB);
  }
}


int gemv_target_waves() {
  static const int t = [] {
    const char *v = getenv("NVFP4_GEMV_WAVES");
    const int n = v ? atoi(v) : 0;
    return n > 0 ? n : 2048;
  }();
  return t;
}

struct GemvShape {
  int kw, g;
};

int gmax_for_rows(int m) { return m == 1 ? 3 : (m == 2 ? 2 : 1); }

// Fewest granules per lane (lightest registers, most waves in flight) that
// keep the workgroup within kMaxKW waves.
GemvShape gemv_shape(int m, int k) {
  const int gran = k / 32;
  GemvShape s;
  s.g = cdiv(gran, 64 * kMaxKW);
  if (s.g < 1) s.g = 1;
  s.kw = cdiv(gran, 64 * s.g);
  (void)m;
  return s;
}

template <int M, int NMAT, int G>
hipError_t launch_g(const GemvArgs &p, int kw, hipStream_t st) {
  // about 2048 waves in flight; every workgroup walks the same number of
  // batches
  const int per_wg = cdiv(p.nbatch * kw, gemv_target_waves());
  const int grid = cdiv(p.nbatch, per_wg);
  if (p.lora_xa)
    hipLaunchKernelGGL((k_gemv<M, NMAT, G, true>), dim3(grid), dim3(64 * kw), 0, st, p);
  else
    hipLaunchKernelGGL((k_gemv<M, NMAT, G, false>), dim3(grid), dim3(64 * kw), 0, st, p);
  return hipGetLastError();
}

template <int M, int NMAT>
hipError_t launch_m(const GemvArgs &p, const GemvShape &s, hipStream_t st) {
  switch (s.g) {
    case 1: return launch_g<M, NMAT, 1>(p, s.kw, st);
    case 2: return launch_g<M, NMAT, (M <= 2 ? 2 : 1)>(p, s.kw, st);
    default: return launch_g<M, NMAT, (M == 1 ? 3 : 1)>(p, s.kw, st);
  }
}

template <int NMAT>
hipError_t launch_n(const GemvArgs &p, const GemvShape &s, hipStream_t st) {
  switch (p.m) {
    case 1: return launch_m<1, NMAT>(p, s, st);
    case 2: return launch_m<2, NMAT>(p, s, st);
    case 3: return launch_m<3, NMAT>(p, s, st);
    default: return launch_m<4, NMAT>(p, s, st);
  }
}

}  // namespace

bool gemv_eligible(int m, int k) {
  if (m < 1 || m > 4) return false;
  const GemvShape s = gemv_shape(m, k);
  return s.kw <= kMaxKW && s.g <= gmax_for_rows(m);
}

hipError_t launch_gemv(const void *x, int m, int k, int n, int nmat, const MatRef *w, void *y,
                       hipStream_t stream, const GemvLora *lora) {
  GemvArgs p{};
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
  p.nbatch = cdiv(n, kCB / nmat);
  if (lora) {
    p.lora_xa = lora->xa;
    p.lora_nkc = lora->nkc;
    p.lora_rmax = lora->rmax;
    for (int i = 0; i < 2; ++i) {
      p.lora_b[i] = (const uint16_t *)lora->b[i];
      p.lora_r[i] = i < nmat ? lora->r[i] : 0;
      p.lora_scale[i] = lora->scale[i];
    }
  }
  const GemvShape s = gemv_shape(m, k);
  return nmat == 1 ? launch_n<1>(p, s, stream) : launch_n<2>(p, s, stream);
}

}  // namespace nvfp4
