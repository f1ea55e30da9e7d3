// k_tiled.hip -- LDS-tiled NVFP4 projection for many rows (gfx950).
//
// Regime: above the small-m edge the pages' prefill GEMM switches to
// M128 tiles (page layers/dense_ffn_prefill.rs, `w4a16_prefill_gemm`); with
// thousands of rows the projection is bound by bf16 MFMA throughput.
//
// Tile: 128 rows x 128 columns x 64 K per step, four waves in a 2x2 grid,
// each owning 64x64 outputs as 2x2 tiles of v_mfma_f32_32x32x16_bf16.
//   * Activations (bf16) are staged through LDS, double-buffered, rows
//     padded by 16 bytes.
//   * Weights never touch LDS: lane (c = lane%32, h = lane/32) loads 16 bytes
//     of codes (K offset 32h of the step) and 2 scale bytes of its column
//     straight into registers -- 4.5 bits per element make this cheap -- and
//     dequantizes them to four bf16 B fragments.  MFMA j of the step sums K
//     offsets {8j..8j+7} U {32+8j..32+8j+7}; the A fragments read the same
//     offsets from LDS.
#include "launchers.h"
#include "nvfp4_common.h"

namespace nvfp4 {

namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDS_LD = BK + 8;  // bf16 per LDS row (144 bytes)

__global__ __launch_bounds__(256) void k_tiled(const uint16_t *__restrict__ x, int m, int k,
                                              const uint8_t *__restrict__ codes,
                                              const uint8_t *__restrict__ scales, float ts,
                                              int n, uint16_t *__restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * LDS_LD];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int row0 = blockIdx.y * BM;
  const int col0 = blockIdx.x * BN;
  const int l32 = lane & 31;
  const int h = lane >> 5;
  const int nk = cdiv(k, BK);

  // weight rows of this lane (two 32-column tiles)
  const uint8_t *crow[2];
  const uint8_t *srow[2];
  bool cok[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    int c = col0 + wn * 64 + ct * 32 + l32;
    cok[ct] = c < n;
    size_t cr = (size_t)(cok[ct] ? c : 0);
    crow[ct] = codes + cr * (size_t)(k >> 1);
    srow[ct] = scales + cr * (size_t)(k >> 4);
  }

  const uint4 z4 = make_uint4(0, 0, 0, 0);
  uint4 areg[4];
  auto load_a = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 256 * i;
      const int r = id >> 3, ch = id & 7;
      const int gr = row0 + r;
      const int kk = kb * BK + ch * 8;
      areg[i] = (gr < m && kk < k) ? *(const uint4 *)(x + (size_t)gr * k + kk) : z4;
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 256 * i;
      const int r = id >> 3, ch = id & 7;
      *(uint4 *)&As[buf][r * LDS_LD + ch * 8] = areg[i];
    }
  };
  uint4 bw[2];
  uint32_t bs[2];
  auto load_b = [&](int kb, uint4 *w, uint32_t *s) {
    const int kk = kb * BK + 32 * h;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const bool ok = cok[ct] && kk < k;
      w[ct] = ok ? *(const uint4 *)(crow[ct] + (kk >> 1)) : z4;
      s[ct] = ok ? (uint32_t)*(const uint16_t *)(srow[ct] + (kk >> 4)) : 0u;
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.f;

  load_a(0);
  load_b(0, bw, bs);
  store_a(0);
  __syncthreads();

  for (int kb = 0; kb < nk; ++kb) {
    const int cur = kb & 1;
    uint4 bw_n[2];
    uint32_t bs_n[2];
    const bool more = kb + 1 < nk;
    if (more) {
      load_a(kb + 1);
      load_b(kb + 1, bw_n, bs_n);
    }
    bf16x8 bf[2][4];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const float s0 = e4m3_to_f32_sel<0>(bs[ct]);
      const float s1 = e4m3_to_f32_sel<1>(bs[ct]);
      bf[ct][0] = dequant8(bw[ct].x, s0);
      bf[ct][1] = dequant8(bw[ct].y, s0);
      bf[ct][2] = dequant8(bw[ct].z, s1);
      bf[ct][3] = dequant8(bw[ct].w, s1);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const uint4 av = *(const uint4 *)&As[cur][(wm * 64 + rt * 32 + l32) * LDS_LD + 32 * h + 8 * j];
        const bf16x8 af = as_bf16x8(av);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
          acc[rt][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf[ct][j], acc[rt][ct], 0, 0, 0);
      }
    }
    if (more) store_a(cur ^ 1);
    __syncthreads();
    if (more) {
      bw[0] = bw_n[0];
      bw[1] = bw_n[1];
      bs[0] = bs_n[0];
      bs[1] = bs_n[1];
    }
  }

  // lane holds rows 8*(e/4) + 4*h + e%4 of column l32 in each 32x32 tile
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int c = col0 + wn * 64 + ct * 32 + l32;
      if (c >= n) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = row0 + wm * 64 + rt * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
        if (r < m) y[(size_t)r * n + c] = __builtin_bit_cast(uint16_t, (__bf16)(acc[rt][ct][e] * ts));
      }
    }
}

}  // namespace

hipError_t launch_tiled(const void *x, int m, int k, int n, const MatRef &w, void *y,
                        hipStream_t stream) {
  dim3 grid(cdiv(n, BN), cdiv(m, BM));
  hipLaunchKernelGGL(k_tiled, grid, dim3(256), 0, stream, (const uint16_t *)x, m, k, w.codes,
                     w.scales, w.ts, n, (uint16_t *)y);
  return hipGetLastError();
}

}  // namespace nvfp4
