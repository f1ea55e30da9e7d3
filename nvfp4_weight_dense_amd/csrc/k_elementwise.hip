// k_elementwise.hip -- silu_mul and the per-row NVFP4 and FP8 activation
// quantizers (gfx950).  All are HBM-bound passes over bf16 rows.
#include <algorithm>

#include "encode_hw.h"
#include "launchers.h"
#include "nvfp4_common.h"

// The quantizer's codes must equal the CPU definition bit for bit: every
// float operation below is one IEEE fp32 operation in the written order (no
// FMA contraction; fp32 division is correctly rounded: the library is
// compiled with -fhip-fp32-correctly-rounded-divide-sqrt), and the
// per-element quotients, computed from a rounded reciprocal with one FMA
// correction, are the correctly rounded ones (encode_hw.h).
#pragma clang fp contract(off)

namespace nvfp4 {

namespace {

// ---- silu_mul: out = bf16(silu(gate) * up), page layers/dense_ffn_fixed.rs,
// `forward_fixed` (`ops::silu_mul`, written over gate) ------------------------

__global__ __launch_bounds__(256) void k_silu_mul(const uint16_t *__restrict__ g,
                                                 const uint16_t *__restrict__ u,
                                                 uint16_t *out, int64_t count) {
  const int64_t nvec = count >> 3;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nvec; i += stride) {
    const uint4 gv = ((const uint4 *)g)[i];
    const uint4 uv = ((const uint4 *)u)[i];
    const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
    const uint32_t uw[4] = {uv.x, uv.y, uv.z, uv.w};
    uint32_t ow[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float g0 = bf16_bits_to_f32(gw[q] & 0xFFFFu), g1 = bf16_bits_to_f32(gw[q] >> 16);
      float u0 = bf16_bits_to_f32(uw[q] & 0xFFFFu), u1 = bf16_bits_to_f32(uw[q] >> 16);
      __bf16 o0 = (__bf16)(silu_f32(g0) * u0);
      __bf16 o1 = (__bf16)(silu_f32(g1) * u1);
      ow[q] = (uint32_t)__builtin_bit_cast(uint16_t, o0) |
              ((uint32_t)__builtin_bit_cast(uint16_t, o1) << 16);
    }
    ((uint4 *)out)[i] = make_uint4(ow[0], ow[1], ow[2], ow[3]);
  }
  for (int64_t i = nvec * 8 + (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += stride) {
    float gv = bf16_bits_to_f32(g[i]), uv = bf16_bits_to_f32(u[i]);
    out[i] = __builtin_bit_cast(uint16_t, (__bf16)(silu_f32(gv) * uv));
  }
}

// ---- per-row NVFP4 quantizer ---------------------------------------------------

// fp32 (>= 0, finite or +inf) -> E4M3FN byte, nearest-even, saturating.
// Below 2^-6 the grid is m * 2^-9: scale by 2^9 (exact) and round to an
// integer.  Above, round the fp32 mantissa to 3 bits (adding half an ulp of
// the target minus one, plus the kept LSB, gives ties-to-even), then move
// the fields (exponent bias 127 -> 7).
__device__ __forceinline__ uint32_t e4m3_encode_sat(float t) {
  const float a = fabsf(t);
  if (!(a < 448.0f)) return 0x7Eu;
  uint32_t v = __float_as_uint(a);
  if (v < 0x3C800000u) return (uint32_t)rintf(a * 512.0f);  // 2^-6
  v = v + 0x7FFFFu + ((v >> 20) & 1u);
  v &= 0xFFF00000u;
  return (((v >> 23) - 120u) << 3) | ((v >> 20) & 7u);
}

// One workgroup per row, one thread per 16-element block (k % 32 == 0): the
// workgroup size follows the row length up to 1024 threads, and each thread
// keeps up to kKeep of its blocks in registers between the row-amax pass and
// the encode pass (longer rows re-read the rest).  With few rows the row is
// cut into gridDim.y slices, one workgroup each: every slice takes the amax
// of the whole row (from cache after the first reads it) and encodes its own
// blocks, so the divisions of one row spread over several CUs.  The row
// amax is a plain maximum, so neither the thread count nor the slicing
// changes any result.
constexpr int kQuantMaxThreads = 1024;
constexpr int kKeep = 4;
constexpr int kSliceThreads = 256;

// The row's absolute maximum, known to every thread.  One slice per row:
// each thread keeps its first kKeep blocks in keep[].
__device__ __forceinline__ float block_amax(const uint4 &v0, const uint4 &v1, float amax) {
  const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    amax = fmaxf(amax, fabsf(bf16_bits_to_f32(w[q] & 0xFFFFu)));
    amax = fmaxf(amax, fabsf(bf16_bits_to_f32(w[q] >> 16)));
  }
  return amax;
}
__device__ __forceinline__ float row_amax(const uint4 *xv4, int nblk, uint4 (&keep)[kKeep][2]) {
  const int nt = blockDim.x, t = threadIdx.x;
  float amax = 0.0f;
  int b = t;
  if (gridDim.y == 1) {
#pragma unroll
    for (int i = 0; i < kKeep; ++i, b += nt) {
      if (b < nblk) {
        keep[i][0] = xv4[2 * b];
        keep[i][1] = xv4[2 * b + 1];
        amax = block_amax(keep[i][0], keep[i][1], amax);
      }
    }
  }
  for (; b < nblk; b += nt) amax = block_amax(xv4[2 * b], xv4[2 * b + 1], amax);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  __shared__ float wmax[kQuantMaxThreads / 64];
  if ((t & 63) == 0) wmax[t >> 6] = amax;
  __syncthreads();
  amax = wmax[0];
  for (int w = 1; w < (nt >> 6); ++w) amax = fmaxf(amax, wmax[w]);
  return amax;
}

// The (row, slice) of this workgroup.  Workgroups go to the eight XCDs in
// turn (dispatch index L to XCD L mod 8), and each XCD takes one contiguous
// run of (row, slice) pairs, rows outermost: the slices of a row share its
// amax reads through one L2, and the 16 rows of an operand tile -- whose
// 16-byte pieces interleave in memory -- are written through one L2, so
// whole lines reach memory instead of pieces from several XCDs.
struct RowSlice {
  int r, s;
};
__device__ __forceinline__ RowSlice row_slice() {
  const int S = (int)gridDim.y, total = (int)gridDim.x * S;
  const int L = (int)blockIdx.x + (int)blockIdx.y * (int)gridDim.x;
  const int q = total >> 3, rem = total & 7, xcd = L & 7;
  const int u = xcd * q + min(xcd, rem) + (L >> 3);
  return RowSlice{u / S, u % S};
}

// Encode this workgroup's blocks: all of the row (one slice: the kept blocks
// from registers), or slice s's run of blocks.
template <class Enc>
__device__ __forceinline__ void encode_blocks(const uint4 *xv4, int nblk, int s, const uint4 (&keep)[kKeep][2],
                                              Enc &&encode_block) {
  const int nt = blockDim.x, t = threadIdx.x;
  if (gridDim.y == 1) {
    int b = t;
#pragma unroll
    for (int i = 0; i < kKeep; ++i, b += nt)
      if (b < nblk) encode_block(b, keep[i][0], keep[i][1]);
    for (; b < nblk; b += nt) encode_block(b, xv4[2 * b], xv4[2 * b + 1]);
  } else {
    const int per = (nblk + (int)gridDim.y - 1) / (int)gridDim.y;
    const int b0 = s * per, b1 = min(nblk, b0 + per);
    for (int b = b0 + t; b < b1; b += nt) encode_block(b, xv4[2 * b], xv4[2 * b + 1]);
  }
}

// Operand tiles (layout in launchers.h): the 16-byte slot of row r holding
// the eight K values from K0 (a multiple of 8), in fp16 units, for the
// NVFP4 (FP8 = false) or FP8 sub-step order.
template <bool FP8>
__device__ __forceinline__ size_t tile_slot(int r, int K0, int nsteps) {
  const int t = K0 >> 7, kw = K0 & 127;
  const int g = FP8 ? (kw >> 4) & 3 : kw >> 5;
  const int j = FP8 ? 2 * (kw >> 6) + ((kw >> 3) & 1) : (kw >> 3) & 3;
  return ((((size_t)(r >> 4) * nsteps + t) * 4 + j) * 64 + (r & 15) + 16 * g) * 8;
}
// Zero the tile slots of K in [k, whole steps) of row r (slice 0 only).
template <bool FP8>
__device__ __forceinline__ void zero_tile_tail(uint16_t *tiles, int r, int s, int k) {
  const int nsteps = (k + 127) >> 7;
  if (s != 0) return;
  for (int K0 = k + 8 * (int)threadIdx.x; K0 < nsteps * 128; K0 += 8 * (int)blockDim.x)
    *(uint4 *)(tiles + tile_slot<FP8>(r, K0, nsteps)) = make_uint4(0u, 0u, 0u, 0u);
}

__global__ __launch_bounds__(kQuantMaxThreads) void k_quantize_rows(const uint16_t *__restrict__ x, int k,
                                                                   uint8_t *__restrict__ codes,
                                                                   uint8_t *__restrict__ scales,
                                                                   float *__restrict__ row_scale,
                                                                   uint16_t *__restrict__ tiles) {
  const RowSlice rs = row_slice();
  const int r = rs.r;
  const int nblk = k >> 4;
  const uint4 *xv4 = (const uint4 *)(x + (size_t)r * k);

  uint4 keep[kKeep][2];
  const float amax = row_amax(xv4, nblk, keep);
  float s_row = amax / 2688.0f;
  if (amax == 0.0f) s_row = 1.0f;
  if (threadIdx.x == 0 && rs.s == 0) row_scale[r] = s_row;

  auto encode_block = [&](int b, const uint4 &v0, const uint4 &v1) {
    const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    float xv[16];
    float amax_b = 0.0f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      xv[2 * q] = bf16_bits_to_f32(w[q] & 0xFFFFu);
      xv[2 * q + 1] = bf16_bits_to_f32(w[q] >> 16);
      amax_b = fmaxf(amax_b, fabsf(xv[2 * q]));
      amax_b = fmaxf(amax_b, fabsf(xv[2 * q + 1]));
    }
    const float d = 6.0f * s_row;
    const float tb = amax_b / d;
    const uint32_t sb = e4m3_encode_sat(tb);
    const float v = e4m3_to_f32(sb);
    const float den = v * s_row;
    uint32_t packed[2] = {0u, 0u};
    if (v == 0.0f) {
      // a zero block scale: every code is the sign of its value
#pragma unroll
      for (int i = 0; i < 16; ++i) packed[i >> 3] |= (__float_as_uint(xv[i]) >> 31) << (4 * (i & 7) + 3);
    } else {
      float q[16];
      if (recip_div_ok(den)) {
        const float y = 1.0f / den;
#pragma unroll
        for (int i = 0; i < 16; ++i) q[i] = div_by_recip(xv[i], den, y);
      } else {
        // (den may underflow to zero here: a zero value keeps its signed zero)
#pragma unroll
        for (int i = 0; i < 16; ++i) q[i] = xv[i] == 0.0f ? xv[i] : xv[i] / den;
      }
      packed[0] = e2m1x8_hw(q);
      packed[1] = e2m1x8_hw(q + 8);
    }
    if (!tiles) {
      *(uint2 *)(codes + (size_t)r * (k >> 1) + 8 * b) = make_uint2(packed[0], packed[1]);
      scales[(size_t)r * nblk + b] = (uint8_t)sb;
    } else {
      // the decoded block (exact in fp16), as the streaming kernels decode it
      const _Float16 sh = e4m3x2_to_f16x2(sb)[0];
      const int nsteps = (k + 127) >> 7;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        *(uint4 *)(tiles + tile_slot<false>(r, 16 * b + 8 * hh, nsteps)) =
            __builtin_bit_cast(uint4, dequant8_f16(packed[hh], sh));
    }
  };
  encode_blocks(xv4, nblk, rs.s, keep, encode_block);
  if (tiles) zero_tile_tail<false>(tiles, r, rs.s, k);
}

// ---- per-row FP8 quantizer of the W8A8 arm ---------------------------------------
// s_row = amax/448 (1 for an all-zero row), code = E4M3(x / s_row) with the
// sign kept.  Same layout of work as k_quantize_rows (row_amax and
// encode_blocks above).

__global__ __launch_bounds__(kQuantMaxThreads) void k_quantize_rows_fp8(const uint16_t *__restrict__ x,
                                                                       int k,
                                                                       uint8_t *__restrict__ codes,
                                                                       float *__restrict__ row_scale,
                                                                       uint16_t *__restrict__ tiles) {
  const RowSlice rs = row_slice();
  const int r = rs.r;
  const int nblk = k >> 4;
  const uint4 *xv4 = (const uint4 *)(x + (size_t)r * k);

  uint4 keep[kKeep][2];
  const float amax = row_amax(xv4, nblk, keep);
  float s_row = amax / 448.0f;
  if (amax == 0.0f) s_row = 1.0f;
  if (threadIdx.x == 0 && rs.s == 0) row_scale[r] = s_row;

  const bool fast = recip_div_ok(s_row);
  const float y_row = 1.0f / s_row;
  auto encode_block = [&](int b, const uint4 &v0, const uint4 &v1) {
    const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    float q[16];
    if (fast) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t h = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
        q[i] = div_by_recip(bf16_bits_to_f32(h), s_row, y_row);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t h = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
        q[i] = bf16_bits_to_f32(h) / s_row;
      }
    }
    uint32_t out[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = e4m3x4_hw(q + 4 * j);
    if (!tiles) {
      *(uint4 *)(codes + (size_t)r * k + 16 * b) = make_uint4(out[0], out[1], out[2], out[3]);
    } else {
      const int nsteps = (k + 127) >> 7;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        *(uint4 *)(tiles + tile_slot<true>(r, 16 * b + 8 * hh, nsteps)) =
            __builtin_bit_cast(uint4, fp8x8_to_f16(out[2 * hh], out[2 * hh + 1]));
    }
  };
  encode_blocks(xv4, nblk, rs.s, keep, encode_block);
  if (tiles) zero_tile_tail<true>(tiles, r, rs.s, k);
}

// Quantizer launch shape: below kQuantSliceRows rows, slices of at least
// 32 blocks so that about that many workgroups share the work (at most 16
// per row; W4A4 FFN at m=32 59.6 -> 57.6 us, m=64 79.3 -> 77.8 us against
// slicing only below 64 rows).
constexpr int kQuantSliceRows = 256;
struct QuantShape {
  dim3 grid, block;
};
QuantShape quant_shape(int m, int k) {
  const int nblk = k >> 4;
  const int slices = (m <= 0 || m >= kQuantSliceRows)
                         ? 1
                         : std::min(std::min(16, (kQuantSliceRows + m - 1) / m), std::max(1, nblk / 32));
  QuantShape q;
  q.grid = dim3(m, slices);
  q.block = dim3(slices == 1 ? std::min(kQuantMaxThreads, (nblk + 63) / 64 * 64) : kSliceThreads);
  return q;
}

// words[i] = 0 for i < count (a plain store kernel: safe to record in a
// graph, unlike a memset node)
__global__ __launch_bounds__(256) void k_zero_words(unsigned *__restrict__ words, int count) {
  const int i = (int)(blockIdx.x * 256 + threadIdx.x);
  if (i < count) words[i] = 0u;
}

}  // namespace

hipError_t launch_zero_words(unsigned *words, int count, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero_words, dim3((count + 255) / 256), dim3(256), 0, stream, words, count);
  return hipGetLastError();
}

size_t operand_tile_bytes(int m, int k) {
  return (size_t)cdiv(m, 16) * 16 * (size_t)cdiv(k, 128) * 128 * 2;
}

hipError_t launch_quantize_rows_fp8(const void *x, int m, int k, uint8_t *codes, float *row_scale,
                                    uint16_t *tiles, hipStream_t stream) {
  const QuantShape q = quant_shape(m, k);
  hipLaunchKernelGGL(k_quantize_rows_fp8, q.grid, q.block, 0, stream, (const uint16_t *)x, k, codes,
                     row_scale, tiles);
  return hipGetLastError();
}

hipError_t launch_silu_mul(const void *gate, const void *up, void *out, int64_t count,
                           hipStream_t stream) {
  int64_t nvec = (count + 7) / 8;
  int64_t blocks = (nvec + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_silu_mul, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const uint16_t *)gate, (const uint16_t *)up, (uint16_t *)out, count);
  return hipGetLastError();
}


hipError_t launch_quantize_rows(const void *x, int m, int k, uint8_t *codes, uint8_t *scales,
                                float *row_scale, uint16_t *tiles, hipStream_t stream) {
  const QuantShape q = quant_shape(m, k);
  hipLaunchKernelGGL(k_quantize_rows, q.grid, q.block, 0, stream, (const uint16_t *)x, k, codes, scales,
                     row_scale, tiles);
  return hipGetLastError();
}

}  // namespace nvfp4
