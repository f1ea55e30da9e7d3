// launchers.h -- host-side launchers of the gfx950 kernels (internal).
// Every launcher assumes its arguments were validated by the C-ABI layer and
// only enqueues work on `stream`; it returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

struct MatRef {
  const uint8_t *codes;   // [n][k/2]
  const uint8_t *scales;  // [n][k/16]
  float ts;
};

// Activation operand of a projection: bf16 rows, or NVFP4 rows produced by
// the per-row quantizer (codes, scales, per-row fp32 scale).
struct ActRef {
  const void *x_bf16;        // [m][k] or nullptr
  const uint8_t *codes;      // [m][k/2]
  const uint8_t *scales;     // [m][k/16]
  const float *row_scale;    // [m]
  const uint16_t *tiles;     // fp16 operand tiles (operand_tile_bytes) or nullptr
};

// fp16 operand tiles of quantized activation rows, written by the row
// quantizers for the many-row fixed-format kernel (which copies them into
// LDS with LDS-DMA).  For row tile rt (16 rows), 128-element K step t and
// MFMA sub-step j there is one 1 KB block, block ((rt * nsteps + t) * 4 + j):
// lane (c, g) = (l % 16, l / 16) holds, at bytes 16 l, the eight exact fp16
// values of row 16 rt + c at K offsets 128 t + 32 g + 8 j + 0..7 (NVFP4
// activations) or 128 t + 16 g + 8 j (j < 2) / 128 t + 64 + 16 g + 8 (j - 2)
// (FP8 activations).  K past k is zero; rows past m are not written.
size_t operand_tile_bytes(int m, int k);

// Weight-streaming projection, nmat = 1 (y = x.W^T) or 2
// (y = bf16(silu(bf16(x.W0^T)) * bf16(x.W1^T))): bf16 activations up to 16
// rows; NVFP4 activations (W4A4) at every row count, from 17 rows through
// the pipelined many-row variant with the same per-output schedule.  With
// ksplit > 1, `partial` must hold stream_partial_floats(...) floats and
// `counters` stream_counter_words(...) words that are zero on entry (the
// kernel leaves them zero).  The plan depends on (n, k) only.
// Reduction length below which no projection splits K over workgroups
// (NVFP4_SPLITK_MIN_K, read once; 0 = split wherever the plan wants).
// Every split plan below honours it; it depends on k only, so the W4A4 and
// W8A8 plans still depend on (n, k) only.
int splitk_min_k();

struct StreamPlan {
  int ksplit;           // workgroups along K
  int steps_per_split;  // 128-element K steps per split
  int tiles;            // workgroups along N
};
StreamPlan stream_plan(int n, int k);
size_t stream_partial_floats(const StreamPlan &pl, int nmat, int m, int n);
size_t stream_counter_words(const StreamPlan &pl, int m);
hipError_t launch_stream(const ActRef &a, int m, int k, int n, int nmat,
                         const MatRef *w, void *y, float *partial,
                         unsigned *counters, const StreamPlan &pl,
                         hipStream_t stream);

// LDS-shared projection (bf16 activations): a workgroup owns 32*mt rows
// and 128 columns; its four waves share each 64-element activation chunk
// through LDS.  Serves projections whose k is not a multiple of 64 (the
// LDS-DMA kernels need whole 64-K steps): 17..64 rows (mt 1 or 2, one row
// block) and more rows (mt 8, 256-row blocks).  Partial/counter rules as above, with
// stream_lds_counter_words(...) counters.
struct LdsPlan {
  int mt;               // 32-row tiles per workgroup
  int row_blocks;       // workgroups along m
  int groups;           // workgroups along N
  int ksplit;
  int steps_per_split;
  int rotate;           // stagger K start per column group (one row block)
};
int lds_row_tiles(int m);
LdsPlan stream_lds_plan(int m, int n, int k, int nmat);
size_t stream_lds_partial_floats(const LdsPlan &pl, int nmat, int m, int n);
size_t stream_lds_counter_words(const LdsPlan &pl);
hipError_t launch_stream_lds(const void *x, int m, int k, int n, int nmat,
                             const MatRef *w, void *y, float *partial,
                             unsigned *counters, const LdsPlan &pl,
                             hipStream_t stream);

// Weight-streaming projection for 17..64 rows (bf16 activations, k % 64
// == 0): one eight-wave workgroup per CU walks an equal share of the
// (column group, 256-K unit) pairs -- column groups of 64 gate + 64 up
// columns (nmat 2, silu fused) or 128 columns (nmat 1) -- and column groups
// split between workgroups are finished in the kernel by the last piece to
// arrive.  `partial` holds smallm_partial_floats(...) floats and `counters`
// smallm_counter_words(...) words that are zero on entry (left zero).
struct SmallPlan {
  int mt;      // 16-row tiles (2 or 4)
  int groups;  // column groups
  int kunits;  // 256-K units per column group
  int units;   // groups * kunits
  int nwg;     // workgroups (at most 256)
};
bool smallm_eligible(int m, int k);
SmallPlan smallm_plan(int m, int n, int k, int nmat);
size_t smallm_partial_floats(const SmallPlan &pl);
size_t smallm_counter_words(const SmallPlan &pl);
hipError_t launch_smallm(const void *x, int m, int k, int n, int nmat,
                         const MatRef *w, void *y, float *partial,
                         unsigned *counters, const SmallPlan &pl,
                         hipStream_t stream);

// Many-row projection (bf16 activations, k % 64 == 0): tiles of 32*mt rows
// (mt in {8, 6, 5, 4, 2}, chosen per shape) x 128 (nmat 2, gate+up+silu
// fused) or 256 (nmat 1) columns over the whole K, walked by one persistent
// workgroup per CU.  Columns [0, n_bulk) take one launch; when n_bulk < n
// the rest take a second launch with tiles of 32*mt2 rows.  Needs no
// scratch.
struct PrefillPlan {
  int mt;    // 32-row tiles per tile
  int nbc;   // 32-column tiles per wave and matrix
  int row_blocks;
  int groups;  // column groups
  int nwg;     // persistent workgroups
  int n_bulk;  // columns of the first launch
  int mt2, row_blocks2, groups2, nwg2;  // second launch (n_bulk < n)
};
PrefillPlan prefill_plan(int m, int n, int k, int nmat);
hipError_t launch_prefill(const void *x, int m, int k, int n, int nmat,
                          const MatRef *w, void *y, const PrefillPlan &pl,
                          hipStream_t stream);

// Vector-ALU projection for 1..4 rows (bf16 activations), nmat as above;
// with a GemvLora, the LoRA deltas are added in the epilogue.
// Eligible when K splits into at most 4 waves of register-resident granules.
// LoRA delta: base[m][n] (bf16, in place) += scale * (x . A^T) . B^T with
// A bf16 [r][k], B bf16 [n][r]; xa is fp32 scratch of lora_xa_floats(m, k,
// pairs) floats.  r % 8 == 0, r <= kMaxRank, k % 8 == 0.
constexpr int kMaxRank = 256;
struct LoraRef {
  const void *a, *b;
  int r;  // 0: no pair
  float scale;
};
size_t lora_xa_floats(int m, int k, int npairs);
hipError_t launch_lora_delta(const void *x, int m, int k, const void *a, const void *b, int r, int n,
                             float scale, void *base, float *xa, hipStream_t stream);
// gate and up deltas (from x) and silu_mul in one pass: g (bf16 [m][n])
// receives act = bf16(silu(bf16(g + dg)) * bf16(u + du)).
hipError_t launch_lora_gate_up_silu(const void *x, int m, int k, const LoraRef &lg, const LoraRef &lu,
                                    int n, void *g, const void *u, float *xa, hipStream_t stream);
// x . A^T partials alone (one or two pairs; lg.r or lu.r may be 0), for a
// GEMV that adds the deltas in its epilogue; lora_chunks(k) K chunks.
hipError_t launch_lora_xa_pair(const void *x, int m, int k, const LoraRef &lg, const LoraRef &lu, float *xa,
                               hipStream_t stream);
int lora_chunks(int k);

bool gemv_eligible(int m, int k);
// LoRA epilogue of the GEMV: matrix i's bf16 value v becomes
// bf16(v + scale[i] * xa_i . B_i[c]) before the silu (nmat 2) or as the
// output (nmat 1), with xa_i the fp32 partials of x . A_i^T written by
// launch_lora_xa_pair ([pair][nkc][m][rmax], summed in chunk order) -- the
// arithmetic of launch_lora_gate_up_silu / launch_lora_delta.
struct GemvLora {
  const float *xa;
  int nkc, rmax;
  const void *b[2];  // B_i bf16 [n][r_i]
  int r[2];          // 0: no pair
  float scale[2];
};
hipError_t launch_gemv(const void *x, int m, int k, int n, int nmat,
                       const MatRef *w, void *y, hipStream_t stream,
                       const GemvLora *lora = nullptr);

// words[0..count) = 0 with a store kernel on `stream`.
hipError_t launch_zero_words(unsigned *words, int count, hipStream_t stream);

hipError_t launch_silu_mul(const void *gate, const void *up, void *out,
                           int64_t count, hipStream_t stream);

// Per-row NVFP4 quantizer: codes, scales and row scales; with `tiles`
// (operand_tile_bytes(m, k) bytes) it writes the row scales and the decoded
// rows as fp16 operand tiles instead of the codes and scales (the many-row
// kernel reads nothing else).
hipError_t launch_quantize_rows(const void *x, int m, int k, uint8_t *codes,
                                uint8_t *scales, float *row_scale, uint16_t *tiles,
                                hipStream_t stream);

// Column tiles per workgroup of the weight-streaming kernels (1 or 2).
int stream_ctw(int n);

// ---- W8A8 fixed format: block-scaled FP8 weights, per-row FP8 activations ----
struct Fp8MatRef {
  const uint8_t *codes;  // E4M3 [n][k]
  const float *scales;   // [ceil(n/128)][ceil(k/128)]
};
struct Fp8ActRef {
  const uint8_t *codes;    // E4M3 [m][k]
  const float *row_scale;  // [m]
  const uint16_t *tiles;   // fp16 operand tiles (operand_tile_bytes) or nullptr
};
// Per-row FP8 quantizer: s_row = amax/448, codes = E4M3(x / s_row); with
// `tiles`, the decoded rows as fp16 operand tiles instead of the codes.
hipError_t launch_quantize_rows_fp8(const void *x, int m, int k, uint8_t *codes,
                                    float *row_scale, uint16_t *tiles, hipStream_t stream);
// ---- packed-Q2 weights: 2-bit codes, fp16 scale per group, bf16 activations ----
struct Q2MatRef {
  const uint8_t *codes;    // [n][k/4]
  const uint16_t *scales;  // fp16 [n][k >> gshift]
};
// Projection (nmat 1) or gate+up+silu (nmat 2) with W = bf16((q - 2) * d);
// plan q2_plan(m, n, k), partials q2_partial_floats, counters as
// stream_counter_words.  group = 1 << gshift, 32 <= group, k % group == 0.
StreamPlan q2_plan(int m, int n, int k);
size_t q2_partial_floats(const StreamPlan &pl, int nmat, int m, int n);
hipError_t launch_q2(const void *x, int m, int k, int n, int gshift, int nmat,
                     const Q2MatRef *w, void *y, float *partial,
                     unsigned *counters, const StreamPlan &pl,
                     hipStream_t stream);

// 17..64 rows on packed-Q2 weights (k % 64 == 0): the kernel of
// launch_smallm with the codes dequantized as bf16((q - 2) * d); plan,
// partials and counters as there.
hipError_t launch_smallm_q2(const void *x, int m, int k, int n, int gshift, int nmat,
                            const Q2MatRef *w, void *y, float *partial,
                            unsigned *counters, const SmallPlan &pl,
                            hipStream_t stream);

// Many-row projection on packed-Q2 weights (k % 64 == 0): the many-row
// kernel of launch_prefill with the weights' codes dequantized in registers
// as bf16((q - 2) * d); plan prefill_plan, no scratch.
hipError_t launch_prefill_q2(const void *x, int m, int k, int n, int gshift, int nmat,
                             const Q2MatRef *w, void *y, const PrefillPlan &pl,
                             hipStream_t stream);

// FP8 projection, nmat 1 or 2 (gate+up+silu) as launch_stream, with its own
// plan (w8a8_plan: depends on n and k only) and partial size
// (w8a8_partial_floats); counters as stream_counter_words.
int w8a8_ctw(int n);
StreamPlan w8a8_plan(int n, int k);
size_t w8a8_partial_floats(const StreamPlan &pl, int nmat, int m, int n);
hipError_t launch_w8a8(const Fp8ActRef &a, int m, int k, int n, int nmat,
                       const Fp8MatRef *w, void *y, float *partial,
                       unsigned *counters, const StreamPlan &pl,
                       hipStream_t stream);

// Many-row fixed-format projections (W4A4 NVFP4 activations, W8A8 FP8),
// from kFixedTallMinRows rows: eight-wave workgroups of 64 or 128 rows
// share every decoded activation fragment, and every output keeps the K
// order of the streaming kernels' plan `pl` (stream_plan for W4A4,
// w8a8_plan for W8A8), so a row's bits do not depend on m.  With
// pl.ksplit > 1, `partial` holds fixed_tall_partial_floats(...) floats and
// `counters` stream_counter_words(pl, m) zero words (left zero).
constexpr int kFixedTallMinRows = 65;
bool fixed_tall_eligible(int m);
size_t fixed_tall_partial_floats(bool fp8, int nmat, int m, int n, int ksplit);
hipError_t launch_fixed_tall_w4a4(const ActRef &a, int m, int k, int n, int nmat,
                                  const MatRef *w, void *y, float *partial,
                                  unsigned *counters, const StreamPlan &pl,
                                  hipStream_t stream);
hipError_t launch_fixed_tall_w8a8(const Fp8ActRef &a, int m, int k, int n, int nmat,
                                  const Fp8MatRef *w, void *y, float *partial,
                                  unsigned *counters, const StreamPlan &pl,
                                  hipStream_t stream);

// Register-only bf16 MFMA loop (a measurement aid): `workgroups` groups of
// four waves, each wave iters x 4 v_mfma_f32_32x32x16_bf16.  sink: 256
// floats, never written in practice.
hipError_t launch_mfma_probe(int workgroups, int iters, float *sink, hipStream_t stream);
// One streaming read of `bytes` (a multiple of 16) at src; see k_probe.hip.
hipError_t launch_read_probe(const void *src, size_t bytes, uint32_t never, float *sink, hipStream_t stream);
hipError_t launch_encode_probe(const float *x, int64_t n, float d, float *q, uint8_t *e2m1, uint8_t *e4m3,
                               hipStream_t stream);

}  // namespace nvfp4
