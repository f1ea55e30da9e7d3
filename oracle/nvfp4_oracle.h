/*
 * nvfp4_oracle.h -- CPU oracle for the NVFP4-weight dense SwiGLU FFN.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link
 * or call this code: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant
 * with the HIP library.
 *
 * What it computes (plain, slow, obviously correct; fp64 accumulation):
 *   - NVFP4 decode: value = e2m1(code) * e4m3(block scale) * tensor scale,
 *     one E4M3 scale per 16 consecutive K elements.  The pages use NVFP4
 *     weights without defining the format; the element/scale encodings are
 *     the standard ones (OCP MX v1.0: E2M1 element, E4M3 "FN" scale).
 *   - W4A16 projection y = x . W^T (page layers/dense_ffn_prefill.rs,
 *     `w4a16_prefill_gemm`: one NVFP4 projection of m rows, n outputs, k in).
 *   - silu_mul: a = silu(g) * u elementwise (page layers/dense_ffn_fixed.rs,
 *     `forward_fixed`, the `ops::silu_mul` step, output written over gate).
 *   - per-row NVFP4 activation quantizer and W4A4 projection (page
 *     layers/dense_ffn_fixed.rs, module doc and `Fixed::W4a4`: NVFP4
 *     activations with a row's bits independent of the row count).
 *   - the dense FFN: gate, up, silu_mul, down (page
 *     layers/dense_ffn_fixed.rs, `forward_fixed`; page
 *     layers/dense_ffn_prefill.rs, `forward_prefill_inner`).
 *   - the LoRA overlay on it (page layers/dense_ffn_overlays.rs,
 *     `apply_lora_gate_up` and `apply_lora_down`): base += dW . input for
 *     m rows, with dW = scale * B . A a low-rank pair; gate and up get their
 *     deltas after the projections and before silu_mul, the output its
 *     delta after the down projection, with silu(gate)*up as input.
 *   - the W8A8 fixed format (page layers/dense_ffn_fixed.rs, `Fixed::W8a8`;
 *     page layers/dense_ffn_overlays.rs, `set_fp8_weights`): block-scaled
 *     FP8 weights, per-row FP8 activations, the same FFN step order.
 *   - packed-Q2 weights (page layers/dense_ffn_prefill.rs, `prefill_q2`):
 *     2-bit codes with an fp16 scale per group, dequantized to bf16, then
 *     the W4A16 step order with bf16 activations.
 *
 * Layout (host memory, row-major):
 *   x, g, u, a, y : bf16 bit patterns (uint16_t) [rows][cols]
 *   codes         : uint8 [n][k/2]; element 2j in the low nibble, 2j+1 high
 *   scales        : uint8 [n][k/16], E4M3 (FN variant)
 *   nibble bits   : s e1 e0 m
 */
#ifndef NVFP4_ORACLE_H
#define NVFP4_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  const uint8_t *codes;  /* [n][k/2] */
  const uint8_t *scales; /* [n][k/16] */
  float ts;              /* per-tensor fp32 scale */
  int n, k;
} nvo_weight;

/* Element and scale decoders (closed form). */
double nvo_e2m1_value(uint8_t code);
double nvo_e4m3_value(uint8_t byte);
double nvo_bf16_value(uint16_t bits);
/* One rounding of a double to bf16, round-to-nearest-even. */
uint16_t nvo_bf16_from_double(double v);
/* fp32 -> E4M3 / E2M1 code: round to nearest, ties to the even code,
 * saturate to the largest finite magnitude, sign kept. */
uint8_t nvo_e4m3_encode(float t);
uint8_t nvo_e2m1_encode(float t);
double nvo_silu(double t);
void nvo_e4m3_encode_n(const float *t, uint8_t *out, int64_t n);
void nvo_e2m1_encode_n(const float *t, uint8_t *out, int64_t n);
void nvo_bf16_from_double_n(const double *v, uint16_t *out, int64_t n);

/* W[r][kk] as doubles, [n][k]. */
void nvo_dequant(const nvo_weight *w, double *out);

/* y[m][n] = bf16(sum_k x[r][k] * W[c][k]); y_exact (optional) keeps the
 * double sum before rounding.  nthreads <= 0: one per online CPU.
 * Returns 0, or -1 on a shape error. */
int nvo_gemm_w4a16(const uint16_t *x, int m, const nvo_weight *w,
                   uint16_t *y, double *y_exact, int nthreads);

void nvo_silu_mul(const uint16_t *g, const uint16_t *u, uint16_t *out,
                  int64_t count);

/* Per-row NVFP4 activation quantizer (fp32 steps, see the .c file). */
int nvo_quantize_rows(const uint16_t *x, int m, int k, uint8_t *codes,
                      uint8_t *scales, float *row_scale);

/* W4A4: quantize x per row, then y = bf16(sum_k xhat * W). */
int nvo_gemm_w4a4(const uint16_t *x, int m, const nvo_weight *w,
                  uint16_t *y, double *y_exact, int nthreads);

/* Dense SwiGLU FFN.  g/u/a (optional, [m][inter]) receive the bf16
 * intermediates; y_exact (optional, [m][hidden]) the double down sum. */
int nvo_dense_ffn(const uint16_t *x, int m, int hidden, int inter,
                  const nvo_weight *wg, const nvo_weight *wu,
                  const nvo_weight *wd, uint16_t *y, double *y_exact,
                  uint16_t *g, uint16_t *u, uint16_t *a, int nthreads);
int nvo_dense_ffn_w4a4(const uint16_t *x, int m, int hidden, int inter,
                       const nvo_weight *wg, const nvo_weight *wu,
                       const nvo_weight *wd, uint16_t *y, double *y_exact,
                       uint16_t *g, uint16_t *u, uint16_t *a, int nthreads);

/* One LoRA pair: a bf16 [r][k], b bf16 [n][r], dW = scale * B . A; r == 0
 * (or a null pointer) means no pair. */
typedef struct {
  const uint16_t *a; /* [r][k] */
  const uint16_t *b; /* [n][r] */
  int r;
  float scale;
} nvo_lora;

/* base[m][n] = bf16(base + scale * sum_j (sum_k x[i][k] A[j][k]) B[c][j]),
 * in place; base_exact (optional) receives the double before rounding.
 * Returns 0, or -1 on a shape error. */
int nvo_lora_delta(const uint16_t *x, int m, int k, const nvo_lora *l, int n,
                   uint16_t *base, double *base_exact);

/* Dense SwiGLU FFN (W4A16) with LoRA pairs on gate, up and down (any may
 * be absent): g = bf16(x.Wg^T) then g += dWg . x; u likewise; a =
 * silu_mul(g, u); y = bf16(a.Wd^T) then y += dWd . a.  y_exact is the
 * double value of the last step before its rounding. */
int nvo_dense_ffn_lora(const uint16_t *x, int m, int hidden, int inter,
                       const nvo_weight *wg, const nvo_weight *wu,
                       const nvo_weight *wd, const nvo_lora *lg,
                       const nvo_lora *lu, const nvo_lora *ld, uint16_t *y,
                       double *y_exact, uint16_t *a, int nthreads);

/* W8A8 fixed format (see the .c file for the readings): FP8 E4M3 weight
 * codes [n][k] with one fp32 scale per 128 x 128 block, grid
 * [ceil(n/128)][ceil(k/128)]; activations quantized per row to E4M3 with
 * one fp32 scale per row. */
typedef struct {
  const uint8_t *codes; /* [n][k] E4M3 (FN) */
  const float *scales;  /* [ceil(n/128)][ceil(k/128)] */
  int n, k;
} nvo_fp8_weight;

void nvo_dequant_fp8(const nvo_fp8_weight *w, double *out);
int nvo_quantize_rows_fp8(const uint16_t *x, int m, int k, uint8_t *codes,
                          float *row_scale);
int nvo_gemm_w8a8(const uint16_t *x, int m, const nvo_fp8_weight *w,
                  uint16_t *y, double *y_exact, int nthreads);
int nvo_dense_ffn_w8a8(const uint16_t *x, int m, int hidden, int inter,
                       const nvo_fp8_weight *wg, const nvo_fp8_weight *wu,
                       const nvo_fp8_weight *wd, uint16_t *y, double *y_exact,
                       uint16_t *g, uint16_t *u, uint16_t *a, int nthreads);

/* Packed-Q2 weights (see the .c file for the reading): 2-bit codes
 * [n][k/4] (element 4j+i in bits 2i..2i+1 of byte j), fp16 scales
 * [n][k/group]; W = bf16((q - 2) * d). */
typedef struct {
  const uint8_t *codes;   /* [n][k/4] */
  const uint16_t *scales; /* [n][k/group], fp16 bit patterns */
  int group;
  int n, k;
} nvo_q2_weight;

double nvo_fp16_value(uint16_t h);
void nvo_dequant_q2(const nvo_q2_weight *w, double *out);
int nvo_gemm_q2(const uint16_t *x, int m, const nvo_q2_weight *w, uint16_t *y,
                double *y_exact, int nthreads);
int nvo_dense_ffn_q2(const uint16_t *x, int m, int hidden, int inter,
                     const nvo_q2_weight *wg, const nvo_q2_weight *wu,
                     const nvo_q2_weight *wd, uint16_t *y, double *y_exact,
                     uint16_t *g, uint16_t *u, uint16_t *a, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
