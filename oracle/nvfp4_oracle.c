/*
 * nvfp4_oracle.c -- CPU oracle for the NVFP4-weight dense SwiGLU FFN.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product path.  Shares nothing
 * with the HIP library.  Build: gcc -O2 -ffp-contract=off (no fast-math), so
 * every float expression below is one IEEE operation, evaluated as written.
 *
 * Sources followed (the pages are rustdoc source listings of the crate
 * metrale_model_layers):
 *   - page layers/dense_ffn_fixed.rs, `DenseFfnLayer::forward_fixed`, W4A4
 *     arm: gate = proj(input), up = proj(input), silu_mul written over gate,
 *     down = proj(gate) into the [m, hidden] output, rows 0..m only (module
 *     doc "Invariants").  The same doc fixes the property the activation
 *     quantizer must keep: a row's output bits do not depend on how many rows
 *     share the launch.
 *   - page layers/dense_ffn_prefill.rs, `w4a16_prefill_gemm`: one NVFP4
 *     projection of m rows with n outputs over k inputs (W4A16: bf16
 *     activations), and `forward_prefill_inner`, whose NVFP4 leg runs the
 *     same gate/up/silu_mul/down sequence.
 *   - page layers/dense_ffn_overlays.rs, `apply_lora_down` doc: the
 *     activation is silu(gate)*up.
 * The NVFP4 format itself is not defined on the pages; the standard one is
 * used: E2M1 element codes, one E4M3 (FN) scale per 16 consecutive K
 * elements, one fp32 tensor scale (OCP MX v1.0 element encodings).
 */
#include "nvfp4_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ---- element formats ---------------------------------------------------- */

/* E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is the
 * subnormal 0.5*m.  Magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6. */
double nvo_e2m1_value(uint8_t code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -mag : mag;
}

/* E4M3 "FN": sign, 4 exponent bits (bias 7), 3 mantissa bits; no infinity,
 * S.1111.111 is NaN, largest finite 448, exponent 0 is subnormal m*2^-9. */
double nvo_e4m3_value(uint8_t b) {
  int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m, -9);
  else
    mag = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

double nvo_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static float bf16_to_float(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Round to the bf16 grid: the spacing in the binade of |v| is 2^(lg-7)
 * (8 significant bits), fixed at 2^-133 below the smallest normal 2^-126.
 * v/q is exact (power-of-two scaling) and rint() rounds ties to the even
 * integer, which is the even mantissa. */
uint16_t nvo_bf16_from_double(double v) {
  if (isnan(v)) return 0x7FC0;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (isinf(a)) return sign | 0x7F80;
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);
  int lg = e - 1; /* floor(log2 a) */
  if (lg < -126) lg = -126;
  double q = ldexp(1.0, lg - 7);
  double r = rint(a / q) * q;
  if (r >= ldexp(1.0, 128)) return sign | 0x7F80; /* rounds past the max */
  float f = (float)r;                             /* exact */
  uint32_t bits;
  memcpy(&bits, &f, 4);
  return sign | (uint16_t)(bits >> 16);
}

/* fp32 -> E4M3: nearest value, ties to even mantissa, saturating at 448. */
uint8_t nvo_e4m3_encode(float t) {
  uint8_t sign = signbit(t) ? 0x80 : 0;
  double a = fabs((double)t);
  if (isnan(a)) return sign | 0x7F;
  if (a >= 448.0) return sign | 0x7E;
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);
  int lg = e - 1;
  if (lg < -6) lg = -6;              /* subnormal range: spacing 2^-9 */
  double q = ldexp(1.0, lg - 3);     /* 3 mantissa bits */
  double r = rint(a / q) * q;        /* <= 448 since a < 448 */
  if (r == 0.0) return sign;
  if (r < ldexp(1.0, -6)) return sign | (uint8_t)(r / ldexp(1.0, -9));
  frexp(r, &e);
  lg = e - 1;
  int mant = (int)(r / ldexp(1.0, lg) * 8.0) - 8;
  return sign | (uint8_t)(((lg + 7) << 3) | mant);
}

/* fp32 -> E2M1: the grid spacing is 0.5 on [0,2), 1 on [2,4), 2 on [4,6];
 * rint() on the scaled value rounds ties to the even code in every
 * interval; |t| >= 6 saturates to 6. */
uint8_t nvo_e2m1_encode(float t) {
  uint8_t sign = signbit(t) ? 8 : 0;
  double a = fabs((double)t);
  if (isnan(a) || a >= 6.0) return sign | 7;
  double q = a < 2.0 ? 0.5 : (a < 4.0 ? 1.0 : 2.0);
  double r = rint(a / q) * q;
  uint8_t mag;
  if (r < 2.0)
    mag = (uint8_t)(r * 2.0);       /* 0, .5, 1, 1.5 -> 0..3 */
  else if (r < 4.0)
    mag = (uint8_t)(r + 2.0);       /* 2, 3 -> 4, 5 */
  else
    mag = r < 6.0 ? 6 : 7;          /* 4 -> 6, 6 -> 7 */
  return sign | mag;
}

double nvo_silu(double t) { return t / (1.0 + exp(-t)); }

/* Array forms of the encoders (same code path, for bulk checks). */
void nvo_e4m3_encode_n(const float *t, uint8_t *out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = nvo_e4m3_encode(t[i]);
}
void nvo_e2m1_encode_n(const float *t, uint8_t *out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = nvo_e2m1_encode(t[i]);
}
void nvo_bf16_from_double_n(const double *v, uint16_t *out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = nvo_bf16_from_double(v[i]);
}

/* ---- weights -------------------------------------------------------------- */

static int weight_ok(const nvo_weight *w) {
  return w && w->codes && w->scales && w->n > 0 && w->k > 0 && w->k % 16 == 0;
}

static void dequant_row(const nvo_weight *w, int c, double *row) {
  const uint8_t *cr = w->codes + (size_t)c * (w->k / 2);
  const uint8_t *sr = w->scales + (size_t)c * (w->k / 16);
  double ts = (double)w->ts;
  for (int kk = 0; kk < w->k; kk++) {
    uint8_t byte = cr[kk >> 1];
    uint8_t code = (kk & 1) ? (byte >> 4) : (byte & 15);
    row[kk] = nvo_e2m1_value(code) * nvo_e4m3_value(sr[kk >> 4]) * ts;
  }
}

void nvo_dequant(const nvo_weight *w, double *out) {
  for (int c = 0; c < w->n; c++) dequant_row(w, c, out + (size_t)c * w->k);
}

/* ---- projection: y = x . W^T, double sums in ascending k ------------------ */

typedef void (*row_decoder)(const void *w, int c, double *row);

typedef struct {
  const double *xd; /* [m][k] activations as doubles */
  int m, n, k;
  const void *w;
  row_decoder decode; /* writes weight row c (k doubles) */
  uint16_t *y;
  double *y_exact;
  int c0, c1;
} proj_job;

static void *proj_worker(void *arg) {
  proj_job *j = (proj_job *)arg;
  int k = j->k, n = j->n;
  double *row = (double *)malloc(sizeof(double) * (size_t)k);
  for (int c = j->c0; c < j->c1; c++) {
    j->decode(j->w, c, row);
    for (int r = 0; r < j->m; r++) {
      const double *xr = j->xd + (size_t)r * k;
      double s = 0.0;
      for (int kk = 0; kk < k; kk++) s += xr[kk] * row[kk];
      j->y[(size_t)r * n + c] = nvo_bf16_from_double(s);
      if (j->y_exact) j->y_exact[(size_t)r * n + c] = s;
    }
  }
  free(row);
  return NULL;
}

static int thread_count(int nthreads, int work) {
  if (nthreads <= 0) {
    long p = sysconf(_SC_NPROCESSORS_ONLN);
    nthreads = p > 0 ? (int)p : 1;
  }
  if (nthreads > work) nthreads = work;
  if (nthreads > 256) nthreads = 256;
  return nthreads < 1 ? 1 : nthreads;
}

/* Projection of m rows whose activations are already doubles, against an
 * [n][k] weight whose rows `decode` produces. */
static void project_rows(const double *xd, int m, int n, int k, const void *w,
                         row_decoder decode, uint16_t *y, double *y_exact,
                         int nthreads) {
  int nt = thread_count(nthreads, n);
  pthread_t th[256];
  proj_job jobs[256];
  for (int t = 0; t < nt; t++) {
    jobs[t].xd = xd;
    jobs[t].m = m;
    jobs[t].n = n;
    jobs[t].k = k;
    jobs[t].w = w;
    jobs[t].decode = decode;
    jobs[t].y = y;
    jobs[t].y_exact = y_exact;
    jobs[t].c0 = (int)((long long)n * t / nt);
    jobs[t].c1 = (int)((long long)n * (t + 1) / nt);
  }
  if (nt == 1) {
    proj_worker(&jobs[0]);
    return;
  }
  for (int t = 0; t < nt; t++) pthread_create(&th[t], NULL, proj_worker, &jobs[t]);
  for (int t = 0; t < nt; t++) pthread_join(th[t], NULL);
}

static void nvfp4_row(const void *w, int c, double *row) {
  dequant_row((const nvo_weight *)w, c, row);
}

static void project(const double *xd, int m, const nvo_weight *w, uint16_t *y,
                    double *y_exact, int nthreads) {
  project_rows(xd, m, w->n, w->k, w, nvfp4_row, y, y_exact, nthreads);
}

int nvo_gemm_w4a16(const uint16_t *x, int m, const nvo_weight *w, uint16_t *y,
                   double *y_exact, int nthreads) {
  if (!weight_ok(w) || m < 0 || (m > 0 && (!x || !y))) return -1;
  if (m == 0) return 0;
  size_t cnt = (size_t)m * w->k;
  double *xd = (double *)malloc(sizeof(double) * cnt);
  for (size_t i = 0; i < cnt; i++) xd[i] = nvo_bf16_value(x[i]);
  project(xd, m, w, y, y_exact, nthreads);
  free(xd);
  return 0;
}

/* ---- silu_mul --------------------------------------------------------------- */

void nvo_silu_mul(const uint16_t *g, const uint16_t *u, uint16_t *out,
                  int64_t count) {
  for (int64_t i = 0; i < count; i++) {
    double gv = nvo_bf16_value(g[i]), uv = nvo_bf16_value(u[i]);
    out[i] = nvo_bf16_from_double(nvo_silu(gv) * uv);
  }
}

/* ---- per-row NVFP4 activation quantizer -----------------------------------
 * Every step is one fp32 IEEE operation, in this order, per row:
 *   1. amax = max |x| over the row.
 *   2. s_row = amax / 2688 (2688 = 6 * 448, the largest NVFP4 magnitude), or
 *      1 for an all-zero row.
 *   3. per 16-element block: d = 6 * s_row, t = amax_block / d,
 *      scale byte = E4M3(t), v = its value.
 *   4. per element: a zero element, or any element of a block whose v is 0,
 *      gets the code sign(x)<<3; otherwise den = v * s_row and
 *      code = E2M1(x / den).
 * The row's own values decide everything, so a row's codes do not depend on
 * any other row. */
int nvo_quantize_rows(const uint16_t *x, int m, int k, uint8_t *codes,
                      uint8_t *scales, float *row_scale) {
  if (m < 0 || k <= 0 || k % 16 != 0) return -1;
  for (int r = 0; r < m; r++) {
    const uint16_t *xr = x + (size_t)r * k;
    float amax = 0.0f;
    for (int kk = 0; kk < k; kk++) {
      float av = fabsf(bf16_to_float(xr[kk]));
      if (av > amax) amax = av;
    }
    float s_row = amax / 2688.0f;
    if (amax == 0.0f) s_row = 1.0f;
    row_scale[r] = s_row;
    for (int b = 0; b < k / 16; b++) {
      float amax_b = 0.0f;
      for (int i = 0; i < 16; i++) {
        float av = fabsf(bf16_to_float(xr[b * 16 + i]));
        if (av > amax_b) amax_b = av;
      }
      float d = 6.0f * s_row;
      float t = amax_b / d;
      uint8_t sb = nvo_e4m3_encode(t);
      float v = (float)nvo_e4m3_value(sb);
      scales[(size_t)r * (k / 16) + b] = sb;
      for (int i = 0; i < 16; i++) {
        int kk = b * 16 + i;
        float xv = bf16_to_float(xr[kk]);
        uint8_t code;
        if (xv == 0.0f || v == 0.0f) {
          code = signbit(xv) ? 8 : 0;
        } else {
          float den = v * s_row;
          float q = xv / den;
          code = nvo_e2m1_encode(q);
        }
        uint8_t *dst = codes + (size_t)r * (k / 2) + (kk >> 1);
        if (kk & 1)
          *dst = (uint8_t)((*dst & 0x0F) | (code << 4));
        else
          *dst = (uint8_t)((*dst & 0xF0) | code);
      }
    }
  }
  return 0;
}

/* Dequantized activations xhat = e2m1 * e4m3 * s_row, in double. */
static double *quantized_rows_as_double(const uint16_t *x, int m, int k) {
  uint8_t *qc = (uint8_t *)calloc((size_t)m * (k / 2), 1);
  uint8_t *qs = (uint8_t *)calloc((size_t)m * (k / 16), 1);
  float *rs = (float *)calloc((size_t)m, sizeof(float));
  double *xd = (double *)malloc(sizeof(double) * (size_t)m * k);
  nvo_quantize_rows(x, m, k, qc, qs, rs);
  for (int r = 0; r < m; r++)
    for (int kk = 0; kk < k; kk++) {
      uint8_t byte = qc[(size_t)r * (k / 2) + (kk >> 1)];
      uint8_t code = (kk & 1) ? (byte >> 4) : (byte & 15);
      xd[(size_t)r * k + kk] = nvo_e2m1_value(code) *
                               nvo_e4m3_value(qs[(size_t)r * (k / 16) + (kk >> 4)]) *
                               (double)rs[r];
    }
  free(qc);
  free(qs);
  free(rs);
  return xd;
}

int nvo_gemm_w4a4(const uint16_t *x, int m, const nvo_weight *w, uint16_t *y,
                  double *y_exact, int nthreads) {
  if (!weight_ok(w) || m < 0 || (m > 0 && (!x || !y))) return -1;
  if (m == 0) return 0;
  double *xd = quantized_rows_as_double(x, m, w->k);
  project(xd, m, w, y, y_exact, nthreads);
  free(xd);
  return 0;
}

/* ---- dense SwiGLU FFN ----------------------------------------------------- */

static int ffn_shapes_ok(int hidden, int inter, const nvo_weight *wg,
                         const nvo_weight *wu, const nvo_weight *wd) {
  return weight_ok(wg) && weight_ok(wu) && weight_ok(wd) && wg->n == inter &&
         wg->k == hidden && wu->n == inter && wu->k == hidden &&
         wd->n == hidden && wd->k == inter;
}

static int dense_ffn(int w4a4, const uint16_t *x, int m, int hidden, int inter,
                     const nvo_weight *wg, const nvo_weight *wu,
                     const nvo_weight *wd, uint16_t *y, double *y_exact,
                     uint16_t *g, uint16_t *u, uint16_t *a, int nthreads) {
  if (m < 0 || !ffn_shapes_ok(hidden, inter, wg, wu, wd)) return -1;
  if (m == 0) return 0;
  size_t mi = (size_t)m * inter;
  uint16_t *gb = g ? g : (uint16_t *)malloc(2 * mi);
  uint16_t *ub = u ? u : (uint16_t *)malloc(2 * mi);
  uint16_t *ab = a ? a : (uint16_t *)malloc(2 * mi);
  if (w4a4) {
    /* gate and up read the same quantized input */
    double *xd = quantized_rows_as_double(x, m, hidden);
    project(xd, m, wg, gb, NULL, nthreads);
    project(xd, m, wu, ub, NULL, nthreads);
    free(xd);
    nvo_silu_mul(gb, ub, ab, (int64_t)mi);
    nvo_gemm_w4a4(ab, m, wd, y, y_exact, nthreads);
  } else {
    nvo_gemm_w4a16(x, m, wg, gb, NULL, nthreads);
    nvo_gemm_w4a16(x, m, wu, ub, NULL, nthreads);
    nvo_silu_mul(gb, ub, ab, (int64_t)mi);
    nvo_gemm_w4a16(ab, m, wd, y, y_exact, nthreads);
  }
  if (!g) free(gb);
  if (!u) free(ub);
  if (!a) free(ab);
  return 0;
}

int nvo_dense_ffn(const uint16_t *x, int m, int hidden, int inter,
                  const nvo_weight *wg, const nvo_weight *wu,
                  const nvo_weight *wd, uint16_t *y, double *y_exact,
                  uint16_t *g, uint16_t *u, uint16_t *a, int nthreads) {
  return dense_ffn(0, x, m, hidden, inter, wg, wu, wd, y, y_exact, g, u, a,
                   nthreads);
}

int nvo_dense_ffn_w4a4(const uint16_t *x, int m, int hidden, int inter,
                       const nvo_weight *wg, const nvo_weight *wu,
                       const nvo_weight *wd, uint16_t *y, double *y_exact,
                       uint16_t *g, uint16_t *u, uint16_t *a, int nthreads) {
  return dense_ffn(1, x, m, hidden, inter, wg, wu, wd, y, y_exact, g, u, a,
                   nthreads);
}

/* ---- LoRA overlay (page layers/dense_ffn_overlays.rs) -----------------------
 * The delta of one pair is dW . input with dW = scale * B . A, taken in two
 * products as the overlay does (first xa = input . A^T, then xa . B^T), in
 * double; it is added to the bf16 base and rounded once. */

static int lora_present(const nvo_lora *l) { return l && l->r > 0 && l->a && l->b; }

int nvo_lora_delta(const uint16_t *x, int m, int k, const nvo_lora *l, int n,
                   uint16_t *base, double *base_exact) {
  if (m < 0 || k <= 0 || n <= 0 || !base) return -1;
  if (!lora_present(l)) {
    if (base_exact)
      for (size_t i = 0; i < (size_t)m * n; i++) base_exact[i] = nvo_bf16_value(base[i]);
    return 0;
  }
  const int r = l->r;
  double *xa = (double *)malloc(sizeof(double) * (size_t)r);
  for (int i = 0; i < m; i++) {
    const uint16_t *xi = x + (size_t)i * k;
    for (int j = 0; j < r; j++) {
      const uint16_t *aj = l->a + (size_t)j * k;
      double s = 0.0;
      for (int kk = 0; kk < k; kk++) s += nvo_bf16_value(xi[kk]) * nvo_bf16_value(aj[kk]);
      xa[j] = s;
    }
    for (int c = 0; c < n; c++) {
      const uint16_t *bc = l->b + (size_t)c * r;
      double d = 0.0;
      for (int j = 0; j < r; j++) d += xa[j] * nvo_bf16_value(bc[j]);
      const double v = nvo_bf16_value(base[(size_t)i * n + c]) + (double)l->scale * d;
      if (base_exact) base_exact[(size_t)i * n + c] = v;
      base[(size_t)i * n + c] = nvo_bf16_from_double(v);
    }
  }
  free(xa);
  return 0;
}

int nvo_dense_ffn_lora(const uint16_t *x, int m, int hidden, int inter,
                       const nvo_weight *wg, const nvo_weight *wu,
                       const nvo_weight *wd, const nvo_lora *lg,
                       const nvo_lora *lu, const nvo_lora *ld, uint16_t *y,
                       double *y_exact, uint16_t *a, int nthreads) {
  if (m < 0 || !ffn_shapes_ok(hidden, inter, wg, wu, wd)) return -1;
  if (m == 0) return 0;
  size_t mi = (size_t)m * inter;
  uint16_t *gb = (uint16_t *)malloc(2 * mi);
  uint16_t *ub = (uint16_t *)malloc(2 * mi);
  uint16_t *ab = a ? a : (uint16_t *)malloc(2 * mi);
  nvo_gemm_w4a16(x, m, wg, gb, NULL, nthreads);
  nvo_gemm_w4a16(x, m, wu, ub, NULL, nthreads);
  int rc = nvo_lora_delta(x, m, hidden, lg, inter, gb, NULL);
  if (!rc) rc = nvo_lora_delta(x, m, hidden, lu, inter, ub, NULL);
  if (!rc) {
    nvo_silu_mul(gb, ub, ab, (int64_t)mi);
    nvo_gemm_w4a16(ab, m, wd, y, y_exact, nthreads);
    if (lora_present(ld)) rc = nvo_lora_delta(ab, m, inter, ld, hidden, y, y_exact);
  }
  free(gb);
  free(ub);
  if (!a) free(ab);
  return rc;
}

/* ---- W8A8 fixed format -----------------------------------------------------
 * Page layers/dense_ffn_fixed.rs, `Fixed::W8a8` (the declared W8A8 layer:
 * per-row FP8 activations at every row count, so a row's bits do not depend
 * on the row count) and page layers/dense_ffn_overlays.rs, `set_fp8_weights`
 * and `set_fp8_gate_up_fused` (block-scaled FP8 weights with a scale grid).
 * The pages define neither grid nor activation recipe; the readings:
 *   weight value W[c][kk] = e4m3(codes[c][kk]) * scales[c/128][kk/128],
 *     one fp32 scale per 128 x 128 block, grid [ceil(n/128)][ceil(k/128)];
 *   activation quantizer, per row, fp32 steps in this order:
 *     1. amax = max |x| over the row;
 *     2. s_row = amax / 448 (the largest E4M3 magnitude), or 1 for an
 *        all-zero row;
 *     3. code = E4M3(x / s_row): nearest, ties to even, saturating at 448,
 *        sign kept;
 *   x_hat = e4m3(code) * s_row, and y = bf16(sum_k x_hat * W) in double. */

static int fp8_weight_ok(const nvo_fp8_weight *w) {
  return w && w->codes && w->scales && w->n > 0 && w->k > 0;
}

static void fp8_row(const void *wv, int c, double *row) {
  const nvo_fp8_weight *w = (const nvo_fp8_weight *)wv;
  const uint8_t *cr = w->codes + (size_t)c * w->k;
  const int kb = (w->k + 127) / 128;
  const float *sr = w->scales + (size_t)(c / 128) * kb;
  for (int kk = 0; kk < w->k; kk++)
    row[kk] = nvo_e4m3_value(cr[kk]) * (double)sr[kk / 128];
}

void nvo_dequant_fp8(const nvo_fp8_weight *w, double *out) {
  for (int c = 0; c < w->n; c++) fp8_row(w, c, out + (size_t)c * w->k);
}

int nvo_quantize_rows_fp8(const uint16_t *x, int m, int k, uint8_t *codes,
                          float *row_scale) {
  if (m < 0 || k <= 0) return -1;
  for (int r = 0; r < m; r++) {
    const uint16_t *xr = x + (size_t)r * k;
    float amax = 0.0f;
    for (int kk = 0; kk < k; kk++) {
      float av = fabsf(bf16_to_float(xr[kk]));
      if (av > amax) amax = av;
    }
    float s_row = amax / 448.0f;
    if (amax == 0.0f) s_row = 1.0f;
    row_scale[r] = s_row;
    for (int kk = 0; kk < k; kk++) {
      float q = bf16_to_float(xr[kk]) / s_row;
      codes[(size_t)r * k + kk] = nvo_e4m3_encode(q);
    }
  }
  return 0;
}

static double *fp8_rows_as_double(const uint16_t *x, int m, int k) {
  uint8_t *qc = (uint8_t *)malloc((size_t)m * k);
  float *rs = (float *)malloc(sizeof(float) * (size_t)m);
  double *xd = (double *)malloc(sizeof(double) * (size_t)m * k);
  nvo_quantize_rows_fp8(x, m, k, qc, rs);
  for (int r = 0; r < m; r++)
    for (int kk = 0; kk < k; kk++)
      xd[(size_t)r * k + kk] = nvo_e4m3_value(qc[(size_t)r * k + kk]) * (double)rs[r];
  free(qc);
  free(rs);
  return xd;
}

int nvo_gemm_w8a8(const uint16_t *x, int m, const nvo_fp8_weight *w,
                  uint16_t *y, double *y_exact, int nthreads) {
  if (!fp8_weight_ok(w) || m < 0 || (m > 0 && (!x || !y))) return -1;
  if (m == 0) return 0;
  double *xd = fp8_rows_as_double(x, m, w->k);
  project_rows(xd, m, w->n, w->k, w, fp8_row, y, y_exact, nthreads);
  free(xd);
  return 0;
}

/* The W8A8 FFN: gate and up from the quantized input, silu_mul, then the
 * down projection of the quantized activation (the same step order as the
 * W4A4 arm of `forward_fixed`). */
int nvo_dense_ffn_w8a8(const uint16_t *x, int m, int hidden, int inter,
                       const nvo_fp8_weight *wg, const nvo_fp8_weight *wu,
                       const nvo_fp8_weight *wd, uint16_t *y, double *y_exact,
                       uint16_t *g, uint16_t *u, uint16_t *a, int nthreads) {
  if (m < 0 || !fp8_weight_ok(wg) || !fp8_weight_ok(wu) || !fp8_weight_ok(wd) ||
      wg->n != inter || wg->k != hidden || wu->n != inter || wu->k != hidden ||
      wd->n != hidden || wd->k != inter)
    return -1;
  if (m == 0) return 0;
  size_t mi = (size_t)m * inter;
  uint16_t *gb = g ? g : (uint16_t *)malloc(2 * mi);
  uint16_t *ub = u ? u : (uint16_t *)malloc(2 * mi);
  uint16_t *ab = a ? a : (uint16_t *)malloc(2 * mi);
  double *xd = fp8_rows_as_double(x, m, hidden);
  project_rows(xd, m, inter, hidden, wg, fp8_row, gb, NULL, nthreads);
  project_rows(xd, m, inter, hidden, wu, fp8_row, ub, NULL, nthreads);
  free(xd);
  nvo_silu_mul(gb, ub, ab, (int64_t)mi);
  nvo_gemm_w8a8(ab, m, wd, y, y_exact, nthreads);
  if (!g) free(gb);
  if (!u) free(ub);
  if (!a) free(ab);
  return 0;
}

/* ---- packed-Q2 weights ------------------------------------------------------
 * Page layers/dense_ffn_prefill.rs, `prefill_q2`: the packed-Q2 FFN, SiLU
 * only, by default dequantizes each projection's Q2_0 weight to BF16
 * (`dequant_q2_0_gn_to_bf16`, groups of `group` elements) and runs the BF16
 * GEMM on it; gate, up, silu_mul (over gate), down.  The pages do not define
 * Q2_0 itself; the reading (by analogy with the GGUF 4-bit Q4_0 form,
 * value = (code - 8) * d): a 2-bit code q per element, four per byte with
 * element 4j+i in bits 2i..2i+1 of byte j, and one fp16 scale d per group of
 * `group` consecutive K elements; value = (q - 2) * d, which the dequant
 * step rounds to bf16 (nearest, ties to even). */

static double fp16_value(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, t = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)t, -24);
  else if (e == 31)
    v = t ? NAN : INFINITY;
  else
    v = ldexp(1.0 + t / 1024.0, e - 15);
  return s ? -v : v;
}

double nvo_fp16_value(uint16_t h) { return fp16_value(h); }

static int q2_weight_ok(const nvo_q2_weight *w) {
  return w && w->codes && w->scales && w->n > 0 && w->k > 0 && w->k % 4 == 0 &&
         w->group > 0 && w->k % w->group == 0;
}

static void q2_row(const void *wv, int c, double *row) {
  const nvo_q2_weight *w = (const nvo_q2_weight *)wv;
  const uint8_t *cr = w->codes + (size_t)c * (w->k / 4);
  const uint16_t *sr = w->scales + (size_t)c * (w->k / w->group);
  for (int kk = 0; kk < w->k; kk++) {
    int q = (cr[kk >> 2] >> (2 * (kk & 3))) & 3;
    double v = (double)(q - 2) * fp16_value(sr[kk / w->group]);
    row[kk] = nvo_bf16_value(nvo_bf16_from_double(v));
  }
}

void nvo_dequant_q2(const nvo_q2_weight *w, double *out) {
  for (int c = 0; c < w->n; c++) q2_row(w, c, out + (size_t)c * w->k);
}

int nvo_gemm_q2(const uint16_t *x, int m, const nvo_q2_weight *w, uint16_t *y,
                double *y_exact, int nthreads) {
  if (!q2_weight_ok(w) || m < 0 || (m > 0 && (!x || !y))) return -1;
  if (m == 0) return 0;
  size_t cnt = (size_t)m * w->k;
  double *xd = (double *)malloc(sizeof(double) * cnt);
  for (size_t i = 0; i < cnt; i++) xd[i] = nvo_bf16_value(x[i]);
  project_rows(xd, m, w->n, w->k, w, q2_row, y, y_exact, nthreads);
  free(xd);
  return 0;
}

int nvo_dense_ffn_q2(const uint16_t *x, int m, int hidden, int inter,
                     const nvo_q2_weight *wg, const nvo_q2_weight *wu,
                     const nvo_q2_weight *wd, uint16_t *y, double *y_exact,
                     uint16_t *g, uint16_t *u, uint16_t *a, int nthreads) {
  if (m < 0 || !q2_weight_ok(wg) || !q2_weight_ok(wu) || !q2_weight_ok(wd) ||
      wg->n != inter || wg->k != hidden || wu->n != inter || wu->k != hidden ||
      wd->n != hidden || wd->k != inter)
    return -1;
  if (m == 0) return 0;
  size_t mi = (size_t)m * inter;
  uint16_t *gb = g ? g : (uint16_t *)malloc(2 * mi);
  uint16_t *ub = u ? u : (uint16_t *)malloc(2 * mi);
  uint16_t *ab = a ? a : (uint16_t *)malloc(2 * mi);
  nvo_gemm_q2(x, m, wg, gb, NULL, nthreads);
  nvo_gemm_q2(x, m, wu, ub, NULL, nthreads);
  nvo_silu_mul(gb, ub, ab, (int64_t)mi);
  nvo_gemm_q2(ab, m, wd, y, y_exact, nthreads);
  if (!g) free(gb);
  if (!u) free(ub);
  if (!a) free(ab);
  return 0;
}
