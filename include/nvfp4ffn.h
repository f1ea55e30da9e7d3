/*
 * nvfp4ffn.h -- C ABI of the MI355X (gfx950) dense SwiGLU FFN with NVFP4
 * weights.
 *
 * The FFN is the one on the pages (rustdoc source of the crate
 * metrale_model_layers): page layers/dense_ffn_fixed.rs,
 * `DenseFfnLayer::forward_fixed`, and page layers/dense_ffn_prefill.rs,
 * `forward_prefill_inner` / `w4a16_prefill_gemm`:
 *
 *     gate = X . Wg^T        [m, inter]   (projection with n = inter, k = hidden)
 *     up   = X . Wu^T        [m, inter]
 *     act  = silu(gate) * up [m, inter]   (`ops::silu_mul`, written over gate)
 *     Y    = act . Wd^T      [m, hidden]  (projection with n = hidden, k = inter)
 *
 * NVFP4 (not defined on the pages; the standard format): each weight
 * element is an E2M1 code, each run of 16 consecutive elements along K
 * shares one E4M3 ("FN": max 448, no inf) scale, and the tensor has one
 * fp32 scale:  W[r][k] = e2m1(code[r][k]) * e4m3(scale[r][k/16]) * ts.
 *
 * Common rules for every entry point
 * ----------------------------------
 * Memory: every array argument is a DEVICE pointer on the current HIP
 *   device, caller-owned, contiguous row-major and 16-byte aligned.  The
 *   library never frees or keeps a caller pointer past the stream work the
 *   call enqueues.  Weights are only read.
 * bf16: activations and outputs are bf16 bit patterns (2 bytes each).
 * Stream: `stream` is a hipStream_t (NULL = the legacy default stream).
 *   Work is enqueued asynchronously; nothing synchronizes unless
 *   NVFP4_PROFILE=1 is set in the environment.
 * Accumulation: fp32.  Intermediates (gate, up, act) are rounded to bf16,
 *   round-to-nearest-even, like the bf16 buffers the pages pass between
 *   the FFN's launches.
 * Rows: only output rows 0..m-1 are written (page layers/dense_ffn_fixed.rs,
 *   module invariants); m == 0 is a no-op returning NVFP4_OK.
 * Errors: a negative status; every check runs before anything is enqueued,
 *   so outputs are untouched on error.  nvfp4_last_error() returns the
 *   calling thread's last message.
 * Scratch: intermediates and split-K partials live in a per-device arena
 *   owned by the library (grown on first use of a larger shape, freed by
 *   nvfp4_release).  Calls that may run concurrently on different streams
 *   of one device race on it; calls on one stream are ordered.
 */
#ifndef NVFP4FFN_H
#define NVFP4FFN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define NVFP4_OK 0
#define NVFP4_EINVAL (-1) /* null/misaligned pointer, negative m, bad count */
#define NVFP4_ESHAPE (-2) /* n or k <= 0 or > 2^21, k % 32 != 0, m > 4194240, inconsistent shapes */
#define NVFP4_ENOMEM (-3) /* the scratch arena could not grow */
#define NVFP4_EHIP (-4)   /* a HIP launch or runtime call failed */

/* One NVFP4 matrix W[n][k] (PyTorch Linear orientation: y = x . W^T).
 *   codes : device, uint8 [n][k/2]; element 2j in the low nibble, 2j+1 in
 *           the high nibble; nibble bits s e1 e0 m.
 *   scales: device, uint8 [n][k/16]; E4M3FN bit patterns.
 *   tensor_scale: fp32 multiplier applied to every element.
 *   k must be a positive multiple of 32. */
typedef struct nvfp4_weight {
  const uint8_t *codes;
  const uint8_t *scales;
  float tensor_scale;
  int32_t n;
  int32_t k;
} nvfp4_weight;

/* W4A16 projection: y[m][n] = bf16( sum_k x[m][k] * W[n][k] ).
 * x: bf16 [m][k]; y: bf16 [m][n].  One NVFP4 projection GEMM of m rows
 * (page layers/dense_ffn_prefill.rs, `w4a16_prefill_gemm`). */
int nvfp4_gemm_w4a16(const void *x, int32_t m, const nvfp4_weight *w,
                     void *y, void *stream);

/* W4A4 projection: x is first quantized per row to NVFP4 (see
 * nvfp4_quantize_rows), then y[r][c] = bf16( s_row[r] * ts *
 * sum_k xq[r][k] * wq[c][k] ) with both operands' NVFP4 values exact.
 * Row r's result bits are the same for every m (page
 * layers/dense_ffn_fixed.rs, module doc and `Fixed::W4a4`:
 * `ops::w4a4_proj::nvfp4_proj_mx`, which takes a bf16 input). */
int nvfp4_gemm_w4a4(const void *x, int32_t m, const nvfp4_weight *w,
                    void *y, void *stream);

/* Per-row NVFP4 activation quantizer (the activation half of the W4A4
 * projection: page layers/dense_ffn_fixed.rs, module doc and the W4A4 arm
 * of `forward_fixed`, where the projection takes the bf16 input and
 * quantizes it to NVFP4 itself; the pages give no recipe, so the one below
 * is this library's reading).  x: bf16 [m][k], k % 32 == 0.  Outputs: codes uint8
 * [m][k/2] (packing as in nvfp4_weight), scales uint8 [m][k/16] (E4M3FN),
 * row_scale fp32 [m].  Per row, in fp32 with IEEE rounding:
 *   s_row = amax/2688 (1 for an all-zero row);
 *   per 16-block: scale = E4M3(amax_block / (6*s_row)), nearest-even,
 *                 saturating at 448;
 *   code = E2M1(x / (e4m3(scale)*s_row)), nearest with ties to the even
 *          code, saturating at 6; zero elements and elements of a
 *          zero-scale block keep only their sign.
 * Depends on nothing outside its row. */
int nvfp4_quantize_rows(const void *x, int32_t m, int32_t k, uint8_t *codes,
                        uint8_t *scales, float *row_scale, void *stream);

/* out[e] = bf16( silu(gate[e]) * up[e] ), silu(t) = t / (1 + exp(-t)),
 * computed in fp32 for e < count.  out may equal gate (every caller on the
 * pages writes over gate: page layers/dense_ffn_fixed.rs, `forward_fixed`,
 * `ops::silu_mul`). */
int silu_mul(const void *gate, const void *up, void *out, int64_t count,
             void *stream);

/* act[m][inter] = bf16( silu(bf16(x.Wg^T)) * bf16(x.Wu^T) ): gate, up and
 * silu_mul in one pass over both weights.  wg, wu: [inter][hidden]. */
int nvfp4_gate_up_silu_w4a16(const void *x, int32_t m, const nvfp4_weight *wg,
                             const nvfp4_weight *wu, void *act, void *stream);

/* Dense SwiGLU FFN, W4A16: out[m][hidden] = down(silu(gate(x)) * up(x)).
 * x: bf16 [m][hidden]; wg, wu: [inter][hidden]; wd: [hidden][inter]
 * (page layers/dense_ffn_prefill.rs, `forward_prefill_inner`, NVFP4 leg;
 * page layers/dense_ffn_fixed.rs, `forward_fixed` for the step order). */
int dense_ffn_forward(const void *x, int32_t m, int32_t hidden, int32_t inter,
                      const nvfp4_weight *wg, const nvfp4_weight *wu,
                      const nvfp4_weight *wd, void *out, void *stream);

/* dense_ffn_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, the same kernels and the same result
 * bits, but act, the split-K partials and the arrival counters live in a
 * fixed 32 MiB device array of the library (one copy per GPU, held until
 * the process ends) instead of the arena.  The call itself allocates
 * nothing.  The first call on a device looks up that array's address and
 * clears its counter region with a kernel on `stream`.  Every call on a
 * GPU shares the array: calls that overlap on one GPU (other streams,
 * other threads) race.  A shape whose scratch exceeds the array (e.g.
 * m * inter * 2 bytes of act beyond about 30 MiB) returns NVFP4_ENOMEM
 * before anything is enqueued; other errors as dense_ffn_forward. */
int dense_ffn_forward_noalloc(const void *x, int32_t m, int32_t hidden,
                              int32_t inter, const nvfp4_weight *wg,
                              const nvfp4_weight *wu, const nvfp4_weight *wd,
                              void *out, void *stream);

/* Dense SwiGLU FFN, fixed-format W4A4: x and act are quantized per row to
 * NVFP4 before each projection; row r's output bits do not depend on m
 * (page layers/dense_ffn_fixed.rs, `forward_fixed`, W4A4 arm). */
int dense_ffn_forward_w4a4(const void *x, int32_t m, int32_t hidden,
                           int32_t inter, const nvfp4_weight *wg,
                           const nvfp4_weight *wu, const nvfp4_weight *wd,
                           void *out, void *stream);

/* Views into one fused gate+up weight [2*inter][hidden]: rows 0..inter-1 are
 * gate and rows inter..2*inter-1 are up, and the E4M3 scale grid is split
 * the same way.  On success *gate and *up point into fused's buffers:
 *   gate->codes  == fused->codes,
 *   up->codes    == fused->codes  + inter * hidden/2,
 *   gate->scales == fused->scales,
 *   up->scales   == fused->scales + inter * hidden/16,
 * both [inter][hidden] with fused's tensor scale.  Host-side pointer
 * arithmetic only: no device access, no allocation, the outputs borrow
 * fused's memory.  NVFP4_EINVAL for a null or misaligned descriptor
 * (a view must stay 16-byte aligned), NVFP4_ESHAPE when fused->n is odd.
 * (page layers/dense_ffn_overlays.rs, `set_fp8_gate_up_fused`: there the
 * FP8 gate and up weights are views into one [2*inter, hidden] buffer at
 * offsets 0 and inter*hidden, scale grid alike; here the same contract for
 * NVFP4.) */
int nvfp4_gate_up_views(const nvfp4_weight *fused, nvfp4_weight *gate,
                        nvfp4_weight *up);

/* Dense SwiGLU FFN, W4A16, on a fused gate+up weight wgu [2*inter][hidden]
 * (layout as in nvfp4_gate_up_views) and wd [hidden][inter].  Runs exactly
 * what dense_ffn_forward runs on the two views (one launch streams both
 * halves and applies silu), so the two give identical bits.  Errors as
 * dense_ffn_forward, plus NVFP4_ESHAPE when wgu is not [2*inter][hidden]. */
int dense_ffn_forward_fused(const void *x, int32_t m, int32_t hidden,
                            int32_t inter, const nvfp4_weight *wgu,
                            const nvfp4_weight *wd, void *out, void *stream);

/* One LoRA pair: dW = scale * B . A, with
 *   a: device bf16 [rank][k] (row-major, K contiguous),
 *   b: device bf16 [n][rank],
 * rank a multiple of 8 and at most 256 (0: no pair; a and b may then be
 * null).  Both buffers 16-byte aligned and owned by the caller. */
typedef struct nvfp4_lora_pair {
  const void *a;
  const void *b;
  int32_t rank;
  float scale;
} nvfp4_lora_pair;

/* The LoRA overlay of one FFN: gate and up pairs act on x ([inter][hidden]
 * deltas), the down pair on act ([hidden][inter]). */
typedef struct nvfp4_lora {
  nvfp4_lora_pair gate, up, down;
} nvfp4_lora;

/* base[m][n] = bf16(base + scale * sum_j (sum_k x[i][k] a[j][k]) b[c][j]),
 * in place: x bf16 [m][k] (k % 8 == 0), base bf16 [m][n].  x . A^T is
 * formed in fp32 first, then its product with B^T (page
 * layers/dense_ffn_overlays.rs, `apply_lora_gate_up`: the overlay keeps
 * an x.A^T buffer and a delta buffer).  rank 0 is a no-op.  NVFP4_EINVAL
 * for null or misaligned pointers, NVFP4_ESHAPE for a rank that is not a
 * multiple of 8 or above 256, or k % 8 != 0. */
int nvfp4_lora_delta(const void *x, int32_t m, int32_t k,
                     const nvfp4_lora_pair *pair, int32_t n, void *base,
                     void *stream);

/* Dense SwiGLU FFN, W4A16, with a LoRA overlay (page
 * layers/dense_ffn_overlays.rs, `set_lora_weights`, `apply_lora_gate_up`,
 * `apply_lora_down`; the overlay needs gate and up materialized, so this
 * takes the split path): gate = bf16(x.Wg^T) then gate += dWg . x; up
 * likewise; act = bf16(silu(gate) * up); out = bf16(act.Wd^T) then out +=
 * dWd . act.  lora == NULL or every rank 0 runs dense_ffn_forward.  Errors
 * as dense_ffn_forward and nvfp4_lora_delta. */
int dense_ffn_forward_lora(const void *x, int32_t m, int32_t hidden,
                           int32_t inter, const nvfp4_weight *wg,
                           const nvfp4_weight *wu, const nvfp4_weight *wd,
                           const nvfp4_lora *lora, void *out, void *stream);

/* ---- W8A8 fixed format ------------------------------------------------------
 * The other fixed activation format of the pages (page
 * layers/dense_ffn_fixed.rs, `Fixed::W8a8`: the declared W8A8 layer, per-row
 * FP8 activations at every row count) on block-scaled FP8 weights (page
 * layers/dense_ffn_overlays.rs, `set_fp8_weights`: FP8 weights that carry
 * their own per-block scale grid).  The pages fix neither the block shape nor the
 * activation recipe; the readings taken here: one fp32 scale per 128 x 128
 * weight block, and one fp32 scale per activation row with amax mapped to
 * 448, the largest E4M3 magnitude. */

/* One block-scaled FP8 matrix W[n][k] (y = x . W^T):
 *   codes : device, uint8 [n][k], E4M3FN bit patterns (0x7F/0xFF are NaN);
 *   scales: device, fp32 [ceil(n/128)][ceil(k/128)], row-major;
 *   W[r][c] = e4m3(codes[r][c]) * scales[r/128][c/128].
 *   k must be a positive multiple of 32; codes 16-byte and scales 4-byte
 *   aligned. */
typedef struct fp8_weight {
  const uint8_t *codes;
  const float *scales;
  int32_t n;
  int32_t k;
} fp8_weight;

/* Per-row FP8 activation quantizer.  x: bf16 [m][k], k % 32 == 0.
 * Outputs: codes uint8 [m][k] (E4M3FN), row_scale fp32 [m].  Per row, in
 * fp32 with IEEE rounding: s_row = amax/448 (1 for an all-zero row);
 * code = E4M3(x / s_row), nearest with ties to the even mantissa,
 * saturating at 448, sign kept.  Depends on nothing outside its row. */
int fp8_quantize_rows(const void *x, int32_t m, int32_t k, uint8_t *codes,
                      float *row_scale, void *stream);

/* W8A8 projection: x is quantized per row (fp8_quantize_rows), then
 * y[r][c] = bf16( s_row[r] * sum_b scales[c/128][b] *
 *                 sum_{k in block b} e4m3(xq[r][k]) * e4m3(wq[c][k]) ),
 * fp32 accumulation.  Both E4M3 operands are converted exactly to fp16 and
 * multiplied on the f16 matrix cores (exact products; gfx950's FP8 matrix
 * forms drop low-order products inside a group, so they are not used).
 * Row r's bits are the same for every m: one kernel and one K order (fixed
 * by n and k) serve every row count.  x: bf16 [m][k]; y: bf16 [m][n]. */
int fp8_gemm_w8a8(const void *x, int32_t m, const fp8_weight *w, void *y,
                  void *stream);

/* Dense SwiGLU FFN, fixed-format W8A8: x and act are quantized per row to
 * FP8 before each projection; gate, up and silu_mul run in one launch;
 * row r's output bits do not depend on m (page layers/dense_ffn_fixed.rs,
 * `forward_fixed`, W8A8 arm).  wg, wu: [inter][hidden]; wd:
 * [hidden][inter].  Errors as dense_ffn_forward. */
int dense_ffn_forward_w8a8(const void *x, int32_t m, int32_t hidden,
                           int32_t inter, const fp8_weight *wg,
                           const fp8_weight *wu, const fp8_weight *wd,
                           void *out, void *stream);

/* ---- packed-Q2 weights -----------------------------------------------------
 * The packed-Q2 FFN of the pages (page layers/dense_ffn_prefill.rs,
 * `prefill_q2`, SiLU only): Q2_0 weights with a group size, dequantized to
 * BF16 and multiplied by the bf16 activations (the default leg there; the
 * W2A8 MMQ leg is opt-in).  Q2_0 is not defined on the pages; the reading:
 *   codes : device, uint8 [n][k/4]; element 4j+i in bits 2i..2i+1 of byte j;
 *   scales: device, fp16 bit patterns [n][k/group];
 *   W[r][c] = bf16((q - 2) * scales[r][c/group]), nearest-even.
 * group is a power of two, at least 32, dividing k (the pages' MMQ leg
 * uses 128); k % 32 == 0; codes 16-byte and scales 2-byte aligned.  The
 * kernels dequantize in registers: no bf16 copy of the weight is made. */
typedef struct q2_weight {
  const uint8_t *codes;
  const uint16_t *scales;
  int32_t group;
  int32_t n;
  int32_t k;
} q2_weight;

/* y[m][n] = bf16( sum_k x[m][k] * W[n][k] ), fp32 accumulation.
 * x: bf16 [m][k]; y: bf16 [m][n]. */
int q2_gemm_w2a16(const void *x, int32_t m, const q2_weight *w, void *y,
                  void *stream);

/* Dense SwiGLU FFN on packed-Q2 weights: gate, up and silu_mul in one
 * launch, then down (page layers/dense_ffn_prefill.rs, `prefill_q2`), at
 * every row count: up to 64 rows the weight-streaming kernel, more rows the
 * many-row kernel (the streaming kernel in 64-row blocks when hidden or
 * inter is not a multiple of 64).  wg, wu: [inter][hidden]; wd:
 * [hidden][inter].  Errors as dense_ffn_forward. */
int dense_ffn_forward_q2(const void *x, int32_t m, int32_t hidden,
                         int32_t inter, const q2_weight *wg,
                         const q2_weight *wu, const q2_weight *wd, void *out,
                         void *stream);

/* The calling thread's last error message ("" if none).  The pages' ops
 * return an error value whose message names the failed check (page
 * layers/dense_ffn_fixed.rs, the `ensure!`/`bail!` checks of
 * `forward_fixed`); a C caller gets the status code from the call and the
 * message from here.  The string stays valid until the thread's next
 * call into the library. */
const char *nvfp4_last_error(void);

/* Frees the scratch arena of every device.  The pages keep per-layer scratch buffers for the FFN's
 * intermediates (page layers/dense_ffn_fixed.rs, the scratch buffers of
 * `forward_fixed`); here they are one arena per device, which this call
 * gives back.  The caller must have synchronized all streams that used the
 * library; the next call grows the arena again. */
void nvfp4_release(void);

/* Measurement aid, not a step of the FFN: enqueues `workgroups` workgroups
 * of four waves, each wave running iters x 4 independent
 * v_mfma_f32_32x32x16_bf16 on register operands (32768 flops each, so
 * workgroups * 4 * iters * 4 * 32768 flops in all).  Timing it with events
 * gives the bf16 matrix throughput the part reaches, which benchmarks print
 * beside the specification's peak.  sink: device fp32 [256], never written
 * in practice (it keeps the loop from being optimized away).  NVFP4_EINVAL
 * for a null sink or a non-positive count. */
int nvfp4_probe_mfma_bf16(int32_t workgroups, int32_t iters, float *sink,
                          void *stream);

/* Measurement aid, not a step of the FFN: enqueues one streaming read of
 * `bytes` bytes of device memory at src (16-byte aligned; bytes a positive
 * multiple of 16): workgroups of 256 lanes, each lane four 16-byte loads in
 * flight, nothing else.  Timing back-to-back calls on buffers that no cache
 * holds gives the HBM read rate a single launch of that size reaches --
 * ramp, latency and drain included -- which benchmarks print beside the
 * specification's 8 TB/s for the memory-bound kernels.  The loaded words are
 * folded with xor; sink (device fp32 [256]) is written only if the fold
 * equals `never`, a word the caller's buffer is not filled with.  src is
 * only read.  NVFP4_EINVAL for a null pointer, a bad size or a misaligned
 * src. */
int nvfp4_probe_read(const void *src, int64_t bytes, uint32_t never, float *sink,
                     void *stream);

/* Test aid, not a step of the FFN: the division and rounding steps of the
 * activation quantizers (nvfp4_quantize_rows, fp8_quantize_rows) applied to
 * arbitrary inputs, so that tests can compare them with their definitions on
 * any fp32 value.  x: device fp32 [n], n a positive multiple of 8.  Outputs
 * (device): q fp32 [n], q[i] = x[i] / d rounded to nearest as the
 * quantizers divide; e2m1 uint8 [n], the E2M1 code of x[i] (nearest, ties to
 * the even code, saturating at 6, sign kept: the code step of
 * nvfp4_quantize_rows); e4m3 uint8 [n], the E4M3FN byte of x[i] (nearest-even,
 * saturating at 448, sign kept: the code step of fp8_quantize_rows).  NaN
 * inputs have no defined codes.  NVFP4_EINVAL for a null pointer, a bad n
 * or a d that is not a positive finite number. */
int nvfp4_probe_encode(const float *x, int64_t n, float d, float *q, uint8_t *e2m1,
                       uint8_t *e4m3, void *stream);

/* ABI version of this header (bumped on incompatible change). */
int32_t nvfp4_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* NVFP4FFN_H */
