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
};

// Weight-streaming projection for few rows, nmat = 1 (y = x.W^T) or 2
// (y = bf16(silu(bf16(x.W0^T)) * bf16(x.W1^T))).  `partial` must hold
// stream_partial_floats(...) floats when that is non-zero.
struct StreamPlan {
  int ksplit;           // workgroups along K
  int steps_per_split;  // 128-element K steps per split
};
StreamPlan stream_plan(int n, int k);
size_t stream_partial_floats(const StreamPlan &pl, int nmat, int m, int n);
hipError_t launch_stream(const ActRef &a, int m, int k, int n, int nmat,
                         const MatRef *w, void *y, float *partial,
                         const StreamPlan &pl, hipStream_t stream);

// LDS-tiled MFMA projection for many rows (bf16 activations only).
hipError_t launch_tiled(const void *x, int m, int k, int n, const MatRef &w,
                        void *y, hipStream_t stream);

hipError_t launch_silu_mul(const void *gate, const void *up, void *out,
                           int64_t count, hipStream_t stream);

hipError_t launch_quantize_rows(const void *x, int m, int k, uint8_t *codes,
                                uint8_t *scales, float *row_scale,
                                hipStream_t stream);

}  // namespace nvfp4
