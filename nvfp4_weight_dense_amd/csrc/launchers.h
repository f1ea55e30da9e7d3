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
// (y = bf16(silu(bf16(x.W0^T)) * bf16(x.W1^T))).  With ksplit > 1,
// `partial` must hold stream_partial_floats(...) floats and `counters`
// stream_counter_words(...) words that are zero on entry (the kernel leaves
// them zero).  The plan depends on (n, k) only.
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

// Weight-streaming projection for 17..64 rows (bf16 activations) with the
// activation chunk shared through LDS; partial/counter rules as above, with
// one counter per column group (`groups` words).
struct LdsPlan {
  int ctw;              // 16-column tiles per wave
  int groups;           // workgroups along N
  int ksplit;
  int steps_per_split;
};
LdsPlan stream_lds_plan(int n, int k, int nmat);
size_t stream_lds_partial_floats(const LdsPlan &pl, int nmat, int m, int n);
hipError_t launch_stream_lds(const void *x, int m, int k, int n, int nmat,
                             const MatRef *w, void *y, float *partial,
                             unsigned *counters, const LdsPlan &pl,
                             hipStream_t stream);

// Vector-ALU projection for 1..4 rows (bf16 activations), nmat as above.
// Eligible when K splits into at most 4 waves of register-resident granules.
bool gemv_eligible(int m, int k);
hipError_t launch_gemv(const void *x, int m, int k, int n, int nmat,
                       const MatRef *w, void *y, hipStream_t stream);

// LDS-tiled MFMA projection for many rows (bf16 activations only).
hipError_t launch_tiled(const void *x, int m, int k, int n, const MatRef &w,
                        void *y, hipStream_t stream);

hipError_t launch_silu_mul(const void *gate, const void *up, void *out,
                           int64_t count, hipStream_t stream);

hipError_t launch_quantize_rows(const void *x, int m, int k, uint8_t *codes,
                                uint8_t *scales, float *row_scale,
                                hipStream_t stream);

}  // namespace nvfp4
