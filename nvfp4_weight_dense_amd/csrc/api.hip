// api.hip -- C ABI of the NVFP4 dense SwiGLU FFN library (declared in
// include/nvfp4ffn.h): argument validation, per-m path choice, the scratch
// arena, error strings and the optional profile/log lines.
//
// Call structure (page layers/dense_ffn_fixed.rs, `forward_fixed`; page
// layers/dense_ffn_prefill.rs, `forward_prefill` / `w4a16_prefill_gemm`):
//   W4A16: gate+up(+silu) -> act, then down -> out.  Up to NVFP4_SMALLM_MAX_M
//          rows (default 64, the pages' small-m edge) take the weight-streaming
//          kernel with gate, up and silu_mul fused; more rows take the
//          many-row kernel (also gate+up+silu fused) when k % 64 == 0, else
//          the LDS-shared streaming kernel with 256-row blocks.
//   W4A4:  quantize x -> gate+up(+silu) -> act -> quantize act -> down.  One
//          kernel and one K order for every m, so row bits do not depend on m.
//   W8A8:  the same sequence with per-row FP8 activations and block-scaled
//          FP8 weights, exact fp16 products on the matrix cores (page
//          layers/dense_ffn_fixed.rs, `Fixed::W8a8`).
//   Q2:    packed-Q2 weights, bf16 activations (page layers/dense_ffn_prefill.rs,
//          `prefill_q2`): up to NVFP4_SMALLM_MAX_M rows the weight-streaming
//          kernel, more rows the many-row kernel when k % 64 == 0 (gate+up+
//          silu fused, then down; the weights dequantized in registers, never
//          copied to bf16), else the streaming kernel with 64-row blocks.
// Every check runs before the first launch; a forced path that cannot serve a
// shape is an error, never a silent fallback (the pages refuse to start with
// a requested but missing variant: page layers/mod.rs, `w4a16_v2_kernel`).
#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <set>
#include <string>
#include <tuple>

#include "launchers.h"
#include "nvfp4_common.h"
#include "nvfp4ffn.h"

using namespace nvfp4;

// ---- fixed device scratch of the allocation-free FFN ------------------------------
// For callers that cannot allocate (graph capture, tight serving loops):
// act, split-K partials and arrival counters of dense_ffn_forward_noalloc
// live in this array, one copy per GPU, held until the process ends.  In
// host code the name is only a stand-in for the symbol; the device address
// comes from hipGetSymbolAddress, once per device (noalloc_scratch below),
// and only that address is passed to kernels.  Calls that overlap on one
// GPU share it and race.
static constexpr size_t kNoAllocBytes = (size_t)32 << 20;
static constexpr size_t kNoAllocCounterBytes = (size_t)64 << 10;  // first 64 KB: counters
static __device__ __align__(256) uint8_t scratch[kNoAllocBytes];

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

enum class Force { Auto, Gemv, Stream, Prefill };
enum class Path { Gemv, Stream, StreamLds, Small, Prefill };

const char *path_name(Path p) {
  switch (p) {
    case Path::Gemv: return "gemv";
    case Path::Stream: return "stream";
    case Path::StreamLds: return "stream-lds";
    case Path::Small: return "small-m";
    default: return "prefill";
  }
}

// weight-streaming kernel for this many rows: plain up to 16; from 17 to 64
// the LDS-DMA weight ring when k % 64 == 0, else LDS-shared activations
Path stream_kind(int m, int k) {
  if (m <= 16) return Path::Stream;
  return smallm_eligible(m, k) ? Path::Small : Path::StreamLds;
}

struct Config {
  int smallm_max_m = 64;
  Force force = Force::Auto;
  bool profile = false;
  bool log = false;
  size_t arena_cap = 0;  // 0: no cap
  int splitk_min_k = 0;  // 0: K may be split at any length
};

const Config &cfg() {
  static Config c = [] {
    Config c;
    if (const char *v = getenv("NVFP4_SMALLM_MAX_M")) c.smallm_max_m = atoi(v);
    if (const char *v = getenv("NVFP4_FORCE_PATH")) {
      if (!strcmp(v, "gemv")) c.force = Force::Gemv;
      if (!strcmp(v, "stream")) c.force = Force::Stream;
      if (!strcmp(v, "prefill")) c.force = Force::Prefill;
    }
    if (const char *v = getenv("NVFP4_PROFILE")) c.profile = !strcmp(v, "1");
    if (const char *v = getenv("NVFP4_LOG")) c.log = !strcmp(v, "1");
    if (const char *v = getenv("NVFP4_ARENA_MAX_BYTES")) c.arena_cap = strtoull(v, nullptr, 10);
    if (const char *v = getenv("NVFP4_SPLITK_MIN_K")) c.splitk_min_k = atoi(v);
    return c;
  }();
  return c;
}

// ---- scratch arena: one grow-only device buffer per device -------------------

constexpr int kMaxDevices = 64;
struct Arena {
  void *ptr = nullptr;
  size_t size = 0;
};
std::mutex g_arena_mu;
Arena g_arena[kMaxDevices];

int arena_get(size_t bytes, void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(NVFP4_EHIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_arena_mu);
  Arena &a = g_arena[dev];
  if (a.size < bytes) {
    size_t want = (bytes + (2u << 20) - 1) & ~(size_t)((2u << 20) - 1);
    if (cfg().arena_cap && want > cfg().arena_cap)
      return fail(NVFP4_ENOMEM, "scratch arena needs %zu bytes, above NVFP4_ARENA_MAX_BYTES=%zu",
                  want, cfg().arena_cap);
    if (a.ptr) {
      // kernels still in flight may read the old buffer
      if (hipDeviceSynchronize() != hipSuccess) return fail(NVFP4_EHIP, "hipDeviceSynchronize failed");
      (void)hipFree(a.ptr);
      a.ptr = nullptr;
      a.size = 0;
    }
    if (hipMalloc(&a.ptr, want) != hipSuccess) {
      a.ptr = nullptr;
      (void)hipGetLastError();
      return fail(NVFP4_ENOMEM, "scratch arena: hipMalloc of %zu bytes failed", want);
    }
    a.size = want;
  }
  *out = a.ptr;
  return NVFP4_OK;
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Split-K arrival counters: a second grow-only buffer per device, zeroed
// when allocated.  Every kernel that uses counters leaves them at zero.
Arena g_counters[kMaxDevices];

int counters_get(size_t words, unsigned **out) {
  *out = nullptr;
  if (words == 0) return NVFP4_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(NVFP4_EHIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_arena_mu);
  Arena &a = g_counters[dev];
  const size_t bytes = words * sizeof(unsigned);
  if (a.size < bytes) {
    size_t want = (bytes + 65535) & ~(size_t)65535;
    if (a.ptr) {
      if (hipDeviceSynchronize() != hipSuccess) return fail(NVFP4_EHIP, "hipDeviceSynchronize failed");
      (void)hipFree(a.ptr);
      a.ptr = nullptr;
      a.size = 0;
    }
    if (hipMalloc(&a.ptr, want) != hipSuccess) {
      a.ptr = nullptr;
      (void)hipGetLastError();
      return fail(NVFP4_ENOMEM, "split-K counters: hipMalloc of %zu bytes failed", want);
    }
    if (hipMemset(a.ptr, 0, want) != hipSuccess) return fail(NVFP4_EHIP, "hipMemset of counters failed");
    a.size = want;
  }
  *out = (unsigned *)a.ptr;
  return NVFP4_OK;
}

// ---- validation ------------------------------------------------------------------

bool misaligned(const void *p) { return ((uintptr_t)p & 15u) != 0; }

constexpr int kMaxDim = 1 << 21;

int check_weight(const nvfp4_weight *w, const char *name) {
  if (!w) return fail(NVFP4_EINVAL, "%s: null weight descriptor", name);
  if (!w->codes || !w->scales) return fail(NVFP4_EINVAL, "%s: null codes or scales pointer", name);
  if (w->n <= 0 || w->k <= 0) return fail(NVFP4_ESHAPE, "%s: n=%d k=%d must be positive", name, w->n, w->k);
  if (w->k % 32 != 0) return fail(NVFP4_ESHAPE, "%s: k=%d is not a multiple of 32", name, w->k);
  // (keeps every buffer range and 32-bit offset of the kernels below 2^31)
  if (w->k > kMaxDim || w->n > kMaxDim)
    return fail(NVFP4_ESHAPE, "%s: n=%d k=%d exceed %d", name, w->n, w->k, kMaxDim);
  if (misaligned(w->codes) || misaligned(w->scales))
    return fail(NVFP4_EINVAL, "%s: codes/scales must be 16-byte aligned", name);
  return NVFP4_OK;
}

int check_act(const void *x, int m, const char *name) {
  if (m < 0) return fail(NVFP4_EINVAL, "%s: m=%d is negative", name, m);
  if (m > 0 && !x) return fail(NVFP4_EINVAL, "%s: null pointer", name);
  if (m > 0 && misaligned(x)) return fail(NVFP4_EINVAL, "%s: must be 16-byte aligned", name);
  if (m > 4194240) return fail(NVFP4_ESHAPE, "%s: m=%d exceeds 4194240 rows", name, m);
  return NVFP4_OK;
}

MatRef mat(const nvfp4_weight *w) { return MatRef{w->codes, w->scales, w->tensor_scale}; }

// W4A16 path of one projection with m rows and reduction length k.  A
// forced path that cannot serve the shape is an error (returns false).
bool choose_path(int m, int k, Path *out) {
  switch (cfg().force) {
    case Force::Gemv:
      *out = Path::Gemv;
      return gemv_eligible(m, k);
    case Force::Stream: *out = stream_kind(m, k); return true;
    case Force::Prefill: *out = Path::Prefill; return k % 64 == 0;
    default:
      if (gemv_eligible(m, k)) *out = Path::Gemv;
      else if (m <= cfg().smallm_max_m) *out = stream_kind(m, k);
      else *out = k % 64 == 0 ? Path::Prefill : Path::StreamLds;
      return true;
  }
}

int path_or_fail(int m, int k, Path *out) {
  if (!choose_path(m, k, out))
    return fail(NVFP4_ESHAPE, "NVFP4_FORCE_PATH=%s cannot serve m=%d k=%d (gemv needs m<=4 and a K "
                "that fits four waves of register-resident activations; prefill needs k %% 64 == 0)",
                cfg().force == Force::Gemv ? "gemv" : "prefill", m, k);
  return NVFP4_OK;
}

int hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return NVFP4_OK;
  return fail(NVFP4_EHIP, "%s: %s", what, hipGetErrorString(e));
}

void log_path(const char *entry, const char *path, int m, int n, int k) {
  if (!cfg().log) return;
  static std::mutex mu;
  static std::set<std::tuple<std::string, int, int, int>> seen;
  std::lock_guard<std::mutex> lk(mu);
  if (seen.insert({std::string(entry) + path, m, n, k}).second)
    fprintf(stderr, "[nvfp4ffn] %s m=%d n=%d k=%d -> %s\n", entry, m, n, k, path);
}

struct ProfileScope {
  const char *what;
  int m;
  hipStream_t s;
  std::chrono::steady_clock::time_point t0;
  bool on;
  ProfileScope(const char *w, int m_, hipStream_t s_) : what(w), m(m_), s(s_), on(cfg().profile) {
    if (on) {
      (void)hipStreamSynchronize(s);
      t0 = std::chrono::steady_clock::now();
    }
  }
  ~ProfileScope() {
    if (!on) return;
    (void)hipStreamSynchronize(s);
    auto us = std::chrono::duration_cast<std::chrono::microseconds>(
                  std::chrono::steady_clock::now() - t0).count();
    fprintf(stderr, "FFN [%s] m=%d: %lldus\n", what, m, (long long)us);
  }
};

// ---- projections with caller-provided scratch ----------------------------------------

// scratch bytes a projection (nmat 1) or gate+up+silu (nmat 2) needs
size_t proj_scratch_bytes(int m, int n, int k, int nmat, Path path) {
  if (path == Path::Gemv) return 0;
  if (path == Path::Stream) return align256(4 * stream_partial_floats(stream_plan(n, k), nmat, m, n));
  if (path == Path::Small) return align256(4 * smallm_partial_floats(smallm_plan(m, n, k, nmat)));
  if (path == Path::StreamLds)
    return align256(4 * stream_lds_partial_floats(stream_lds_plan(m, n, k, nmat), nmat, m, n));
  return 0;  // many-row kernel: no scratch
}

// split-K arrival counters a projection needs (zero on entry, left zero)
size_t proj_counter_words(int m, int n, int k, int nmat, Path path) {
  if (path == Path::Small) return smallm_counter_words(smallm_plan(m, n, k, nmat));
  if (path == Path::StreamLds) {
    const LdsPlan pl = stream_lds_plan(m, n, k, nmat);
    return pl.ksplit > 1 ? stream_lds_counter_words(pl) : 0;
  }
  if (path == Path::Stream) return stream_counter_words(stream_plan(n, k), m);
  return 0;
}

// `counters`: null to take them from the library's counter buffer, else a
// caller region of at least proj_counter_words(...) zero words
int run_proj(const ActRef &a, int m, int k, int n, int nmat, const MatRef *w, void *y,
             void *scratch, Path path, hipStream_t s, unsigned *counters_in = nullptr) {
  if (path == Path::Gemv)
    return hip_status(launch_gemv(a.x_bf16, m, k, n, nmat, w, y, s), "gemv projection launch");
  if (path == Path::Prefill)
    return hip_status(launch_prefill(a.x_bf16, m, k, n, nmat, w, y, prefill_plan(m, n, k, nmat), s),
                      "many-row projection launch");
  if (path == Path::Small) {
    SmallPlan pl = smallm_plan(m, n, k, nmat);
    unsigned *counters = counters_in;
    if (!counters) {
      int rc = counters_get(smallm_counter_words(pl), &counters);
      if (rc) return rc;
    }
    return hip_status(launch_smallm(a.x_bf16, m, k, n, nmat, w, y, (float *)scratch, counters, pl, s),
                      "small-m projection launch");
  }
  if (path == Path::StreamLds) {
    LdsPlan pl = stream_lds_plan(m, n, k, nmat);
    unsigned *counters = counters_in;
    if (pl.ksplit > 1 && !counters) {
      int rc = counters_get(stream_lds_counter_words(pl), &counters);
      if (rc) return rc;
    }
    return hip_status(launch_stream_lds(a.x_bf16, m, k, n, nmat, w, y, (float *)scratch, counters, pl, s),
                      "weight-streaming (LDS) projection launch");
  }
  if (path == Path::Stream) {
    StreamPlan pl = stream_plan(n, k);
    unsigned *counters = counters_in;
    if (!counters) {
      int rc = counters_get(stream_counter_words(pl, m), &counters);
      if (rc) return rc;
    }
    return hip_status(launch_stream(a, m, k, n, nmat, w, y, (float *)scratch, counters, pl, s),
                      "weight-streaming projection launch");
  }
  return fail(NVFP4_EINVAL, "internal: no kernel for path %s", path_name(path));
}

int check_ffn(const void *x, int m, int hidden, int inter, const nvfp4_weight *wg,
              const nvfp4_weight *wu, const nvfp4_weight *wd, const void *out) {
  int rc;
  if ((rc = check_act(x, m, "x")) || (rc = check_act(out, m, "out"))) return rc;
  if (hidden <= 0 || inter <= 0)
    return fail(NVFP4_ESHAPE, "hidden=%d inter=%d must be positive", hidden, inter);
  if ((rc = check_weight(wg, "wg")) || (rc = check_weight(wu, "wu")) || (rc = check_weight(wd, "wd")))
    return rc;
  if (wg->n != inter || wg->k != hidden || wu->n != inter || wu->k != hidden)
    return fail(NVFP4_ESHAPE, "wg/wu must be [inter=%d][hidden=%d], got [%d][%d] and [%d][%d]",
                inter, hidden, wg->n, wg->k, wu->n, wu->k);
  if (wd->n != hidden || wd->k != inter)
    return fail(NVFP4_ESHAPE, "wd must be [hidden=%d][inter=%d], got [%d][%d]", hidden, inter,
                wd->n, wd->k);
  return NVFP4_OK;
}

// quantized activation rows: codes, scales and row scales; from
// kFixedTallMinRows rows the row scales and fp16 operand tiles instead
// (all the many-row kernel reads)
struct QuantBuf {
  uint8_t *codes;
  uint8_t *scales;
  float *rs;
  uint16_t *tiles;
  size_t bytes;
};

QuantBuf quant_layout(char *base, int m, int k) {
  QuantBuf q;
  const bool tiled = fixed_tall_eligible(m);
  const size_t c = tiled ? 0 : align256((size_t)m * k / 2), s = tiled ? 0 : align256((size_t)m * k / 16);
  const size_t r = align256((size_t)m * 4), t = tiled ? align256(operand_tile_bytes(m, k)) : 0;
  q.codes = base && !tiled ? (uint8_t *)base : nullptr;
  q.scales = base && !tiled ? (uint8_t *)(base + c) : nullptr;
  q.rs = base ? (float *)(base + c + s) : nullptr;
  q.tiles = base && tiled ? (uint16_t *)(base + c + s + r) : nullptr;
  q.bytes = c + s + r + t;
  return q;
}

// ---- W8A8 ------------------------------------------------------------------------------

int check_fp8_weight(const fp8_weight *w, const char *name) {
  if (!w) return fail(NVFP4_EINVAL, "%s: null weight descriptor", name);
  if (!w->codes || !w->scales) return fail(NVFP4_EINVAL, "%s: null codes or scales pointer", name);
  if (w->n <= 0 || w->k <= 0) return fail(NVFP4_ESHAPE, "%s: n=%d k=%d must be positive", name, w->n, w->k);
  if (w->k % 32 != 0) return fail(NVFP4_ESHAPE, "%s: k=%d is not a multiple of 32", name, w->k);
  // n*k codes stay below 2^31 bytes, the range of one buffer resource
  if (w->k > kMaxDim || w->n > kMaxDim || (int64_t)w->n * w->k > 0x7FFFFFFFll)
    return fail(NVFP4_ESHAPE, "%s: n=%d k=%d exceed the limits (each <= %d, n*k < 2^31)", name, w->n,
                w->k, kMaxDim);
  if (misaligned(w->codes) || ((uintptr_t)w->scales & 3u))
    return fail(NVFP4_EINVAL, "%s: codes must be 16-byte and scales 4-byte aligned", name);
  return NVFP4_OK;
}

// rows of an FP8 activation buffer: m*k codes stay below 2^31 bytes
int check_fp8_rows(int m, int k, const char *name) {
  if ((int64_t)m * k > 0x7FFFFFFFll)
    return fail(NVFP4_ESHAPE, "%s: m=%d rows of k=%d exceed 2^31 bytes of FP8 codes", name, m, k);
  return NVFP4_OK;
}

Fp8MatRef fp8_mat(const fp8_weight *w) { return Fp8MatRef{w->codes, w->scales}; }

struct Fp8QuantBuf {
  uint8_t *codes;
  float *rs;
  uint16_t *tiles;
  size_t bytes;
};

Fp8QuantBuf fp8_quant_layout(char *base, int m, int k) {
  Fp8QuantBuf q;
  const bool tiled = fixed_tall_eligible(m);  // as quant_layout: tiles instead of codes
  const size_t c = tiled ? 0 : align256((size_t)m * k), r = align256((size_t)m * 4);
  const size_t t = tiled ? align256(operand_tile_bytes(m, k)) : 0;
  q.codes = base && !tiled ? (uint8_t *)base : nullptr;
  q.rs = base ? (float *)(base + c) : nullptr;
  q.tiles = base && tiled ? (uint16_t *)(base + c + r) : nullptr;
  q.bytes = c + r + t;
  return q;
}

size_t w8a8_scratch_bytes(int m, int n, int k, int nmat) {
  return align256(4 * w8a8_partial_floats(w8a8_plan(n, k), nmat, m, n));
}

int run_w8a8(const Fp8ActRef &a, int m, int k, int n, int nmat, const Fp8MatRef *w, void *y,
             void *scratch, hipStream_t s) {
  StreamPlan pl = w8a8_plan(n, k);
  unsigned *counters = nullptr;
  int rc = counters_get(stream_counter_words(pl, m), &counters);
  if (rc) return rc;
  return hip_status(launch_w8a8(a, m, k, n, nmat, w, y, (float *)scratch, counters, pl, s),
                    "W8A8 projection launch");
}

// ---- packed Q2 ----------------------------------------------------------------------

int check_q2_weight(const q2_weight *w, const char *name, int *gshift) {
  if (!w) return fail(NVFP4_EINVAL, "%s: null weight descriptor", name);
  if (!w->codes || !w->scales) return fail(NVFP4_EINVAL, "%s: null codes or scales pointer", name);
  if (w->n <= 0 || w->k <= 0) return fail(NVFP4_ESHAPE, "%s: n=%d k=%d must be positive", name, w->n, w->k);
  if (w->k % 32 != 0) return fail(NVFP4_ESHAPE, "%s: k=%d is not a multiple of 32", name, w->k);
  if (w->k > kMaxDim || w->n > kMaxDim)
    return fail(NVFP4_ESHAPE, "%s: n=%d k=%d exceed %d", name, w->n, w->k, kMaxDim);
  int sh = 5;
  while (sh < 21 && (1 << sh) != w->group) ++sh;
  if (w->group < 32 || (1 << sh) != w->group || w->k % w->group != 0)
    return fail(NVFP4_ESHAPE, "%s: group=%d must be a power of two >= 32 dividing k=%d", name,
                w->group, w->k);
  if (misaligned(w->codes) || ((uintptr_t)w->scales & 1u))
    return fail(NVFP4_EINVAL, "%s: codes must be 16-byte and scales 2-byte aligned", name);
  *gshift = sh;
  return NVFP4_OK;
}

Q2MatRef q2_mat(const q2_weight *w) { return Q2MatRef{w->codes, w->scales}; }

size_t q2_scratch_bytes(int m, int n, int k, int nmat) {
  if (smallm_eligible(m, k)) return align256(4 * smallm_partial_floats(smallm_plan(m, n, k, nmat)));
  return align256(4 * q2_partial_floats(q2_plan(m, n, k), nmat, m, n));
}

// ---- many rows on packed-Q2 weights: the many-row kernel --------------------------
// (page layers/dense_ffn_prefill.rs, `prefill_q2`: the default leg runs a BF16
// GEMM on the dequantized weight; here the many-row kernel dequantizes each
// weight fragment in registers, so no bf16 copy of the weight exists).
bool q2_tiled(int m, int k) { return m > cfg().smallm_max_m && k % 64 == 0; }


// up to 64 rows: 17..64 (k % 64 == 0) on the small-m kernel, else the
// packed-Q2 streaming kernel
int run_q2(const void *x, int m, int k, int n, int gshift, int nmat, const Q2MatRef *w, void *y,
           void *scratch, hipStream_t s) {
  if (smallm_eligible(m, k)) {
    const SmallPlan sp = smallm_plan(m, n, k, nmat);
    unsigned *counters = nullptr;
    int rc = counters_get(smallm_counter_words(sp), &counters);
    if (rc) return rc;
    return hip_status(launch_smallm_q2(x, m, k, n, gshift, nmat, w, y, (float *)scratch, counters, sp, s),
                      "packed-Q2 small-m projection launch");
  }
  StreamPlan pl = q2_plan(m, n, k);
  unsigned *counters = nullptr;
  int rc = counters_get(stream_counter_words(pl, m), &counters);
  if (rc) return rc;
  return hip_status(launch_q2(x, m, k, n, gshift, nmat, w, y, (float *)scratch, counters, pl, s),
                    "packed-Q2 projection launch");
}

struct NoAllocDev {
  bool ready = false;
  void *ptr = nullptr;
};
std::mutex g_noalloc_mu;
NoAllocDev g_noalloc[kMaxDevices];

// This device's copy of `scratch`; on first use the symbol's address is
// looked up and the counter region cleared (by a store kernel on `s`, so a
// capture records no memset node).  Kernels leave the counters at zero.
int noalloc_scratch(hipStream_t s, void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(NVFP4_EHIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_noalloc_mu);
  NoAllocDev &d = g_noalloc[dev];
  if (!d.ready) {
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(NVFP4_EHIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    int rc = hip_status(launch_zero_words((unsigned *)ptr, (int)(kNoAllocCounterBytes / 4), s),
                        "scratch counter clear");
    if (rc) return rc;
    d.ptr = ptr;
    d.ready = true;
  }
  *out = d.ptr;
  return NVFP4_OK;
}

}  // namespace

// (declared in launchers.h: the plans of the split-K kernels read it)
int nvfp4::splitk_min_k() { return cfg().splitk_min_k; }

// ---- C ABI ---------------------------------------------------------------------------

extern "C" {

int32_t nvfp4_abi_version(void) { return 1; }

int nvfp4_probe_mfma_bf16(int32_t workgroups, int32_t iters, float *sink, void *stream) {
  g_err.clear();
  if (workgroups <= 0 || iters <= 0) return fail(NVFP4_EINVAL, "probe: workgroups and iters must be positive");
  if (!sink) return fail(NVFP4_EINVAL, "probe: null sink");
  return hip_status(launch_mfma_probe(workgroups, iters, sink, (hipStream_t)stream), "probe launch");
}

int nvfp4_probe_read(const void *src, int64_t bytes, uint32_t never, float *sink, void *stream) {
  g_err.clear();
  if (!src || !sink) return fail(NVFP4_EINVAL, "read probe: null pointer");
  if (bytes <= 0 || bytes % 16 != 0) return fail(NVFP4_EINVAL, "read probe: bytes must be a positive multiple of 16");
  if (((uintptr_t)src & 15u) != 0) return fail(NVFP4_EINVAL, "read probe: src must be 16-byte aligned");
  if (bytes / 16 > (int64_t)0xFFFFFFFFll * 1024) return fail(NVFP4_EINVAL, "read probe: too many bytes");
  return hip_status(launch_read_probe(src, (size_t)bytes, never, sink, (hipStream_t)stream), "read probe launch");
}

int nvfp4_probe_encode(const float *x, int64_t n, float d, float *q, uint8_t *e2m1, uint8_t *e4m3,
                       void *stream) {
  g_err.clear();
  if (!x || !q || !e2m1 || !e4m3) return fail(NVFP4_EINVAL, "encode probe: null pointer");
  if (n <= 0 || n % 8 != 0 || n / 8 > (int64_t)0x7FFFFFFF * 256)
    return fail(NVFP4_EINVAL, "encode probe: n must be a positive multiple of 8");
  if (!(d > 0.0f) || !(d < INFINITY)) return fail(NVFP4_EINVAL, "encode probe: d must be positive and finite");
  return hip_status(launch_encode_probe(x, n, d, q, e2m1, e4m3, (hipStream_t)stream), "encode probe launch");
}

const char *nvfp4_last_error(void) { return g_err.c_str(); }

void nvfp4_release(void) {
  std::lock_guard<std::mutex> lk(g_arena_mu);
  int cur = 0;
  (void)hipGetDevice(&cur);
  for (int d = 0; d < kMaxDevices; ++d) {
    for (Arena *a : {&g_arena[d], &g_counters[d]}) {
      if (!a->ptr) continue;
      (void)hipSetDevice(d);
      (void)hipFree(a->ptr);
      a->ptr = nullptr;
      a->size = 0;
    }
  }
  (void)hipSetDevice(cur);
}

int silu_mul(const void *gate, const void *up, void *out, int64_t count, void *stream) {
  g_err.clear();
  if (count < 0) return fail(NVFP4_EINVAL, "silu_mul: count=%lld is negative", (long long)count);
  if (count == 0) return NVFP4_OK;
  if (!gate || !up || !out) return fail(NVFP4_EINVAL, "silu_mul: null pointer");
  if (misaligned(gate) || misaligned(up) || misaligned(out))
    return fail(NVFP4_EINVAL, "silu_mul: pointers must be 16-byte aligned");
  return hip_status(launch_silu_mul(gate, up, out, count, (hipStream_t)stream), "silu_mul launch");
}

int nvfp4_quantize_rows(const void *x, int32_t m, int32_t k, uint8_t *codes, uint8_t *scales,
                        float *row_scale, void *stream) {
  g_err.clear();
  int rc;
  if ((rc = check_act(x, m, "x"))) return rc;
  if (k <= 0 || k % 32 != 0) return fail(NVFP4_ESHAPE, "quantize_rows: k=%d must be a positive multiple of 32", k);
  if (m == 0) return NVFP4_OK;
  if (!codes || !scales || !row_scale) return fail(NVFP4_EINVAL, "quantize_rows: null output pointer");
  if (misaligned(codes) || ((uintptr_t)row_scale & 3u))
    return fail(NVFP4_EINVAL, "quantize_rows: codes must be 16-byte and row_scale 4-byte aligned");
  return hip_status(launch_quantize_rows(x, m, k, codes, scales, row_scale, nullptr, (hipStream_t)stream),
                    "quantize_rows launch");
}

int nvfp4_gemm_w4a16(const void *x, int32_t m, const nvfp4_weight *w, void *y, void *stream) {
  g_err.clear();
  int rc;
  if ((rc = check_act(x, m, "x")) || (rc = check_act(y, m, "y")) || (rc = check_weight(w, "w")))
    return rc;
  if (m == 0) return NVFP4_OK;
  hipStream_t s = (hipStream_t)stream;
  Path path;
  if ((rc = path_or_fail(m, w->k, &path))) return rc;
  log_path("gemm_w4a16", path_name(path), m, w->n, w->k);
  void *scr = nullptr;
  size_t need = proj_scratch_bytes(m, w->n, w->k, 1, path);
  if (need && (rc = arena_get(need, &scr))) return rc;
  ProfileScope ps("gemm_w4a16", m, s);
  MatRef wm = mat(w);
  return run_proj(ActRef{x, nullptr, nullptr, nullptr}, m, w->k, w->n, 1, &wm, y, scr, path, s);
}

int nvfp4_gate_up_silu_w4a16(const void *x, int32_t m, const nvfp4_weight *wg,
                             const nvfp4_weight *wu, void *act, void *stream) {
  g_err.clear();
  int rc;
  if ((rc = check_act(x, m, "x")) || (rc = check_act(act, m, "act")) ||
      (rc = check_weight(wg, "wg")) || (rc = check_weight(wu, "wu")))
    return rc;
  if (wg->n != wu->n || wg->k != wu->k)
    return fail(NVFP4_ESHAPE, "wg [%d][%d] and wu [%d][%d] differ", wg->n, wg->k, wu->n, wu->k);
  if (m == 0) return NVFP4_OK;
  hipStream_t s = (hipStream_t)stream;
  Path path;
  if ((rc = path_or_fail(m, wg->k, &path))) return rc;
  log_path("gate_up_silu_w4a16", path_name(path), m, wg->n, wg->k);
  void *scr = nullptr;
  size_t need = proj_scratch_bytes(m, wg->n, wg->k, 2, path);
  if (need && (rc = arena_get(need, &scr))) return rc;
  ProfileScope ps("gate_up_silu_w4a16", m, s);
  MatRef w2[2] = {mat(wg), mat(wu)};
  return run_proj(ActRef{x, nullptr, nullptr, nullptr}, m, wg->k, wg->n, 2, w2, act, scr, path, s);
}

int dense_ffn_forward(const void *x, int32_t m, int32_t hidden, int32_t inter,
                      const nvfp4_weight *wg, const nvfp4_weight *wu, const nvfp4_weight *wd,
                      void *out, void *stream) {
  g_err.clear();
  int rc;
  if ((rc = check_ffn(x, m, hidden, inter, wg, wu, wd, out))) return rc;
  if (m == 0) return NVFP4_OK;
  hipStream_t s = (hipStream_t)stream;
  Path p_up, p_down;
  if ((rc = path_or_fail(m, hidden, &p_up)) || (rc = path_or_fail(m, inter, &p_down))) return rc;
  log_path("dense_ffn_forward gate+up", path_name(p_up), m, inter, hidden);
  log_path("dense_ffn_forward down", path_name(p_down), m, hidden, inter);
  const size_t act_b = align256((size_t)2 * m * inter);
  size_t scr_b = proj_scratch_bytes(m, inter, hidden, 2, p_up);
  size_t down_b = proj_scratch_bytes(m, hidden, inter, 1, p_down);
  if (down_b > scr_b) scr_b = down_b;
  void *base = nullptr;
  if ((rc = arena_get(act_b + scr_b, &base))) return rc;
  char *act = (char *)base;
  char *scr = act + act_b;
  ProfileScope ps("dense_total", m, s);
  MatRef w2[2] = {mat(wg), mat(wu)};
  MatRef wdm = mat(wd);
  if ((rc = run_proj(ActRef{x, nullptr, nullptr, nullptr}, m, hidden, inter, 2, w2, act, scr, p_up, s)))
    return rc;
  return run_proj(ActRef{act, nullptr, nullptr, nullptr}, m, inter, hidden, 1, &wdm, out, scr, p_down, s);
}

int dense_ffn_forward_noalloc(const void *x, int32_t m, int32_t hidden, int32_t inter,
                              const nvfp4_weight *wg, const nvfp4_weight *wu,
                              const nvfp4_weight *wd, void *out, void *stream) {
  g_err.clear();
  int rc;
  if ((rc = check_ffn(x, m, hidden, inter, wg, wu, wd, out))) return rc;
  if (m == 0) return NVFP4_OK;
  hipStream_t s = (hipStream_t)stream;
  Path p_up, p_down;
  if ((rc = path_or_fail(m, hidden, &p_up)) || (rc = path_or_fail(m, inter, &p_down))) return rc;
  const size_t act_b = align256((size_t)2 * m * inter);
  const size_t scr_b = std::max(proj_scratch_bytes(m, inter, hidden, 2, p_up),
                                proj_scratch_bytes(m, hidden, inter, 1, p_down));
  const size_t words = std::max(proj_counter_words(m, inter, hidden, 2, p_up),
                                proj_counter_words(m, hidden, inter, 1, p_down));
  const size_t need = kNoAllocCounterBytes + act_b + scr_b;
  if (need > kNoAllocBytes || words * 4 > kNoAllocCounterBytes)
    return fail(NVFP4_ENOMEM,
                "dense_ffn_forward_noalloc: m=%d hidden=%d inter=%d needs %zu bytes of scratch "
                "(%zu counter words); the fixed scratch holds %zu bytes (%zu words)",
                m, hidden, inter, need, words, kNoAllocBytes, kNoAllocCounterBytes / 4);
  log_path("dense_ffn_forward_noalloc gate+up", path_name(p_up), m, inter, hidden);
  log_path("dense_ffn_forward_noalloc down", path_name(p_down), m, hidden, inter);
  void *base = nullptr;
  if ((rc = noalloc_scratch(s, &base))) return rc;
  unsigned *counters = (unsigned *)base;
  char *act = (char *)base + kNoAllocCounterBytes;
  char *scr = act + act_b;
  ProfileScope ps("dense_total noalloc", m, s);
  MatRef w2[2] = {mat(wg), mat(wu)};
  MatRef wdm = mat(wd);
  if ((rc = run_proj(ActRef{x, nullptr, nullptr, nullptr}, m, hidden, inter, 2, w2, act, scr, p_up, s,
                     counters)))
    return rc;
  return run_proj(ActRef{act, nullptr, nullptr, nullptr}, m, inter, hidden, 1, &wdm, out, scr, p_down, s,
                  counters);
}

int nvfp4_gate_up_views(const nvfp4_weight *fused, nvfp4_weight *gate, nvfp4_weight *up) {
  g_err.clear();
  int rc;
  if ((rc = check_weight(fused, "fused"))) return rc;
  if (!gate || !up) return fail(NVFP4_EINVAL, "gate_up_views: null output descriptor");
  if (fused->n % 2 != 0)
    return fail(NVFP4_ESHAPE, "gate_up_views: fused n=%d is not 2*inter", fused->n);
  const int inter = fused->n / 2;
  const size_t off_codes = (size_t)inter * (size_t)(fused->k / 2);
  const size_t off_scales = (size_t)inter * (size_t)(fused->k / 16);
  nvfp4_weight g = {fused->codes, fused->scales, fused->tensor_scale, inter, fused->k};
  nvfp4_weight u = {fused->codes + off_codes, fused->scales + off_scales, fused->tensor_scale, inter,
                    fused->k};
  if ((rc = check_weight(&u, "up view"))) return rc;
  *gate = g;
  *up = u;
  return NVFP4_OK;
}

int dense_ffn_forward_fused(const void *x, int32_t m, int32_t hidden, int32_t inter,
                            const nvfp4_weight *wgu, const nvfp4_weight *wd, void *out,
                            void *stream) {
  g_err.clear();
  int rc;
  nvfp4_weight wg, wu;
  if ((rc = nvfp4_gate_up_views(wgu, &wg, &wu))) return rc;
  if ((int64_t)wgu->n != 2 * (int64_t)inter || wgu->k != hidden)
    return fail(NVFP4_ESHAPE, "wgu must be [2*inter=%lld][hidden=%d], got [%d][%d]",
                2 * (long long)inter, hidden, wgu->n, wgu->k);
  return dense_ffn_forward(x, m, hidden, inter, &wg, &wu, wd, out, stream);
}

int check_lora(const nvfp4_lora_pair *l, int k, int n, const char *name) {
  if (!l || l->rank == 0) return NVFP4_OK;
  if (l->rank < 0 || l->rank % 8 != 0 || l->rank > kMaxRank)
    return fail(NVFP4_ESHAPE, "%s: rank=%d must be a multiple of 8 in 8..%d", name, l->rank, kMaxRank);
  if (!l->a || !l->b) return fail(NVFP4_EINVAL, "%s: null a or b", name);
  if (misaligned(l->a) || misaligned(l->b))
    return fail(NVFP4_EINVAL, "%s: a and b must be 16-byte aligned", name);
  if (k % 8 != 0) return fail(NVFP4_ESHAPE, "%s: k=%d is not a multiple of 8", name, k);
  (void)n;
  return NVFP4_OK;
}

bool lora_on(const nvfp4_lora_pair &l) { return l.rank > 0; }

int nvfp4_lora_delta(const void *x, int32_t m, int32_t k, const nvfp4_lora_pair *pair, int32_t n,
                     void *base, void *stream) {
  g_err.clear();
  int rc;
  if (!pair) return fail(NVFP4_EINVAL, "lora_delta: null pair");
  if ((rc = check_act(x, m, "x")) || (rc = check_act(base, m, "base"))) return rc;
  if (k <= 0 || n <= 0 || k > kMaxDim || n > kMaxDim)
    return fail(NVFP4_ESHAPE, "lora_delta: k=%d n=%d out of range", k, n);
  if ((rc = check_lora(pair, k, n, "lora_delta"))) return rc;
  if (m == 0 || pair->rank == 0) return NVFP4_OK;
  void *xa = nullptr;
  if ((rc = arena_get(align256(4 * lora_xa_floats(m, k, 1)), &xa))) return rc;
  return hip_status(launch_lora_delta(x, m, k, pair->a, pair->b, pair->rank, n, pair->scale,
                                      base, (float *)xa, (hipStream_t)stream),
                    "lora delta launch");
}

int dense_ffn_forward_lora(const void *x, int32_t m, int32_t hidden, int32_t inter,
                           const nvfp4_weight *wg, const nvfp4_weight *wu, const nvfp4_weight *wd,
                           const nvfp4_lora *lora, void *out, void *stream) {
  g_err.clear();
  int rc;
  if (!lora || (!lora_on(lora->gate) && !lora_on(lora->up) && !lora_on(lora->down)))
    return dense_ffn_forward(x, m, hidden, inter, wg, wu, wd, out, stream);
  if ((rc = check_ffn(x, m, hidden, inter, wg, wu, wd, out))) return rc;
  if ((rc = check_lora(&lora->gate, hidden, inter, "lora.gate")) ||
      (rc = check_lora(&lora->up, hidden, inter, "lora.up")) ||
      (rc = check_lora(&lora->down, inter, hidden, "lora.down")))
    return rc;
  if (m == 0) return NVFP4_OK;
  hipStream_t s = (hipStream_t)stream;
  Path p_up, p_down;
  if ((rc = path_or_fail(m, hidden, &p_up)) || (rc = path_or_fail(m, inter, &p_down))) return rc;
  log_path("dense_ffn_forward_lora gate/up", path_name(p_up), m, inter, hidden);
  log_path("dense_ffn_forward_lora down", path_name(p_down), m, hidden, inter);
  // arena: gate (then act), up, xa, projection scratch
  const size_t gu_b = align256((size_t)2 * m * inter);
  const size_t xa_b = align256(4 * std::max(lora_xa_floats(m, hidden, 2), lora_xa_floats(m, inter, 1)));
  size_t scr_b = proj_scratch_bytes(m, inter, hidden, 1, p_up);
  const size_t down_b = proj_scratch_bytes(m, hidden, inter, 1, p_down);
  if (down_b > scr_b) scr_b = down_b;
  void *base = nullptr;
  if ((rc = arena_get(2 * gu_b + xa_b + scr_b, &base))) return rc;
  char *g = (char *)base, *u = g + gu_b;
  float *xa = (float *)(u + gu_b);
  char *scr = (char *)xa + xa_b;
  ProfileScope ps("dense_total lora", m, s);
  MatRef mg = mat(wg), mu = mat(wu), md = mat(wd);
  const ActRef ax{x, nullptr, nullptr, nullptr};
  auto ref = [](const nvfp4_lora_pair &l) {
    return lora_on(l) ? LoraRef{l.a, l.b, l.rank, l.scale} : LoraRef{nullptr, nullptr, 0, 0.f};
  };
  const LoraRef lg = ref(lora->gate), lu = ref(lora->up), ld = ref(lora->down);
  const LoraRef none{nullptr, nullptr, 0, 0.f};
  if (p_up == Path::Gemv) {
    // x . A^T of both pairs, then one GEMV launch streams both weights and
    // adds the deltas and silu_mul in its epilogue (act over gate)
    const MatRef w2[2] = {mg, mu};
    const GemvLora gl{xa, lora_chunks(hidden), std::max(lg.r, lu.r), {lg.b, lu.b}, {lg.r, lu.r},
                      {lg.scale, lu.scale}};
    if ((rc = hip_status(launch_lora_xa_pair(x, m, hidden, lg, lu, xa, s), "lora x.A launch")) ||
        (rc = hip_status(launch_gemv(x, m, hidden, inter, 2, w2, g, s, &gl), "gemv projection launch")))
      return rc;
  } else if ((rc = run_proj(ax, m, hidden, inter, 1, &mg, g, scr, p_up, s)) ||
             (rc = run_proj(ax, m, hidden, inter, 1, &mu, u, scr, p_up, s)) ||
             // gate and up deltas, then silu_mul, in one pass over gate/up (act over gate)
             (rc = hip_status(launch_lora_gate_up_silu(x, m, hidden, lg, lu, inter, g, u, xa, s),
                              "lora gate/up + silu launch"))) {
    return rc;
  }
  const ActRef aact{g, nullptr, nullptr, nullptr};
  if (ld.r == 0) return run_proj(aact, m, inter, hidden, 1, &md, out, scr, p_down, s);
  if (p_down == Path::Gemv) {
    // act . A^T, then the down GEMV adds the delta in its epilogue
    const GemvLora gl{xa, lora_chunks(inter), ld.r, {ld.b, nullptr}, {ld.r, 0}, {ld.scale, 0.f}};
    if ((rc = hip_status(launch_lora_xa_pair(g, m, inter, ld, none, xa, s), "lora act.A launch"))) return rc;
    return hip_status(launch_gemv(g, m, inter, hidden, 1, &md, out, s, &gl), "gemv projection launch");
  }
  if ((rc = run_proj(aact, m, inter, hidden, 1, &md, out, scr, p_down, s))) return rc;
  return hip_status(launch_lora_delta(g, m, inter, ld.a, ld.b, ld.r, hidden, ld.scale, out, xa, s),
                    "lora delta launch");
}

int nvfp4_gemm_w4a4(const void *x, int32_t m, const nvfp4_weight *w, void *y, void *stream) {
  g_err.clear();
  int rc;
  if ((rc = check_act(x, m, "x")) || (rc = check_act(y, m, "y")) || (rc = check_weight(w, "w")))
    return rc;
  if (m == 0) return NVFP4_OK;
  hipStream_t s = (hipStream_t)stream;
  log_path("gemm_w4a4", "stream", m, w->n, w->k);
  QuantBuf q = quant_layout(nullptr, m, w->k);
  size_t part = proj_scratch_bytes(m, w->n, w->k, 1, Path::Stream);
  void *base = nullptr;
  if ((rc = arena_get(q.bytes + part, &base))) return rc;
  q = quant_layout((char *)base, m, w->k);
  ProfileScope ps("gemm_w4a4", m, s);
  if ((rc = hip_status(launch_quantize_rows(x, m, w->k, q.codes, q.scales, q.rs, q.tiles, s), "quantize launch")))
    return rc;
  MatRef wm = mat(w);
  return run_proj(ActRef{nullptr, q.codes, q.scales, q.rs, q.tiles}, m, w->k, w->n, 1, &wm, y,
                  (char *)base + q.bytes, Path::Stream, s);
}

int dense_ffn_forward_w4a4(const void *x, int32_t m, int32_t hidden, int32_t inter,
                           const nvfp4_weight *wg, const nvfp4_weight *wu, const nvfp4_weight *wd,
                           void *out, void *stream) {
  g_err.clear();
  int rc;
  if ((rc = check_ffn(x, m, hidden, inter, wg, wu, wd, out))) return rc;
  if (m == 0) return NVFP4_OK;
  hipStream_t s = (hipStream_t)stream;
  log_path("dense_ffn_forward_w4a4", "stream", m, inter, hidden);
  QuantBuf qx = quant_layout(nullptr, m, hidden);
  QuantBuf qa = quant_layout(nullptr, m, inter);
  const size_t act_b = align256((size_t)2 * m * inter);
  size_t part = proj_scratch_bytes(m, inter, hidden, 2, Path::Stream);
  size_t part_d = proj_scratch_bytes(m, hidden, inter, 1, Path::Stream);
  if (part_d > part) part = part_d;
  void *base = nullptr;
  if ((rc = arena_get(qx.bytes + qa.bytes + act_b + part, &base))) return rc;
  char *p = (char *)base;
  qx = quant_layout(p, m, hidden);
  qa = quant_layout(p + qx.bytes, m, inter);
  char *act = p + qx.bytes + qa.bytes;
  char *scr = act + act_b;
  ProfileScope ps("dense_total w4a4", m, s);
  MatRef w2[2] = {mat(wg), mat(wu)};
  MatRef wdm = mat(wd);
  if ((rc = hip_status(launch_quantize_rows(x, m, hidden, qx.codes, qx.scales, qx.rs, qx.tiles, s),
                       "quantize launch")))
    return rc;
  if ((rc = run_proj(ActRef{nullptr, qx.codes, qx.scales, qx.rs, qx.tiles}, m, hidden, inter, 2, w2, act, scr,
                     Path::Stream, s)))
    return rc;
  if ((rc = hip_status(launch_quantize_rows(act, m, inter, qa.codes, qa.scales, qa.rs, qa.tiles, s),
                       "quantize launch")))
    return rc;
  return run_proj(ActRef{nullptr, qa.codes, qa.scales, qa.rs, qa.tiles}, m, inter, hidden, 1, &wdm, out, scr,
                  Path::Stream, s);
}

int fp8_quantize_rows(const void *x, int32_t m, int32_t k, uint8_t *codes, float *row_scale,
                      void *stream) {
  g_err.clear();
  int rc;
  if ((rc = check_act(x, m, "x"))) return rc;
  if (k <= 0 || k % 32 != 0 || k > kMaxDim)
    return fail(NVFP4_ESHAPE, "fp8_quantize_rows: k=%d must be a positive multiple of 32 up to %d", k,
                kMaxDim);
  if ((rc = check_fp8_rows(m, k, "fp8_quantize_rows"))) return rc;
  if (m == 0) return NVFP4_OK;
  if (!codes || !row_scale) return fail(NVFP4_EINVAL, "fp8_quantize_rows: null output pointer");
  if (misaligned(codes) || ((uintptr_t)row_scale & 3u))
    return fail(NVFP4_EINVAL, "fp8_quantize_rows: codes must be 16-byte and row_scale 4-byte aligned");
  return hip_status(launch_quantize_rows_fp8(x, m, k, codes, row_scale, nullptr, (hipStream_t)stream),
                    "fp8 quantize_rows launch");
}

int fp8_gemm_w8a8(const void *x, int32_t m, const fp8_weight *w, void *y, void *stream) {
  g_err.clear();
  int rc;
  if ((rc = check_act(x, m, "x")) || (rc = check_act(y, m, "y")) || (rc = check_fp8_weight(w, "w")) ||
      (rc = check_fp8_rows(m, w->k, "x")))
    return rc;
  if (m == 0) return NVFP4_OK;
  hipStream_t s = (hipStream_t)stream;
  log_path("gemm_w8a8", "w8a8", m, w->n, w->k);
  Fp8QuantBuf q = fp8_quant_layout(nullptr, m, w->k);
  const size_t part = w8a8_scratch_bytes(m, w->n, w->k, 1);
  void *base = nullptr;
  if ((rc = arena_get(q.bytes + part, &base))) return rc;
  q = fp8_quant_layout((char *)base, m, w->k);
  ProfileScope ps("gemm_w8a8", m, s);
  if ((rc = hip_status(launch_quantize_rows_fp8(x, m, w->k, q.codes, q.rs, q.tiles, s), "fp8 quantize launch")))
    return rc;
  Fp8MatRef wm = fp8_mat(w);
  return run_w8a8(Fp8ActRef{q.codes, q.rs, q.tiles}, m, w->k, w->n, 1, &wm, y, (char *)base + q.bytes, s);
}

int dense_ffn_forward_w8a8(const void *x, int32_t m, int32_t hidden, int32_t inter,
                           const fp8_weight *wg, const fp8_weight *wu, const fp8_weight *wd,
                           void *out, void *stream) {
  g_err.clear();
  int rc;
  if ((rc = check_act(x, m, "x")) || (rc = check_act(out, m, "out"))) return rc;
  if (hidden <= 0 || inter <= 0)
    return fail(NVFP4_ESHAPE, "hidden=%d inter=%d must be positive", hidden, inter);
  if ((rc = check_fp8_weight(wg, "wg")) || (rc = check_fp8_weight(wu, "wu")) ||
      (rc = check_fp8_weight(wd, "wd")))
    return rc;
  if (wg->n != inter || wg->k != hidden || wu->n != inter || wu->k != hidden)
    return fail(NVFP4_ESHAPE, "wg/wu must be [inter=%d][hidden=%d], got [%d][%d] and [%d][%d]",
                inter, hidden, wg->n, wg->k, wu->n, wu->k);
  if (wd->n != hidden || wd->k != inter)
    return fail(NVFP4_ESHAPE, "wd must be [hidden=%d][inter=%d], got [%d][%d]", hidden, inter,
                wd->n, wd->k);
  if ((rc = check_fp8_rows(m, hidden, "x")) || (rc = check_fp8_rows(m, inter, "act"))) return rc;
  if (m == 0) return NVFP4_OK;
  hipStream_t s = (hipStream_t)stream;
  log_path("dense_ffn_forward_w8a8", "w8a8", m, inter, hidden);
  Fp8QuantBuf qx = fp8_quant_layout(nullptr, m, hidden);
  Fp8QuantBuf qa = fp8_quant_layout(nullptr, m, inter);
  const size_t act_b = align256((size_t)2 * m * inter);
  size_t part = w8a8_scratch_bytes(m, inter, hidden, 2);
  const size_t part_d = w8a8_scratch_bytes(m, hidden, inter, 1);
  if (part_d > part) part = part_d;
  void *base = nullptr;
  if ((rc = arena_get(qx.bytes + qa.bytes + act_b + part, &base))) return rc;
  char *p = (char *)base;
  qx = fp8_quant_layout(p, m, hidden);
  qa = fp8_quant_layout(p + qx.bytes, m, inter);
  char *act = p + qx.bytes + qa.bytes;
  char *scr = act + act_b;
  ProfileScope ps("dense_total w8a8", m, s);
  Fp8MatRef w2[2] = {fp8_mat(wg), fp8_mat(wu)};
  Fp8MatRef wdm = fp8_mat(wd);
  if ((rc = hip_status(launch_quantize_rows_fp8(x, m, hidden, qx.codes, qx.rs, qx.tiles, s), "fp8 quantize launch")))
    return rc;
  if ((rc = run_w8a8(Fp8ActRef{qx.codes, qx.rs, qx.tiles}, m, hidden, inter, 2, w2, act, scr, s))) return rc;
  if ((rc = hip_status(launch_quantize_rows_fp8(act, m, inter, qa.codes, qa.rs, qa.tiles, s), "fp8 quantize launch")))
    return rc;
  return run_w8a8(Fp8ActRef{qa.codes, qa.rs, qa.tiles}, m, inter, hidden, 1, &wdm, out, scr, s);
}

int q2_gemm_w2a16(const void *x, int32_t m, const q2_weight *w, void *y, void *stream) {
  g_err.clear();
  int rc, gs = 0;
  if ((rc = check_act(x, m, "x")) || (rc = check_act(y, m, "y")) || (rc = check_q2_weight(w, "w", &gs)))
    return rc;
  if (m == 0) return NVFP4_OK;
  hipStream_t s = (hipStream_t)stream;
  Q2MatRef wm = q2_mat(w);
  if (q2_tiled(m, w->k)) {
    log_path("gemm_q2", "prefill", m, w->n, w->k);
    ProfileScope ps("gemm_q2", m, s);
    return hip_status(launch_prefill_q2(x, m, w->k, w->n, gs, 1, &wm, y, prefill_plan(m, w->n, w->k, 1), s),
                      "packed-Q2 many-row projection launch");
  }
  log_path("gemm_q2", "q2", m, w->n, w->k);
  const size_t part = q2_scratch_bytes(m, w->n, w->k, 1);
  void *scr = nullptr;
  if (part && (rc = arena_get(part, &scr))) return rc;
  ProfileScope ps("gemm_q2", m, s);
  return run_q2(x, m, w->k, w->n, gs, 1, &wm, y, scr, s);
}

int dense_ffn_forward_q2(const void *x, int32_t m, int32_t hidden, int32_t inter, const q2_weight *wg,
                         const q2_weight *wu, const q2_weight *wd, void *out, void *stream) {
  g_err.clear();
  int rc, gsg = 0, gsu = 0, gsd = 0;
  if ((rc = check_act(x, m, "x")) || (rc = check_act(out, m, "out"))) return rc;
  if (hidden <= 0 || inter <= 0)
    return fail(NVFP4_ESHAPE, "hidden=%d inter=%d must be positive", hidden, inter);
  if ((rc = check_q2_weight(wg, "wg", &gsg)) || (rc = check_q2_weight(wu, "wu", &gsu)) ||
      (rc = check_q2_weight(wd, "wd", &gsd)))
    return rc;
  if (wg->n != inter || wg->k != hidden || wu->n != inter || wu->k != hidden)
    return fail(NVFP4_ESHAPE, "wg/wu must be [inter=%d][hidden=%d], got [%d][%d] and [%d][%d]",
                inter, hidden, wg->n, wg->k, wu->n, wu->k);
  if (wd->n != hidden || wd->k != inter)
    return fail(NVFP4_ESHAPE, "wd must be [hidden=%d][inter=%d], got [%d][%d]", hidden, inter,
                wd->n, wd->k);
  if (gsg != gsu)
    return fail(NVFP4_ESHAPE, "wg and wu must share one group size (got %d and %d)", wg->group, wu->group);
  if (m == 0) return NVFP4_OK;
  hipStream_t s = (hipStream_t)stream;
  Q2MatRef mg = q2_mat(wg), mu = q2_mat(wu), md = q2_mat(wd);
  const bool up_tiled = q2_tiled(m, hidden), down_tiled = q2_tiled(m, inter);
  if (up_tiled || down_tiled) {
    // gate+up+silu in one launch, then down; the many-row kernel where
    // k % 64 == 0, else the streaming kernel with 64-row blocks
    log_path("dense_ffn_forward_q2 gate+up", up_tiled ? "prefill" : "q2", m, inter, hidden);
    log_path("dense_ffn_forward_q2 down", down_tiled ? "prefill" : "q2", m, hidden, inter);
    const size_t act_b = align256((size_t)2 * m * inter);
    const size_t part = std::max(up_tiled ? 0 : q2_scratch_bytes(m, inter, hidden, 2),
                                 down_tiled ? 0 : q2_scratch_bytes(m, hidden, inter, 1));
    void *base = nullptr;
    if ((rc = arena_get(act_b + part, &base))) return rc;
    char *act = (char *)base;
    char *scr = act + act_b;
    ProfileScope ps("dense_total q2", m, s);
    Q2MatRef w2[2] = {mg, mu};
    if (up_tiled)
      rc = hip_status(launch_prefill_q2(x, m, hidden, inter, gsg, 2, w2, act, prefill_plan(m, inter, hidden, 2), s),
                      "packed-Q2 many-row projection launch");
    else
      rc = run_q2(x, m, hidden, inter, gsg, 2, w2, act, scr, s);
    if (rc) return rc;
    if (down_tiled)
      return hip_status(launch_prefill_q2(act, m, inter, hidden, gsd, 1, &md, out, prefill_plan(m, hidden, inter, 1), s),
                        "packed-Q2 many-row projection launch");
    return run_q2(act, m, inter, hidden, gsd, 1, &md, out, scr, s);
  }
  log_path("dense_ffn_forward_q2", "q2", m, inter, hidden);
  const size_t act_b = align256((size_t)2 * m * inter);
  size_t part = q2_scratch_bytes(m, inter, hidden, 2);
  const size_t part_d = q2_scratch_bytes(m, hidden, inter, 1);
  if (part_d > part) part = part_d;
  void *base = nullptr;
  if ((rc = arena_get(act_b + part, &base))) return rc;
  char *act = (char *)base;
  char *scr = act + act_b;
  ProfileScope ps("dense_total q2", m, s);
  Q2MatRef w2[2] = {mg, mu};
  if ((rc = run_q2(x, m, hidden, inter, gsg, 2, w2, act, scr, s))) return rc;
  return run_q2(act, m, inter, hidden, gsd, 1, &md, out, scr, s);
}

}  // extern "C"
