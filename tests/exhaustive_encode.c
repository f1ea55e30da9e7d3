/* Exhaustive check of the oracle's fp32 -> E4M3 and fp32 -> E2M1 encoders.
 *
 * TEST INFRASTRUCTURE.  Every one of the 2^32 fp32 bit patterns is encoded by
 * the oracle library (loaded with dlopen) and compared with the code chosen
 * here by a different method: the value set of each format is decoded from its
 * bit fields (OCP Microscaling Formats spec, E4M3 and E2M1 element encodings,
 * as the NVFP4 pages use them), and the code of a magnitude is the nearest
 * entry of that sorted set, found by walking the set alongside the fp32 values
 * in increasing order and comparing with the exact midpoint of the two
 * neighbouring entries.  Ties go to the even code, magnitudes at or above the
 * largest finite value saturate to it, and the sign bit is kept (also for a
 * value that rounds to zero).
 *
 * NaN inputs follow the oracle's stated convention: E4M3FN has a NaN code
 * (0x7F with the sign), E2M1 has none and saturates (code 7 with the sign).
 *
 * Usage: exhaustive_encode <liboracle.so> <threads>
 * Prints one line per format, "<fmt> checked=<n> mismatches=<m>", then up to
 * eight mismatches, and exits 0 only when both formats match everywhere.
 */
#include <dlfcn.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef uint8_t (*encode_fn)(float);

typedef struct {
  const char *name;
  encode_fn enc;
  double vals[128];  /* positive finite values, index = code */
  int nvals;         /* number of positive finite codes */
  uint8_t sign_bit;
  uint8_t nan_code;  /* magnitude code an input NaN maps to */
} format;

/* E4M3FN: 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is
 * subnormal with spacing 2^-9; 0x7F is NaN, so codes 0..0x7E are finite. */
static void make_e4m3(format *f) {
  f->name = "e4m3";
  f->nvals = 127;
  for (int c = 0; c < 127; c++) {
    int e = c >> 3, m = c & 7;
    f->vals[c] = e == 0 ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 7 - 3);
  }
  f->sign_bit = 0x80;
  f->nan_code = 0x7F;
}

/* E2M1: 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is subnormal
 * with spacing 1/2; all eight magnitude codes are finite. */
static void make_e2m1(format *f) {
  f->name = "e2m1";
  f->nvals = 8;
  for (int c = 0; c < 8; c++) {
    int e = c >> 1, m = c & 1;
    f->vals[c] = e == 0 ? 0.5 * m : ldexp(2.0 + m, e - 1 - 1);
  }
  f->sign_bit = 8;
  f->nan_code = 7;
}

typedef struct {
  const format *f;
  uint64_t lo, hi;   /* magnitude bit patterns [lo, hi) */
  uint64_t checked, bad;
  uint32_t bad_bits[8];
  uint8_t bad_got[8], bad_want[8];
} job;

static void note(job *j, uint32_t bits, uint8_t got, uint8_t want) {
  if (j->bad < 8) {
    j->bad_bits[j->bad] = bits;
    j->bad_got[j->bad] = got;
    j->bad_want[j->bad] = want;
  }
  j->bad++;
}

static void *run(void *arg) {
  job *j = (job *)arg;
  const format *f = j->f;
  const double top = f->vals[f->nvals - 1];
  int i = 0;  /* vals[i] <= a < vals[i + 1] for the current finite a < top */
  for (uint64_t b = j->lo; b < j->hi; b++) {
    uint32_t bits = (uint32_t)b;
    float t;
    memcpy(&t, &bits, 4);
    uint8_t want;
    if (bits > 0x7F800000u) {
      want = f->nan_code;
    } else {
      double a = (double)t;
      if (a >= top) {
        want = (uint8_t)(f->nvals - 1);
      } else {
        while (f->vals[i + 1] <= a) i++;
        double mid = 0.5 * (f->vals[i] + f->vals[i + 1]);  /* exact: few bits */
        if (a < mid) want = (uint8_t)i;
        else if (a > mid) want = (uint8_t)(i + 1);
        else want = (uint8_t)((i & 1) ? i + 1 : i);
      }
    }
    for (int s = 0; s < 2; s++) {
      uint32_t sb = bits | (s ? 0x80000000u : 0u);
      float ts;
      memcpy(&ts, &sb, 4);
      uint8_t w = want | (s ? f->sign_bit : 0);
      uint8_t got = f->enc(ts);
      if (got != w) note(j, sb, got, w);
    }
    j->checked += 2;
  }
  return NULL;
}

static int check(const format *f, int nthreads) {
  job *jobs = calloc((size_t)nthreads, sizeof(job));
  pthread_t *tid = calloc((size_t)nthreads, sizeof(pthread_t));
  const uint64_t total = 0x80000000ull;  /* magnitudes; each runs with both signs */
  for (int t = 0; t < nthreads; t++) {
    jobs[t].f = f;
    jobs[t].lo = total * t / nthreads;
    jobs[t].hi = total * (t + 1) / nthreads;
  }
  for (int t = 0; t < nthreads; t++) pthread_create(&tid[t], NULL, run, &jobs[t]);
  uint64_t checked = 0, bad = 0;
  for (int t = 0; t < nthreads; t++) {
    pthread_join(tid[t], NULL);
    checked += jobs[t].checked;
    bad += jobs[t].bad;
  }
  printf("%s checked=%llu mismatches=%llu\n", f->name, (unsigned long long)checked,
         (unsigned long long)bad);
  int shown = 0;
  for (int t = 0; t < nthreads && shown < 8; t++)
    for (uint64_t q = 0; q < jobs[t].bad && q < 8 && shown < 8; q++, shown++) {
      float v;
      memcpy(&v, &jobs[t].bad_bits[q], 4);
      printf("  %s bits=0x%08x (%.9g) got=0x%02x want=0x%02x\n", f->name, jobs[t].bad_bits[q],
             (double)v, jobs[t].bad_got[q], jobs[t].bad_want[q]);
    }
  free(jobs);
  free(tid);
  return bad == 0;
}

int main(int argc, char **argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s <liboracle.so> <threads>\n", argv[0]);
    return 2;
  }
  int nthreads = atoi(argv[2]);
  if (nthreads < 1 || nthreads > 256) nthreads = 1;
  void *h = dlopen(argv[1], RTLD_NOW | RTLD_LOCAL);
  if (!h) {
    fprintf(stderr, "dlopen: %s\n", dlerror());
    return 2;
  }
  format e4m3, e2m1;
  make_e4m3(&e4m3);
  make_e2m1(&e2m1);
  e4m3.enc = (encode_fn)dlsym(h, "nvo_e4m3_encode");
  e2m1.enc = (encode_fn)dlsym(h, "nvo_e2m1_encode");
  if (!e4m3.enc || !e2m1.enc) {
    fprintf(stderr, "missing encoder symbols\n");
    return 2;
  }
  /* the value sets must be strictly increasing in the code for the walk */
  for (int c = 1; c < e4m3.nvals; c++)
    if (!(e4m3.vals[c] > e4m3.vals[c - 1])) return 3;
  for (int c = 1; c < e2m1.nvals; c++)
    if (!(e2m1.vals[c] > e2m1.vals[c - 1])) return 3;
  if (e4m3.vals[126] != 448.0 || e4m3.vals[1] != ldexp(1.0, -9) || e2m1.vals[7] != 6.0) return 3;
  int ok = check(&e4m3, nthreads);
  ok &= check(&e2m1, nthreads);
  fflush(stdout);
  return ok ? 0 : 1;
}
