/*
 * inputs_gen.c -- counter-based seeded normal samples for the synthetic
 * inputs of the tests and the benchmark (host side, plain C, threads).
 *
 * Holds none of the shard path's arithmetic: it only draws numbers.  Every
 * element is a pure function of (key, global row, column), so a rank's shard,
 * a few rows of it, or the whole tensor can be drawn independently on any
 * machine and always give the same bytes:
 *
 *   pair p   = (row * cols + col) / 2
 *   u        = mix64(key + (p + 1) * 0x9E3779B97F4A7C15)      (SplitMix64)
 *   u1       = ((u >> 40) + 1) / 2^24  in (0, 1],  u2 = (u & 0xFFFFFF) / 2^24
 *   z        = sqrtf(-2 logf u1) * (cosf 2 pi u2 for even elements, sinf for odd)
 *                                            (Box-Muller, single precision)
 *   value    = float(mu + sigma * z)   (in double, one rounding to f32)
 *   bf16     = the f32 value rounded to nearest even
 *
 * key = mix64(mix64(seed) + tensor * 0xD1B54A32D192ED03 + source * 0xABC98388FB8FAC03).
 */
#define _GNU_SOURCE /* sincosf */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

static uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t sprms_inputs_key(uint64_t seed, uint64_t tensor, uint64_t source) {
  return mix64(mix64(seed) + tensor * 0xD1B54A32D192ED03ull + source * 0xABC98388FB8FAC03ull);
}

static const float kTwoPiF = 6.28318530717958647692f;

/* elements 2p and 2p + 1 of the stream as f32 (one Box-Muller pair; the
 * radius and angle in single precision, mu + sigma * z in double) */
static void sample_pair(uint64_t key, uint64_t p, double mu, double sigma, float* even, float* odd) {
  const uint64_t u = mix64(key + (p + 1) * 0x9E3779B97F4A7C15ull);
  const float u1 = (float)((double)((u >> 40) + 1) * (1.0 / 16777216.0));  /* (0, 1], 24 bits */
  const float u2 = (float)((double)(u & 0xFFFFFFull) * (1.0 / 16777216.0)); /* [0, 1), 24 bits */
  const float r = sqrtf(-2.0f * logf(u1));
  float s, c;
  sincosf(kTwoPiF * u2, &s, &c);
  *even = (float)(mu + sigma * (double)(r * c));
  *odd = (float)(mu + sigma * (double)(r * s));
}

static uint16_t bf16_rne(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  if ((b & 0x7F800000u) == 0x7F800000u) return (uint16_t)((b >> 16) | ((b & 0xFFFFu) ? 0x40u : 0u));
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

typedef struct {
  uint64_t key;
  int64_t row0, rows, cols;
  double mu, sigma;
  int bf16;
  void* out;
} job;

static void put(const job* j, int64_t i, float v) {
  if (j->bf16)
    ((uint16_t*)j->out)[i] = bf16_rne(v);
  else
    ((float*)j->out)[i] = v;
}

static void run(const job* j, int64_t r_lo, int64_t r_hi) {
  for (int64_t r = r_lo; r < r_hi; ++r) {
    const uint64_t base = (uint64_t)(j->row0 + r) * (uint64_t)j->cols;
    for (int64_t c = 0; c < j->cols;) {
      const uint64_t e = base + (uint64_t)c;
      float ev, od;
      sample_pair(j->key, e >> 1, j->mu, j->sigma, &ev, &od);
      if ((e & 1) == 0 && c + 1 < j->cols) {  /* both elements of the pair are in this row */
        put(j, r * j->cols + c, ev);
        put(j, r * j->cols + c + 1, od);
        c += 2;
      } else {
        put(j, r * j->cols + c, (e & 1) ? od : ev);
        c += 1;
      }
    }
  }
}

typedef struct {
  const job* j;
  int64_t lo, hi;
} slice;

static void* run_slice(void* p) {
  const slice* s = (const slice*)p;
  run(s->j, s->lo, s->hi);
  return NULL;
}

/* rows [row0, row0 + rows) of a [.][cols] tensor into out (f32 or bf16 bits),
 * split over up to `threads` threads (at most 64).  Returns 0, or -1 on bad
 * arguments. */
int sprms_inputs_normal(uint64_t key, int64_t row0, int64_t rows, int64_t cols, double mu, double sigma,
                        int bf16, void* out, int threads) {
  if (row0 < 0 || rows < 0 || cols < 1 || (rows > 0 && !out)) return -1;
  job j = {key, row0, rows, cols, mu, sigma, bf16, out};
  if (threads > 64) threads = 64;
  if (threads < 1 || rows * cols < (1 << 16)) threads = 1;
  if (threads > rows) threads = (int)(rows > 0 ? rows : 1);
  if (threads == 1) {
    run(&j, 0, rows);
    return 0;
  }
  pthread_t tid[64];
  slice sl[64];
  int created[64];
  for (int t = 0; t < threads; ++t) {
    sl[t].j = &j;
    sl[t].lo = rows * t / threads;
    sl[t].hi = rows * (t + 1) / threads;
    created[t] = pthread_create(&tid[t], NULL, run_slice, &sl[t]) == 0;
    if (!created[t]) run(&j, sl[t].lo, sl[t].hi); /* no thread: do that slice here */
  }
  for (int t = 0; t < threads; ++t)
    if (created[t]) pthread_join(tid[t], NULL);
  return 0;
}
