/*
 * synth.c - seeded, counter-based synthetic inputs (see synth.h).
 *
 * Generation recipe, matching the MoE decode workloads: weights are uniform
 * E2M1 codes with log-uniform E4M3 block scales, activations and router
 * logits are standard normals, skewed routing adds a normal per-expert bias
 * or draws Zipf popularity through Gumbel noise.
 */
#include "synth.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

uint64_t synth_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint64_t a, uint64_t b, uint64_t c, uint64_t d) {
  uint64_t k = synth_mix(seed + GOLDEN);
  k = synth_mix(k ^ (a + 1) * GOLDEN);
  k = synth_mix(k ^ (b + 1) * GOLDEN);
  k = synth_mix(k ^ (c + 1) * GOLDEN);
  k = synth_mix(k ^ (d + 1) * GOLDEN);
  return k;
}

uint64_t synth_u64(uint64_t key, uint64_t i) { return synth_mix(key + (i + 1) * GOLDEN); }

/* Uniform double in [0, 1) on the 53-bit grid. */
static double unit53(uint64_t v) { return (double)(v >> 11) * (1.0 / 9007199254740992.0); }

/* ---- threaded range fills ------------------------------------------------ */

typedef void (*range_fn)(void* ctx, int64_t begin, int64_t end);
typedef struct {
  range_fn fn;
  void* ctx;
  int64_t begin, end;
} range_job;

static void* run_job(void* p) {
  range_job* j = (range_job*)p;
  j->fn(j->ctx, j->begin, j->end);
  return NULL;
}

static void parallel_range(range_fn fn, void* ctx, int64_t n, int64_t grain, int nthreads) {
  if (nthreads <= 0) {
    long c = sysconf(_SC_NPROCESSORS_ONLN);
    nthreads = c > 16 ? 16 : (c < 1 ? 1 : (int)c);
  }
  if (n < grain * 2 || nthreads == 1) {
    fn(ctx, 0, n);
    return;
  }
  int64_t parts = (n + grain - 1) / grain;
  if (parts < nthreads) nthreads = (int)parts;
  pthread_t th[64];
  range_job jobs[64];
  if (nthreads > 64) nthreads = 64;
  int64_t per = (n + nthreads - 1) / nthreads;
  per = (per + 7) & ~(int64_t)7; /* whole 8-byte words per thread */
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    int64_t b = (int64_t)t * per, e = b + per;
    if (b >= n) break;
    if (e > n) e = n;
    jobs[t].fn = fn;
    jobs[t].ctx = ctx;
    jobs[t].begin = b;
    jobs[t].end = e;
    if (pthread_create(&th[t], NULL, run_job, &jobs[t]) != 0) {
      run_job(&jobs[t]);
      th[t] = 0;
    }
    started = t + 1;
  }
  for (int t = 0; t < started; ++t)
    if (th[t]) pthread_join(th[t], NULL);
}

/* ---- bytes ---------------------------------------------------------------- */

typedef struct {
  uint64_t key;
  uint8_t* out;
} bytes_ctx;

/* Byte j of a stream is byte (j % 8), little-endian, of counter j / 8. */
static void bytes_span(uint64_t key, uint8_t* out, int64_t b, int64_t e) {
  int64_t j = b;
  while (j < e && (j & 7)) {
    out[j] = (uint8_t)(synth_u64(key, (uint64_t)(j >> 3)) >> (8 * (j & 7)));
    ++j;
  }
  for (; j + 8 <= e; j += 8) {
    uint64_t w = synth_u64(key, (uint64_t)(j >> 3));
    for (int q = 0; q < 8; ++q) out[j + q] = (uint8_t)(w >> (8 * q));
  }
  for (; j < e; ++j) out[j] = (uint8_t)(synth_u64(key, (uint64_t)(j >> 3)) >> (8 * (j & 7)));
}

static void bytes_range(void* p, int64_t b, int64_t e) {
  bytes_ctx* c = (bytes_ctx*)p;
  bytes_span(c->key, c->out, b, e);
}

void synth_fill_bytes(uint64_t key, uint8_t* out, int64_t n, int nthreads) {
  bytes_ctx c = {key, out};
  parallel_range(bytes_range, &c, n, 1 << 20, nthreads);
}

/* ---- log-uniform E4M3 scale codes ---------------------------------------- */

typedef struct {
  uint64_t key;
  uint8_t* out;
  double lo, span;
  double frac_edge[8]; /* log2(1 + (q + 1/2) / 8): rounding edges inside an octave */
} scale_ctx;

static void scales_range(void* p, int64_t b, int64_t e) {
  scale_ctx* c = (scale_ctx*)p;
  for (int64_t j = b; j < e; ++j) {
    double u = c->lo + c->span * unit53(synth_u64(c->key, (uint64_t)j));
    double oct = floor(u);
    double f = u - oct;
    int q = 0;
    while (q < 8 && f >= c->frac_edge[q]) ++q;
    int ex = (int)oct;
    if (q == 8) {
      q = 0;
      ex += 1;
    }
    c->out[j] = (uint8_t)(((ex + 7) << 3) | q);
  }
}

int synth_fill_scales(uint64_t key, uint8_t* out, int64_t n, double lo_log2, double hi_log2,
                      int nthreads) {
  if (!(lo_log2 >= -6.0 && hi_log2 <= 8.0 && lo_log2 < hi_log2)) return -1;
  scale_ctx c;
  c.key = key;
  c.out = out;
  c.lo = lo_log2;
  c.span = hi_log2 - lo_log2;
  for (int q = 0; q < 8; ++q) c.frac_edge[q] = log2(1.0 + (q + 0.5) / 8.0);
  parallel_range(scales_range, &c, n, 1 << 18, nthreads);
  return 0;
}

/* ---- normals -------------------------------------------------------------- */

/* Box-Muller on counters 2i and 2i+1: u1 in (0, 1], u2 in [0, 1). */
static double normal_at(uint64_t key, int64_t i) {
  double u1 = 1.0 - unit53(synth_u64(key, (uint64_t)(2 * i)));
  double u2 = unit53(synth_u64(key, (uint64_t)(2 * i + 1)));
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}

void synth_fill_normal_f32(uint64_t key, float* out, int64_t n, double mean, double std) {
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(mean + std * normal_at(key, i));
}

static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

void synth_fill_normal_bf16(uint64_t key, uint16_t* out, int64_t n, double mean, double std) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne((float)(mean + std * normal_at(key, i)));
}

/* ---- Zipf popularity through Gumbel noise ---------------------------------- */

void synth_fill_zipf_gumbel(uint64_t key, uint64_t perm_key, float* out, int64_t M, int64_t E,
                            double s) {
  int64_t* rank = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
  double* lp = (double*)malloc(sizeof(double) * (size_t)E);
  for (int64_t e = 0; e < E; ++e) rank[e] = e;
  for (int64_t i = E - 1; i > 0; --i) { /* Fisher-Yates */
    int64_t j = (int64_t)(synth_u64(perm_key, (uint64_t)i) % (uint64_t)(i + 1));
    int64_t t = rank[i];
    rank[i] = rank[j];
    rank[j] = t;
  }
  double z = 0.0;
  for (int64_t r = 1; r <= E; ++r) z += pow((double)r, -s);
  for (int64_t e = 0; e < E; ++e) lp[e] = log(pow((double)(rank[e] + 1), -s) / z);
  for (int64_t m = 0; m < M; ++m)
    for (int64_t e = 0; e < E; ++e) {
      double u = 1.0 - unit53(synth_u64(key, (uint64_t)(m * E + e))); /* (0, 1] */
      double gum = -log(-log(u > 0.9999999999999999 ? 0.9999999999999999 : u));
      out[m * E + e] = (float)(lp[e] + gum);
    }
  free(rank);
  free(lp);
}

/* ---- many streams at once: one key per matrix, threads across matrices ---- */

typedef struct {
  const uint64_t* keys;
  uint8_t* out;
  int64_t per;
  int is_scale;
  double lo, span;
  double frac_edge[8];
} multi_ctx;

static void multi_range(void* p, int64_t b, int64_t e) {
  multi_ctx* c = (multi_ctx*)p;
  for (int64_t g = b; g < e; ++g) {
    if (!c->is_scale) {
      bytes_span(c->keys[g], c->out + g * c->per, 0, c->per);
    } else {
      scale_ctx s;
      s.key = c->keys[g];
      s.out = c->out + g * c->per;
      s.lo = c->lo;
      s.span = c->span;
      memcpy(s.frac_edge, c->frac_edge, sizeof(s.frac_edge));
      scales_range(&s, 0, c->per);
    }
  }
}

void synth_fill_bytes_keys(const uint64_t* keys, int64_t G, uint8_t* out, int64_t per,
                           int nthreads) {
  multi_ctx c;
  memset(&c, 0, sizeof(c));
  c.keys = keys;
  c.out = out;
  c.per = per;
  parallel_range(multi_range, &c, G, 1, nthreads);
}

int synth_fill_scales_keys(const uint64_t* keys, int64_t G, uint8_t* out, int64_t per,
                           double lo_log2, double hi_log2, int nthreads) {
  if (!(lo_log2 >= -6.0 && hi_log2 <= 8.0 && lo_log2 < hi_log2)) return -1;
  multi_ctx c;
  memset(&c, 0, sizeof(c));
  c.keys = keys;
  c.out = out;
  c.per = per;
  c.is_scale = 1;
  c.lo = lo_log2;
  c.span = hi_log2 - lo_log2;
  for (int q = 0; q < 8; ++q) c.frac_edge[q] = log2(1.0 + (q + 0.5) / 8.0);
  parallel_range(multi_range, &c, G, 1, nthreads);
  return 0;
}
