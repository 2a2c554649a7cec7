/*
 * Seeded synthetic inputs for the routed-expert FFN path.
 *
 * This module is shared by the CPU oracle and by the GPU tests/bench. It holds
 * no arithmetic of the method itself (no routing, no dequantization, no FFN):
 * it draws random numbers and writes them out, including the *encoding* of
 * float weights into the record byte layout described below (the decoders on
 * both sides are written independently from that description).
 *
 * Random numbers: SplitMix64 (Steele, Lea & Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014), used counter-based: the j-th
 * draw of a stream is mix64(key + (j + 1) * GAMMA), where the key is derived
 * from (seed, tag, a, b).  Any record or row can therefore be regenerated on
 * its own.
 *
 * Approximate normal draws: the sum of the four 16-bit fields of one 64-bit
 * draw (Irwin-Hall, n = 4), centred and scaled to unit variance.
 *
 * Record layout (one record = every tensor of one (layer, expert)):
 *   gate payload [I x H] | up payload [I x H] | down payload [H x I] |
 *   gate scales | up scales | down scales
 * The tensor order follows the expert record of the NVMe streaming page
 * ("엔진", item 1).  Each matrix (N output rows, Kd input columns, N % 16 == 0,
 * Kd % 32 == 0) is cut into tiles of 16 rows x 32 inputs, tile index
 * (n / 16) * (Kd / 32) + k / 32 (row slices outer, inputs inner).  A tile's 256
 * payload bytes hold element (n, k) at byte (q * 16 + r) * 4 + i / 2 with
 * r = n % 16, q = (k % 32) / 8, i = k % 8, even i in the low nibble.  Its 32
 * scale bytes (scale area, same tile index): int4 -> bf16 scale of (n, k / 32)
 * at r * 2; NVFP4 -> e4m3 scale of (n, k / 16) at ((k % 32) / 16) * 16 + r.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint64_t tag, uint64_t a, uint64_t b) {
  uint64_t k = mix64(seed ^ mix64(tag + GAMMA));
  k = mix64(k ^ mix64(a + 2 * GAMMA));
  k = mix64(k ^ mix64(b + 3 * GAMMA));
  return k;
}

static inline uint64_t draw(uint64_t key, uint64_t j) { return mix64(key + (j + 1) * GAMMA); }

static const double IH4_MEAN = 131070.0; /* 4 * 65535 / 2 */

static inline double approx_normal(uint64_t r) {
  const double inv_sd = 1.0 / sqrt(4.0 * (65536.0 * 65536.0 - 1.0) / 12.0); /* folded at compile time */
  double s = (double)(r & 0xFFFF) + (double)((r >> 16) & 0xFFFF) + (double)((r >> 32) & 0xFFFF) +
             (double)(r >> 48);
  return (s - IH4_MEAN) * inv_sd;
}

static inline double uniform01(uint64_t r) { return ((double)(r >> 11) + 0.5) * (1.0 / 9007199254740992.0); }

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t bias = 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)((u + bias) >> 16);
}

static inline float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* ---------------------------------------------------------------- plain tensors */

void synth_normal_f32(uint64_t seed, uint64_t tag, uint64_t a, uint64_t b, int64_t n, double scale,
                      float* out) {
  uint64_t key = synth_key(seed, tag, a, b);
  for (int64_t j = 0; j < n; ++j) out[j] = (float)(scale * approx_normal(draw(key, (uint64_t)j)));
}

void synth_normal_bf16(uint64_t seed, uint64_t tag, uint64_t a, uint64_t b, int64_t n, double scale,
                       uint16_t* out) {
  uint64_t key = synth_key(seed, tag, a, b);
  for (int64_t j = 0; j < n; ++j)
    out[j] = f32_to_bf16_rne((float)(scale * approx_normal(draw(key, (uint64_t)j))));
}

void synth_uniform_f64(uint64_t seed, uint64_t tag, uint64_t a, uint64_t b, int64_t n, double* out) {
  uint64_t key = synth_key(seed, tag, a, b);
  for (int64_t j = 0; j < n; ++j) out[j] = uniform01(draw(key, (uint64_t)j));
}

/* ---------------------------------------------------------------- encoders */

/* e4m3 (OCP E4M3FN) value of a code: bias 7, subnormals, S.1111.111 is NaN. */
static double e4m3_value(int code) {
  int e = (code >> 3) & 15, m = code & 7;
  double v = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  return (code & 0x80) ? -v : v;
}

/* nearest positive e4m3 code (0x00..0x7E), ties to the even code; clamps to 448.
 * Within a binade 2^e * (1 + m/8) the nearest m is rint of the scaled mantissa (ties to even
 * m, i.e. the even code); m = 8 carries into the next binade; below 2^-6 the codes are the
 * subnormals m * 2^-9 with the same spacing. */
static uint8_t e4m3_encode_pos(double v) {
  if (!(v > 0.0)) return 0;
  if (v >= 448.0) return 0x7E;
  if (v < 0.015625) return (uint8_t)rint(v * 512.0); /* 0..8; 8 is 2^-6, code 0x08 */
  int ex;
  double f = frexp(v, &ex);                           /* v = f * 2^ex, f in [0.5, 1) */
  int e = ex - 1;
  int m = (int)rint((2.0 * f - 1.0) * 8.0);
  if (m == 8) { m = 0; e += 1; }
  int code = ((e + 7) << 3) | m;
  return (uint8_t)(code > 0x7E ? 0x7E : code);
}

/* nearest e2m1 code for v (sign kept, magnitude clamped to 6), ties to the even code.
 * Magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6; midpoints .25 .75 1.25 1.75 2.5 3.5 5 go to the even
 * code of the two (codes 0, 2, 2, 4, 4, 6, 6). */
static inline uint8_t e2m1_encode(double v) {
  double a = fabs(v);
  int c = (a > 0.25) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5) + (a >= 3.5) + (a > 5.0);
  return (uint8_t)(c | ((v < 0.0) ? 8 : 0));
}

/* ---------------------------------------------------------------- record layout (writer side) */

static inline int64_t scale_tile_off(int64_t Kd, int64_t n, int64_t k) {
  return ((n / 16) * (Kd / 32) + k / 32) * 32;
}

int64_t synth_record_bytes(int64_t H, int64_t I) { return 3 * H * I / 2 + 3 * H * I / 16; }

enum { FMT_INT4_G32_BF16 = 0, FMT_NVFP4_G16_E4M3 = 1 };
enum { TAG_WEIGHT = 1 };

/* float weights of matrix m (0 gate [I,H], 1 up [I,H], 2 down [H,I]) of expert (l, e). */
void synth_weights_f32(uint64_t seed, int64_t E, int64_t l, int64_t e, int m, int64_t H, int64_t I,
                       double sigma, float* out) {
  int64_t N = (m == 2) ? H : I, Kd = (m == 2) ? I : H;
  synth_normal_f32(seed, TAG_WEIGHT, (uint64_t)(l * E + e), (uint64_t)m, N * Kd, sigma, out);
}

/* Store the 32 codes of inputs 32*kb .. 32*kb+31 of row n (one chunk) into the payload. */
static inline void put_chunk(uint8_t* pay, int64_t Kd, int64_t n, int64_t kb, const uint8_t* codes) {
  int64_t tile = (n / 16) * (Kd / 32) + kb;
  int64_t r = n % 16;
  for (int q = 0; q < 4; ++q) {
    uint8_t* dst = pay + tile * 256 + (q * 16 + r) * 4;
    for (int j = 0; j < 4; ++j)
      dst[j] = (uint8_t)((codes[q * 8 + 2 * j] & 15) | ((codes[q * 8 + 2 * j + 1] & 15) << 4));
  }
}

/* Encode one matrix (row-major floats w[N][Kd]) into payload + scale bytes. */
static void encode_matrix(const float* w, int64_t N, int64_t Kd, int fmt, uint8_t* pay, uint8_t* sc,
                          float* tensor_scale) {
  uint8_t codes[32];
  /* chunks are visited in the payload's own order (input block outer, row inner) */
  if (fmt == FMT_INT4_G32_BF16) {
    for (int64_t g = 0; g < Kd / 32; ++g) {
      for (int64_t n = 0; n < N; ++n) {
        const float* wg = w + n * Kd + g * 32;
        double amax = 0.0;
        for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs((double)wg[i]));
        uint16_t sbits = f32_to_bf16_rne((float)(amax / 7.0));
        double s = (double)bf16_to_f32(sbits);
        if (!(s > 0.0)) { sbits = 0x3F80; s = 1.0; } /* all-zero group: codes 8 -> 0.0 */
        int64_t so = scale_tile_off(Kd, n, g * 32) + (n % 16) * 2;
        memcpy(sc + so, &sbits, 2);
        const double inv = 1.0 / s;
        for (int i = 0; i < 32; ++i) {
          double qd = nearbyint((double)wg[i] * inv); /* round-half-even (default FP mode) */
          if (qd < -8) qd = -8;
          if (qd > 7) qd = 7;
          codes[i] = (uint8_t)((int)qd + 8);
        }
        put_chunk(pay, Kd, n, g, codes);
      }
    }
    *tensor_scale = 1.0f;
  } else {
    double amax = 0.0;
    for (int64_t j = 0; j < N * Kd; ++j) amax = fmax(amax, fabs((double)w[j]));
    float ts = (float)(amax / (6.0 * 448.0));
    if (!(ts > 0.0f)) ts = 1.0f;
    *tensor_scale = ts;
    for (int64_t g = 0; g < Kd / 32; ++g) {
      for (int64_t n = 0; n < N; ++n) {
        for (int h = 0; h < 2; ++h) {
          const float* wg = w + n * Kd + g * 32 + h * 16;
          double bmax = 0.0;
          for (int i = 0; i < 16; ++i) bmax = fmax(bmax, fabs((double)wg[i]));
          uint8_t sb = e4m3_encode_pos(bmax / (6.0 * (double)ts));
          double sv = e4m3_value(sb) * (double)ts;
          int64_t k0 = g * 32 + h * 16;
          int64_t so = scale_tile_off(Kd, n, k0) + ((k0 % 32) / 16) * 16 + (n % 16);
          sc[so] = sb;
          if (sv > 0.0) {
            const double inv = 1.0 / sv;
            for (int i = 0; i < 16; ++i) codes[h * 16 + i] = e2m1_encode((double)wg[i] * inv);
          } else {
            for (int i = 0; i < 16; ++i) codes[h * 16 + i] = 0;
          }
        }
        put_chunk(pay, Kd, n, g, codes);
      }
    }
  }
}

/* Write the record of expert (l, e) into rec (synth_record_bytes bytes); ts3 gets the
 * three tensor scales (1.0 for int4). scratch must hold max(I*H) floats. */
void synth_record(uint64_t seed, int64_t E, int64_t l, int64_t e, int64_t H, int64_t I, int fmt,
                  double sigma, uint8_t* rec, float* ts3, float* scratch) {
  int64_t pay_m = H * I / 2, sc_m = H * I / 16;
  for (int m = 0; m < 3; ++m) {
    int64_t N = (m == 2) ? H : I, Kd = (m == 2) ? I : H;
    synth_weights_f32(seed, E, l, e, m, H, I, sigma, scratch);
    encode_matrix(scratch, N, Kd, fmt, rec + m * pay_m, rec + 3 * pay_m + m * sc_m, &ts3[m]);
  }
}

typedef struct {
  uint64_t seed;
  int64_t E, H, I, first, count, R;
  int fmt;
  double sigma;
  uint8_t* pool;
  float* ts;
  int64_t next; /* shared work counter */
  pthread_mutex_t mu;
} fill_job;

static void* fill_worker(void* arg) {
  fill_job* J = (fill_job*)arg;
  float* scratch = (float*)malloc(sizeof(float) * (size_t)(J->H * J->I));
  if (!scratch) return (void*)1;
  for (;;) {
    pthread_mutex_lock(&J->mu);
    int64_t i = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (i >= J->count) break;
    int64_t flat = J->first + i;
    int64_t l = flat / J->E, e = flat % J->E;
    synth_record(J->seed, J->E, l, e, J->H, J->I, J->fmt, J->sigma, J->pool + i * J->R,
                 J->ts + 3 * i, scratch);
  }
  free(scratch);
  return NULL;
}

/* Fill `count` consecutive records starting at flat id `first` (= layer * E + expert). */
int synth_fill_records(uint64_t seed, int64_t E, int64_t H, int64_t I, int fmt, double sigma,
                       int64_t first, int64_t count, uint8_t* pool, float* ts, int nthreads) {
  if (H % 64 || I % 64 || nthreads < 1) return -1; /* 32 | inputs, 16 | rows, and the library's 64 */
  fill_job J;
  J.seed = seed; J.E = E; J.H = H; J.I = I; J.first = first; J.count = count;
  J.R = synth_record_bytes(H, I); J.fmt = fmt; J.sigma = sigma; J.pool = pool; J.ts = ts; J.next = 0;
  pthread_mutex_init(&J.mu, NULL);
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  int started = 0, rc = 0;
  for (int t = 0; t < nthreads; ++t)
    if (pthread_create(&th[t], NULL, fill_worker, &J) == 0) started++;
  if (started == 0) rc = -2;
  for (int t = 0; t < started; ++t) {
    void* ret = NULL;
    pthread_join(th[t], &ret);
    if (ret) rc = -3;
  }
  pthread_mutex_destroy(&J.mu);
  return rc;
}

/* ---------------------------------------------------------------- routing traces */

enum { TAG_PERM = 11, TAG_GUMBEL = 12, TAG_SPEC = 13 };

/* Popularity of layer l: a seeded permutation pi (Fisher-Yates), p[pi[i]] ~ 1/(i+1)^s. */
void synth_zipf_logp(uint64_t seed, int64_t l, int64_t E, double s, double* logp) {
  int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  if (!perm) return;
  for (int64_t i = 0; i < E; ++i) perm[i] = (int32_t)i;
  uint64_t key = synth_key(seed, TAG_PERM, (uint64_t)l, 0);
  for (int64_t i = E - 1; i > 0; --i) {
    int64_t j = (int64_t)(uniform01(draw(key, (uint64_t)i)) * (double)(i + 1));
    if (j > i) j = i;
    int32_t t = perm[i]; perm[i] = perm[j]; perm[j] = t;
  }
  double z = 0.0;
  for (int64_t i = 0; i < E; ++i) z += pow((double)(i + 1), -s);
  for (int64_t i = 0; i < E; ++i) logp[perm[i]] = -s * log((double)(i + 1)) - log(z);
  free(perm);
}

/* Trace logits of layer l for tokens [t0, t0 + n): logp + Gumbel; the top-K of each row is a
 * draw of K experts without replacement, proportional to p (Gumbel-top-k). out[n][E], fp32. */
void synth_trace_logits(uint64_t seed, int64_t l, int64_t E, double s, int64_t t0, int64_t n,
                        float* out) {
  double* logp = (double*)malloc(sizeof(double) * (size_t)E);
  if (!logp) return;
  synth_zipf_logp(seed, l, E, s, logp);
  for (int64_t t = 0; t < n; ++t) {
    uint64_t key = synth_key(seed, TAG_GUMBEL, (uint64_t)l, (uint64_t)(t0 + t));
    for (int64_t e = 0; e < E; ++e) {
      double u = uniform01(draw(key, (uint64_t)e));
      out[t * E + e] = (float)(logp[e] - log(-log(u)));
    }
  }
  free(logp);
}

/* Predicted ids for a speculative request: each id of the true set `truth[K]` is kept with
 * probability keep; every dropped one is replaced by a fresh draw from p (rejection of ids
 * already in the true set or already chosen).  out[K]. */
void synth_spec_ids(uint64_t seed, int64_t l, int64_t E, double s, int64_t t, const int32_t* truth,
                    int K, double keep, int32_t* out) {
  double* logp = (double*)malloc(sizeof(double) * (size_t)E);
  double* cdf = (double*)malloc(sizeof(double) * (size_t)E);
  if (!logp || !cdf) { free(logp); free(cdf); return; }
  synth_zipf_logp(seed, l, E, s, logp);
  double acc = 0.0;
  for (int64_t e = 0; e < E; ++e) { acc += exp(logp[e]); cdf[e] = acc; }
  uint64_t key = synth_key(seed, TAG_SPEC, (uint64_t)l, (uint64_t)t);
  uint64_t j = 0;
  for (int k = 0; k < K; ++k) out[k] = -1;
  for (int k = 0; k < K; ++k)
    if (uniform01(draw(key, j++)) < keep) out[k] = truth[k];
  for (int k = 0; k < K; ++k) {
    if (out[k] >= 0) continue;
    for (int tries = 0; tries < 100000; ++tries) {
      double u = uniform01(draw(key, j++)) * acc;
      int64_t lo = 0, hi = E - 1;
      while (lo < hi) { int64_t mid = (lo + hi) / 2; if (cdf[mid] < u) lo = mid + 1; else hi = mid; }
      int32_t c = (int32_t)lo;
      int dup = 0;
      for (int q = 0; q < K; ++q) if (truth[q] == c || out[q] == c) dup = 1;
      if (!dup) { out[k] = c; break; }
    }
  }
  free(logp);
  free(cdf);
}
