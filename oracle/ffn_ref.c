/*
 * Oracle (test infrastructure only): the SwiGLU expert down(silu(gate(x)) * up(x))
 * evaluated in double precision by plain loops, straight from one record's bytes.
 * Same definitions as oracle/formats.py and oracle/ffn.py, restated in C so that
 * full-size shapes (4096 x 2048 matrices) finish in seconds.  Shares no code with
 * the HIP library.
 *
 * Formats: int4 value (u - 8) * bf16 scale per 32 inputs; NVFP4 value
 * e2m1(c) * e4m3(s) * tensor scale, e4m3 per 16 inputs.  Layout: see
 * oracle/formats.py (16 x 32 tiles, tile = (n / 16) * (Kd / 32) + k / 32).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double e2m1(int c) {
  int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -mag : mag;
}

static double e4m3(int c) {
  int s = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

static double bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* decode row n of matrix m into out[Kd] */
static void decode_row(const uint8_t* rec, int fmt, int64_t H, int64_t I, int m, int64_t n, double ts,
                       double* out) {
  int64_t N = (m == 2) ? H : I, Kd = (m == 2) ? I : H;
  const uint8_t* pay = rec + m * (H * I / 2);
  const uint8_t* sca = rec + 3 * (H * I / 2) + m * (H * I / 16);
  (void)N;
  for (int64_t k = 0; k < Kd; ++k) {
    int64_t tile = (n / 16) * (Kd / 32) + k / 32;
    int64_t r = n % 16, q = (k % 32) / 8, i = k % 8;
    int64_t off = tile * 256 + (q * 16 + r) * 4 + i / 2;
    int code = (i % 2 == 0) ? (pay[off] & 15) : (pay[off] >> 4);
    if (fmt == 0) {
      int64_t so = tile * 32 + r * 2;
      uint16_t sb = (uint16_t)(sca[so] | (sca[so + 1] << 8));
      out[k] = (double)(code - 8) * bf16(sb);
    } else {
      int64_t so = tile * 32 + ((k % 32) / 16) * 16 + r;
      out[k] = e2m1(code) * e4m3(sca[so]) * ts;
    }
  }
}

/* y[nt][H] = expert(x[nt][H]) for one record. */
void oracle_expert_ffn(const uint8_t* rec, int fmt, int64_t H, int64_t I, const float* ts3,
                       const double* x, int nt, double* y) {
  double* row = (double*)malloc(sizeof(double) * (size_t)(H > I ? H : I));
  double* a = (double*)malloc(sizeof(double) * (size_t)(I * nt));
  double* g = (double*)malloc(sizeof(double) * (size_t)nt);
  if (!row || !a || !g) { free(row); free(a); free(g); return; }
  for (int64_t n = 0; n < I; ++n) {
    decode_row(rec, fmt, H, I, 0, n, ts3[0], row);
    for (int t = 0; t < nt; ++t) {
      double acc = 0.0;
      for (int64_t k = 0; k < H; ++k) acc += row[k] * x[t * H + k];
      g[t] = acc;
    }
    decode_row(rec, fmt, H, I, 1, n, ts3[1], row);
    for (int t = 0; t < nt; ++t) {
      double acc = 0.0;
      for (int64_t k = 0; k < H; ++k) acc += row[k] * x[t * H + k];
      a[t * I + n] = g[t] / (1.0 + exp(-g[t])) * acc;
    }
  }
  for (int64_t n = 0; n < H; ++n) {
    decode_row(rec, fmt, H, I, 2, n, ts3[2], row);
    for (int t = 0; t < nt; ++t) {
      double acc = 0.0;
      for (int64_t k = 0; k < I; ++k) acc += row[k] * a[t * I + k];
      y[t * H + n] = acc;
    }
  }
  free(row); free(a); free(g);
}

typedef struct {
  const uint8_t* rec;
  const float* ts3;
  const double* x;
  double* y;
  int nt;
} ffn_job;

typedef struct {
  const ffn_job* jobs;
  int njobs, fmt;
  int64_t H, I;
  int next;
  pthread_mutex_t mu;
} ffn_batch;

static void* batch_worker(void* arg) {
  ffn_batch* B = (ffn_batch*)arg;
  for (;;) {
    pthread_mutex_lock(&B->mu);
    int j = B->next++;
    pthread_mutex_unlock(&B->mu);
    if (j >= B->njobs) break;
    const ffn_job* J = &B->jobs[j];
    oracle_expert_ffn(J->rec, B->fmt, B->H, B->I, J->ts3, J->x, J->nt, J->y);
  }
  return NULL;
}

/* Run njobs independent expert evaluations on nthreads threads. */
int oracle_expert_ffn_batch(const ffn_job* jobs, int njobs, int fmt, int64_t H, int64_t I, int nthreads) {
  ffn_batch B;
  B.jobs = jobs; B.njobs = njobs; B.fmt = fmt; B.H = H; B.I = I; B.next = 0;
  pthread_mutex_init(&B.mu, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 128) nthreads = 128;
  pthread_t th[128];
  int started = 0;
  for (int t = 0; t < nthreads; ++t)
    if (pthread_create(&th[t], NULL, batch_worker, &B) == 0) started++;
  if (started == 0) batch_worker(&B);
  for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
  pthread_mutex_destroy(&B.mu);
  return 0;
}
