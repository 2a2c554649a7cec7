// Host share of a decode step: the same SwiGLU expert on the CPU, straight from
// the pinned pool, for the entries the split left to the host.
//
// [FT-deep] §4 design pattern ③: the host executor receives the routed ids with
// -1 wherever the GPU owns the entry and skips those; §7: it runs one thread per
// physical core because decode on the host is bound by memory bandwidth
// ([FT-blog] §三.2).  fp32 accumulation, fixed order per output row.
#include <immintrin.h>

#include <chrono>
#include <cmath>
#include <cstring>
#include <vector>

#include "eff_internal.h"

namespace eff {

namespace {

struct Tables {
  float e4m3[256];
  float e2m1[16];
  Tables() {
    for (int c = 0; c < 256; ++c) {
      int s = (c >> 7) & 1, ex = (c >> 3) & 15, m = c & 7;
      float v = (ex == 0) ? std::ldexp((float)m, -9) : std::ldexp(1.0f + m / 8.0f, ex - 7);
      if (ex == 15 && m == 7) v = NAN;
      e4m3[c] = s ? -v : v;
    }
    static const float mag[8] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};
    for (int c = 0; c < 16; ++c) e2m1[c] = (c & 8) ? -mag[c & 7] : mag[c & 7];
  }
};
const Tables& tables() {
  static Tables t;
  return t;
}

inline float bf16f(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}
inline uint16_t f2bf_trunc(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}
inline uint16_t f2bf_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// A slice kernel: rows 16*sl .. 16*sl+15 of one matrix (KB tiles of 16 rows x 32 inputs, the
// slice's tiles contiguous at pay + (sl*KB + kb)*256, scales at sca + (sl*KB + kb)*32) against
// `nrows` bf16 input rows; row i accumulates into token i % nt (so a value can come as a hi + lo
// pair of rows).  out[r * nt + j] = tscale * sum_k W[16*sl + r][k] * x_j[k], fp32.
typedef void (*SliceFn)(const uint8_t* pay, const uint8_t* sca, int KB, int sl, int fmt,
                        const uint16_t* const* xr, int nrows, int nt, float tscale, float* out);

// AVX2 + FMA: per row, 8-wide fp32 FMAs over the row's 32 inputs of each tile, reduced at the end.
// The 4 bytes of row r, inputs 8q..8q+7 of a tile are its dword (q*16 + r).
void slice_avx2(const uint8_t* pay, const uint8_t* sca, int KB, int sl, int fmt, const uint16_t* const* xr,
                int nrows, int nt, float tscale, float* out) {
  const __m256i shifts = _mm256_setr_epi32(0, 4, 8, 12, 16, 20, 24, 28);
  const __m256i m15 = _mm256_set1_epi32(15), m7 = _mm256_set1_epi32(7), m8 = _mm256_set1_epi32(8);
  const __m256 eight = _mm256_set1_ps(8.f);
  const __m256 mag = _mm256_setr_ps(0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f);
  const Tables& T = tables();
  __m256 acc[16 * kMaxTokens];
  for (int i = 0; i < 16 * nt; ++i) acc[i] = _mm256_setzero_ps();
  for (int kb = 0; kb < KB; ++kb) {
    const int64_t tile = (int64_t)sl * KB + kb;
    const uint32_t* sp = reinterpret_cast<const uint32_t*>(pay + tile * 256);
    const uint8_t* sb = sca + tile * 32;
    __m256 xv[2 * kMaxTokens][4];
    for (int i = 0; i < nrows; ++i)
      for (int q = 0; q < 4; ++q) {
        const __m128i b = _mm_loadu_si128(reinterpret_cast<const __m128i*>(xr[i] + kb * 32 + q * 8));
        xv[i][q] = _mm256_castsi256_ps(_mm256_slli_epi32(_mm256_cvtepu16_epi32(b), 16));
      }
    for (int r = 0; r < 16; ++r) {
      __m256 w[4];
      for (int q = 0; q < 4; ++q) {
        const __m256i c = _mm256_and_si256(_mm256_srlv_epi32(_mm256_set1_epi32((int)sp[q * 16 + r]), shifts), m15);
        if (fmt == EFF_WFMT_INT4_G32_BF16) {
          w[q] = _mm256_sub_ps(_mm256_cvtepi32_ps(c), eight);
        } else {
          const __m256 v = _mm256_permutevar8x32_ps(mag, _mm256_and_si256(c, m7));
          const __m256i sgn = _mm256_slli_epi32(_mm256_and_si256(c, m8), 28);
          w[q] = _mm256_xor_ps(v, _mm256_castsi256_ps(sgn));
        }
      }
      float s0, s1;
      if (fmt == EFF_WFMT_INT4_G32_BF16) {
        uint16_t sbits;
        std::memcpy(&sbits, sb + r * 2, 2);
        s0 = s1 = bf16f(sbits);
      } else {
        s0 = T.e4m3[sb[r]];
        s1 = T.e4m3[sb[16 + r]];
      }
      const __m256 vs0 = _mm256_set1_ps(s0), vs1 = _mm256_set1_ps(s1);
      for (int i = 0; i < nrows; ++i) {
        __m256 h0 = _mm256_mul_ps(w[0], xv[i][0]);
        h0 = _mm256_fmadd_ps(w[1], xv[i][1], h0);
        __m256 h1 = _mm256_mul_ps(w[2], xv[i][2]);
        h1 = _mm256_fmadd_ps(w[3], xv[i][3], h1);
        __m256& a = acc[(size_t)r * nt + (i % nt)];
        a = _mm256_fmadd_ps(h0, vs0, a);
        a = _mm256_fmadd_ps(h1, vs1, a);
      }
    }
  }
  for (int r = 0; r < 16; ++r)
    for (int j = 0; j < nt; ++j) {
      alignas(32) float v[8];
      _mm256_store_ps(v, acc[(size_t)r * nt + j]);
      out[r * nt + j] = (((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]))) * tscale;
    }
}

// AVX-512 BF16: the 16 rows of a tile are the 16 dword lanes of a zmm.  For byte m of a row's
// dword (nibbles 2m, 2m+1), vpermt2b gathers the two nibbles of every lane into the low byte
// of each 16-bit half and vpermw maps them to bf16 weights (exact for int4 and e2m1), which
// vdpbf16ps multiplies with the broadcast bf16 input pair (x[8q+2m], x[8q+2m+1]): products exact,
// fp32 accumulation.  Scales per (row, group) are applied per tile in fp32.
__attribute__((target("avx512f,avx512bw,avx512vbmi,avx512bf16"))) void slice_avx512(
    const uint8_t* pay, const uint8_t* sca, int KB, int sl, int fmt, const uint16_t* const* xr, int nrows, int nt,
    float tscale, float* out) {
  alignas(64) uint16_t tab[32];
  for (int u = 0; u < 32; ++u) {
    float v = 0.f;
    if (u < 16) v = (fmt == EFF_WFMT_INT4_G32_BF16) ? (float)(u - 8) : tables().e2m1[u];
    tab[u] = f2bf_trunc(v);  // exact
  }
  const __m512i table = _mm512_load_si512(tab);
  alignas(64) uint8_t ib[4][64];
  for (int m = 0; m < 4; ++m)
    for (int r = 0; r < 16; ++r) {
      ib[m][4 * r + 0] = (uint8_t)(4 * r + m);
      ib[m][4 * r + 1] = 0;
      ib[m][4 * r + 2] = (uint8_t)(64 + 4 * r + m);
      ib[m][4 * r + 3] = 0;
    }
  const __m512i idx0 = _mm512_load_si512(ib[0]), idx1 = _mm512_load_si512(ib[1]);
  const __m512i idx2 = _mm512_load_si512(ib[2]), idx3 = _mm512_load_si512(ib[3]);
  const __mmask64 keep = 0x5555555555555555ull;
  const __m512i m0f = _mm512_set1_epi32(0x0F0F0F0F);
  __m512 tot[kMaxTokens];
  for (int j = 0; j < nt; ++j) tot[j] = _mm512_setzero_ps();
  for (int kb = 0; kb < KB; ++kb) {
    const int64_t tile = (int64_t)sl * KB + kb;
    const uint8_t* tp = pay + tile * 256;
    __m512i w[16];
    for (int q = 0; q < 4; ++q) {
      const __m512i d = _mm512_loadu_si512(tp + 64 * q);
      const __m512i v1 = _mm512_and_si512(d, m0f);                        // nibbles 0, 2, 4, 6
      const __m512i v2 = _mm512_and_si512(_mm512_srli_epi32(d, 4), m0f);  // nibbles 1, 3, 5, 7
      w[q * 4 + 0] = _mm512_permutexvar_epi16(_mm512_maskz_permutex2var_epi8(keep, v1, idx0, v2), table);
      w[q * 4 + 1] = _mm512_permutexvar_epi16(_mm512_maskz_permutex2var_epi8(keep, v1, idx1, v2), table);
      w[q * 4 + 2] = _mm512_permutexvar_epi16(_mm512_maskz_permutex2var_epi8(keep, v1, idx2, v2), table);
      w[q * 4 + 3] = _mm512_permutexvar_epi16(_mm512_maskz_permutex2var_epi8(keep, v1, idx3, v2), table);
    }
    const uint8_t* sp = sca + tile * 32;
    __m512 s0, s1;
    if (fmt == EFF_WFMT_INT4_G32_BF16) {
      const __m256i b = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(sp));
      s0 = s1 = _mm512_castsi512_ps(_mm512_slli_epi32(_mm512_cvtepu16_epi32(b), 16));
    } else {
      // e4m3 -> fp32: magnitude bits placed under the fp32 exponent/mantissa, times 2^120
      // (normals and subnormals alike), then the sign
      const __m512 k120 = _mm512_set1_ps(1.329227995784916e36f);  // 2^120
      const __m512i c0 = _mm512_cvtepu8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(sp)));
      const __m512i c1 = _mm512_cvtepu8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(sp + 16)));
      const __m512i x7f = _mm512_set1_epi32(0x7F), x80 = _mm512_set1_epi32(0x80);
      s0 = _mm512_mul_ps(_mm512_castsi512_ps(_mm512_slli_epi32(_mm512_and_si512(c0, x7f), 20)), k120);
      s1 = _mm512_mul_ps(_mm512_castsi512_ps(_mm512_slli_epi32(_mm512_and_si512(c1, x7f), 20)), k120);
      s0 = _mm512_castsi512_ps(_mm512_or_si512(_mm512_castps_si512(s0), _mm512_slli_epi32(_mm512_and_si512(c0, x80), 24)));
      s1 = _mm512_castsi512_ps(_mm512_or_si512(_mm512_castps_si512(s1), _mm512_slli_epi32(_mm512_and_si512(c1, x80), 24)));
    }
    for (int i = 0; i < nrows; ++i) {
      const int32_t* xk = reinterpret_cast<const int32_t*>(xr[i] + kb * 32);  // 16 bf16 pairs
      __m512 a0 = _mm512_setzero_ps(), a1 = _mm512_setzero_ps();
      for (int z = 0; z < 8; ++z)
        a0 = _mm512_dpbf16_ps(a0, (__m512bh)w[z], (__m512bh)_mm512_set1_epi32(xk[z]));
      for (int z = 8; z < 16; ++z)
        a1 = _mm512_dpbf16_ps(a1, (__m512bh)w[z], (__m512bh)_mm512_set1_epi32(xk[z]));
      __m512& t = tot[i % nt];
      t = _mm512_fmadd_ps(s0, a0, t);
      t = _mm512_fmadd_ps(s1, a1, t);
    }
  }
  const __m512 ts = _mm512_set1_ps(tscale);
  for (int j = 0; j < nt; ++j) {
    alignas(64) float v[16];
    _mm512_store_ps(v, _mm512_mul_ps(tot[j], ts));
    for (int r = 0; r < 16; ++r) out[r * nt + j] = v[r];
  }
}

SliceFn pick_slice(int isa) { return isa == 1 ? slice_avx512 : slice_avx2; }

}  // namespace

int host_isa_best() {
  __builtin_cpu_init();
  return (__builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
          __builtin_cpu_supports("avx512vbmi") && __builtin_cpu_supports("avx512bf16"))
             ? 1
             : 0;
}

// Host share of one call: entries with cpu_ids[p] >= 0 get y[p] = W_d (silu(W_g x) * (W_u x)) of
// expert cpu_ids[p] of `layer`, x the entry's token row (bf16).  One parallel pass: the 16-row
// slices of gate+up of every host expert first, then the slices of down; a down task waits
// until its expert's gate/up slices are done (tasks are claimed in order, so this cannot
// deadlock).  The down input a = silu(g)*u goes in as a bf16 hi + lo pair (error ~2^-16).
void host_ffn(eff_engine* e, int layer, const uint16_t* x, const int32_t* cpu_ids, int B, float* y) {
  const eff_config& c = e->cfg;
  const int K = c.top_k, H = c.hidden, I = c.inter, E = c.num_experts;
  HostScratch& hs = e->hscratch;
  // unique host experts, ascending, and their entries (at most one per token)
  int U = 0;
  for (int p = 0; p < B * K; ++p) {
    const int id = cpu_ids[p];
    if (id < 0 || id >= E) continue;
    int u = 0;
    while (u < U && hs.uexp[u] < id) ++u;
    if (u < U && hs.uexp[u] == id) {
      if (hs.ucnt[u] < kMaxTokens) hs.uent[u][hs.ucnt[u]++] = p;
      continue;
    }
    for (int v = U; v > u; --v) {
      hs.uexp[v] = hs.uexp[v - 1];
      hs.ucnt[v] = hs.ucnt[v - 1];
      std::memcpy(hs.uent[v], hs.uent[v - 1], sizeof(hs.uent[v]));
    }
    hs.uexp[u] = id;
    hs.ucnt[u] = 1;
    hs.uent[u][0] = p;
    ++U;
  }
  if (U == 0) return;
  // SwiGLU activations (hi and lo bf16 rows) per (expert, token)
  int off[kMaxEntries + 1];
  off[0] = 0;
  for (int u = 0; u < U; ++u) off[u + 1] = off[u] + hs.ucnt[u];
  const size_t need = (size_t)off[U] * I * 2;
  if (hs.a.size() < need) hs.a.resize(need);
  for (int u = 0; u < U; ++u) hs.done[u].store(0, std::memory_order_relaxed);
  const SliceFn slice = pick_slice(e->host_isa);
  const int64_t pay = (int64_t)H * I / 2, sca = (int64_t)H * I / 16;
  const int SI = I / 16, SH = H / 16;
  const int n1 = U * SI;
  e->pool_threads->parallel_for(n1 + U * SH, [&](int task) {
    if (task < n1) {  // gate and up: 16 rows of a
      const int u = task / SI, sl = task % SI;
      const int nt = hs.ucnt[u];
      const int64_t flat = (int64_t)layer * E + hs.uexp[u];
      const uint8_t* rec = e->pool + flat * e->R;
      const uint16_t* xr[kMaxTokens];
      for (int j = 0; j < nt; ++j) xr[j] = x + (size_t)(hs.uent[u][j] / K) * H;
      float g[16 * kMaxTokens], v[16 * kMaxTokens];
      slice(rec, rec + 3 * pay, H / 32, sl, c.wformat, xr, nt, nt, e->h_ts[flat * 3 + 0], g);
      slice(rec + pay, rec + 3 * pay + sca, H / 32, sl, c.wformat, xr, nt, nt, e->h_ts[flat * 3 + 1], v);
      uint16_t* ahi = hs.a.data() + (size_t)off[u] * I * 2;
      for (int r = 0; r < 16; ++r)
        for (int j = 0; j < nt; ++j) {
          const float gg = g[r * nt + j], uu = v[r * nt + j];
          const float a = gg / (1.f + std::exp(-gg)) * uu;
          const uint16_t hi = f2bf_trunc(a);
          ahi[(size_t)j * I + sl * 16 + r] = hi;                                   // row j
          ahi[(size_t)(nt + j) * I + sl * 16 + r] = f2bf_rne(a - bf16f(hi));      // row nt + j
        }
      hs.done[u].fetch_add(1, std::memory_order_release);
      return;
    }
    const int t2 = task - n1, u = t2 / SH, sl = t2 % SH;  // down: 16 rows of y
    while (hs.done[u].load(std::memory_order_acquire) < SI) _mm_pause();
    const int nt = hs.ucnt[u];
    const int64_t flat = (int64_t)layer * E + hs.uexp[u];
    const uint8_t* rec = e->pool + flat * e->R;
    const uint16_t* ar[2 * kMaxTokens];
    const uint16_t* abase = hs.a.data() + (size_t)off[u] * I * 2;
    for (int i = 0; i < 2 * nt; ++i) ar[i] = abase + (size_t)i * I;
    float out[16 * kMaxTokens];
    slice(rec + 2 * pay, rec + 3 * pay + 2 * sca, I / 32, sl, c.wformat, ar, 2 * nt, nt, e->h_ts[flat * 3 + 2],
          out);
    for (int r = 0; r < 16; ++r)
      for (int j = 0; j < nt; ++j) y[(int64_t)hs.uent[u][j] * H + sl * 16 + r] = out[r * nt + j];
  });
}

// ----------------------------------------------------------------------------------- pool
ThreadPool::ThreadPool(int n) {
  for (int i = 0; i < n - 1; ++i) workers_.emplace_back([this] { loop(); });
}

ThreadPool::~ThreadPool() {
  {
    std::lock_guard<std::mutex> g(mu_);
    stop_.store(true);
  }
  cv_.notify_all();
  for (auto& t : workers_) t.join();
}

void ThreadPool::run_tasks(uint64_t g, const std::function<void(int)>* fn, int n) {
  const uint64_t tag = (g & 0xFFFFFFFFull) << 32;
  for (;;) {
    uint64_t v = next_.load(std::memory_order_acquire);
    if ((v & ~0xFFFFFFFFull) != tag || (int64_t)(v & 0xFFFFFFFFull) >= n) return;
    if (!next_.compare_exchange_weak(v, v + 1, std::memory_order_acq_rel)) continue;
    (*fn)((int)(v & 0xFFFFFFFFull));
    done_.fetch_add(1, std::memory_order_release);
  }
}

void ThreadPool::loop() {
  uint64_t seen = gen_.load(std::memory_order_acquire);
  while (!stop_.load(std::memory_order_relaxed)) {
    uint64_t g = seen;
    const auto t0 = std::chrono::steady_clock::now();
    for (int it = 0;; ++it) {
      g = gen_.load(std::memory_order_acquire);
      if (g != seen || stop_.load(std::memory_order_relaxed)) break;
      _mm_pause();
      if ((it & 1023) == 1023 && std::chrono::steady_clock::now() - t0 > std::chrono::milliseconds(2)) break;
    }
    if (g == seen) {  // idle: sleep until a new job or shutdown
      std::unique_lock<std::mutex> lk(mu_);
      sleepers_.fetch_add(1);
      cv_.wait(lk, [&] { return stop_.load() || gen_.load() != seen; });
      sleepers_.fetch_sub(1);
      continue;
    }
    seen = g;
    run_tasks(g, fn_.load(std::memory_order_acquire), n_.load(std::memory_order_acquire));
  }
}

void ThreadPool::parallel_for(int n, const std::function<void(int)>& fn) {
  if (n <= 0) return;
  const uint64_t g = gen_.load(std::memory_order_relaxed) + 1;
  fn_.store(&fn, std::memory_order_relaxed);
  n_.store(n, std::memory_order_relaxed);
  done_.store(0, std::memory_order_relaxed);
  next_.store((g & 0xFFFFFFFFull) << 32, std::memory_order_relaxed);
  gen_.store(g, std::memory_order_release);
  if (sleepers_.load() > 0) {
    std::lock_guard<std::mutex> lk(mu_);
    cv_.notify_all();
  }
  run_tasks(g, &fn, n);
  while (done_.load(std::memory_order_acquire) < n) _mm_pause();
}

}  // namespace eff
