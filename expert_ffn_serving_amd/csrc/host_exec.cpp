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
#include <map>
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

// One 16-row slice (rows 16*sl .. 16*sl+15) of one matrix times nt input rows:
// out[r * nt + j] = scale_m * sum_k W[16*sl + r][k] * xs[j][k], AVX2 + FMA, fp32.
// The slice is KB contiguous tiles; the 4 bytes for row r, inputs 8q..8q+7 of tile kb are at
// pay + (sl*KB + kb)*256 + (q*16 + r)*4 (8 nibbles, low first), its scales at sca + (sl*KB + kb)*32.
void slice_dot(const uint8_t* pay, const uint8_t* sca, int KB, int sl, int fmt, const float* xs, int ld,
               int nt, float tscale, float* out) {
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
      for (int j = 0; j < nt; ++j) {
        const float* xj = xs + (int64_t)j * ld + kb * 32;
        __m256 h0 = _mm256_mul_ps(w[0], _mm256_loadu_ps(xj));
        h0 = _mm256_fmadd_ps(w[1], _mm256_loadu_ps(xj + 8), h0);
        __m256 h1 = _mm256_mul_ps(w[2], _mm256_loadu_ps(xj + 16));
        h1 = _mm256_fmadd_ps(w[3], _mm256_loadu_ps(xj + 24), h1);
        __m256& a = acc[(size_t)r * nt + j];
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

}  // namespace

void host_ffn(eff_engine* e, int layer, const uint16_t* x, const int32_t* cpu_ids, int B, float* y) {
  const eff_config& c = e->cfg;
  const int K = c.top_k, H = c.hidden, I = c.inter, E = c.num_experts;
  // unique host experts, ascending, with their entries
  std::map<int, std::vector<int>> groups;
  for (int p = 0; p < B * K; ++p)
    if (cpu_ids[p] >= 0 && cpu_ids[p] < E) groups[cpu_ids[p]].push_back(p);
  if (groups.empty()) return;
  std::vector<int> experts;
  std::vector<std::vector<int>> entries;
  for (auto& kv : groups) {
    experts.push_back(kv.first);
    entries.push_back(kv.second);
  }
  const int U = (int)experts.size();
  // per expert: its tokens' x rows (fp32) and the SwiGLU activations
  std::vector<std::vector<float>> xs(U), a(U);
  for (int u = 0; u < U; ++u) {
    const int nt = (int)entries[u].size();
    xs[u].resize((size_t)nt * H);
    for (int j = 0; j < nt; ++j) {
      const uint16_t* xr = x + (size_t)(entries[u][j] / K) * H;
      for (int k = 0; k < H; ++k) xs[u][(size_t)j * H + k] = bf16f(xr[k]);
    }
    a[u].assign((size_t)nt * I, 0.f);
  }
  const int64_t pay = (int64_t)H * I / 2, sca = (int64_t)H * I / 16;
  const int SI = I / 16, SH = H / 16;
  // phase 1: 16-row slices of gate and up -> a = silu(g) * u
  e->pool_threads->parallel_for(U * SI, [&](int task) {
    const int u = task / SI, sl = task % SI;
    const int nt = (int)entries[u].size();
    const int64_t flat = (int64_t)layer * E + experts[u];
    const uint8_t* rec = e->pool + flat * e->R;
    float g[16 * kMaxTokens], v[16 * kMaxTokens];
    const float tsg = e->h_ts[flat * 3 + 0], tsu = e->h_ts[flat * 3 + 1];
    slice_dot(rec, rec + 3 * pay, H / 32, sl, c.wformat, xs[u].data(), H, nt, tsg, g);
    slice_dot(rec + pay, rec + 3 * pay + sca, H / 32, sl, c.wformat, xs[u].data(), H, nt, tsu, v);
    for (int r = 0; r < 16; ++r)
      for (int j = 0; j < nt; ++j) {
        const float gg = g[r * nt + j], uu = v[r * nt + j];
        a[u][(size_t)j * I + sl * 16 + r] = gg / (1.f + std::exp(-gg)) * uu;
      }
  });
  // phase 2: 16-row slices of down -> y of each entry
  e->pool_threads->parallel_for(U * SH, [&](int task) {
    const int u = task / SH, sl = task % SH;
    const int nt = (int)entries[u].size();
    const int64_t flat = (int64_t)layer * E + experts[u];
    const uint8_t* rec = e->pool + flat * e->R;
    float out[16 * kMaxTokens];
    slice_dot(rec + 2 * pay, rec + 3 * pay + 2 * sca, I / 32, sl, c.wformat, a[u].data(), I, nt,
              e->h_ts[flat * 3 + 2], out);
    for (int r = 0; r < 16; ++r)
      for (int j = 0; j < nt; ++j) y[(int64_t)entries[u][j] * H + sl * 16 + r] = out[r * nt + j];
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
