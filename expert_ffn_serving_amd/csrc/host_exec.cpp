// Host share of a decode step: the same SwiGLU expert on the CPU, straight from
// the pinned pool, for the entries the split left to the host.
//
// [FT-deep] §4 design pattern ③: the host executor receives the routed ids with
// -1 wherever the GPU owns the entry and skips those; §7: it runs one thread per
// physical core because decode on the host is bound by memory bandwidth
// ([FT-blog] §三.2).  fp32 accumulation, fixed order per output row.
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

// acc[row * nt + j] += sum over the block's 32 inputs of w[row][k] * xs[j][k0 + k], for the
// 64 rows of payload block `blk` of one matrix; xs: nt rows of length ld.
void block_dot(const uint8_t* pay, const uint8_t* sca, int64_t blk, int fmt, const float* xs, int ld, int nt,
               int k0, float* acc) {
  const Tables& T = tables();
  const uint8_t* pb = pay + blk * 1024;
  const uint8_t* sb = sca + blk * 128;
  float w[8];
  for (int q = 0; q < 4; ++q) {
    for (int r = 0; r < 16; ++r) {
      for (int t = 0; t < 4; ++t) {
        const uint8_t* lanep = pb + t * 256 + (q * 16 + r) * 4;
        const int row = t * 16 + r;
        float s;
        if (fmt == EFF_WFMT_INT4_G32_BF16) {
          uint16_t sbits;
          std::memcpy(&sbits, sb + (r * 4 + t) * 2, 2);
          s = bf16f(sbits);
          for (int i = 0; i < 8; ++i) {
            const uint8_t byte = lanep[i / 2];
            const int u = (i & 1) ? (byte >> 4) : (byte & 15);
            w[i] = (float)(u - 8);
          }
        } else {
          s = T.e4m3[sb[((q >> 1) * 16 + r) * 4 + t]];
          for (int i = 0; i < 8; ++i) {
            const uint8_t byte = lanep[i / 2];
            w[i] = T.e2m1[(i & 1) ? (byte >> 4) : (byte & 15)];
          }
        }
        for (int j = 0; j < nt; ++j) {
          const float* xj = xs + (int64_t)j * ld + k0 + q * 8;
          float d = 0.f;
          for (int i = 0; i < 8; ++i) d += w[i] * xj[i];
          acc[row * nt + j] += s * d;
        }
      }
    }
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
  std::vector<float> xf((size_t)B * H);
  for (int64_t i = 0; i < (int64_t)B * H; ++i) xf[i] = bf16f(x[i]);
  // per expert: its tokens' x rows, gathered
  std::vector<std::vector<float>> xs(U), a(U);
  for (int u = 0; u < U; ++u) {
    const int nt = (int)entries[u].size();
    xs[u].resize((size_t)nt * H);
    for (int j = 0; j < nt; ++j)
      std::memcpy(&xs[u][(size_t)j * H], &xf[(size_t)(entries[u][j] / K) * H], sizeof(float) * H);
    a[u].assign((size_t)nt * I, 0.f);
  }
  const int64_t pay = (int64_t)H * I / 2, sca = (int64_t)H * I / 16;
  const int NBI = I / 64, NBH = H / 64;
  // phase 1: gate/up row blocks -> a = silu(g) * u
  e->pool_threads->parallel_for(U * NBI, [&](int task) {
    const int u = task / NBI, nb = task % NBI;
    const int nt = (int)entries[u].size();
    const int64_t flat = (int64_t)layer * E + experts[u];
    const uint8_t* rec = e->pool + flat * e->R;
    std::vector<float> g((size_t)64 * nt, 0.f), v((size_t)64 * nt, 0.f);
    for (int kb = 0; kb < H / 32; ++kb) {
      const int64_t blk = (int64_t)kb * NBI + nb;
      block_dot(rec, rec + 3 * pay, blk, c.wformat, xs[u].data(), H, nt, kb * 32, g.data());
      block_dot(rec + pay, rec + 3 * pay + sca, blk, c.wformat, xs[u].data(), H, nt, kb * 32, v.data());
    }
    const float tsg = e->h_ts.empty() ? 1.f : e->h_ts[flat * 3 + 0];
    const float tsu = e->h_ts.empty() ? 1.f : e->h_ts[flat * 3 + 1];
    for (int row = 0; row < 64; ++row)
      for (int j = 0; j < nt; ++j) {
        const float gg = g[row * nt + j] * tsg, uu = v[row * nt + j] * tsu;
        a[u][(size_t)j * I + nb * 64 + row] = gg / (1.f + std::exp(-gg)) * uu;
      }
  });
  // phase 2: down row blocks -> y of each entry
  e->pool_threads->parallel_for(U * NBH, [&](int task) {
    const int u = task / NBH, nb = task % NBH;
    const int nt = (int)entries[u].size();
    const int64_t flat = (int64_t)layer * E + experts[u];
    const uint8_t* rec = e->pool + flat * e->R;
    std::vector<float> acc((size_t)64 * nt, 0.f);
    for (int kb = 0; kb < I / 32; ++kb) {
      const int64_t blk = (int64_t)kb * NBH + nb;
      block_dot(rec + 2 * pay, rec + 3 * pay + 2 * sca, blk, c.wformat, a[u].data(), I, nt, kb * 32,
                acc.data());
    }
    const float tsd = e->h_ts.empty() ? 1.f : e->h_ts[flat * 3 + 2];
    for (int row = 0; row < 64; ++row)
      for (int j = 0; j < nt; ++j)
        y[(int64_t)entries[u][j] * H + nb * 64 + row] = acc[row * nt + j] * tsd;
  });
}

// ----------------------------------------------------------------------------------- pool
ThreadPool::ThreadPool(int n) {
  for (int i = 0; i < n - 1; ++i) workers_.emplace_back([this] { loop(); });
}

ThreadPool::~ThreadPool() {
  {
    std::lock_guard<std::mutex> g(mu_);
    stop_ = true;
  }
  cv_.notify_all();
  for (auto& t : workers_) t.join();
}

void ThreadPool::loop() {
  uint64_t seen = 0;
  for (;;) {
    const std::function<void(int)>* fn;
    int n;
    {
      std::unique_lock<std::mutex> lk(mu_);
      cv_.wait(lk, [&] { return stop_ || gen_ != seen; });
      if (stop_) return;
      seen = gen_;
      if (!fn_) continue;  // woke after that job completed: nothing to join
      fn = fn_;
      n = n_;
      ++active_;  // the job cannot complete (nor the next one start) until this worker leaves it
    }
    for (int i = next_.fetch_add(1); i < n; i = next_.fetch_add(1)) (*fn)(i);
    {
      std::lock_guard<std::mutex> g(mu_);
      if (--active_ == 0) done_cv_.notify_all();
    }
  }
}

void ThreadPool::parallel_for(int n, const std::function<void(int)>& fn) {
  if (n <= 0) return;
  {
    std::lock_guard<std::mutex> g(mu_);
    fn_ = &fn;
    n_ = n;
    next_.store(0);
    ++gen_;
  }
  cv_.notify_all();
  for (int i = next_.fetch_add(1); i < n; i = next_.fetch_add(1)) fn(i);
  std::unique_lock<std::mutex> lk(mu_);
  done_cv_.wait(lk, [&] { return active_ == 0 && next_.load() >= n; });
  fn_ = nullptr;
}

}  // namespace eff
