// libeff host side: engine lifecycle, the C ABI entry points, the eager decode-layer
// orchestration and prefill streaming.
#include <immintrin.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "eff_internal.h"

namespace eff {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }
int fail(int code, const std::string& msg) {
  set_error(msg);
  return code;
}

static bool capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &st) != hipSuccess) return false;
  return st != hipStreamCaptureStatusNone;
}

static int validate(const eff_config* c, std::string* why) {
  auto bad = [&](const char* m) {
    *why = m;
    return EFF_EINVAL;
  };
  if (!c) return bad("config is NULL");
  if (c->num_layers < 1) return bad("num_layers must be >= 1");
  if (c->num_experts < 1 || c->num_experts > kMaxExperts) return bad("num_experts must be in [1, 4096]");
  if (c->top_k < 1 || c->top_k > kMaxTopK || c->top_k > c->num_experts) return bad("top_k must be in [1, min(32, E)]");
  if (c->hidden < 64 || c->hidden % 64) return bad("hidden must be a positive multiple of 64");
  if (c->inter < 64 || c->inter % 64 || c->inter > 4096) return bad("inter must be a multiple of 64 in [64, 4096]");
  if (c->wformat != EFF_WFMT_INT4_G32_BF16 && c->wformat != EFF_WFMT_NVFP4_G16_E4M3) return bad("unknown wformat");
  if (c->num_slots < 0 || c->num_slots > kMaxSlots) return bad("num_slots must be in [0, 16384]");
  if (c->max_tokens < 1 || c->max_tokens > kMaxTokens) return bad("max_tokens must be in [1, 32]");
  if (c->max_tokens * c->top_k > kMaxEntries) return bad("max_tokens * top_k must be <= 512");
  if (c->max_prefill_tokens < 0) return bad("max_prefill_tokens must be >= 0");
  if (c->fetch_frac_q16 > 65536u) return bad("fetch_frac_q16 must be in [0, 65536]");
  if (c->host_threads < 0 || c->host_threads > 256) return bad("host_threads must be in [0, 256]");
  if (c->flags & ~(uint32_t)(EFF_CFG_TIMING | EFF_CFG_SYNC_HOST)) return bad("unknown config flags");
  if ((int64_t)c->num_layers * c->num_experts > (int64_t)1 << 30) return bad("L*E too large");
  return EFF_OK;
}

static int64_t record_bytes(const eff_config* c) {
  return 3 * (int64_t)c->hidden * c->inter / 2 + 3 * (int64_t)c->hidden * c->inter / 16;
}

template <typename T>
static hipError_t dalloc(T** p, size_t count) {
  return hipMalloc((void**)p, std::max<size_t>(1, count) * sizeof(T));
}

static void stop_worker(eff_engine* e);

static void release(eff_engine* e) {
  if (!e) return;
  stop_worker(e);
  void* dev[] = {e->d_arena, e->d_table, e->d_owner, e->d_usage, e->d_recency, e->d_clock, e->d_ts,
                 e->d_pending, e->d_fetch, e->d_err, e->d_seq, e->d_stats, e->d_plan, e->d_a, e->d_ids, e->d_w, e->d_slots, e->d_cpu, e->d_counts, e->d_spec_ids,
                 e->d_spec_cpu, e->d_logits, e->d_ygpu, e->d_yhost, e->d_pf_count, e->d_pf_rows,
                 e->d_pf_a, e->d_pf_x, e->d_pf_y, e->d_pf_meta, e->d_pf_slot_of, e->d_pf_experts};
  for (void* p : dev)
    if (p) (void)hipFree(p);
  void* host[] = {e->h_fetch, e->h_x, e->h_cpu, e->h_call, e->h_done, e->h_yhost, e->h_pf_ids, e->h_pf_meta,
                  e->h_tq};
  for (void* p : host)
    if (p) (void)hipHostFree(p);
  hipEvent_t evs[] = {e->ev_copy, e->ev_pf[0], e->ev_pf[1], e->ev_pf_done[0], e->ev_pf_done[1]};
  for (hipEvent_t v : evs)
    if (v) (void)hipEventDestroy(v);
  for (auto& tc : e->timed)
    for (hipEvent_t v : tc.ev)
      if (v) (void)hipEventDestroy(v);
  for (hipEvent_t v : e->free_events) (void)hipEventDestroy(v);
  delete e->pool_threads;
  delete e;
}

static int alloc_all(eff_engine* e) {
  const eff_config& c = e->cfg;
  const int64_t L = c.num_layers, E = c.num_experts, S = c.num_slots, H = c.hidden, I = c.inter;
  const int64_t K = c.top_k, B = c.max_tokens, T = c.max_prefill_tokens;
  EFF_HIP_TRY(dalloc(&e->d_arena, S > 0 ? (size_t)(S * e->R + kArenaTail) : 0));
  EFF_HIP_TRY(dalloc(&e->d_table, L * E));
  EFF_HIP_TRY(dalloc(&e->d_owner, S));
  EFF_HIP_TRY(dalloc(&e->d_usage, S));
  EFF_HIP_TRY(dalloc(&e->d_recency, L * E));
  EFF_HIP_TRY(dalloc(&e->d_clock, 3));
  EFF_HIP_TRY(dalloc(&e->d_ts, L * E * 3));
  EFF_HIP_TRY(dalloc(&e->d_pending, 1));
  EFF_HIP_TRY(dalloc(&e->d_fetch, kFetchLists));
  EFF_HIP_TRY(dalloc(&e->d_err, 1));
  EFF_HIP_TRY(dalloc(&e->d_seq, 1));
  EFF_HIP_TRY(dalloc(&e->d_stats, ST_COUNT));
  // host-mapped control words are coherent (fine-grained): the host reads them while kernels run
  const unsigned mapped = hipHostMallocMapped | hipHostMallocCoherent;
  EFF_HIP_TRY(hipHostMalloc((void**)&e->h_fetch, kFetchLists * sizeof(FetchList), mapped));
  EFF_HIP_TRY(hipHostGetDevicePointer((void**)&e->h_fetch_dev, e->h_fetch, 0));
  // decode scratch
  e->maxU = (int)std::min<int64_t>(B * K, E);
  EFF_HIP_TRY(dalloc(&e->d_plan, 1));
  EFF_HIP_TRY(hipMemset(e->d_plan, 0, sizeof(eff::DecodePlan)));  // every unit starts empty
  EFF_HIP_TRY(dalloc(&e->d_a, (size_t)e->maxU * B * I));
  // orchestrator
  EFF_HIP_TRY(dalloc(&e->d_ids, B * K));
  EFF_HIP_TRY(dalloc(&e->d_w, B * K));
  EFF_HIP_TRY(dalloc(&e->d_slots, B * K));
  EFF_HIP_TRY(dalloc(&e->d_cpu, B * K));
  EFF_HIP_TRY(dalloc(&e->d_counts, 6));
  EFF_HIP_TRY(dalloc(&e->d_spec_ids, B * K));
  EFF_HIP_TRY(dalloc(&e->d_spec_cpu, B * K));
  EFF_HIP_TRY(dalloc(&e->d_logits, std::max(B, T) * E));
  EFF_HIP_TRY(dalloc(&e->d_ygpu, B * K * H));
  EFF_HIP_TRY(dalloc(&e->d_yhost, B * K * H));
  EFF_HIP_TRY(hipHostMalloc((void**)&e->h_x, (size_t)(B * H) * 2, mapped));
  EFF_HIP_TRY(hipHostMalloc((void**)&e->h_cpu, (size_t)(B * K) * 4, mapped));
  EFF_HIP_TRY(hipHostMalloc((void**)&e->h_call, kCallRing * sizeof(uint64_t), mapped));
  EFF_HIP_TRY(hipHostMalloc((void**)&e->h_done, 64, mapped));
  EFF_HIP_TRY(hipHostMalloc((void**)&e->h_yhost, (size_t)(B * K * H) * 4, mapped));
  EFF_HIP_TRY(hipHostMalloc((void**)&e->h_tq, kTimedMax * 2 * sizeof(int32_t), 0));
  EFF_HIP_TRY(hipHostGetDevicePointer((void**)&e->h_x_dev, e->h_x, 0));
  EFF_HIP_TRY(hipHostGetDevicePointer((void**)&e->h_cpu_dev, e->h_cpu, 0));
  EFF_HIP_TRY(hipHostGetDevicePointer((void**)&e->h_call_dev, e->h_call, 0));
  EFF_HIP_TRY(hipHostGetDevicePointer((void**)&e->h_done_dev, e->h_done, 0));
  e->h_err = reinterpret_cast<int32_t*>(e->h_done + 1);  // shares the 64-byte block
  e->h_err_dev = reinterpret_cast<int32_t*>(e->h_done_dev + 1);
  EFF_HIP_TRY(hipHostGetDevicePointer((void**)&e->h_yhost_dev, e->h_yhost, 0));
  std::memset(e->h_call, 0, kCallRing * sizeof(uint64_t));
  std::memset(e->h_done, 0, 64);
  // prefill
  if (T > 0) {
    EFF_HIP_TRY(dalloc(&e->d_pf_count, E + 1));
    EFF_HIP_TRY(dalloc(&e->d_pf_rows, T * K));
    EFF_HIP_TRY(dalloc(&e->d_pf_a, (size_t)(T * K * I)));
    EFF_HIP_TRY(dalloc(&e->d_pf_x, (size_t)(T * H)));
    EFF_HIP_TRY(dalloc(&e->d_pf_y, (size_t)(T * K * H)));
    EFF_HIP_TRY(dalloc(&e->d_pf_slot_of, E));
    EFF_HIP_TRY(dalloc(&e->d_pf_experts, E));
    EFF_HIP_TRY(hipHostMalloc((void**)&e->h_pf_ids, (size_t)(T * K) * 4, 0));
    EFF_HIP_TRY(hipHostMalloc((void**)&e->h_pf_meta, (size_t)(2 * E) * 4, 0));
  }
  EFF_HIP_TRY(hipEventCreateWithFlags(&e->ev_copy, hipEventDisableTiming));
  for (int b = 0; b < 2; ++b) {
    EFF_HIP_TRY(hipEventCreateWithFlags(&e->ev_pf[b], hipEventDisableTiming));
    EFF_HIP_TRY(hipEventCreateWithFlags(&e->ev_pf_done[b], hipEventDisableTiming));
  }
  // initial state: empty cache
  EFF_HIP_TRY(hipMemset(e->d_table, 0xFF, (size_t)(L * E) * 4));
  EFF_HIP_TRY(hipMemset(e->d_owner, 0xFF, (size_t)std::max<int64_t>(1, S) * 4));
  EFF_HIP_TRY(hipMemset(e->d_usage, 0xFF, (size_t)std::max<int64_t>(1, S) * 8));
  EFF_HIP_TRY(hipMemset(e->d_recency, 0xFF, (size_t)(L * E) * 8));
  EFF_HIP_TRY(hipMemset(e->d_clock, 0, 24));
  EFF_HIP_TRY(hipMemset(e->d_pending, 0, sizeof(Pending)));
  EFF_HIP_TRY(hipMemset(e->d_err, 0, 4));
  EFF_HIP_TRY(hipMemset(e->d_seq, 0, 8));
  EFF_HIP_TRY(hipMemset(e->d_stats, 0, ST_COUNT * 8));
  std::memset(e->h_fetch, 0, kFetchLists * sizeof(FetchList));
  EFF_HIP_TRY(split_kernel_setup((int)S, (int)E));
  EFF_HIP_TRY(decode_kernels_setup(c.wformat, (int)B, (int)H, (int)I));
  EFF_HIP_TRY(hipDeviceSynchronize());
  return EFF_OK;
}

// ---------------------------------------------------------------------------------- timing
static hipEvent_t take_event(eff_engine* e) {
  if (!e->free_events.empty()) {
    hipEvent_t ev = e->free_events.back();
    e->free_events.pop_back();
    return ev;
  }
  hipEvent_t ev = nullptr;
  if (hipEventCreate(&ev) != hipSuccess) return nullptr;
  return ev;
}

// Adds the durations of every recorded call (waits for them) and recycles the events.
static void resolve_timing(eff_engine* e) {
  for (auto& tc : e->timed) {
    bool ok = tc.ev[0] && tc.ev[1] && tc.ev[2] && tc.ev[3] && hipEventSynchronize(tc.ev[3]) == hipSuccess;
    float a = 0.f, b = 0.f;
    if (ok && hipEventElapsedTime(&a, tc.ev[0], tc.ev[1]) == hipSuccess &&
        hipEventElapsedTime(&b, tc.ev[2], tc.ev[3]) == hipSuccess) {
      e->t_ms[tc.kind] += a;
      e->t_ms[tc.kind + 1] += b;
      e->t_launches[tc.kind] += 1;
      e->t_launches[tc.kind + 1] += 1;
      const int32_t* tq = e->h_tq + 2 * (&tc - e->timed.data());
      if (tc.has_q && tq[0] == 0) {
        e->t_units_nf += tq[1];
        e->t_ms_nf[tc.kind] += a;
        e->t_ms_nf[tc.kind + 1] += b;
        e->t_launches_nf[tc.kind] += 1;
        e->t_launches_nf[tc.kind + 1] += 1;
      }
    }
    for (hipEvent_t ev : tc.ev)
      if (ev) e->free_events.push_back(ev);
  }
  e->timed.clear();
}

int timing_begin(eff_engine* e, int kind, hipStream_t s, bool record_first) {
  if (!(e->cfg.flags & EFF_CFG_TIMING)) return -1;
  if (e->timed.size() >= (size_t)kTimedMax) resolve_timing(e);  // bounded number of live events
  eff_engine::TimedCall tc;
  tc.kind = kind;
  for (int i = 0; i < 4; ++i) tc.ev[i] = take_event(e);
  const int slot = (int)e->timed.size();
  // the call's fetch count and GPU expert count, copied before the launch's first event (stream order)
  tc.has_q = e->timing_q_src &&
             hipMemcpyAsync(e->h_tq + 2 * slot, e->timing_q_src, sizeof(int32_t), hipMemcpyDeviceToHost, s) ==
                 hipSuccess &&
             hipMemcpyAsync(e->h_tq + 2 * slot + 1, &e->d_plan->nu, sizeof(int32_t), hipMemcpyDeviceToHost, s) ==
                 hipSuccess;
  e->timed.push_back(tc);
  if (record_first) timing_mark(e, slot, 0, s);
  return slot;
}

hipEvent_t timing_event(eff_engine* e, int slot, int i) {
  if (slot < 0 || slot >= (int)e->timed.size()) return nullptr;
  return e->timed[slot].ev[i];
}

bool stream_capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(s, &st) == hipSuccess && st != hipStreamCaptureStatusNone;
}

void timing_mark(eff_engine* e, int slot, int i, hipStream_t s) {
  if (slot < 0 || slot >= (int)e->timed.size()) return;
  hipEvent_t ev = e->timed[slot].ev[i];
  if (ev) (void)hipEventRecord(ev, s);
}

static int check_engine(eff_engine* e) {
  if (!e) return fail(EFF_EINVAL, "engine is NULL");
  return EFF_OK;
}

static int read_device_error(eff_engine* e) {
  for (int w = 0; w < kFetchLists; ++w) {
    const int err = e->h_fetch[w].err;
    if (err) {
      e->h_fetch[w].err = 0;
      return fail(EFF_EDEVICE, (err & 1)    ? "an expert id was outside [0, E) (entries skipped)"
                               : (err & 16) ? "victim selection found fewer candidates than it counted"
                                            : "split ran without a pending ensure");
    }
  }
  return EFF_OK;
}


// ---------------------------------------------------------------------------- host share
static int64_t ns_since(std::chrono::steady_clock::time_point t) {
  return std::chrono::duration_cast<std::chrono::nanoseconds>(std::chrono::steady_clock::now() - t).count();
}

static void set_async_error(eff_engine* e, const std::string& msg) {
  std::lock_guard<std::mutex> g(e->async_mu);
  if (!e->async_err.load()) {
    e->async_msg = msg;
    e->async_err.store(1, std::memory_order_release);
  }
}

static int check_async_error(eff_engine* e) {
  const int32_t dev_err = __atomic_exchange_n(e->h_err, 0, __ATOMIC_ACQ_REL);  // sticky device error bits
  if (dev_err)
    return fail(EFF_EDEVICE, (dev_err & 1) ? "an expert id was outside [0, E) (entries skipped)"
                             : (dev_err & 4) ? "a combine gave up waiting for its host share"
                             : (dev_err & 8) ? "a prefill activation or SwiGLU output exceeded the fp16 range (65504)"
                             : (dev_err & 16) ? "victim selection found fewer candidates than it counted"
                                             : "device error");
  if (!e->async_err.load(std::memory_order_acquire)) return EFF_OK;
  std::lock_guard<std::mutex> g(e->async_mu);
  return fail(EFF_EHIP, "host share of an earlier decode call: " + e->async_msg);
}

// Waits for the control kernel's word of call `seq`: the number of entries the host computes,
// 0 when a later call already overwrote the word (only calls without host entries let the
// device run ahead), or -1 (error recorded) when the word does not come.  With a stream given,
// the wait also ends when that stream fails or drains without publishing.
// Fields of a call word (see kCallRing).
static inline uint32_t word_seq(uint64_t w) { return (uint32_t)(w >> 32); }
static inline int word_host(uint64_t w) { return (int)(w & kCallHostMask); }
static inline int word_batch(uint64_t w) { return (int)((w >> kCallBShift) & kCallBMask) + 1; }
static inline int word_layer(uint64_t w) { return (int)((w >> kCallLayerShift) & kCallLayerMask); }
// order of two call numbers from their low 32 bits (calls in flight are far fewer than 2^31 apart)
static inline int32_t seq_order(uint32_t a, uint64_t b) { return (int32_t)(a - (uint32_t)b); }

// EFF_CFG_SYNC_HOST: waits for call `seq`'s word; returns its host entries (-1 on failure).
static int wait_call(eff_engine* e, uint64_t seq, hipStream_t cs) {
  const auto t0 = std::chrono::steady_clock::now();
  volatile uint64_t* word = e->h_call + seq % kCallRing;
  int nhost = -1;
  for (uint64_t spin = 1;; ++spin) {
    const uint64_t w = *word;
    const int32_t d = seq_order(word_seq(w), seq);
    if (d == 0) {
      nhost = word_host(w);
      break;
    }
    if (d > 0) {
      nhost = 0;
      break;
    }
    if ((spin & 4095) == 0) {
      const hipError_t q = hipStreamQuery(cs);
      if (q == hipSuccess && seq_order(word_seq(*word), seq) < 0) {
        set_async_error(e, "control kernel finished without publishing its call");
        break;
      }
      if (q != hipSuccess && q != hipErrorNotReady) {
        set_async_error(e, std::string("control kernel: ") + hipGetErrorString(q));
        break;
      }
      if (ns_since(t0) > (int64_t)30 * 1000 * 1000 * 1000) {
        set_async_error(e, "no control kernel result within 30 s");
        break;
      }
    }
    _mm_pause();
  }
  std::atomic_thread_fence(std::memory_order_acquire);
  e->wait_ns += ns_since(t0);
  return nhost;
}

// The host-share worker (asynchronous mode) follows the call ring in call order, so it needs no
// message from the enqueuing thread and a captured decode step drives it like an eager one.  For a
// call with host entries it runs the host share from the host-mapped x and host ids, then stores
// h_done = seq, which releases that call's combine kernel.  x and the host ids stay valid meanwhile:
// the next control kernel runs after that combine.  A ring slot already holding a later call was
// overwritten while the worker lagged, which only a call without host entries can be (a call with
// host entries holds its stream until h_done): it is skipped.
static void worker_loop(eff_engine* e) {
  if (e->host_pin && !e->host_cpus.empty() && pin_this_thread(e->host_cpus[0])) e->worker_pinned.store(true);
  uint64_t next = e->worker_seq.load(std::memory_order_relaxed) + 1, idle = 0;
  auto t_wait = std::chrono::steady_clock::now();
  for (;;) {
    const uint64_t w = *(volatile uint64_t*)(e->h_call + next % kCallRing);
    const int32_t d = seq_order(word_seq(w), next);
    if (d < 0) {  // not published yet
      if (e->worker_stop.load(std::memory_order_acquire)) break;
      if (++idle < 100000) _mm_pause();
      else std::this_thread::sleep_for(std::chrono::microseconds(20));
      continue;
    }
    idle = 0;
    std::atomic_thread_fence(std::memory_order_acquire);
    if (d == 0 && word_host(w) > 0) {
      const auto t1 = std::chrono::steady_clock::now();
      e->wait_ns += std::chrono::duration_cast<std::chrono::nanoseconds>(t1 - t_wait).count();
      host_ffn(e, word_layer(w), e->h_x, e->h_cpu, word_batch(w), e->h_yhost);
      e->host_ns += ns_since(t1);
      e->host_calls_a += 1;
      std::atomic_thread_fence(std::memory_order_release);
      __atomic_store_n(e->h_done, next, __ATOMIC_RELEASE);
      t_wait = std::chrono::steady_clock::now();
    }
    e->worker_seq.store(next, std::memory_order_release);
    ++next;
  }
}

// Waits until the worker has handled every decode call issued so far (synchronizes the device).
static void drain_worker(eff_engine* e) {
  if (!e->async_host) return;
  uint64_t last = 0;
  if (hipDeviceSynchronize() != hipSuccess || hipMemcpy(&last, e->d_seq, 8, hipMemcpyDeviceToHost) != hipSuccess)
    return;
  const auto t0 = std::chrono::steady_clock::now();
  while (e->worker_seq.load(std::memory_order_acquire) < last) {
    if (ns_since(t0) > (int64_t)30 * 1000 * 1000 * 1000) {
      set_async_error(e, "host-share worker did not catch up within 30 s");
      return;
    }
    std::this_thread::sleep_for(std::chrono::microseconds(20));
  }
}

static void stop_worker(eff_engine* e) {
  if (!e->worker.joinable()) return;
  e->worker_stop.store(true, std::memory_order_release);
  e->worker.join();
}

}  // namespace eff

using namespace eff;

extern "C" {

const char* eff_last_error(void) { return g_last_error.c_str(); }

int64_t eff_record_bytes(const eff_config* cfg) {
  std::string why;
  if (validate(cfg, &why) != EFF_OK) return 0;
  return record_bytes(cfg);
}

int eff_host_alloc(size_t bytes, void** out) {
  if (!out || bytes == 0) return fail(EFF_EINVAL, "eff_host_alloc: bad arguments");
  hipError_t err = hipHostMalloc(out, bytes, hipHostMallocMapped | hipHostMallocPortable);
  if (err != hipSuccess) return fail(EFF_ENOMEM, std::string("hipHostMalloc: ") + hipGetErrorString(err));
  return EFF_OK;
}

int eff_host_free(void* p) {
  if (!p) return EFF_OK;
  EFF_HIP_TRY(hipHostFree(p));
  return EFF_OK;
}

int eff_create(const eff_config* cfg, const void* host_pool, const float* tensor_scales, eff_engine** out) {
  std::string why;
  if (!out) return fail(EFF_EINVAL, "out is NULL");
  *out = nullptr;
  if (validate(cfg, &why) != EFF_OK) return fail(EFF_EINVAL, why);
  if (!host_pool) return fail(EFF_EINVAL, "host_pool is NULL");
  if (cfg->wformat == EFF_WFMT_NVFP4_G16_E4M3 && !tensor_scales)
    return fail(EFF_EINVAL, "NVFP4 needs tensor_scales");
  const int64_t R = record_bytes(cfg);
  // the pool must be pinned host memory covering L*E records
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, host_pool) != hipSuccess || attr.type != hipMemoryTypeHost) {
    (void)hipGetLastError();
    return fail(EFF_EINVAL, "host_pool is not pinned host memory (use hipHostMalloc / eff_host_alloc)");
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(EFF_EHIP, "no HIP device");
  size_t free_b = 0, total_b = 0;
  if (hipMemGetInfo(&free_b, &total_b) == hipSuccess &&
      (uint64_t)cfg->num_slots * (uint64_t)R > (uint64_t)free_b)
    return fail(EFF_ENOMEM, "slot arena does not fit in free device memory");
  eff_engine* e = new (std::nothrow) eff_engine();
  if (!e) return fail(EFF_ENOMEM, "engine allocation failed");
  e->cfg = *cfg;
  e->R = R;
  e->pool = (const uint8_t*)host_pool;
  e->device = dev;
  int rc = alloc_all(e);
  if (rc != EFF_OK) {
    std::string msg = g_last_error;
    release(e);
    return fail(rc == EFF_EHIP ? EFF_ENOMEM : rc, msg);
  }
  const size_t nts = (size_t)cfg->num_layers * cfg->num_experts * 3;
  e->h_ts.assign(nts, 1.0f);
  if (tensor_scales) std::memcpy(e->h_ts.data(), tensor_scales, nts * sizeof(float));
  if (hipMemcpy(e->d_ts, e->h_ts.data(), nts * sizeof(float), hipMemcpyHostToDevice) != hipSuccess) {
    release(e);
    return fail(EFF_EHIP, "copying tensor scales failed");
  }
  void* pdev = nullptr;
  if (hipHostGetDevicePointer(&pdev, const_cast<void*>(host_pool), 0) != hipSuccess || !pdev) {
    (void)hipGetLastError();
    release(e);
    return fail(EFF_EINVAL, "host_pool is not mapped into the device address space (use eff_host_alloc)");
  }
  e->pool_dev = (const uint8_t*)pdev;
  // the address of this device's copy of the no-allocation scratch (eff_expert_ffn_decode_noalloc)
  if (hipError_t err = noalloc_setup(dev); err != hipSuccess) {
    release(e);
    return fail(EFF_EHIP, std::string("noalloc_setup (hipGetSymbolAddress of the static scratch): ") +
                              hipGetErrorString(err));
  }
  // the host executor: one thread per physical core ([FT-deep] §7), SMT siblings excluded, one core
  // left to the thread that enqueues the GPU work; each pinned to its core.  An explicit thread count
  // is pinned the same way when there are enough cores for it.
  e->host_cpus = physical_core_cpus();
  e->host_physical = (int)e->host_cpus.size();
  int nth = cfg->host_threads;
  if (nth == 0) nth = std::max(1, e->host_physical - (e->host_physical > 1 ? 1 : 0));
  e->host_pin = e->host_physical > 0 && nth <= e->host_physical;
  e->async_host = !(cfg->flags & EFF_CFG_SYNC_HOST);
  // in the synchronous mode the caller's thread runs its share unpinned; the pool keeps cpus[1..]
  e->pool_threads = new (std::nothrow) ThreadPool(nth, e->host_pin ? &e->host_cpus : nullptr);
  if (!e->pool_threads) {
    release(e);
    return fail(EFF_ENOMEM, "thread pool");
  }
  e->host_isa = e->host_isa_max = host_isa_best();
  if (e->async_host) {
    try {
      e->worker = std::thread(worker_loop, e);
    } catch (...) {
      release(e);
      return fail(EFF_ENOMEM, "host worker thread");
    }
  }
  *out = e;
  return EFF_OK;
}

int eff_destroy(eff_engine* e) {
  if (!e) return EFF_OK;
  drain_worker(e);
  (void)hipDeviceSynchronize();
  release(e);
  return EFF_OK;
}

int eff_route(eff_engine* e, const void* x, const void* w_router, int B, int32_t* ids, float* w,
              eff_stream_t stream) {
  if (int rc = check_engine(e)) return rc;
  const int maxB = std::max(e->cfg.max_tokens, e->cfg.max_prefill_tokens);
  if (!x || !w_router || !ids || !w || B < 1 || B > maxB) return fail(EFF_EINVAL, "eff_route: bad arguments");
  hipStream_t s = (hipStream_t)stream;
  EFF_HIP_TRY(launch_route_logits((const uint16_t*)x, (const uint16_t*)w_router, B, e->cfg.num_experts,
                                  e->cfg.hidden, e->d_logits, s));
  EFF_HIP_TRY(launch_topk(e->d_logits, B, e->cfg.num_experts, e->cfg.top_k, ids, w, s));
  return EFF_OK;
}

int eff_last_logits(eff_engine* e, const float** logits) {
  if (int rc = check_engine(e)) return rc;
  if (!logits) return fail(EFF_EINVAL, "eff_last_logits: logits is NULL");
  *logits = e->d_logits;
  return EFF_OK;
}

int eff_route_logits(eff_engine* e, const float* logits, int B, int32_t* ids, float* w, eff_stream_t stream) {
  if (int rc = check_engine(e)) return rc;
  const int maxB = std::max(e->cfg.max_tokens, e->cfg.max_prefill_tokens);
  if (!logits || !ids || !w || B < 1 || B > maxB) return fail(EFF_EINVAL, "eff_route_logits: bad arguments");
  EFF_HIP_TRY(launch_topk(logits, B, e->cfg.num_experts, e->cfg.top_k, ids, w, (hipStream_t)stream));
  return EFF_OK;
}

int eff_ensure_experts(eff_engine* e, int layer, int32_t* ids_inout, int n, uint32_t flags, eff_stream_t stream) {
  if (int rc = check_engine(e)) return rc;
  if (!ids_inout || layer < 0 || layer >= e->cfg.num_layers || n < 1 || n > e->cfg.max_tokens * e->cfg.top_k)
    return fail(EFF_EINVAL, "eff_ensure_experts: bad arguments");
  if (flags & ~(uint32_t)EFF_SPECULATIVE) return fail(EFF_EINVAL, "eff_ensure_experts: unknown flags");
  if (e->pending_host) return fail(EFF_ESTATE, "an ensure is already pending its split");
  // the fetch list of an earlier split of the same kind is read by eff_copy_missing
  if ((flags & EFF_SPECULATIVE) ? e->spec_split_pending : e->real_split_pending)
    return fail(EFF_ESTATE, "the copies of the previous split of this kind have not been issued (eff_copy_missing)");
  EFF_HIP_TRY(launch_ensure(e, layer, ids_inout, n, (flags & EFF_SPECULATIVE) ? 1 : 0, (hipStream_t)stream));
  e->pending_host = true;
  e->spec_pending_call = (flags & EFF_SPECULATIVE) != 0;
  if (e->spec_pending_call) e->spec_list = spec_fetch_list(layer);
  return EFF_OK;
}

int eff_split_misses(eff_engine* e, int32_t* ids_inout, int32_t* cpu_ids, int32_t* counts, eff_stream_t stream) {
  if (int rc = check_engine(e)) return rc;
  if (!ids_inout) return fail(EFF_EINVAL, "eff_split_misses: ids is NULL");
  if (!e->pending_host) return fail(EFF_ESTATE, "split without a pending ensure");
  EFF_HIP_TRY(launch_split(e, ids_inout, cpu_ids, counts, 0, (hipStream_t)stream));
  e->pending_host = false;
  if (e->spec_pending_call) e->spec_split_pending = true;
  else e->real_split_pending = true;
  return EFF_OK;
}

int64_t eff_qstar(int64_t m, uint32_t f) {
  if (m < 0 || m > ((int64_t)1 << 40) || f > 65536u) return -1;
  return qstar_host(m, f);
}

int eff_qstar_batch(const int32_t* m, const uint32_t* f, int32_t* q, int n, eff_stream_t stream) {
  if ((!m || !f || !q) && n > 0) return fail(EFF_EINVAL, "eff_qstar_batch: NULL pointer");
  if (n < 0) return fail(EFF_EINVAL, "eff_qstar_batch: n < 0");
  EFF_HIP_TRY(launch_qstar_batch(m, f, q, n, (hipStream_t)stream));
  return EFF_OK;
}

uint32_t eff_frac_q16(double bp, double bh) {
  if (std::isnan(bp) || std::isnan(bh) || bp < 0 || bh < 0) return 0xFFFFFFFFu;
  if (bp == 0) return 0;
  if (bh == 0 || std::isinf(bp)) return 65536u;
  if (std::isinf(bh)) return 0;
  // the integer part of bp * 65536 / bh, exactly: the quotient's floor, then corrected by the
  // sign of q*bh - bp*65536 (one rounding in the fma keeps the sign; bp*65536 is exact)
  const double num = bp * 65536.0;
  double q = std::floor(num / bh);
  if (q >= 65536.0) return 65536u;
  if (std::fma(q, bh, -num) > 0) q -= 1;
  else if (std::fma(q + 1, bh, -num) <= 0) q += 1;
  return q >= 65536.0 ? 65536u : (uint32_t)q;
}

int eff_set_speculation(eff_engine* e, int max_fetch, int in_gap) {
  if (int rc = check_engine(e)) return rc;
  if (max_fetch < -1 || (in_gap != 0 && in_gap != 1))
    return fail(EFF_EINVAL, "eff_set_speculation: max_fetch >= -1 and in_gap 0 or 1");
  e->spec_budget = max_fetch;
  e->spec_in_gap = in_gap != 0;
  return EFF_OK;
}

int eff_set_speculation_link(eff_engine* e, int link_records) {
  if (int rc = check_engine(e)) return rc;
  if (link_records < -1) return fail(EFF_EINVAL, "eff_set_speculation_link: link_records >= -1");
  e->spec_link = link_records;
  return EFF_OK;
}

int eff_set_fetch_frac(eff_engine* e, uint32_t frac_q16) {
  if (int rc = check_engine(e)) return rc;
  if (frac_q16 > 65536u) return fail(EFF_EINVAL, "fetch_frac_q16 must be in [0, 65536]");
  e->cfg.fetch_frac_q16 = frac_q16;
  return EFF_OK;
}

// The host side of the profile: `calls` host shares of one token with K experts each (a layer's
// experts in turn, layers cycling first, so consecutive calls read distinct records).
static double host_profile_pass(eff_engine* e, int calls, const uint16_t* x, float* y) {
  const eff_config& c = e->cfg;
  std::vector<int32_t> cpu(c.top_k);
  const auto t0 = std::chrono::steady_clock::now();
  for (int i = 0; i < calls; ++i) {
    const int layer = i % c.num_layers, base = (i / c.num_layers) * c.top_k;
    for (int k = 0; k < c.top_k; ++k) cpu[k] = (base + k) % c.num_experts;
    host_ffn(e, layer, x, cpu.data(), 1, y);
  }
  return std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
}

int eff_profile_bandwidth(eff_engine* e, int records, eff_bw_profile* out) {
  if (int rc = check_engine(e)) return rc;
  if (!out) return fail(EFF_EINVAL, "eff_profile_bandwidth: out is NULL");
  const eff_config& c = e->cfg;
  const int64_t n_flat = (int64_t)c.num_layers * c.num_experts;
  if (records < 1 || records > n_flat) return fail(EFF_EINVAL, "records must be in [1, L*E]");
  if (capturing(nullptr)) return fail(EFF_ECAPTURE, "eff_profile_bandwidth waits on the host");
  drain_worker(e);
  if (int rc = check_async_error(e)) return rc;
  hipStream_t s = nullptr;
  hipEvent_t ev[2] = {nullptr, nullptr};
  uint8_t* dst = nullptr;
  int rc = EFF_OK;
  const int64_t stride = std::max<int64_t>(1, n_flat / records);
  const int K = c.top_k, calls = (records + K - 1) / K;
  const double host_bytes = (double)calls * K * e->R;
  std::vector<uint16_t> x(c.hidden);
  std::vector<float> y((size_t)K * c.hidden);
  uint32_t lcg = 12345u;  // a fixed token: bf16 values in about [-2, 2)
  for (auto& v : x) {
    lcg = lcg * 1664525u + 1013904223u;
    const float f = ((lcg >> 8) * (1.0f / 16777216.0f)) * 4.0f - 2.0f;
    uint32_t u;
    std::memcpy(&u, &f, 4);
    v = (uint16_t)(u >> 16);
  }
  auto gpu_pass = [&](int n, float* ms) -> hipError_t {
    hipError_t err = hipEventRecord(ev[0], s);
    if (err == hipSuccess) err = launch_bw_copy(e, 0, stride, n, dst, s);
    if (err == hipSuccess) err = hipEventRecord(ev[1], s);
    return err;
  };
  auto gpu_done = [&](float* ms) -> hipError_t {
    hipError_t err = hipEventSynchronize(ev[1]);
    if (err == hipSuccess) err = hipEventElapsedTime(ms, ev[0], ev[1]);
    return err;
  };
  do {
    if (hipStreamCreate(&s) != hipSuccess || hipEventCreate(&ev[0]) != hipSuccess ||
        hipEventCreate(&ev[1]) != hipSuccess) {
      rc = fail(EFF_EHIP, "eff_profile_bandwidth: stream or events");
      break;
    }
    if (hipMalloc((void**)&dst, 2 * (size_t)e->R) != hipSuccess) {
      rc = fail(EFF_ENOMEM, "eff_profile_bandwidth: scratch");
      break;
    }
    float ms = 0.f;
    // warm-up, then the link alone
    if (gpu_pass(std::min(records, 4), &ms) != hipSuccess || gpu_done(&ms) != hipSuccess ||
        gpu_pass(records, &ms) != hipSuccess || gpu_done(&ms) != hipSuccess) {
      rc = fail(EFF_EHIP, "eff_profile_bandwidth: copy kernel");
      break;
    }
    const double t_p = std::max(1e-9, ms * 1e-3);
    // the host alone (one warm-up call)
    host_profile_pass(e, 1, x.data(), y.data());
    const double t_h = std::max(1e-9, host_profile_pass(e, calls, x.data(), y.data()));
    // both at once: enough records on the link to cover the host pass
    const int n2 = (int)std::min<double>(n_flat, std::max(1.0, std::round(records * t_h / t_p)));
    if (gpu_pass(n2, &ms) != hipSuccess) {
      rc = fail(EFF_EHIP, "eff_profile_bandwidth: copy kernel");
      break;
    }
    const double t_h2 = std::max(1e-9, host_profile_pass(e, calls, x.data(), y.data()));
    if (gpu_done(&ms) != hipSuccess) {
      rc = fail(EFF_EHIP, "eff_profile_bandwidth: copy kernel");
      break;
    }
    const double t_p2 = std::max(1e-9, ms * 1e-3);
    out->pcie_alone = (double)records * e->R / t_p;
    out->host_alone = host_bytes / t_h;
    out->pcie_concurrent = (double)n2 * e->R / t_p2;
    out->host_concurrent = host_bytes / t_h2;
    out->frac_q16 = eff_frac_q16(out->pcie_concurrent, out->host_concurrent);
    out->frac_q16_alone = eff_frac_q16(out->pcie_alone, out->host_alone);
    out->record_bytes = e->R;
    out->records = records;
    out->pad = 0;
  } while (false);
  if (s) (void)hipStreamSynchronize(s);
  if (dst) (void)hipFree(dst);
  for (hipEvent_t v : ev)
    if (v) (void)hipEventDestroy(v);
  if (s) (void)hipStreamDestroy(s);
  return rc;
}

int eff_rebuild_cache(eff_engine* e, int num_slots, uint64_t max_arena_bytes) {
  if (int rc = check_engine(e)) return rc;
  if (capturing(nullptr)) return fail(EFF_ECAPTURE, "eff_rebuild_cache waits on the host");
  const eff_config& c = e->cfg;
  const int64_t L = c.num_layers, E = c.num_experts;
  // geometry and budget, before anything else
  if (num_slots < 0 || num_slots > kMaxSlots) return fail(EFF_EREJECTED, "num_slots must be in [0, 16384]");
  const uint64_t slot_bytes = (uint64_t)num_slots * (uint64_t)e->R;
  if (max_arena_bytes > 0 && slot_bytes > max_arena_bytes)
    return fail(EFF_EREJECTED, "the slot arena does not fit the byte budget");
  const uint64_t arena = num_slots > 0 ? slot_bytes + kArenaTail : 0;
  // a safe point: no call half done
  if (e->pending_host) return fail(EFF_EREJECTED, "an ensure is waiting for its split");
  if (e->real_split_pending || e->spec_split_pending)
    return fail(EFF_EREJECTED, "a split's copies have not been issued (eff_copy_missing)");
  if (e->pf_streamed[0] || e->pf_streamed[1])
    return fail(EFF_EREJECTED, "a streamed prefill layer has not been computed");
  drain_worker(e);
  if (int rc = check_async_error(e)) return rc;
  // the new buffers first; on any failure only they are released
  uint8_t* arena_new = nullptr;
  int32_t* owner_new = nullptr;
  int64_t* usage_new = nullptr;
  auto reject = [&](const std::string& why) {
    (void)hipGetLastError();
    if (arena_new) (void)hipFree(arena_new);
    if (owner_new) (void)hipFree(owner_new);
    if (usage_new) (void)hipFree(usage_new);
    return fail(EFF_EREJECTED, why);
  };
  const size_t S1 = (size_t)std::max(1, num_slots);
  if (arena > 0 && hipMalloc((void**)&arena_new, arena) != hipSuccess)
    return reject("the slot arena cannot be allocated");
  if (hipMalloc((void**)&owner_new, S1 * sizeof(int32_t)) != hipSuccess ||
      hipMalloc((void**)&usage_new, S1 * sizeof(int64_t)) != hipSuccess)
    return reject("the slot tables cannot be allocated");
  if (hipMemset(owner_new, 0xFF, S1 * sizeof(int32_t)) != hipSuccess ||
      hipMemset(usage_new, 0xFF, S1 * sizeof(int64_t)) != hipSuccess)
    return reject("clearing the new slot tables failed");
  if (num_slots > c.num_slots && split_kernel_setup(num_slots, (int)E) != hipSuccess)
    return reject("the victim sort cannot take that many slots");
  // commit: nothing resident, the old cache released, the clock and recency kept
  if (hipMemset(e->d_table, 0xFF, (size_t)(L * E) * sizeof(int32_t)) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess)
    return reject("clearing the table failed");
  if (e->d_arena) (void)hipFree(e->d_arena);
  (void)hipFree(e->d_owner);
  (void)hipFree(e->d_usage);
  e->d_arena = arena_new;
  e->d_owner = owner_new;
  e->d_usage = usage_new;
  e->cfg.num_slots = num_slots;
  std::memset(e->h_fetch, 0, kFetchLists * sizeof(FetchList));
  EFF_HIP_TRY(hipMemset(e->d_fetch, 0, kFetchLists * sizeof(FetchList)));  // no list names an old slot
  return EFF_OK;
}

static int issue_copies(eff_engine* e, int which, hipStream_t side) {
  const FetchList& fl = e->h_fetch[which];
  for (int i = 0; i < fl.count; ++i) {
    const int64_t flat = fl.flat[i], slot = fl.slot[i];
    EFF_HIP_TRY(hipMemcpyAsync(e->d_arena + slot * e->R, e->pool + flat * e->R, (size_t)e->R,
                               hipMemcpyHostToDevice, side));
  }
  if (which == 0) e->host_bytes_fetched += (int64_t)fl.count * e->R;
  else e->host_spec_fetched += fl.count;
  return EFF_OK;
}

// Issues the pending fetches (real, then speculative) on `side` and makes `compute` wait for
// every copy issued so far (the side stream is in order, so this also covers speculative copies
// issued one layer earlier that this layer now hits).  The host must have waited for the split.
static int issue_pending_copies(eff_engine* e, hipStream_t cs, hipStream_t ss) {
  if (int rc = read_device_error(e)) return rc;
  if (e->real_split_pending) {
    if (int rc = issue_copies(e, 0, ss)) return rc;
    e->real_split_pending = false;
  }
  if (e->spec_split_pending) {
    if (int rc = issue_copies(e, e->spec_list, ss)) return rc;
    e->spec_split_pending = false;
  }
  EFF_HIP_TRY(hipEventRecord(e->ev_copy, ss));
  EFF_HIP_TRY(hipStreamWaitEvent(cs, e->ev_copy, 0));
  return EFF_OK;
}

static double now_ms() {
  return std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now().time_since_epoch()).count();
}

int eff_copy_missing(eff_engine* e, eff_stream_t compute, eff_stream_t side) {
  if (int rc = check_engine(e)) return rc;
  hipStream_t cs = (hipStream_t)compute, ss = (hipStream_t)side;
  if (capturing(cs) || capturing(ss)) return fail(EFF_ECAPTURE, "eff_copy_missing waits on the host");
  EFF_HIP_TRY(hipStreamSynchronize(cs));
  return issue_pending_copies(e, cs, ss);
}

int eff_expert_ffn_decode(eff_engine* e, int layer, const void* x, const int32_t* slots, int B, float* y,
                          eff_stream_t stream) {
  if (int rc = check_engine(e)) return rc;
  if (!x || !slots || !y || B < 1 || B > e->cfg.max_tokens || layer < 0 || layer >= e->cfg.num_layers)
    return fail(EFF_EINVAL, "eff_expert_ffn_decode: bad arguments");
  EFF_HIP_TRY(launch_ffn_decode(e, layer, (const uint16_t*)x, slots, B, y, (hipStream_t)stream));
  return EFF_OK;
}

int eff_expert_ffn_decode_noalloc(eff_engine* e, int layer, const void* x, const int32_t* slots, int B, float* y,
                                  eff_stream_t stream) {
  if (int rc = check_engine(e)) return rc;
  if (!x || !slots || !y || B < 1 || B > e->cfg.max_tokens || layer < 0 || layer >= e->cfg.num_layers)
    return fail(EFF_EINVAL, "eff_expert_ffn_decode_noalloc: bad arguments");
  const size_t need = noalloc_need(e, B);
  if (need > kNoAllocScratchBytes)
    return fail(EFF_EINVAL, "eff_expert_ffn_decode_noalloc: this call needs " + std::to_string(need) +
                                " bytes of scratch (plan + 3 * min(B*K, units) * max_tokens * inter), more than the " +
                                std::to_string(kNoAllocScratchBytes) + " of the static scratch");
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != e->device)
    return fail(EFF_EINVAL, "eff_expert_ffn_decode_noalloc: the current device is not the engine's");
  const hipError_t err = launch_ffn_decode_noalloc(e, (const uint16_t*)x, slots, B, y, (hipStream_t)stream);
  if (err == hipErrorNotInitialized)
    return fail(EFF_ESTATE, "eff_expert_ffn_decode_noalloc: no scratch address for this device");
  EFF_HIP_TRY(err);
  return EFF_OK;
}

int eff_host_ffn_decode(eff_engine* e, int layer, const void* x_host, const int32_t* cpu_ids_host, int B,
                        float* y_host) {
  if (int rc = check_engine(e)) return rc;
  if (!x_host || !cpu_ids_host || !y_host || B < 1 || B > e->cfg.max_tokens || layer < 0 ||
      layer >= e->cfg.num_layers)
    return fail(EFF_EINVAL, "eff_host_ffn_decode: bad arguments");
  host_ffn(e, layer, (const uint16_t*)x_host, cpu_ids_host, B, y_host);
  return EFF_OK;
}

int eff_combine(eff_engine* e, const float* y_gpu, const float* y_host, const int32_t* slots, const float* w,
                int B, void* out, eff_stream_t stream) {
  if (int rc = check_engine(e)) return rc;
  if (!y_gpu || !slots || !w || !out || B < 1 || B > std::max(e->cfg.max_tokens, e->cfg.max_prefill_tokens))
    return fail(EFF_EINVAL, "eff_combine: bad arguments");
  EFF_HIP_TRY(launch_combine(y_gpu, y_host ? y_host : y_gpu, slots, w, B, e->cfg.top_k, e->cfg.hidden,
                             (uint16_t*)out, (hipStream_t)stream));
  return EFF_OK;
}

int eff_decode_layer(eff_engine* e, int layer, const void* x, const void* w_router, const float* logits, int B,
                     const int32_t* spec_ids, void* out, eff_stream_t compute, eff_stream_t side) {
  if (int rc = check_engine(e)) return rc;
  if (int rc = check_async_error(e)) return rc;
  const eff_config& c = e->cfg;
  if (!x || !out || (!w_router && !logits) || B < 1 || B > c.max_tokens || layer < 0 || layer >= c.num_layers)
    return fail(EFF_EINVAL, "eff_decode_layer: bad arguments");
  if (e->pending_host) return fail(EFF_ESTATE, "an ensure is pending its split");
  hipStream_t cs = (hipStream_t)compute, ss = (hipStream_t)side;
  if (!e->async_host && (capturing(cs) || capturing(ss)))
    return fail(EFF_ECAPTURE, "eff_decode_layer waits on the host (EFF_CFG_SYNC_HOST)");
  if ((c.flags & EFF_CFG_TIMING) && (capturing(cs) || capturing(ss)))
    return fail(EFF_ECAPTURE, "eff_decode_layer: timing events cannot be captured (EFF_CFG_TIMING)");
  const int K = c.top_k;
  const float* lg = logits;
  if (w_router) {
    EFF_HIP_TRY(launch_route_logits((const uint16_t*)x, (const uint16_t*)w_router, B, c.num_experts, c.hidden,
                                    e->d_logits, cs));
    lg = e->d_logits;
  }
  // top-K, ensure, split, the speculative request and the decode plan in one workgroup; host ids
  // and x land in host-mapped memory, then the call word
  const bool spec = spec_ids && layer + 1 < c.num_layers;
  EFF_HIP_TRY(launch_control(e, layer, lg, B, (const uint16_t*)x, spec ? spec_ids : nullptr, cs));
  // GPU experts; a unit installed by this call reads its record from the pool and fills its slot.
  // This layer's speculative fetches ride along as extra workgroups of its gate/up kernel (beside
  // the layer's own fetches) or, in the gap, of its down kernel: their victims are slots this call
  // does not use, and the next layer's kernels follow them in stream order, with no launch or event
  // of their own.  A budget or link cap of 0 lets the request fetch nothing (it still stamps its
  // hits), so nothing rides along then.
  SpecCopy sc;
  if (spec && e->spec_budget != 0 && e->spec_link != 0) {
    sc.fl = e->d_fetch + spec_fetch_list(layer + 1);
    sc.nwg = kSpecCopyWGs;
    sc.S = c.num_slots;
    sc.n_flat = (int64_t)c.num_layers * c.num_experts;
  }
  e->timing_q_src = e->d_counts + 1;  // this call's fetch count (real split)
  const hipError_t ffn_err = launch_ffn_decode(e, layer, (const uint16_t*)x, e->d_slots, B, e->d_ygpu, cs, true, sc,
                                               e->spec_in_gap);
  e->timing_q_src = nullptr;
  EFF_HIP_TRY(ffn_err);
  if (e->async_host) {
    // the combine waits for the host share (or the control kernel's own release of the call)
    EFF_HIP_TRY(launch_combine(e->d_ygpu, e->h_yhost_dev, e->d_slots, e->d_w, B, K, c.hidden, (uint16_t*)out, cs,
                               e->h_done_dev, e->d_seq, e->h_err_dev));
    return EFF_OK;
  }
  const int nhost = wait_call(e, ++e->sync_seq, cs);
  if (nhost < 0) return fail(EFF_EHIP, e->async_msg);
  if (nhost > 0) {
    const auto t1 = std::chrono::steady_clock::now();
    host_ffn(e, layer, e->h_x, e->h_cpu, B, e->h_yhost);  // overlaps the GPU expert kernels
    e->host_ns += ns_since(t1);
    e->host_calls_a += 1;
  }
  EFF_HIP_TRY(launch_combine(e->d_ygpu, e->h_yhost_dev, e->d_slots, e->d_w, B, K, c.hidden, (uint16_t*)out, cs));
  return EFF_OK;
}

int eff_last_layer_info(eff_engine* e, const int32_t** ids, const float** w, const int32_t** slots,
                        const int32_t** cpu_ids, const int32_t** counts) {
  if (int rc = check_engine(e)) return rc;
  if (ids) *ids = e->d_ids;
  if (w) *w = e->d_w;
  if (slots) *slots = e->d_slots;
  if (cpu_ids) *cpu_ids = e->d_cpu;
  if (counts) *counts = e->d_counts;
  return EFF_OK;
}

int eff_prefill_stream_layer(eff_engine* e, int layer, eff_stream_t side) {
  if (int rc = check_engine(e)) return rc;
  const eff_config& c = e->cfg;
  if (layer < 0 || layer >= c.num_layers) return fail(EFF_EINVAL, "eff_prefill_stream_layer: bad layer");
  if (c.num_slots < 2 * c.num_experts) return fail(EFF_EINVAL, "double buffering needs S >= 2E");
  hipStream_t ss = (hipStream_t)side;
  const int b = layer % 2;
  // the buffer is free once the layer that used it last has finished computing
  if (e->pf_done_recorded[b]) EFF_HIP_TRY(hipStreamWaitEvent(ss, e->ev_pf_done[b], 0));
  EFF_HIP_TRY(launch_prefill_install(e, layer, ss));
  const int64_t E = c.num_experts;
  EFF_HIP_TRY(hipMemcpyAsync(e->d_arena + (int64_t)b * E * e->R, e->pool + (int64_t)layer * E * e->R,
                             (size_t)(E * e->R), hipMemcpyHostToDevice, ss));
  EFF_HIP_TRY(hipEventRecord(e->ev_pf[b], ss));
  e->pf_layer[b] = layer;
  e->pf_streamed[b] = true;
  return EFF_OK;
}

int eff_expert_ffn_prefill_layer(eff_engine* e, int layer, const void* x, const int32_t* ids, const float* w,
                                 int T, void* out, eff_stream_t stream) {
  if (int rc = check_engine(e)) return rc;
  if (int rc = check_async_error(e)) return rc;
  const eff_config& c = e->cfg;
  if (!x || !ids || !w || !out || T < 1 || T > c.max_prefill_tokens || layer < 0 || layer >= c.num_layers)
    return fail(EFF_EINVAL, "eff_expert_ffn_prefill_layer: bad arguments");
  hipStream_t cs = (hipStream_t)stream;
  const int E = c.num_experts, K = c.top_k;
  if (c.num_slots >= 2 * E) {
    const int b = layer % 2;
    if (!e->pf_streamed[b] || e->pf_layer[b] != layer)
      return fail(EFF_ESTATE, "layer was not streamed (call eff_prefill_stream_layer first)");
    EFF_HIP_TRY(hipStreamWaitEvent(cs, e->ev_pf[b], 0));
    EFF_HIP_TRY(launch_prefill(e, layer, (const uint16_t*)x, ids, w, T, (uint16_t*)out, nullptr, b * E, true, cs));
    EFF_HIP_TRY(hipEventRecord(e->ev_pf_done[b], cs));
    e->pf_done_recorded[b] = true;
    e->pf_streamed[b] = false;
    return EFF_OK;
  }
  // on-demand fallback: routed experts ascending, in groups of min(S, E), copy then compute
  if (capturing(cs)) return fail(EFF_ECAPTURE, "the prefill fallback waits on the host");
  if (c.num_slots < 1) return fail(EFF_EINVAL, "prefill needs at least one slot");
  EFF_HIP_TRY(hipMemcpyAsync(e->h_pf_ids, ids, (size_t)T * K * 4, hipMemcpyDeviceToHost, cs));
  EFF_HIP_TRY(hipStreamSynchronize(cs));
  std::vector<char> used(E, 0);
  for (int p = 0; p < T * K; ++p)
    if (e->h_pf_ids[p] >= 0 && e->h_pf_ids[p] < E) used[e->h_pf_ids[p]] = 1;
  std::vector<int> routed;
  for (int x2 = 0; x2 < E; ++x2)
    if (used[x2]) routed.push_back(x2);
  const int G = std::min(c.num_slots, E);
  for (size_t g0 = 0; g0 < routed.size(); g0 += G) {
    const int n = (int)std::min<size_t>(G, routed.size() - g0);
    int32_t* slot_of = e->h_pf_meta;
    int32_t* experts = e->h_pf_meta + E;
    for (int x2 = 0; x2 < E; ++x2) slot_of[x2] = -1;
    for (int i = 0; i < n; ++i) {
      experts[i] = routed[g0 + i];
      slot_of[routed[g0 + i]] = i;
    }
    EFF_HIP_TRY(hipMemcpyAsync(e->d_pf_slot_of, slot_of, (size_t)E * 4, hipMemcpyHostToDevice, cs));
    EFF_HIP_TRY(hipMemcpyAsync(e->d_pf_experts, experts, (size_t)n * 4, hipMemcpyHostToDevice, cs));
    EFF_HIP_TRY(launch_fallback_install(e, layer, e->d_pf_experts, n, cs));
    for (int i = 0; i < n; ++i)
      EFF_HIP_TRY(hipMemcpyAsync(e->d_arena + (int64_t)i * e->R,
                                 e->pool + ((int64_t)layer * E + routed[g0 + i]) * e->R, (size_t)e->R,
                                 hipMemcpyHostToDevice, cs));
    EFF_HIP_TRY(launch_prefill(e, layer, (const uint16_t*)x, ids, w, T, (uint16_t*)out, e->d_pf_slot_of, -1,
                               false, cs));
    // staging buffers are reused by the next group
    EFF_HIP_TRY(hipStreamSynchronize(cs));
  }
  EFF_HIP_TRY(launch_combine(e->d_pf_y, nullptr, nullptr, w, T, K, c.hidden, (uint16_t*)out, cs));
  return EFF_OK;
}

int eff_snapshot_tables(eff_engine* e, int32_t* table, int32_t* owner, int64_t* usage, int64_t* recency,
                        int64_t* clock) {
  if (int rc = check_engine(e)) return rc;
  EFF_HIP_TRY(hipDeviceSynchronize());
  const eff_config& c = e->cfg;
  const size_t LE = (size_t)c.num_layers * c.num_experts, S = (size_t)c.num_slots;
  if (table) EFF_HIP_TRY(hipMemcpy(table, e->d_table, LE * 4, hipMemcpyDeviceToHost));
  if (owner && S) EFF_HIP_TRY(hipMemcpy(owner, e->d_owner, S * 4, hipMemcpyDeviceToHost));
  if (usage && S) EFF_HIP_TRY(hipMemcpy(usage, e->d_usage, S * 8, hipMemcpyDeviceToHost));
  if (recency) EFF_HIP_TRY(hipMemcpy(recency, e->d_recency, LE * 8, hipMemcpyDeviceToHost));
  if (clock) EFF_HIP_TRY(hipMemcpy(clock, e->d_clock, 16, hipMemcpyDeviceToHost));
  if (int rc = check_async_error(e)) return rc;
  return read_device_error(e);
}

int eff_get_stats(eff_engine* e, eff_stats* out) {
  if (int rc = check_engine(e)) return rc;
  if (!out) return fail(EFF_EINVAL, "eff_get_stats: out is NULL");
  int64_t st[ST_COUNT];
  EFF_HIP_TRY(hipDeviceSynchronize());
  drain_worker(e);
  EFF_HIP_TRY(hipMemcpy(st, e->d_stats, sizeof(st), hipMemcpyDeviceToHost));
  std::memset(out, 0, sizeof(*out));
  out->calls = st[ST_CALLS];
  out->hits = st[ST_HITS];
  out->fetched = st[ST_FETCHED];
  out->host = st[ST_HOST];
  out->spec_fetched = st[ST_SPEC_FETCHED];
  out->bytes_fetched = (st[ST_FETCHED] + st[ST_SPEC_FETCHED]) * e->R;
  for (int i = 0; i < 17; ++i) out->qstar_hist[i] = st[ST_HIST0 + i];
  resolve_timing(e);
  for (int i = 0; i < 4; ++i) {
    out->launches[i] = e->t_launches[i];
    out->kernel_ms[i] = e->t_ms[i];
    out->launches_nofetch[i] = e->t_launches_nf[i];
    out->kernel_ms_nofetch[i] = e->t_ms_nf[i];
  }
  out->gpu_experts_nofetch = e->t_units_nf;
  out->host_ms = e->host_ns.load() * 1e-6;
  out->wait_ms = e->wait_ns.load() * 1e-6;
  out->host_calls = e->host_calls_a.load();
  return EFF_OK;
}

int eff_get_host_info(eff_engine* e, eff_host_info* out) {
  if (int rc = check_engine(e)) return rc;
  if (!out) return fail(EFF_EINVAL, "eff_get_host_info: out is NULL");
  const int threads = e->pool_threads->size();
  const int pinned = e->pool_threads->pinned_workers() + (e->worker_pinned.load() ? 1 : 0);
  out->isa = e->host_isa;
  out->isa_best = e->host_isa_max;
  out->threads = threads;
  out->pinned = (e->host_pin && e->async_host && pinned == threads) ? 1 : 0;
  out->physical_cores = e->host_physical;
  out->pad = 0;
  return EFF_OK;
}

int eff_set_host_isa(eff_engine* e, int isa) {
  if (int rc = check_engine(e)) return rc;
  if (isa < EFF_HOST_ISA_SCALAR || isa > e->host_isa_max)
    return fail(EFF_EINVAL, "eff_set_host_isa: unknown level or one this CPU does not support");
  if (capturing(nullptr)) return fail(EFF_ECAPTURE, "eff_set_host_isa waits for the host-share worker");
  drain_worker(e);
  if (int rc = check_async_error(e)) return rc;
  e->host_isa = isa;
  return EFF_OK;
}

int eff_set_flags(eff_engine* e, uint32_t flags) {
  if (int rc = check_engine(e)) return rc;
  if (flags & ~(uint32_t)(EFF_CFG_TIMING | EFF_CFG_SYNC_HOST)) return fail(EFF_EINVAL, "unknown config flags");
  if ((flags ^ e->cfg.flags) & EFF_CFG_SYNC_HOST) return fail(EFF_EINVAL, "EFF_CFG_SYNC_HOST is fixed at create");
  e->cfg.flags = flags;
  return EFF_OK;
}

int eff_reset_stats(eff_engine* e) {
  if (int rc = check_engine(e)) return rc;
  EFF_HIP_TRY(hipDeviceSynchronize());
  drain_worker(e);
  resolve_timing(e);
  for (int i = 0; i < 4; ++i) {
    e->t_launches[i] = e->t_launches_nf[i] = 0;
    e->t_ms[i] = e->t_ms_nf[i] = 0.0;
  }
  e->t_units_nf = 0;
  e->host_bytes_fetched = 0;
  e->host_spec_fetched = 0;
  e->host_ns = 0;
  e->wait_ns = 0;
  e->host_calls_a = 0;
  EFF_HIP_TRY(hipMemset(e->d_stats, 0, ST_COUNT * 8));
  return EFF_OK;
}

int eff_slot_ptr(eff_engine* e, int slot, const void** out) {
  if (int rc = check_engine(e)) return rc;
  if (!out || slot < 0 || slot >= e->cfg.num_slots) return fail(EFF_EINVAL, "eff_slot_ptr: bad slot");
  *out = e->d_arena + (int64_t)slot * e->R;
  return EFF_OK;
}

}  // extern "C"
