// Internal declarations shared by the libeff translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <condition_variable>
#include <cstdint>
#include <functional>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "../../include/eff.h"

namespace eff {

constexpr int kMaxTokens = 32;       // decode batch bound
constexpr int kTimedMax = 4096;      // timed launches held before their events are resolved
constexpr int kMaxTopK = 32;
constexpr int kMaxEntries = 512;     // entries (B*K) of one decode call
constexpr int kMaxSlots = 16384;      // single-workgroup victim sort (keys in LDS)
constexpr int kMaxExperts = 4096;

// Error reporting -----------------------------------------------------------------------------
void set_error(const std::string& msg);
int fail(int code, const std::string& msg);
#define EFF_HIP_TRY(expr)                                                                  \
  do {                                                                                     \
    hipError_t _e = (expr);                                                                \
    if (_e != hipSuccess)                                                                  \
      return ::eff::fail(EFF_EHIP, std::string(#expr) + ": " + hipGetErrorString(_e));     \
  } while (0)

// Pending ensure (device-resident) ----------------------------------------------------------------
struct Pending {
  int32_t valid;       // 1 while an ensure waits for its split
  int32_t layer;
  int32_t n;           // entries
  int32_t spec;        // speculative call
  int64_t s;           // step of the call
  int64_t floor_;      // victims need usage < floor_
  int32_t nuniq, nmiss;
  int32_t ids[kMaxEntries];    // routed expert ids of the call
  int32_t slot[kMaxEntries];   // slot of each entry after the ensure (hits), else -1
  int32_t uniq[kMaxEntries];   // unique ids ascending
  int32_t miss[kMaxEntries];   // unique missing ids ascending
};

// Fetch lists written by the split kernel (device memory and a host-mapped mirror): list 0 for real
// calls, lists 1 and 2 for speculative requests of even and odd layers.  A speculative request made
// during layer l (for layer l+1) is copied by extra workgroups of layer l's own expert kernels; the
// request that reuses its list is made two layers later, after those kernels in stream order.
constexpr int kFetchLists = 3;
// Bytes allocated after the last slot of the arena: a decode wave loads a whole 1 KiB run (and its
// 128 scale bytes) even where a slice ends inside it, and past its last run it loads that run again
// so that no load sits behind a branch; such bytes are never used.
constexpr int64_t kArenaTail = 4096;
__host__ __device__ inline int spec_fetch_list(int layer) { return 1 + (layer & 1); }
// ------------------------------------------------------------------------------------------------
struct FetchList {
  int32_t count;
  int32_t err;         // device error word of the ensure/split pair (bit 1: bad id, bit 2: no pending,
                       // bit 16: victim count)
  int32_t flat[kMaxEntries];
  int32_t slot[kMaxEntries];
};

// Plan of one decode expert-FFN call: distinct GPU slots and their entries ----------------------
// One distinct slot: everything a decode workgroup needs comes from one record.  Units at
// index >= nu have count 0 (so a kernel never needs nu before its own unit).
struct DecodeUnit {
  int32_t slot;
  int32_t count;
  int32_t flat;                  // layer * E + expert held by the slot (tensor scales)
  int32_t fetch;                 // 1: installed by this call; the FFN kernels read the record
                                 //    from the host pool and write it into the slot
  int32_t entry[kMaxTokens];     // entry p = t*K + k, ascending
};
struct DecodePlan {
  int32_t nu;
  int32_t pad[3];
  DecodeUnit unit[kMaxEntries];
};

// Decode calls publish one word each in a host-mapped ring, at seq % kCallRing.  seq counts the
// engine's decode calls from 1 in device memory (the control kernel increments it), so a captured
// and replayed decode step numbers its calls like eager ones.  Word: seq (low 32 bits) << 32 |
// layer << 16 | (B - 1) << 10 | host entries.  The host-share worker follows the ring in seq order.
constexpr int kCallRing = 256;
constexpr int kCallLayerShift = 16, kCallBShift = 10;
constexpr uint64_t kCallHostMask = 0x3FF, kCallBMask = 0x3F, kCallLayerMask = 0xFFFF;
static_assert(kMaxEntries <= kCallHostMask && kMaxTokens <= kCallBMask + 1, "call word fields");
// polls of the host-share word by the combine kernel before it gives up (about 2 s)
constexpr uint32_t kCombineSpinLimit = 1u << 20;

// Device stats counters (int64) ----------------------------------------------------------------
enum { ST_CALLS, ST_HITS, ST_FETCHED, ST_HOST, ST_SPEC_FETCHED, ST_HIST0, ST_COUNT = ST_HIST0 + 17 };

// Host thread pool for the host executor --------------------------------------------------------
// Workers spin on the job generation for a couple of milliseconds after each job (decode calls
// come every few hundred microseconds), then sleep on a condition variable.  A task index is
// claimed by compare-and-swap on (generation << 32 | index), so a worker that wakes late can
// never run a task of a finished or newer job.
class ThreadPool {
 public:
  // n threads in all: n - 1 workers plus the thread that calls parallel_for.  With `pin`, worker i
  // is pinned to logical CPU pin[i + 1] (pin[0] is left for the calling thread).
  explicit ThreadPool(int n, const std::vector<int>* pin = nullptr);
  int pinned_workers() const { return pinned_.load(); }
  ~ThreadPool();
  // run fn(i) for i in [0, n) on the pool and the calling thread; returns when all are done
  void parallel_for(int n, const std::function<void(int)>& fn);
  int size() const { return (int)workers_.size() + 1; }

 private:
  void loop();
  void run_tasks(uint64_t g, const std::function<void(int)>* fn, int n);
  std::vector<std::thread> workers_;
  // idle workers spin on gen_ while tasks are claimed through next_ and counted in done_: each
  // on a cache line of its own, so that neither write traffic stalls the spinning readers
  alignas(128) std::atomic<uint64_t> gen_{0};
  std::atomic<const std::function<void(int)>*> fn_{nullptr};
  std::atomic<int> n_{0};
  std::atomic<bool> stop_{false};
  alignas(128) std::atomic<uint64_t> next_{0};
  alignas(128) std::atomic<int> done_{0};
  alignas(128) std::atomic<int> sleepers_{0};
  std::atomic<int> pinned_{0};
  std::mutex mu_;
  std::condition_variable cv_;
};

// One logical CPU per physical core the process may use: the affinity mask, SMT siblings
// dropped (first sibling kept), at most as many as the cgroup's CPU quota allows.
std::vector<int> physical_core_cpus();
// Pins the calling thread to one logical CPU; true on success.
bool pin_this_thread(int cpu);

// Host-share scratch, reused across calls (no allocation per call once grown).
struct HostScratch {
  int32_t uexp[kMaxEntries];
  int32_t ucnt[kMaxEntries];
  int32_t uent[kMaxEntries][kMaxTokens];
  struct alignas(128) Counter {
    std::atomic<int> v{0};
  };
  Counter done[kMaxEntries];  // gate/up slices finished per host expert
  std::vector<uint16_t> a;   // per (expert, token): hi row, then lo row of silu(g)*u, bf16
  std::vector<uint16_t> xp;  // the call's token rows in the AVX-512 kernel's paired order
};

}  // namespace eff

struct eff_engine {
  eff_config cfg;
  int64_t R = 0;              // record bytes
  const uint8_t* pool = nullptr;
  int device = 0;

  // slot arena and tables (device)
  uint8_t* d_arena = nullptr;
  int32_t* d_table = nullptr;
  int32_t* d_owner = nullptr;
  int64_t* d_usage = nullptr;
  int64_t* d_recency = nullptr;
  int64_t* d_clock = nullptr;     // {step, last_real, fetches of the last real call}
  float* d_ts = nullptr;          // [L*E*3]
  eff::Pending* d_pending = nullptr;
  eff::FetchList* d_fetch = nullptr;   // [kFetchLists]: real, speculative (even layer), speculative (odd layer)
  eff::FetchList* h_fetch = nullptr;   // host-mapped mirror [kFetchLists] (host view)
  eff::FetchList* h_fetch_dev = nullptr;  // the same memory as seen by kernels
  int32_t* d_err = nullptr;            // device error word
  int64_t* d_stats = nullptr;
  bool pending_host = false;           // host-side mirror of Pending::valid
  bool spec_pending_call = false;      // the pending ensure is speculative
  bool spec_split_pending = false;     // a speculative split's fetches not yet copied
  int spec_list = 1;                   // fetch list of the pending speculative ensure/split
  bool real_split_pending = false;

  // decode scratch
  eff::DecodePlan* d_plan = nullptr;
  float* d_a = nullptr;           // SwiGLU activations: [maxU][maxB][I] fp16, then [maxU][maxB][I/8] float2
  int maxU = 0;

  // orchestrator buffers (device)
  int32_t* d_ids = nullptr;
  float* d_w = nullptr;
  int32_t* d_slots = nullptr;
  int32_t* d_cpu = nullptr;
  int32_t* d_counts = nullptr;    // [6]
  int32_t* d_spec_ids = nullptr;
  int32_t* d_spec_cpu = nullptr;
  float* d_logits = nullptr;      // [maxT or maxB][E]
  float* d_ygpu = nullptr;        // [maxB*K*H]
  float* d_yhost = nullptr;       // [maxB*K*H]
  // pinned host staging
  uint16_t* h_x = nullptr;        // [maxB*H] host-mapped
  int32_t* h_cpu = nullptr;       // [maxB*K] host-mapped
  uint16_t* h_x_dev = nullptr;    // device views of the two above
  int32_t* h_cpu_dev = nullptr;
  uint64_t* h_call = nullptr;     // host-mapped ring [kCallRing] of call words (see kCallRing)
  uint64_t* h_call_dev = nullptr;
  uint64_t* h_done = nullptr;     // host-mapped: the last call whose host share is in h_yhost
  uint64_t* h_done_dev = nullptr;
  int32_t* h_err = nullptr;       // host-mapped sticky device error bits (bad id 1, combine wait 4, prefill fp16 range 8,
                                  // victim count 16)
  int32_t* h_err_dev = nullptr;
  uint64_t* d_seq = nullptr;      // device: the last decode call's seq
  uint64_t sync_seq = 0;          // EFF_CFG_SYNC_HOST: the host's count of decode calls (= *d_seq)
  float* h_yhost = nullptr;       // [maxB*K*H] host-mapped: the host share's outputs
  float* h_yhost_dev = nullptr;
  const uint8_t* pool_dev = nullptr;  // device view of the pinned pool (in-kernel fetches)
  bool async_host = false;        // host share on the worker thread, the stream waits on h_done
  int spec_budget = -1;           // eff_set_speculation: records per speculative request (-1: any)
  int spec_link = -1;              // eff_set_speculation_link: link records per layer (-1: no cap)
  bool spec_in_gap = false;       // eff_set_speculation: speculative copies ride in the down kernel
  // host-share worker (async mode)
  std::thread worker;
  std::atomic<uint64_t> worker_seq{0};  // every call up to this seq has been handled
  std::atomic<bool> worker_stop{false};
  std::atomic<int> async_err{0};
  std::mutex async_mu;
  std::string async_msg;
  std::atomic<int64_t> host_ns{0}, wait_ns{0}, host_calls_a{0};

  // prefill scratch
  int32_t* d_pf_count = nullptr;  // [E+1] per-expert counts / offsets
  int32_t* d_pf_rows = nullptr;   // [T*K] sorted entries (t*K+k)
  uint16_t* d_pf_a = nullptr;     // [T*K][I] fp16 SwiGLU activations
  uint16_t* d_pf_x = nullptr;     // [T][H] fp16 copy of the tokens' bf16 inputs
  float* d_pf_y = nullptr;        // [T*K][H] fp32 expert outputs
  int32_t* d_pf_meta = nullptr;   // misc
  hipEvent_t ev_copy = nullptr, ev_pf[2] = {nullptr, nullptr};
  bool pf_streamed[2] = {false, false};
  int pf_layer[2] = {-1, -1};

  std::vector<float> h_ts;        // host copy of the tensor scales (host executor)
  hipEvent_t ev_pf_done[2] = {nullptr, nullptr};
  bool pf_done_recorded[2] = {false, false};
  int32_t* d_pf_slot_of = nullptr;  // [E] slot per expert (fallback prefill)
  int32_t* d_pf_experts = nullptr;  // [E] expert list of a fallback group
  int32_t* h_pf_ids = nullptr;      // pinned [T*K]
  int32_t* h_pf_meta = nullptr;     // pinned [2E]
  eff::ThreadPool* pool_threads = nullptr;
  int host_isa = 0;               // host slice kernels: EFF_HOST_ISA_*
  int host_isa_max = 0;           // the best the CPU supports
  std::vector<int> host_cpus;     // pinned: cpus[0] for the engine's worker, cpus[i] for pool worker i - 1
  bool host_pin = false;
  std::atomic<bool> worker_pinned{false};
  int host_physical = 0;
  eff::HostScratch hscratch;
  // kernel timing (EFF_CFG_TIMING): events (start, end) of each of two kernels per call
  struct TimedCall { int kind; hipEvent_t ev[4]; bool has_q; };
  std::vector<TimedCall> timed;     // recorded, not yet resolved (at most kTimedMax)
  std::vector<hipEvent_t> free_events;
  int64_t t_launches[4] = {0, 0, 0, 0};
  double t_ms[4] = {0, 0, 0, 0};
  int64_t t_launches_nf[4] = {0, 0, 0, 0};  // calls that fetched nothing
  double t_ms_nf[4] = {0, 0, 0, 0};
  int64_t t_units_nf = 0;                   // their distinct GPU experts
  int32_t* h_tq = nullptr;                  // pinned [kTimedMax][2]: fetch count, GPU experts per timed call
  const int32_t* timing_q_src = nullptr;    // device fetch count of the call being launched, if any
  int64_t host_bytes_fetched = 0;
  int64_t host_spec_fetched = 0;
};

// Kernel launchers (implemented in the .hip files) -------------------------------------------------
namespace eff {
hipError_t launch_route_logits(const uint16_t* x, const uint16_t* wr, int B, int E, int H, float* logits,
                               hipStream_t s);
hipError_t launch_topk(const float* logits, int B, int E, int K, int32_t* ids, float* w, hipStream_t s);
hipError_t launch_ensure(eff_engine* e, int layer, int32_t* ids, int n, int spec, hipStream_t s);
hipError_t launch_split(eff_engine* e, int32_t* ids, int32_t* cpu_ids, int32_t* counts, int which,
                        hipStream_t s);
hipError_t launch_qstar_batch(const int32_t* m, const uint32_t* f, int32_t* q, int n, hipStream_t s);
hipError_t launch_prefill_install(eff_engine* e, int layer, hipStream_t s);
hipError_t launch_fallback_install(eff_engine* e, int layer, const int32_t* experts, int n,
                                   hipStream_t s);
// A speculative fetch list copied by extra workgroups at the front of an expert kernel's grid
// (fl null: none), so that the copy needs no launch or event of its own and the next layer's
// kernels follow it in stream order.  n_flat = L*E, S: the bounds every entry is checked against.
struct SpecCopy {
  const FetchList* fl = nullptr;
  int nwg = 0;
  int S = 0;
  int64_t n_flat = 0;
};
constexpr int kSpecCopyWGs = 64;  // workgroups that carry a speculative copy (the link is the bound)
// spec: a speculative copy carried by the gate/up kernel (in_down false) or by the down kernel
hipError_t launch_ffn_decode(eff_engine* e, int layer, const uint16_t* x, const int32_t* slots, int B,
                             float* y, hipStream_t s, bool plan_ready = false, SpecCopy spec = SpecCopy(),
                             bool in_down = false);
// n records from the pool (flat ids first + i*stride modulo L*E) into dst[2][R] (bandwidth profile)
hipError_t launch_bw_copy(eff_engine* e, int64_t first, int64_t stride, int n, uint8_t* dst, hipStream_t s);
// the decode plan of n entries into `plan`, units [0, maxU) written (count 0 past the last)
hipError_t launch_plan(eff_engine* e, const int32_t* slots, int n, hipStream_t s, DecodePlan* plan, int maxU);
// The no-allocation decode: plan and SwiGLU staging in a file-scope device array (per device, its
// address taken once at engine creation).  noalloc_setup: for the current device; noalloc_need:
// scratch bytes a call of B tokens needs; launch_ffn_decode_noalloc: as launch_ffn_decode without
// events or engine scratch.
constexpr size_t kNoAllocScratchBytes = 8u << 20;
hipError_t noalloc_setup(int device);
size_t noalloc_need(const eff_engine* e, int B);
hipError_t launch_ffn_decode_noalloc(eff_engine* e, const uint16_t* x, const int32_t* slots, int B, float* y,
                                     hipStream_t s);
hipError_t launch_control(eff_engine* e, int layer, const float* logits, int B, const uint16_t* x,
                          const int32_t* spec_ids, hipStream_t s);
// timing hooks: returns the call's event slot (or -1 when timing is off); mark(i) records event i
// (record_first = false: event 0 is left for the launch itself to set)
int timing_begin(eff_engine* e, int kind, hipStream_t s, bool record_first = true);
void timing_mark(eff_engine* e, int slot, int i, hipStream_t s);
// event i of a timed call (nullptr when the slot is -1): a launcher can hand events 0/1 and 2/3 to
// hipExtLaunchKernelGGL, which sets them at its kernel's start and end (the kernel's own duration)
hipEvent_t timing_event(eff_engine* e, int slot, int i);
bool stream_capturing(hipStream_t s);
hipError_t launch_combine(const float* ygpu, const float* yhost, const int32_t* slots, const float* w,
                          int B, int K, int H, uint16_t* out, hipStream_t s, const uint64_t* done = nullptr,
                          const uint64_t* seq = nullptr, int32_t* err = nullptr);
hipError_t launch_prefill(eff_engine* e, int layer, const uint16_t* x, const int32_t* ids,
                          const float* w, int T, uint16_t* out, const int32_t* slot_of_expert,
                          int slot_base, bool combine, hipStream_t s);
hipError_t split_kernel_setup(int S, int E);
hipError_t decode_kernels_setup(int fmt, int maxB, int H, int I);
int64_t qstar_host(int64_t m, int64_t f);
// host executor
void host_ffn(eff_engine* e, int layer, const uint16_t* x, const int32_t* cpu_ids, int B, float* y);
int host_isa_best();
}  // namespace eff
