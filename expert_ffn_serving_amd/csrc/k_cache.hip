// Slot-cache control kernels: ensure, split (q*), q* batch, prefill installs.
//
// All routing-dependent control flow runs on the device as data, in one
// workgroup per call ([FT-blog] §六: one kernel deduplicates, checks residency,
// computes q, picks victims and rewrites ids to a slot or the host marker;
// [FT-deep] §4 design pattern ② explains why: the miss count exists only on the
// device while the decode step is captured).
#include <algorithm>
#include <cstddef>

#include "eff_internal.h"

namespace eff {
namespace {

constexpr int kThreads = 1024;
constexpr uint64_t kInfKey = ~0ull;
constexpr int kArgminMax = 4;  // victims chosen by block-wide argmin rounds; more by radix select

// q*(m, f): floor of the balance point m*f/65536 or the next integer, whichever
// has the smaller max(F*(65536-f), (m-F)*f) (the lower one on a tie), capped at m
// ([FT-deep] §4 design pattern ②; [FT-blog] §六).  f = 0 fetches nothing.
__device__ __host__ inline int64_t qstar_dev(int64_t m, int64_t f) {
  if (f <= 0 || m <= 0) return 0;
  int64_t lo = (m * f) >> 16;
  int64_t c_lo = max(lo * (65536 - f), (m - lo) * f);
  int64_t c_hi = max((lo + 1) * (65536 - f), (m - lo - 1) * f);
  int64_t best = (c_lo <= c_hi) ? lo : lo + 1;
  return best < m ? best : m;
}

struct CacheState {
  int E, S;
  uint32_t f;
  int32_t* table;
  int32_t* owner;
  int64_t* usage;
  int64_t* recency;
  int64_t* clock;
  Pending* pd;
  FetchList* fl_dev;
  FetchList* fl_host;  // host-mapped mirror (device view)
  int64_t* stats;
  int32_t* err;
  int32_t* host_err;  // host-mapped sticky error bits
  int sort_pow2;
  int spec_budget;  // most records a speculative call fetches (-1: no budget)
  int spec_link;     // records the link carries per layer; a speculative call fetches at most this minus
                    // the latest real call's fetches (-1: no such cap)
};

// Barrier for data exchanged through LDS only: waits for this wave's LDS accesses, not for its
// global stores (those are committed together at the end of a call and need no barrier).
__device__ inline void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One ensure + split call, kept in LDS.  The call reads the slot state from device memory and
// writes every change in one commit at the end.
struct alignas(16) CallLds {
  int32_t id[kMaxEntries];      // expert id of each entry (-1: invalid)
  int32_t hit[kMaxEntries];     // slot the ensure found (resident), else -1
  int32_t slot[kMaxEntries];    // the partition after the split
  int32_t first[kMaxEntries];   // entry is the first with its id
  int32_t uniq[kMaxEntries];    // unique valid ids, ascending
  int32_t miss[kMaxEntries];    // unique missing ids, ascending
  int32_t ranked[kMaxEntries];  // misses by (recency desc, id asc)
  int32_t victim[kMaxEntries];  // victims by (usage, slot)
  int32_t vold[kMaxEntries];    // previous owner of each victim
  int32_t mrank[kMaxEntries];   // rank of each miss (index into miss)
  int32_t hist[256];            // radix select: one digit's histogram
  int64_t mrec[kMaxEntries];    // recency of each miss (then the selected victim keys)
  uint64_t red[kThreads / 64];
  int nvw[kThreads / 64];       // prebuilt victim keys below the floor, per wave
  int64_t s, floor_;
  uint64_t rs_and, rs_or;       // radix select: AND and OR of the candidate keys
  int layer, n, spec, nu, nm, nv, qq, err;
  int rs_bin, rs_rem, rs_n;     // radix select: the chosen digit, the rank left, keys selected
};
// ranked, victim, vold and mrank are written by the split only: until then the ensure uses them
// as one table of up to kEnsureTab experts
constexpr int kEnsureTab = 4 * kMaxEntries;
static_assert(offsetof(CallLds, mrank) == offsetof(CallLds, ranked) + 3 * kMaxEntries * sizeof(int32_t),
              "one contiguous table");
static_assert(kEnsureTab % kThreads == 0, "whole ids per thread");

__device__ inline void stat_add(int64_t* p, int64_t v) {
  atomicAdd(reinterpret_cast<unsigned long long*>(p), (unsigned long long)v);
}

// first[p]: entry p is the first one with its (valid) id.  Entry p = thread p; each sweeps all
// n entries in order, a loop of the same length on every lane whose loads read one LDS word for
// the whole wave (a broadcast) and do not wait for each other.
static_assert(kMaxEntries <= kThreads && kMaxEntries % 32 == 0, "one entry per thread; whole batches");

// f(q, a[q]) (and b[q] for the two-array forms) for q = 0 .. n-1, the same sequence on every lane:
// batches of 16 values read with 4 (8) LDS vector loads issued together, which every lane reads
// at one address (a broadcast), so the loop waits for the LDS once per batch.  a, b: 16-byte
// aligned LDS arrays of kMaxEntries (read past n up to the batch's end, never past the array).
constexpr int kSweepB = 16;
static_assert(kMaxEntries % kSweepB == 0, "whole batches");
template <typename F>
__device__ inline void sweep(const int32_t* a, int n_, F f) {
  const int n = __builtin_amdgcn_readfirstlane(n_);  // uniform: scalar loop bounds
  for (int q0 = 0; q0 < n; q0 += kSweepB) {
    int4 x[kSweepB / 4];
#pragma unroll
    for (int i = 0; i < kSweepB / 4; ++i) x[i] = reinterpret_cast<const int4*>(a + q0)[i];
    if (q0 + kSweepB <= n) {  // a whole batch: no check per value
#pragma unroll
      for (int i = 0; i < kSweepB / 4; ++i) {
        const int q = q0 + 4 * i;
        f(q, x[i].x);
        f(q + 1, x[i].y);
        f(q + 2, x[i].z);
        f(q + 3, x[i].w);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kSweepB / 4; ++i) {
        const int q = q0 + 4 * i;
        if (q < n) f(q, x[i].x);
        if (q + 1 < n) f(q + 1, x[i].y);
        if (q + 2 < n) f(q + 2, x[i].z);
        if (q + 3 < n) f(q + 3, x[i].w);
      }
    }
  }
}
template <typename F>
__device__ inline void sweep2(const int32_t* a, const int32_t* b, int n_, F f) {
  const int n = __builtin_amdgcn_readfirstlane(n_);
  for (int q0 = 0; q0 < n; q0 += kSweepB) {
    int4 x[kSweepB / 4], y[kSweepB / 4];
#pragma unroll
    for (int i = 0; i < kSweepB / 4; ++i) {
      x[i] = reinterpret_cast<const int4*>(a + q0)[i];
      y[i] = reinterpret_cast<const int4*>(b + q0)[i];
    }
    if (q0 + kSweepB <= n) {
#pragma unroll
      for (int i = 0; i < kSweepB / 4; ++i) {
        const int q = q0 + 4 * i;
        f(q, x[i].x, y[i].x);
        f(q + 1, x[i].y, y[i].y);
        f(q + 2, x[i].z, y[i].z);
        f(q + 3, x[i].w, y[i].w);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kSweepB / 4; ++i) {
        const int q = q0 + 4 * i;
        if (q < n) f(q, x[i].x, y[i].x);
        if (q + 1 < n) f(q + 1, x[i].y, y[i].y);
        if (q + 2 < n) f(q + 2, x[i].z, y[i].z);
        if (q + 3 < n) f(q + 3, x[i].w, y[i].w);
      }
    }
  }
}
// f(q, a[q], b[q]) with b 64-bit (a may be null: 0 is passed)
template <typename F>
__device__ inline void sweep_i64(const int32_t* a, const uint64_t* b, int n_, F f) {
  const int n = __builtin_amdgcn_readfirstlane(n_);
  for (int q0 = 0; q0 < n; q0 += kSweepB) {
    int4 x[kSweepB / 4];
    ulonglong2 y[kSweepB / 2];
#pragma unroll
    for (int i = 0; i < kSweepB / 4; ++i) x[i] = a ? reinterpret_cast<const int4*>(a + q0)[i] : make_int4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < kSweepB / 2; ++i) y[i] = reinterpret_cast<const ulonglong2*>(b + q0)[i];
    if (q0 + kSweepB <= n) {
#pragma unroll
      for (int i = 0; i < kSweepB / 4; ++i) {
        const int q = q0 + 4 * i;
        f(q, x[i].x, (uint64_t)y[2 * i].x);
        f(q + 1, x[i].y, (uint64_t)y[2 * i].y);
        f(q + 2, x[i].z, (uint64_t)y[2 * i + 1].x);
        f(q + 3, x[i].w, (uint64_t)y[2 * i + 1].y);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kSweepB / 4; ++i) {
        const int q = q0 + 4 * i;
        if (q < n) f(q, x[i].x, (uint64_t)y[2 * i].x);
        if (q + 1 < n) f(q + 1, x[i].y, (uint64_t)y[2 * i].y);
        if (q + 2 < n) f(q + 2, x[i].z, (uint64_t)y[2 * i + 1].x);
        if (q + 3 < n) f(q + 3, x[i].w, (uint64_t)y[2 * i + 1].y);
      }
    }
  }
}

__device__ inline void mark_first(CallLds& C, int n) {
  const int p = threadIdx.x;
  if ((p & ~63) < n) {  // waves holding entries
    const int id = p < n ? C.id[p] : -1;
    bool dup = false;
    sweep(C.id, n, [&](int q, int o) { dup |= q < p && o == id; });
    if (p < n) C.first[p] = id >= 0 && !dup;
  }
}

// ensure: dedup and residency ([FT-deep] §4 ⑤; [FT-blog] §六).  In: C.id[0..n).  Out, in LDS:
// C.hit, C.first, C.uniq, C.miss, step and floor.  Reads the table; writes nothing to memory.
__device__ __attribute__((always_inline)) void ensure_body(const CacheState& c, int layer, int n, int spec, CallLds& C) {
  const int tid = threadIdx.x, E = c.E;
  if (tid == 0) {
    const int64_t s = c.clock[0] + 1;
    C.s = s;
    C.floor_ = spec ? c.clock[1] : s;
    C.nu = 0;
    C.nm = 0;
    C.layer = layer;
    C.n = n;
    C.spec = spec;
    C.err = 0;
  }
  if (n <= 64) {
    // one wave, lane p = entry p: the table lookup, then one uniform readlane sweep gives each lane
    // the entries with the same id and with smaller ids (registers only; no LDS round trips).
    // Wave 0 also holds tid 0, whose initialisation above it follows in program order.
    if (tid < 64) {
      int v = tid < n ? C.id[tid] : -1;
      const bool bad = tid < n && (v < 0 || v >= E);
      if (bad) v = -1;
      const int hit = (v >= 0) ? c.table[(int64_t)layer * E + v] : -1;
      uint64_t same = 0, less = 0;
      for (int q = 0; q < n; ++q) {
        const int vq = __builtin_amdgcn_readlane(v, q);
        same |= (uint64_t)(vq == v) << q;
        less |= (uint64_t)(vq < v) << q;
      }
      const bool first = v >= 0 && (same & ((1ull << tid) - 1)) == 0;
      const uint64_t fm = __ballot(first), mm = __ballot(first && hit < 0), badm = __ballot(bad);
      if (tid < n) {
        C.id[tid] = v;
        C.hit[tid] = hit;
        C.first[tid] = first;
      }
      if (first) {
        C.uniq[__popcll(less & fm)] = v;
        if (hit < 0) C.miss[__popcll(less & mm)] = v;
      }
      if (tid == 0) {
        C.nu = __popcll(fm);
        C.nm = __popcll(mm);
        C.err = badm ? 1 : 0;
      }
    }
    lds_sync();
    return;
  }
  if (E <= kEnsureTab) {
    // more entries, few experts: entry p = thread p, and a table over the experts.  Each entry's
    // id takes the largest (n - p) of its entries (its first entry) with the missing bit; then
    // one exclusive scan over the experts numbers the distinct and the distinct missing ids.
    int32_t* tab = C.ranked;
    for (int e = tid; e < E; e += kThreads) tab[e] = 0;
    int v = -1, hit = -1;
    if (tid < n) {
      v = C.id[tid];
      if (v < 0 || v >= E) {
        atomicOr(&C.err, 1);
        v = -1;
      }
      hit = (v >= 0) ? c.table[(int64_t)layer * E + v] : -1;
      C.id[tid] = v;
      C.hit[tid] = hit;
    }
    lds_sync();
    if (v >= 0) atomicMax(&tab[v], (n - tid) << 1 | (hit < 0 ? 1 : 0));
    lds_sync();
    if (tid < n) C.first[tid] = v >= 0 && (tab[v] >> 1) == n - tid;
    constexpr int kPer = kEnsureTab / kThreads;  // experts tid*kPer .. +kPer-1 of this thread
    int cnt[kPer], local = 0;  // per expert: present + (missing << 16)
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = tid * kPer + i;
      const int t = e < E ? tab[e] : 0;
      cnt[i] = t ? 1 + ((t & 1) << 16) : 0;
      local += cnt[i];
    }
    const int lane = tid & 63, wave = tid >> 6;
    int incl = local;
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d);
      if (lane >= d) incl += o;
    }
    if (lane == 63) C.hist[wave] = incl;  // the histogram is free until the split
    lds_sync();
    int before = incl - local;
    for (int w = 0; w < wave; ++w) before += C.hist[w];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (cnt[i]) {
        const int e = tid * kPer + i;
        C.uniq[before & 0xFFFF] = e;
        if (cnt[i] >> 16) C.miss[before >> 16] = e;
      }
      before += cnt[i];
    }
    if (tid == kThreads - 1) {
      C.nu = before & 0xFFFF;
      C.nm = before >> 16;
    }
    lds_sync();
    return;
  }
  // more entries: entry p = thread p.  The table lookups, then two sweeps over all entries (as in
  // mark_first): is the entry the first with its id, and how many distinct (missing) ids are
  // smaller.  C.slot holds each first entry's (id, missing) packed until the split overwrites it.
  int v = -1, hit = -1;
  if (tid < n) {
    v = C.id[tid];
    if (v < 0 || v >= E) {
      atomicOr(&C.err, 1);
      v = -1;
    }
    hit = (v >= 0) ? c.table[(int64_t)layer * E + v] : -1;
    C.id[tid] = v;
    C.hit[tid] = hit;
  }
  lds_sync();
  const bool wv = (tid & ~63) < n;  // waves holding entries
  bool first = false;
  if (wv) {
    bool dup = false;
    sweep(C.id, n, [&](int q, int o) { dup |= q < tid && o == v; });
    first = tid < n && v >= 0 && !dup;
    if (tid < n) {
      C.first[tid] = first;
      C.slot[tid] = first ? (v << 1 | (hit < 0 ? 1 : 0)) : -1;
    }
  }
  lds_sync();
  if (wv) {
    int ru = 0, rm = 0;
    sweep(C.slot, n, [&](int, int pk) {
      const bool lt = pk >= 0 && (pk >> 1) < v;
      ru += lt;
      rm += lt && (pk & 1);
    });
    if (first) {
      C.uniq[ru] = v;
      if (hit < 0) C.miss[rm] = v;
    }
  }
  const uint64_t fm = __ballot(first), mm = __ballot(first && hit < 0);
  if ((tid & 63) == 0 && fm) {
    atomicAdd(&C.nu, __popcll(fm));
    if (mm) atomicAdd(&C.nm, __popcll(mm));
  }
  lds_sync();
}

// Block-wide min of a 64-bit key; every thread gets the result.
// Minimum over the wave of a 64-bit value, with DPP moves of both halves (no LDS round trips);
// lanes outside a DPP source row see the identity (all ones).
__device__ inline uint64_t wave_min_u64(uint64_t v) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
#define EFF_DPP_MIN64(ctrl, rmask)                                                                      \
  {                                                                                                     \
    const uint32_t ol = (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)lo, ctrl, rmask, 0xF, false);    \
    const uint32_t oh = (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)hi, ctrl, rmask, 0xF, false);    \
    const bool lt = oh < hi || (oh == hi && ol < lo);                                                   \
    lo = lt ? ol : lo;                                                                                  \
    hi = lt ? oh : hi;                                                                                  \
  }
  EFF_DPP_MIN64(0xB1, 0xF)   // quad_perm [1,0,3,2]
  EFF_DPP_MIN64(0x4E, 0xF)   // quad_perm [2,3,0,1]
  EFF_DPP_MIN64(0x124, 0xF)  // row_ror:4
  EFF_DPP_MIN64(0x128, 0xF)  // row_ror:8
  EFF_DPP_MIN64(0x142, 0xA)  // row_bcast:15 into rows 1, 3
  EFF_DPP_MIN64(0x143, 0xC)  // row_bcast:31 into rows 2, 3
#undef EFF_DPP_MIN64
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, 63) << 32) |
         (uint32_t)__builtin_amdgcn_readlane((int)lo, 63);
}

__device__ inline uint64_t block_min_u64(uint64_t v, uint64_t* s_red) {
  v = wave_min_u64(v);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) s_red[wave] = v;
  lds_sync();
  uint64_t r = s_red[0];
  for (int i = 1; i < kThreads / 64; ++i) r = s_red[i] < r ? s_red[i] : r;
  lds_sync();
  return r;
}

// The victim key of every slot for a real call, from the usage before the call (the split reads it
// only when it fetches, but the keys cost nothing on the critical path when waves that would
// otherwise wait build them at the start): ((usage + 1) << 14 | slot) below floor = clock + 1, else
// kInfKey.  Threads [kKeyT0, kThreads); C.nvw[w] = keys below the floor built by wave w.
constexpr int kKeyT0 = 320;  // waves 1-4 copy x for the host meanwhile
__device__ void prebuild_keys(const CacheState& c, CallLds& C, uint64_t* s_key) {
  constexpr int kNt = kThreads - kKeyT0, kPer = (kMaxSlots + kNt - 1) / kNt;
  const int t = threadIdx.x - kKeyT0, S = c.S;
  const int64_t floor_ = c.clock[0] + 1;
  int64_t us[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int v = t + i * kNt;
    us[i] = v < S ? c.usage[v] : 0;
  }
  int wave_nv = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int v = t + i * kNt;
    const bool below = v < S && us[i] < floor_;
    if (v < c.sort_pow2) s_key[v] = below ? (((uint64_t)(us[i] + 1) << 14) | (uint64_t)v) : kInfKey;
    wave_nv += __popcll(__ballot(below));
  }
  if ((threadIdx.x & 63) == 0) C.nvw[threadIdx.x >> 6] = wave_nv;
}

// split: q*, recency ranking, LRU victims and the -1 partition, computed in LDS (C.victim,
// C.ranked, C.vold, C.qq, C.slot).  Reads recency, usage and owner; writes nothing to memory.
// The call's hit slots are never victims (their stamp of this step is committed later).
// s_key: sort_pow2 uint64 of LDS.
// keys_ready: s_key and C.nvw were prebuilt (prebuild_keys) from the usage this call sees.
// real_q: the latest real call's fetch count when the caller has it (the fused control kernel, whose
// real split precedes its speculative one), else -1: read from clock[2].
__device__ __attribute__((always_inline)) void split_body(const CacheState& c, CallLds& C, uint64_t* s_key, bool keys_ready = false,
                           int real_q = -1) {
  const int tid = threadIdx.x;
  const int E = c.E, S = c.S;
  const int n = C.n, m = C.nm;
  const int64_t floor_ = C.floor_;
  const int64_t base = (int64_t)C.layer * E;
  int q = (int)qstar_dev(m, c.f);
  if (C.spec && c.spec_budget >= 0) q = min(q, c.spec_budget);  // q' = min(q*, victims, budget, gap)
  if (C.spec && c.spec_link >= 0) q = min(q, max(0, c.spec_link - (real_q >= 0 ? real_q : (int)c.clock[2])));
  int qq = 0;
  if (q > 0) {
    if (tid == 0) {
      int nv = 0;
      if (keys_ready)
        for (int w = kKeyT0 / 64; w < kThreads / 64; ++w) nv += C.nvw[w];
      C.nv = nv;
      C.rs_and = ~0ull;
      C.rs_or = 0;
      C.rs_n = 0;
      C.rs_bin = 0;
      C.rs_rem = 1;
    }
    lds_sync();
    // the misses' recency and the victim keys: every load is issued before any is used (a loop that
    // consumed each load in turn would pay one global round trip per slot a thread owns)
    static_assert(kMaxEntries <= kThreads && kMaxSlots % kThreads == 0, "one miss per thread, whole rounds");
    constexpr int kPer = kMaxSlots / kThreads;
    const int64_t mr = tid < m ? c.recency[base + C.miss[tid]] : 0;
    if (!keys_ready) {
      int64_t us[kPer];
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int v = tid + i * kThreads;
        us[i] = v < S ? c.usage[v] : 0;
      }
      int wave_nv = 0;  // counted per wave with ballots: one LDS atomic per wave, not per thread
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int v = tid + i * kThreads;
        const bool below = v < S && us[i] < floor_;  // slots with usage below the floor, by (usage, slot)
        if (v < c.sort_pow2) s_key[v] = below ? (((uint64_t)(us[i] + 1) << 14) | (uint64_t)v) : kInfKey;
        wave_nv += __popcll(__ballot(below));
      }
      if ((tid & 63) == 0 && wave_nv) atomicAdd(&C.nv, wave_nv);
    }
    if (tid < m) C.mrec[tid] = mr;
    lds_sync();
    for (int p = tid; p < n; p += kThreads) {
      const int v = C.hit[p];
      if (C.first[p] && v >= 0 && v < S && s_key[v] != kInfKey) {
        s_key[v] = kInfKey;
        atomicSub(&C.nv, 1);
      }
    }
    // Misses ranked by (recency desc, id asc) ([FT-deep] §4 ⑤: prefer recently active experts).
    if ((tid & ~63) < m) {  // waves holding misses (one per thread)
      const int e = tid < m ? C.miss[tid] : 0;
      const int64_t r = tid < m ? C.mrec[tid] : 0;
      int rank = 0;
      sweep_i64(C.miss, reinterpret_cast<const uint64_t*>(C.mrec), m, [&](int, int o, uint64_t u) {
        const int64_t ro = (int64_t)u;
        rank += (ro > r) || (ro == r && o < e);
      });
      if (tid < m) {
        C.ranked[rank] = e;
        C.mrank[tid] = rank;
      }
    }
    lds_sync();
    qq = min(q, C.nv);
    if (qq > 0 && qq <= kArgminMax) {
      // few fetches: qq rounds of block-wide argmin
      for (int i = 0; i < qq; ++i) {
        uint64_t lm = kInfKey;
        for (int v = tid; v < S; v += kThreads) lm = s_key[v] < lm ? s_key[v] : lm;
        const uint64_t g = block_min_u64(lm, C.red);
        const int v = (int)(g & 0x3FFF);
        if (tid == 0) {
          C.victim[i] = v;
          s_key[v] = kInfKey;
        }
        lds_sync();
      }
    } else if (qq > kArgminMax) {
      // more fetches: radix select of the qq smallest keys (distinct: the slot is in the low bits),
      // 8 bits a pass from the highest bit in which the candidates differ, then their ranks
      uint64_t kand = ~0ull, kor = 0;
      for (int v = tid; v < S; v += kThreads) {
        const uint64_t k = s_key[v];
        if (k != kInfKey) {
          kand &= k;
          kor |= k;
        }
      }
      for (int d = 32; d >= 1; d >>= 1) {
        kand &= __shfl_xor(kand, d);
        kor |= __shfl_xor(kor, d);
      }
      if ((tid & 63) == 0) {
        atomicAnd(&C.rs_and, kand);
        atomicOr(&C.rs_or, kor);
      }
      lds_sync();
      const uint64_t diff = C.rs_and ^ C.rs_or;
      int shift = diff ? ((63 - __builtin_clzll(diff)) & ~7) : 0;
      uint64_t prefix = C.rs_and & (shift >= 56 ? 0ull : ~0ull << (shift + 8));  // bits every candidate shares
      int rem = qq;  // the rem-th smallest key among those that match prefix above the digit
      for (;;) {
        const uint64_t hm = shift >= 56 ? 0ull : ~0ull << (shift + 8);
        if (tid < 256) C.hist[tid] = 0;
        lds_sync();
        for (int v = tid; v < S; v += kThreads) {
          const uint64_t k = s_key[v];
          if (k != kInfKey && (k & hm) == prefix) atomicAdd(&C.hist[(k >> shift) & 255], 1);
        }
        lds_sync();
        if (tid < 64) {  // lane l: bins 4l..4l+3; the bin where the running count reaches rem
          const int h0 = C.hist[4 * tid], h1 = C.hist[4 * tid + 1], h2 = C.hist[4 * tid + 2], h3 = C.hist[4 * tid + 3];
          const int sum = h0 + h1 + h2 + h3;
          int incl = sum;
          for (int d = 1; d < 64; d <<= 1) {
            const int o = __shfl_up(incl, d);
            if (tid >= d) incl += o;
          }
          int acc = incl - sum;
          if (acc < rem && rem <= incl) {
            int b = 0;
            if (rem > acc + h0) {
              acc += h0;
              b = 1;
              if (rem > acc + h1) {
                acc += h1;
                b = 2;
                if (rem > acc + h2) {
                  acc += h2;
                  b = 3;
                }
              }
            }
            C.rs_bin = 4 * tid + b;
            C.rs_rem = rem - acc;
          }
        }
        lds_sync();
        prefix |= (uint64_t)C.rs_bin << shift;
        rem = C.rs_rem;
        if (shift == 0) break;
        shift -= 8;
      }
      // prefix is now the qq-th smallest key: the keys up to it, unordered, then each one's rank
      uint64_t* sel = reinterpret_cast<uint64_t*>(C.mrec);  // the misses' recency is used up
      for (int v = tid; v < S; v += kThreads) {
        const uint64_t k = s_key[v];
        if (k <= prefix) {
          const int i = atomicAdd(&C.rs_n, 1);
          if (i < kMaxEntries) sel[i] = k;
        }
      }
      lds_sync();
      if (C.rs_n != qq) {  // the keys disagree with the count of candidates: never seen; fetch fewer
        if (tid == 0) atomicOr(&C.err, 16);
        qq = min(qq, C.rs_n);
      }
      if ((tid & ~63) < qq) {
        const uint64_t k = tid < qq ? sel[tid] : 0;
        int r = 0;
        sweep_i64(nullptr, sel, qq, [&](int, int, uint64_t o) { r += o < k; });
        if (tid < qq) C.victim[r] = (int)(k & 0x3FFF);
      }
      lds_sync();
    }
    for (int i = tid; i < qq; i += kThreads) C.vold[i] = c.owner[C.victim[i]];
  }
  // The -1 partition ([FT-deep] §4 ③): i-th ranked miss -> i-th victim; hits keep their slot.  A
  // missing entry finds its id in the ascending miss list, then that miss's rank.
  for (int p = tid; p < n; p += kThreads) {
    const int id = C.id[p];
    int slot = C.hit[p];
    if (slot < 0 && id >= 0 && qq > 0) {
      int lo = 0, hi = m - 1;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (C.miss[mid] < id) lo = mid + 1;
        else hi = mid;
      }
      const int r = C.mrank[lo];
      if (r < qq) slot = C.victim[r];
    }
    C.slot[p] = slot;
  }
  if (tid == 0) C.qq = qq;
  lds_sync();
}

// Commit a call: hit stamps (when stamp_hits), installs, the fetch list, outputs, recency,
// clocks, counts and stats.  Host-mapped outputs (cpu_host, the fetch list mirror) are written
// by wave 0 only, so that one wave's system fence publishes them.  All arrays may be null.
__device__ __attribute__((always_inline)) void commit_body(const CacheState& c, const CallLds& C, bool stamp_hits, int32_t* __restrict__ slots_out,
                            int32_t* __restrict__ cpu_out, int32_t* __restrict__ cpu_host,
                            int32_t* __restrict__ counts) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = C.n, spec = C.spec, m = C.nm, nu = C.nu, qq = C.qq;
  const int64_t s = C.s, base = (int64_t)C.layer * c.E;
  // a speculative request for layer l fills list 1 + l % 2: consecutive requests never share a list,
  // whichever kernel carries their copies
  const int li = spec ? spec_fetch_list(C.layer) : 0;
  FetchList* fl = c.fl_dev + li;
  FetchList* flh = c.fl_host + li;
  if (stamp_hits)
    for (int p = tid; p < n; p += kThreads)
      if (C.first[p] && C.hit[p] >= 0) c.usage[C.hit[p]] = s;  // hit: stamped as used now
  for (int i = tid; i < qq; i += kThreads) {
    const int v = C.victim[i], e = C.ranked[i], old = C.vold[i];
    if (old >= 0) c.table[old] = -1;
    c.owner[v] = (int32_t)(base + e);
    c.table[base + e] = v;
    c.usage[v] = s;
    fl->flat[i] = (int32_t)(base + e);
    fl->slot[i] = v;
  }
  for (int p = tid; p < n; p += kThreads) {
    const int slot = C.slot[p], id = C.id[p];
    if (slots_out) slots_out[p] = slot;
    if (cpu_out) cpu_out[p] = (!spec && slot < 0 && id >= 0) ? id : -1;
  }
  if (!spec)
    for (int u = tid; u < nu; u += kThreads) c.recency[base + C.uniq[u]] = s;
  if (wave == 0) {
    for (int i = lane; i < qq; i += 64) {
      flh->flat[i] = (int32_t)(base + C.ranked[i]);
      flh->slot[i] = C.victim[i];
    }
    if (cpu_host)
      for (int p = lane; p < n; p += 64) {
        const int slot = C.slot[p], id = C.id[p];
        cpu_host[p] = (!spec && slot < 0 && id >= 0) ? id : -1;
      }
  }
  if (tid == 0) {
    c.clock[0] = s;
    if (!spec) {
      c.clock[1] = s;
      c.clock[2] = qq;  // the real call's fetches (speculative link cap)
    }
    if (counts) {
      counts[0] = m;
      counts[1] = qq;
      counts[2] = spec ? 0 : m - qq;
    }
    const int err = C.err | atomicExch(c.err, 0);
    if (err) __hip_atomic_fetch_or(c.host_err, err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    fl->count = qq;
    flh->count = qq;
    fl->err = err;
    flh->err = err;
    c.pd->valid = 0;
    stat_add(&c.stats[ST_CALLS], 1);
    if (spec) {
      stat_add(&c.stats[ST_SPEC_FETCHED], qq);
    } else {
      stat_add(&c.stats[ST_HITS], nu - m);
      stat_add(&c.stats[ST_FETCHED], qq);
      stat_add(&c.stats[ST_HOST], m - qq);
      stat_add(&c.stats[ST_HIST0 + (qq < 16 ? qq : 16)], 1);
    }
  }
}

// The call, kept in device memory between a separate ensure and split.
__device__ void store_pending(const CacheState& c, const CallLds& C) {
  const int tid = threadIdx.x;
  Pending* pd = c.pd;
  for (int p = tid; p < C.n; p += kThreads) {
    pd->ids[p] = C.id[p];
    pd->slot[p] = C.hit[p];
  }
  for (int u = tid; u < C.nu; u += kThreads) pd->uniq[u] = C.uniq[u];
  for (int u = tid; u < C.nm; u += kThreads) pd->miss[u] = C.miss[u];
  if (tid == 0) {
    pd->valid = 1;
    pd->layer = C.layer;
    pd->n = C.n;
    pd->spec = C.spec;
    pd->s = C.s;
    pd->floor_ = C.floor_;
    pd->nuniq = C.nu;
    pd->nmiss = C.nm;
    if (C.err) atomicOr(c.err, C.err);
  }
}

// Returns false (and flags the error) when no ensure is pending.
__device__ bool load_pending(const CacheState& c, CallLds& C) {
  const int tid = threadIdx.x;
  const Pending* pd = c.pd;
  __shared__ int s_ok;
  if (tid == 0) {
    s_ok = pd->valid;
    C.layer = pd->layer;
    C.n = pd->n;
    C.spec = pd->spec;
    C.s = pd->s;
    C.floor_ = pd->floor_;
    C.nu = pd->nuniq;
    C.nm = pd->nmiss;
    C.err = 0;
  }
  lds_sync();
  if (!s_ok) {
    if (tid == 0) atomicOr(c.err, 2);
    return false;
  }
  for (int p = tid; p < C.n; p += kThreads) {
    C.id[p] = pd->ids[p];
    C.hit[p] = pd->slot[p];
  }
  for (int u = tid; u < C.nu; u += kThreads) C.uniq[u] = pd->uniq[u];
  for (int u = tid; u < C.nm; u += kThreads) C.miss[u] = pd->miss[u];
  lds_sync();
  mark_first(C, C.n);
  lds_sync();
  return true;
}

// Whole-wave reductions on DPP row operations (no LDS crossbar): the result is read from lane 63
// and is the same on every lane.  Lanes outside a DPP source row contribute the identity.
template <bool MAX>
__device__ inline uint32_t wave_reduce_u32(uint32_t v) {
  constexpr int kId = MAX ? 0 : -1;
#define EFF_DPP_STEP(ctrl, rmask)                                                              \
  {                                                                                            \
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(kId, (int)v, ctrl, rmask, 0xF, false); \
    v = MAX ? (o > v ? o : v) : (o < v ? o : v);                                               \
  }
  EFF_DPP_STEP(0xB1, 0xF)   // quad_perm [1,0,3,2]
  EFF_DPP_STEP(0x4E, 0xF)   // quad_perm [2,3,0,1]
  EFF_DPP_STEP(0x124, 0xF)  // row_ror:4
  EFF_DPP_STEP(0x128, 0xF)  // row_ror:8  (every lane of a row holds the row's result)
  EFF_DPP_STEP(0x142, 0xA)  // row_bcast:15 into rows 1, 3
  EFF_DPP_STEP(0x143, 0xC)  // row_bcast:31 into rows 2, 3
#undef EFF_DPP_STEP
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ inline float wave_sum_f32(float v) {
#define EFF_DPP_ADD(ctrl, rmask) \
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, rmask, 0xF, false));
  EFF_DPP_ADD(0xB1, 0xF)
  EFF_DPP_ADD(0x4E, 0xF)
  EFF_DPP_ADD(0x124, 0xF)
  EFF_DPP_ADD(0x128, 0xF)
  EFF_DPP_ADD(0x142, 0xA)
  EFF_DPP_ADD(0x143, 0xC)
#undef EFF_DPP_ADD
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Order-preserving key of a float (larger value -> larger key; -0 is taken as +0).
__device__ inline uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// top-K of one logits row by (logit desc, id asc) and the softmax of the K selected, by one
// wave.  Lane l holds experts l, l+64, ... (E <= 64*NJ) as order keys in registers; each of the
// K rounds takes the wave's largest key, then the lowest id holding it.  NJ = 0: E up to 4096,
// the row is re-read from memory in each round.  lds_ids (may be null) receives the ids too.
// Logits must not be NaN.
template <int NJ>
__device__ void wave_topk(const float* __restrict__ row, int E, int K, int32_t* __restrict__ ids,
                          float* __restrict__ w, int32_t* lds_ids) {
  const int lane = threadIdx.x & 63;
  uint32_t key[NJ > 0 ? NJ : 1];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    key[j] = e < E ? order_key(row[e]) : 0u;
  }
  uint64_t taken = 0;  // element lane + 64*j is taken when bit j is set
  float mysel = 0.f;   // lane k keeps the k-th selected logit
  int myid = 0;
  for (int k = 0; k < K; ++k) {
    uint32_t best = 0u;
    int bj = -1;
    if (NJ > 0) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const bool ok = !((taken >> j) & 1) && key[j] > best;
        best = ok ? key[j] : best;
        bj = ok ? j : bj;
      }
    } else {
      int j = 0;
      for (int e = lane; e < E; e += 64, ++j) {
        const uint32_t kj = order_key(row[e]);
        const bool ok = !((taken >> j) & 1) && kj > best;
        best = ok ? kj : best;
        bj = ok ? j : bj;
      }
    }
    const uint32_t m = wave_reduce_u32<true>(best);
    const uint32_t cand = (bj >= 0 && best == m) ? (uint32_t)(bj * 64 + lane) : 0xFFFFFFFFu;
    const int id = (int)wave_reduce_u32<false>(cand);
    if ((id & 63) == lane) taken |= 1ull << (id >> 6);
    if (lane == k) {
      mysel = key_value(m);
      myid = id;
    }
  }
  // softmax over the K selected logits, relative to the largest (lane 0's)
  const float top = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mysel), 0));
  const float ex = lane < K ? expf(mysel - top) : 0.f;
  const float sum = wave_sum_f32(ex);
  if (lane < K) {
    ids[lane] = myid;
    w[lane] = ex / sum;
    if (lds_ids) lds_ids[lane] = myid;
  }
}

// The same selection with each lane's keys sorted once, by (key desc, element asc): a lane's
// candidate is then the head of its list.  A round is one wave max over the heads; when a single
// lane holds that key (the common case) it is the winner, since a lane's later keys are no larger
// and its elements are in id order.  Equal keys in several lanes fall back to the lowest id among
// them.  The winner shifts its list.
template <int NJ>
__device__ void wave_topk_sorted(const float* __restrict__ row, int E, int K, int32_t* __restrict__ ids,
                                 float* __restrict__ w, int32_t* lds_ids) {
  const int lane = threadIdx.x & 63;
  uint32_t key[NJ];
  int el[NJ];  // element id lane + 64*j of each key
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int e = lane + 64 * j;
    key[j] = e < E ? order_key(row[e]) : 0u;
    el[j] = e;
  }
  // insertion sort, descending; a strict comparison keeps equal keys in element order
#pragma unroll
  for (int i = 1; i < NJ; ++i)
#pragma unroll
    for (int j = i; j > 0; --j) {
      const bool sw = key[j] > key[j - 1];
      const uint32_t ka = key[j - 1], kb = key[j];
      const int ea = el[j - 1], eb = el[j];
      key[j - 1] = sw ? kb : ka;
      key[j] = sw ? ka : kb;
      el[j - 1] = sw ? eb : ea;
      el[j] = sw ? ea : eb;
    }
  float mysel = 0.f;  // lane k keeps the k-th selected logit
  int myid = 0;
  for (int k = 0; k < K; ++k) {
    const uint32_t m = wave_reduce_u32<true>(key[0]);
    const uint64_t hold = __ballot(key[0] == m);
    int win;
    if (__popcll(hold) == 1) {
      win = __builtin_ctzll(hold);
    } else {
      const uint32_t cand = key[0] == m ? (uint32_t)el[0] : 0xFFFFFFFFu;
      win = (int)(wave_reduce_u32<false>(cand) & 63);
    }
    const int id = __builtin_amdgcn_readlane(el[0], win);
    if (lane == win) {
#pragma unroll
      for (int j = 0; j + 1 < NJ; ++j) {
        key[j] = key[j + 1];
        el[j] = el[j + 1];
      }
      key[NJ - 1] = 0u;
    }
    if (lane == k) {
      mysel = key_value(m);
      myid = id;
    }
  }
  // softmax over the K selected logits, relative to the largest (lane 0's)
  const float top = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mysel), 0));
  const float ex = lane < K ? expf(mysel - top) : 0.f;
  const float sum = wave_sum_f32(ex);
  if (lane < K) {
    ids[lane] = myid;
    w[lane] = ex / sum;
    if (lds_ids) lds_ids[lane] = myid;
  }
}

__device__ inline void topk_row(const float* row, int E, int K, int32_t* ids, float* w, int32_t* lds_ids) {
  if (E <= 256) wave_topk_sorted<4>(row, E, K, ids, w, lds_ids);
  else if (E <= 512) wave_topk_sorted<8>(row, E, K, ids, w, lds_ids);
  else if (E <= 1024) wave_topk_sorted<16>(row, E, K, ids, w, lds_ids);
  else wave_topk<0>(row, E, K, ids, w, lds_ids);
}

// Decode plan (distinct GPU slots and their entries) by one workgroup, from the entries' slots
// in LDS.  flat id of a unit: base + lds_id[p] when ids are known, else owner[slot].  lds_hit
// (may be null): the slot the ensure found; a unit whose slot was installed by this call
// (hit < 0) is marked fetch.  scratch: 3*kMaxEntries int32 of LDS (16-byte aligned).
// The decode plan of a call of at most 64 entries, by wave 0 alone (no barrier): each lane
// learns which lanes share its slot and which hold a smaller slot from one uniform readlane sweep
// (registers only; no LDS round trips).  Call with tid < 64.
__device__ __attribute__((always_inline)) void plan_wave0(const int32_t* lds_slot, const int32_t* lds_id, const int32_t* lds_hit, int64_t base,
                           const int32_t* __restrict__ owner, int n, int S, int maxU, int maxB, DecodePlan* plan) {
  const int tid = threadIdx.x;
  int v = -1;
  if (tid < n) {
    const int sl = lds_slot[tid];
    v = (sl >= 0 && sl < S) ? sl : -1;  // slots outside the arena are never read
  }
  uint64_t same = 0, less = 0;
  for (int q = 0; q < n; ++q) {
    const int vq = __builtin_amdgcn_readlane(v, q);
    same |= (uint64_t)(vq == v) << q;
    less |= (uint64_t)(vq < v) << q;
  }
  const bool first = v >= 0 && (same & ((1ull << tid) - 1)) == 0;
  const uint64_t fm = __ballot(first);
  // units by descending token count, then ascending slot: the workgroups of the busiest experts
  // start first and the short ones fill in behind them (one entry each: ascending slot)
  const int c = min(__popcll(same), maxB);
  uint64_t before = less;
  if (__ballot(first && c > 1)) {
    before = 0;
    for (int q = 0; q < n; ++q) {
      const int vq = __builtin_amdgcn_readlane(v, q), cq = __builtin_amdgcn_readlane(c, q);
      before |= (uint64_t)(cq > c || (cq == c && vq < v)) << q;
    }
  }
  const int rank = __popcll(before & fm);
  const int nu = min(__popcll(fm), maxU);
  if (first && rank < maxU) {  // more distinct slots than a layer has experts: not computed
    DecodeUnit& un = plan->unit[rank];
    int cnt = 0;
    for (uint64_t m = same; m && cnt < maxB; m &= m - 1)  // a slot appears at most once per token
      un.entry[cnt++] = __builtin_ctzll(m);
    un.slot = v;
    un.count = cnt;
    un.flat = lds_id ? (int32_t)(base + lds_id[tid]) : owner[v];
    un.fetch = (lds_hit && lds_hit[tid] < 0) ? 1 : 0;
  }
  for (int u = nu + tid; u < maxU; u += 64) {
    plan->unit[u].count = 0;
    plan->unit[u].slot = 0;
    plan->unit[u].flat = 0;
    plan->unit[u].fetch = 0;
  }
  if (tid == 0) plan->nu = nu;
}

__device__ __attribute__((always_inline)) void plan_body(const int32_t* lds_slot, const int32_t* lds_id, const int32_t* lds_hit, int64_t base,
                          const int32_t* __restrict__ owner, int n, int S, int maxU, int maxB, DecodePlan* plan,
                          int32_t* scratch) {
  const int tid = threadIdx.x;
  if (n <= 64) {
    if (tid < 64) plan_wave0(lds_slot, lds_id, lds_hit, base, owner, n, S, maxU, maxB, plan);
    lds_sync();
    return;
  }
  // more entries: entry p = thread p.  One sweep over all entries (as in mark_first) gives each
  // entry its slot's first entry, its place among the slot's entries and the slot's entry count; a
  // second ranks the units; then every entry writes itself into its unit.
  int32_t* s_sl = scratch;
  int32_t* s_first = scratch + kMaxEntries;     // at a slot's first entry: its count (<= maxB), else 0
  int32_t* s_rank = scratch + 2 * kMaxEntries;  // at a slot's first entry: its unit, or maxU
  __shared__ int s_nu;
  if (tid == 0) s_nu = 0;
  int v = -1;
  if (tid < n) {
    const int sl = lds_slot[tid];
    v = (sl >= 0 && sl < S) ? sl : -1;  // slots outside the arena are never read
    s_sl[tid] = v;
  }
  lds_sync();
  const bool wv = (tid & ~63) < n;  // waves holding entries
  int c = 0, pos = 0, fq = 0;
  if (wv) {
    int cnt = 0;
    fq = kMaxEntries;
    sweep(s_sl, n, [&](int q, int o) {
      const bool same = o == v;
      cnt += same;
      pos += same && q < tid;
      fq = same && fq == kMaxEntries ? q : fq;
    });
    if (tid < n && v >= 0 && pos == 0) c = min(cnt, maxB);
  }
  if (tid < n) s_first[tid] = c;
  lds_sync();
  int rank = maxU;
  if (wv) {
    // units by descending token count, then ascending slot (as in plan_wave0)
    int rk = 0;
    sweep2(s_first, s_sl, n, [&](int, int cq, int sq) { rk += cq > c || (cq == c && sq < v); });
    if (c > 0) rank = min(rk, maxU);  // more distinct slots than a layer has experts: not computed
  }
  if (tid < n) s_rank[tid] = rank;
  lds_sync();
  if (tid < n && v >= 0 && pos < maxB) {  // a slot appears at most once per token
    const int r = s_rank[fq];
    if (r < maxU) plan->unit[r].entry[pos] = tid;
  }
  if (rank < maxU) {
    DecodeUnit& un = plan->unit[rank];
    un.slot = v;
    un.count = c;
    un.flat = lds_id ? (int32_t)(base + lds_id[tid]) : owner[v];
    un.fetch = (lds_hit && lds_hit[tid] < 0) ? 1 : 0;
  }
  const uint64_t um = __ballot(rank < maxU);
  if ((tid & 63) == 0 && um) atomicAdd(&s_nu, __popcll(um));
  lds_sync();
  const int nu = min(s_nu, maxU);
  for (int u = nu + tid; u < maxU; u += blockDim.x) {
    plan->unit[u].count = 0;
    plan->unit[u].slot = 0;
    plan->unit[u].flat = 0;
    plan->unit[u].fetch = 0;
  }
  if (tid == 0) plan->nu = nu;
  lds_sync();
}

__global__ void __launch_bounds__(kThreads)
k_ensure(CacheState c, int layer, int32_t* __restrict__ ids, int n, int spec) {
  __shared__ CallLds C;
  for (int p = threadIdx.x; p < n; p += kThreads) C.id[p] = ids[p];
  lds_sync();
  ensure_body(c, layer, n, spec, C);
  for (int p = threadIdx.x; p < n; p += kThreads) {
    ids[p] = C.hit[p];
    if (C.first[p] && C.hit[p] >= 0) c.usage[C.hit[p]] = C.s;  // hit: stamped as used now
  }
  if (threadIdx.x == 0) c.clock[0] = C.s;
  store_pending(c, C);
}

__global__ void __launch_bounds__(kThreads)
k_split(CacheState c, int32_t* __restrict__ ids_out, int32_t* __restrict__ cpu_out, int32_t* __restrict__ counts) {
  extern __shared__ __attribute__((aligned(16))) uint64_t s_key[];
  __shared__ CallLds C;
  if (!load_pending(c, C)) return;
  split_body(c, C, s_key);
  commit_body(c, C, false, ids_out, cpu_out, nullptr, counts);
}

__global__ void __launch_bounds__(kThreads)
k_topk(const float* __restrict__ logits, int B, int E, int K, int32_t* __restrict__ ids, float* __restrict__ w) {
  const int wave = threadIdx.x >> 6;
  for (int t = blockIdx.x * (kThreads / 64) + wave; t < B; t += gridDim.x * (kThreads / 64))
    topk_row(logits + (int64_t)t * E, E, K, ids + (int64_t)t * K, w + (int64_t)t * K, nullptr);
}

__global__ void __launch_bounds__(kThreads)
k_plan(const int32_t* __restrict__ slots, int n, int S, int maxU, int maxB, const int32_t* __restrict__ owner,
       DecodePlan* plan) {
  __shared__ int32_t s_slot[kMaxEntries];
  __shared__ __attribute__((aligned(16))) int32_t scratch[3 * kMaxEntries];
  for (int p = threadIdx.x; p < n; p += kThreads) s_slot[p] = slots[p];
  lds_sync();
  plan_body(s_slot, nullptr, nullptr, 0, owner, n, S, maxU, maxB, plan, scratch);
}

// One decode layer's control path in one workgroup: top-K of the B logits rows, ensure, split,
// the decode plan (units installed by this call are fetched by the FFN kernels), the commit,
// (speculative ensure + split + commit for the next layer), and the host's inputs (host ids, x)
// in host-mapped memory.  Last, wave 0 fences at system scope, numbers the call (seq = ++*seq_ctr,
// device memory) and publishes its word (seq, layer, B, host entries) at call_ring[seq % kCallRing];
// a call with no host entries also sets *host_done = seq itself (nothing for the host to add).
// Wave 0, last: the call word after a system-scope fence (which covers wave 0's host ids and x,
// whose stores waves 1-4 completed before a barrier that wave 0 passed since).
__device__ inline void publish_call(uint64_t* call_ring, uint64_t* host_done, uint64_t* seq_ctr, int layer, int B,
                                    int nhost) {
  if (!call_ring) return;
  __threadfence_system();
  if (threadIdx.x == 0) {
    // this call's number, then the word; relaxed stores after the release fence (a release store
    // would write back the L2 again)
    const uint64_t seq = *seq_ctr + 1;
    *seq_ctr = seq;
    const uint64_t word = ((seq & 0xFFFFFFFFull) << 32) | ((uint64_t)layer << kCallLayerShift) |
                          ((uint64_t)(B - 1) << kCallBShift) | (uint64_t)nhost;
    __hip_atomic_store(call_ring + seq % kCallRing, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    if (nhost == 0) __hip_atomic_store(host_done, seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

__global__ void __launch_bounds__(kThreads)
k_control(CacheState c, const float* __restrict__ logits, int B, int K, int layer, int32_t* __restrict__ ids,
          float* __restrict__ w, int32_t* __restrict__ slots, int32_t* __restrict__ cpu, int32_t* __restrict__ counts,
          const int32_t* __restrict__ spec_ids, int32_t* __restrict__ spec_slots, int32_t* __restrict__ cpu_host,
          const uint16_t* __restrict__ x, uint16_t* __restrict__ x_host, int H, int maxU, int maxB,
          DecodePlan* plan, uint64_t* call_ring, uint64_t* host_done, uint64_t* seq_ctr) {
  extern __shared__ __attribute__((aligned(16))) uint64_t s_key[];  // victim keys, plan scratch (16-byte aligned)
  __shared__ CallLds C;
  const int tid = threadIdx.x;
  const int n = B * K;
  if (tid >= kKeyT0) prebuild_keys(c, C, s_key);  // waves 5.., before their top-K rows
  for (int t = tid >> 6; t < B; t += kThreads / 64)
    topk_row(logits + (int64_t)t * c.E, c.E, K, ids + (int64_t)t * K, w + (int64_t)t * K, C.id + t * K);
  if (tid >= 64 && tid < kKeyT0) {
    // waves 1-4 copy x for the host after their top-K rows (whose loads would otherwise wait for
    // these stores).  They wait for the stores to complete only after the split (below), before
    // the plan's barrier; wave 0's system-scope fence before the call word then publishes them
    // together with its own stores.  A completed store to coherent host memory is not yet visible
    // to the host without that fence (measured: host ids published with completed system-scope
    // stores and no fence were read stale), and one fence for the workgroup is enough: a fence per
    // wave would write back the L2 once per wave, which costs microseconds.
    for (int i = tid - 64; i < B * H / 8; i += kKeyT0 - 64)
      reinterpret_cast<uint4*>(x_host)[i] = reinterpret_cast<const uint4*>(x)[i];
  }
  lds_sync();
  ensure_body(c, layer, n, 0, C);
  if (n <= 64 && !spec_ids && qstar_dev(C.nm, c.f) == 0) {
    // nothing to fetch (q* = 0, uniform): no victims are needed, so wave 0 finishes the call alone,
    // without a block barrier per phase.  One barrier orders the x copies before wave 0's fence.
    if (tid >= 64 && tid < kKeyT0 && call_ring) __builtin_amdgcn_s_waitcnt(0);  // x_host stores complete
    lds_sync();
    if (tid >= 64) return;
    if (tid < n) C.slot[tid] = C.hit[tid];  // the -1 partition: hits keep their slot
    if (tid == 0) C.qq = 0;
    // the lanes of this wave read each other's entries from LDS next (in order within a wave)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    plan_wave0(C.slot, C.id, C.hit, (int64_t)layer * c.E, c.owner, n, c.S, maxU, maxB, plan);
    commit_body(c, C, true, slots, cpu, cpu_host, counts);
    int nhost = __popcll(__ballot(tid < n && C.slot[tid] < 0 && C.id[tid] >= 0));
    publish_call(call_ring, host_done, seq_ctr, layer, B, nhost);
    return;
  }
  split_body(c, C, s_key, true);
  if (tid >= 64 && tid < kKeyT0 && call_ring) __builtin_amdgcn_s_waitcnt(0);  // x_host stores complete (above)
  plan_body(C.slot, C.id, C.hit, (int64_t)layer * c.E, c.owner, n, c.S, maxU, maxB, plan,
            reinterpret_cast<int32_t*>(s_key));
  commit_body(c, C, true, slots, cpu, cpu_host, counts);
  int nhost = 0;  // wave 0: entries of the real call the host computes
  if (tid < 64)
    for (int p0 = 0; p0 < n; p0 += 64) {
      const int p = p0 + tid;
      nhost += __popcll(__ballot(p < n && C.slot[p] < 0 && C.id[p] >= 0));
    }
  if (spec_ids) {
    const int real_q = C.qq;  // the real call's fetches, before the speculative call reuses C
    __syncthreads();  // the real call's commit is visible to the speculative ensure
    for (int p = tid; p < n; p += kThreads) C.id[p] = spec_ids[p];
    lds_sync();
    ensure_body(c, layer + 1, n, 1, C);
    split_body(c, C, s_key, false, real_q);
    commit_body(c, C, true, spec_slots, nullptr, nullptr, counts + 3);
  }
  if (tid < 64) publish_call(call_ring, host_done, seq_ctr, layer, B, nhost);
}

__global__ void k_qstar_batch(const int32_t* __restrict__ m, const uint32_t* __restrict__ f,
                              int32_t* __restrict__ q, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) q[i] = (int32_t)qstar_dev(m[i], f[i]);
}

// Installs flat ids into target slots in the given order with exactly the
// sequential semantics of one-at-a-time installs (evict the target's owner,
// free the expert's previous slot), carried out on LDS images by one thread.
// mode 0: whole layer, expert e -> slot (layer%2)*E + e.  mode 1: experts[i] -> slot i.
__global__ void __launch_bounds__(256)
k_install(int layer, int E, int mode, const int32_t* __restrict__ experts, int n,
          int32_t* __restrict__ table, int32_t* __restrict__ owner, int64_t* __restrict__ usage,
          int64_t* __restrict__ clock) {
  extern __shared__ int32_t s_dyn[];
  int32_t* s_tab = s_dyn;              // [E] table image of this layer
  int32_t* s_own = s_dyn + E;          // [E] owner image of the target slot range
  int32_t* s_ext_tab = s_dyn + 2 * E;  // [E] flat ids outside the layer whose table entry is cleared
  int32_t* s_ext_slot = s_dyn + 3 * E; // [E] slots outside the target range that are freed
  __shared__ int s_nt, s_ns;
  __shared__ int64_t s_step;
  const int tid = threadIdx.x;
  const int64_t base = (int64_t)layer * E;
  const int tbase = (mode == 0) ? (layer % 2) * E : 0;  // first target slot
  const int tcount = (mode == 0) ? E : n;
  for (int e = tid; e < E; e += blockDim.x) s_tab[e] = table[base + e];
  for (int i = tid; i < tcount; i += blockDim.x) s_own[i] = owner[tbase + i];
  if (tid == 0) {
    s_nt = 0;
    s_ns = 0;
    s_step = clock[0] + 1;
  }
  __syncthreads();
  if (tid == 0) {
    for (int i = 0; i < tcount; ++i) {
      int e = (mode == 0) ? i : experts[i];
      int v = tbase + i;
      int w = s_tab[e];
      if (w == v) continue;
      int old = s_own[i];
      if (old >= 0) {
        if (old >= base && old < base + E) s_tab[old - base] = -1;
        else s_ext_tab[s_nt++] = old;
      }
      if (w >= 0) {
        if (w >= tbase && w < tbase + tcount) s_own[w - tbase] = -1;
        else s_ext_slot[s_ns++] = w;
      }
      s_own[i] = (int32_t)(base + e);
      s_tab[e] = v;
    }
  }
  __syncthreads();
  const int64_t st = s_step;
  for (int i = tid; i < s_nt; i += blockDim.x) table[s_ext_tab[i]] = -1;
  for (int i = tid; i < s_ns; i += blockDim.x) {
    owner[s_ext_slot[i]] = -1;
    usage[s_ext_slot[i]] = -1;
  }
  for (int e = tid; e < E; e += blockDim.x) table[base + e] = s_tab[e];
  for (int i = tid; i < tcount; i += blockDim.x) {
    owner[tbase + i] = s_own[i];
    usage[tbase + i] = st;  // every target slot holds its install of this step
  }
  if (tid == 0) {
    clock[0] = st;
    clock[1] = st;
  }
}

}  // namespace

static int sort_pow2_of(int S) {
  int p = 1024;
  while (p < S) p <<= 1;
  return p;
}

static CacheState state_of(eff_engine* e) {
  CacheState c;
  c.E = e->cfg.num_experts;
  c.S = e->cfg.num_slots;
  c.f = e->cfg.fetch_frac_q16;
  c.table = e->d_table;
  c.owner = e->d_owner;
  c.usage = e->d_usage;
  c.recency = e->d_recency;
  c.clock = e->d_clock;
  c.pd = e->d_pending;
  c.fl_dev = e->d_fetch;
  c.fl_host = e->h_fetch_dev;
  c.stats = e->d_stats;
  c.err = e->d_err;
  c.host_err = e->h_err_dev;
  c.sort_pow2 = sort_pow2_of(c.S);
  c.spec_budget = e->spec_budget;
  c.spec_link = e->spec_link;
  return c;
}

// dynamic LDS of the control kernel: victim keys and the plan scratch
static size_t control_lds(int S, int E) {
  (void)E;
  return std::max((size_t)sort_pow2_of(S) * sizeof(uint64_t), (size_t)3 * kMaxEntries * sizeof(int32_t));
}

hipError_t launch_ensure(eff_engine* e, int layer, int32_t* ids, int n, int spec, hipStream_t s) {
  hipLaunchKernelGGL(k_ensure, dim3(1), dim3(kThreads), 0, s, state_of(e), layer, ids, n, spec);
  return hipGetLastError();
}

hipError_t launch_split(eff_engine* e, int32_t* ids, int32_t* cpu_ids, int32_t* counts, int which,
                        hipStream_t s) {
  (void)which;
  const CacheState c = state_of(e);
  hipLaunchKernelGGL(k_split, dim3(1), dim3(kThreads), (size_t)c.sort_pow2 * sizeof(uint64_t), s, c, ids, cpu_ids,
                     counts);
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int B, int E, int K, int32_t* ids, float* w, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  const int per = kThreads / 64;
  hipLaunchKernelGGL(k_topk, dim3((B + per - 1) / per), dim3(kThreads), 0, s, logits, B, E, K, ids, w);
  return hipGetLastError();
}

hipError_t launch_plan(eff_engine* e, const int32_t* slots, int n, hipStream_t s, DecodePlan* plan, int maxU) {
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(kThreads), 0, s, slots, n, e->cfg.num_slots, maxU,
                     e->cfg.max_tokens, e->d_owner, plan);
  return hipGetLastError();
}

hipError_t launch_control(eff_engine* e, int layer, const float* logits, int B, const uint16_t* x,
                          const int32_t* spec_ids, hipStream_t s) {
  const eff_config& cf = e->cfg;
  const size_t lds = control_lds(cf.num_slots, cf.num_experts);
  hipLaunchKernelGGL(k_control, dim3(1), dim3(kThreads), lds, s, state_of(e), logits, B,
                     cf.top_k, layer, e->d_ids, e->d_w, e->d_slots, e->d_cpu, e->d_counts, spec_ids,
                     e->d_spec_ids, e->h_cpu_dev, x, e->h_x_dev, cf.hidden, e->maxU, cf.max_tokens, e->d_plan,
                     e->h_call_dev, e->h_done_dev, e->d_seq);
  return hipGetLastError();
}

hipError_t split_kernel_setup(int S, int E) {
  const int P = sort_pow2_of(S);
  hipError_t err = hipFuncSetAttribute((const void*)k_split, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)(P * sizeof(uint64_t)));
  if (err != hipSuccess) return err;
  return hipFuncSetAttribute((const void*)k_control, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)control_lds(S, E));
}

hipError_t launch_qstar_batch(const int32_t* m, const uint32_t* f, int32_t* q, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_qstar_batch, dim3((n + 255) / 256), dim3(256), 0, s, m, f, q, n);
  return hipGetLastError();
}

hipError_t launch_prefill_install(eff_engine* e, int layer, hipStream_t s) {
  hipLaunchKernelGGL(k_install, dim3(1), dim3(256), (size_t)16 * e->cfg.num_experts, s, layer,
                     e->cfg.num_experts, 0,
                     (const int32_t*)nullptr, e->cfg.num_experts, e->d_table, e->d_owner, e->d_usage,
                     e->d_clock);
  return hipGetLastError();
}

hipError_t launch_fallback_install(eff_engine* e, int layer, const int32_t* experts, int n,
                                   hipStream_t s) {
  hipLaunchKernelGGL(k_install, dim3(1), dim3(256), (size_t)16 * e->cfg.num_experts, s, layer,
                     e->cfg.num_experts, 1, experts, n,
                     e->d_table, e->d_owner, e->d_usage, e->d_clock);
  return hipGetLastError();
}

int64_t qstar_host(int64_t m, int64_t f) { return qstar_dev(m, f); }

}  // namespace eff
