// Slot-cache control kernels: ensure, split (q*), q* batch, prefill installs.
//
// All routing-dependent control flow runs on the device as data, in one
// workgroup per call ([FT-blog] §六: one kernel deduplicates, checks residency,
// computes q, picks victims and rewrites ids to a slot or the host marker;
// [FT-deep] §4 design pattern ② explains why: the miss count exists only on the
// device while the decode step is captured).
#include "eff_internal.h"

namespace eff {
namespace {

constexpr int kThreads = 1024;
constexpr uint64_t kInfKey = ~0ull;

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
  int sort_pow2;
};

// LDS the control bodies need besides the dynamic key buffer.
struct SplitLds {
  int32_t ranked[kMaxEntries];
  int32_t victim[kMaxEntries];
  int32_t mid[kMaxEntries];
  int64_t mrec[kMaxEntries];
  uint64_t red[kThreads / 64];
  int nv;
};

// ensure: dedup, residency, hits stamped at this step, ids rewritten to slot-or--1, call kept
// pending.  scratch: 3 * kMaxEntries int32 of LDS (free outside this body).
__device__ void ensure_body(const CacheState& c, int layer, int32_t* __restrict__ ids, int n, int spec,
                            int32_t* scratch) {
  int32_t* s_id = scratch;
  int32_t* s_slot = scratch + kMaxEntries;
  int32_t* s_first = scratch + 2 * kMaxEntries;
  __shared__ int64_t s_step, s_floor;
  __shared__ int s_nu, s_nm;
  const int tid = threadIdx.x, E = c.E;
  if (tid == 0) {
    s_step = c.clock[0] + 1;
    s_floor = spec ? c.clock[1] : s_step;
    s_nu = 0;
    s_nm = 0;
  }
  for (int p = tid; p < n; p += kThreads) {
    int v = ids[p];
    if (v < 0 || v >= E) {
      atomicOr(c.err, 1);
      v = -1;
    }
    s_id[p] = v;
    s_slot[p] = (v >= 0) ? c.table[(int64_t)layer * E + v] : -1;
  }
  __syncthreads();
  for (int p = tid; p < n; p += kThreads) {
    int id = s_id[p], first = id >= 0;
    for (int q = 0; q < p && first; ++q) first = (s_id[q] != id);
    s_first[p] = first;
  }
  __syncthreads();
  const int64_t s = s_step;
  for (int p = tid; p < n; p += kThreads) {
    if (!s_first[p]) continue;
    int id = s_id[p], ru = 0, rm = 0;
    bool miss = s_slot[p] < 0;
    for (int q = 0; q < n; ++q) {
      if (!s_first[q]) continue;
      int o = s_id[q];
      ru += (o < id);
      rm += (o < id) && (s_slot[q] < 0);
    }
    c.pd->uniq[ru] = id;
    if (miss) {
      c.pd->miss[rm] = id;
      atomicAdd(&s_nm, 1);
    } else {
      c.usage[s_slot[p]] = s;  // hit: stamped as used now
    }
    atomicAdd(&s_nu, 1);
  }
  for (int p = tid; p < n; p += kThreads) {
    c.pd->ids[p] = s_id[p];
    ids[p] = s_slot[p];
  }
  __syncthreads();
  if (tid == 0) {
    c.clock[0] = s;
    c.pd->valid = 1;
    c.pd->layer = layer;
    c.pd->n = n;
    c.pd->spec = spec;
    c.pd->s = s;
    c.pd->floor_ = s_floor;
    c.pd->nuniq = s_nu;
    c.pd->nmiss = s_nm;
  }
  __syncthreads();
}

// Block-wide min of a 64-bit key; every thread gets the result.
__device__ inline uint64_t block_min_u64(uint64_t v, uint64_t* s_red) {
  for (int o = 32; o >= 1; o >>= 1) {
    uint64_t w = __shfl_xor(v, o);
    v = w < v ? w : v;
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  uint64_t r = s_red[0];
  for (int i = 1; i < kThreads / 64; ++i) r = s_red[i] < r ? s_red[i] : r;
  __syncthreads();
  return r;
}

// split: q*, recency ranking, LRU victims, installs, the -1 partition, recency and counts.
// cpu_host (may be null): a host-mapped copy of cpu_ids.  s_key: sort_pow2 uint64 of LDS.
__device__ void split_body(const CacheState& c, int32_t* __restrict__ ids_out, int32_t* __restrict__ cpu_out,
                           int32_t* __restrict__ cpu_host, int32_t* __restrict__ counts, SplitLds& L,
                           uint64_t* s_key) {
  const int tid = threadIdx.x;
  Pending* pd = c.pd;
  if (!pd->valid) {
    if (tid == 0) atomicOr(c.err, 2);
    return;
  }
  const int E = c.E, S = c.S;
  const int layer = pd->layer, n = pd->n, spec = pd->spec, m = pd->nmiss, nu = pd->nuniq;
  const int64_t s = pd->s, floor_ = pd->floor_;
  const int64_t base = (int64_t)layer * E;
  const int q = (int)qstar_dev(m, c.f);

  int qq = 0;
  if (q > 0) {
    // Misses ranked by (recency desc, id asc) ([FT-deep] §4 ⑤: prefer recently active experts).
    for (int i = tid; i < m; i += kThreads) {
      int e = pd->miss[i];
      L.mid[i] = e;
      L.mrec[i] = c.recency[base + e];
    }
    if (tid == 0) L.nv = 0;
    __syncthreads();
    for (int i = tid; i < m; i += kThreads) {
      int e = L.mid[i];
      int64_t r = L.mrec[i];
      int rank = 0;
      for (int j = 0; j < m; ++j) {
        int o = L.mid[j];
        int64_t ro = L.mrec[j];
        rank += (ro > r) || (ro == r && o < e);
      }
      L.ranked[rank] = e;
    }
    // Victim keys: slots with usage below the floor, ordered by (usage, slot).
    int local_nv = 0;
    for (int v = tid; v < c.sort_pow2; v += kThreads) {
      uint64_t key = kInfKey;
      if (v < S) {
        int64_t u = c.usage[v];
        if (u < floor_) {
          key = ((uint64_t)(u + 1) << 14) | (uint64_t)v;
          ++local_nv;
        }
      }
      s_key[v] = key;
    }
    if (local_nv) atomicAdd(&L.nv, local_nv);
    __syncthreads();
    qq = min(q, L.nv);
    if (qq > 0 && qq <= 16) {
      // few fetches: qq rounds of block-wide argmin
      for (int i = 0; i < qq; ++i) {
        uint64_t lm = kInfKey;
        for (int v = tid; v < S; v += kThreads) lm = s_key[v] < lm ? s_key[v] : lm;
        uint64_t g = block_min_u64(lm, L.red);
        int v = (int)(g & 0x3FFF);
        if (tid == 0) {
          L.victim[i] = v;
          s_key[v] = kInfKey;
        }
        __syncthreads();
      }
    } else if (qq > 16) {
      // many fetches: bitonic sort of all keys (ascending)
      for (int k = 2; k <= c.sort_pow2; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
          for (int i = tid; i < c.sort_pow2; i += kThreads) {
            int ixj = i ^ j;
            if (ixj > i) {
              uint64_t a = s_key[i], b = s_key[ixj];
              bool up = (i & k) == 0;
              if ((a > b) == up) {
                s_key[i] = b;
                s_key[ixj] = a;
              }
            }
          }
          __syncthreads();
        }
      }
      for (int i = tid; i < qq; i += kThreads) L.victim[i] = (int)(s_key[i] & 0x3FFF);
      __syncthreads();
    }
  }
  // Installs: i-th ranked miss -> i-th oldest victim.
  FetchList* fl = c.fl_dev + (spec ? 1 : 0);
  FetchList* flh = c.fl_host + (spec ? 1 : 0);
  for (int i = tid; i < qq; i += kThreads) {
    int v = L.victim[i], e = L.ranked[i];
    int old = c.owner[v];
    if (old >= 0) c.table[old] = -1;
    c.owner[v] = (int32_t)(base + e);
    c.table[base + e] = v;
    c.usage[v] = s;
    fl->flat[i] = (int32_t)(base + e);
    fl->slot[i] = v;
    flh->flat[i] = (int32_t)(base + e);
    flh->slot[i] = v;
  }
  __syncthreads();
  // The -1 partition ([FT-deep] §4 ③): GPU owns entries with a slot, the host the rest.
  for (int p = tid; p < n; p += kThreads) {
    int id = pd->ids[p];
    int slot = (id >= 0) ? c.table[base + id] : -1;
    ids_out[p] = slot;
    const int cpu = (!spec && slot < 0 && id >= 0) ? id : -1;
    if (cpu_out) cpu_out[p] = cpu;
    if (cpu_host) cpu_host[p] = cpu;
  }
  if (!spec)
    for (int u = tid; u < nu; u += kThreads) c.recency[base + pd->uniq[u]] = s;
  __syncthreads();
  if (tid == 0) {
    if (!spec) c.clock[1] = s;
    if (counts) {
      counts[0] = m;
      counts[1] = qq;
      counts[2] = spec ? 0 : m - qq;
    }
    fl->count = qq;
    flh->count = qq;
    fl->err = *c.err;
    flh->err = *c.err;
    *c.err = 0;
    pd->valid = 0;
    c.stats[ST_CALLS] += 1;
    if (spec) {
      c.stats[ST_SPEC_FETCHED] += qq;
    } else {
      c.stats[ST_HITS] += nu - m;
      c.stats[ST_FETCHED] += qq;
      c.stats[ST_HOST] += m - qq;
      c.stats[ST_HIST0 + (qq < 16 ? qq : 16)] += 1;
    }
  }
  __syncthreads();
}

__device__ inline bool better(float a, int ia, float b, int ib) { return a > b || (a == b && ia < ib); }

// top-K of one logits row by (logit desc, id asc) and the softmax of the K selected, by one wave.
// sel: kMaxTopK floats of LDS for this wave.
__device__ void wave_topk(const float* __restrict__ row, int E, int K, int32_t* __restrict__ ids,
                          float* __restrict__ w, float* sel) {
  const int lane = threadIdx.x & 63;
  uint64_t taken = 0;  // element lane + 64*j is taken when bit j is set
  for (int k = 0; k < K; ++k) {
    float bv = 0.f;
    int bi = 0x7FFFFFFF;
    int j = 0;
    for (int e = lane; e < E; e += 64, ++j) {
      if ((taken >> j) & 1) continue;
      const float v = row[e];
      if (bi == 0x7FFFFFFF || better(v, e, bv, bi)) {
        bv = v;
        bi = e;
      }
    }
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o);
      if (oi != 0x7FFFFFFF && (bi == 0x7FFFFFFF || better(ov, oi, bv, bi))) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1ull << (bi >> 6);
    if (lane == 0) {
      sel[k] = bv;
      ids[k] = bi;
    }
  }
  if (lane == 0) {
    // softmax over the K selected logits, relative to the largest
    float sum = 0.f;
    for (int k = 0; k < K; ++k) sum += expf(sel[k] - sel[0]);
    for (int k = 0; k < K; ++k) w[k] = expf(sel[k] - sel[0]) / sum;
  }
}

// decode plan (distinct GPU slots and their entries), by one workgroup; scratch: 2*kMaxEntries.
__device__ void plan_body(const int32_t* __restrict__ slots, int n, int S, int maxU, int maxB,
                          const int32_t* __restrict__ owner, DecodePlan* plan, int32_t* scratch) {
  int32_t* s_sl = scratch;
  int32_t* s_first = scratch + kMaxEntries;
  __shared__ int s_nu;
  const int tid = threadIdx.x;
  if (tid == 0) s_nu = 0;
  for (int p = tid; p < n; p += blockDim.x) {
    const int v = slots[p];
    s_sl[p] = (v >= 0 && v < S) ? v : -1;  // slots outside the arena are never read
  }
  __syncthreads();
  for (int p = tid; p < n; p += blockDim.x) {
    int v = s_sl[p], first = v >= 0;
    for (int q = 0; q < p && first; ++q) first = s_sl[q] != v;
    s_first[p] = first;
  }
  __syncthreads();
  for (int p = tid; p < n; p += blockDim.x) {
    if (!s_first[p]) continue;
    int v = s_sl[p], rank = 0, cnt = 0;
    for (int q = 0; q < n; ++q) rank += s_first[q] && s_sl[q] < v;
    if (rank >= maxU) continue;  // more distinct slots than a layer has experts: not computed
    DecodeUnit& un = plan->unit[rank];
    for (int q = 0; q < n && cnt < maxB; ++q)  // a slot appears at most once per token
      if (s_sl[q] == v) un.entry[cnt++] = q;
    un.slot = v;
    un.count = cnt;
    un.flat = owner[v];
    atomicAdd(&s_nu, 1);
  }
  __syncthreads();
  const int nu = min(s_nu, maxU);
  for (int u = nu + tid; u < maxU; u += blockDim.x) {
    plan->unit[u].count = 0;
    plan->unit[u].slot = 0;
    plan->unit[u].flat = 0;
  }
  if (tid == 0) plan->nu = nu;
  __syncthreads();
}

__global__ void __launch_bounds__(kThreads)
k_ensure(CacheState c, int layer, int32_t* __restrict__ ids, int n, int spec) {
  __shared__ int32_t scratch[3 * kMaxEntries];
  ensure_body(c, layer, ids, n, spec, scratch);
}

__global__ void __launch_bounds__(kThreads)
k_split(CacheState c, int32_t* __restrict__ ids_out, int32_t* __restrict__ cpu_out, int32_t* __restrict__ counts) {
  extern __shared__ uint64_t s_key[];
  __shared__ SplitLds L;
  split_body(c, ids_out, cpu_out, nullptr, counts, L, s_key);
}

__global__ void __launch_bounds__(kThreads)
k_topk(const float* __restrict__ logits, int B, int E, int K, int32_t* __restrict__ ids, float* __restrict__ w) {
  __shared__ float s_sel[kThreads / 64][kMaxTopK];
  const int wave = threadIdx.x >> 6;
  for (int t = blockIdx.x * (kThreads / 64) + wave; t < B; t += gridDim.x * (kThreads / 64))
    wave_topk(logits + (int64_t)t * E, E, K, ids + (int64_t)t * K, w + (int64_t)t * K, s_sel[wave]);
}

__global__ void __launch_bounds__(kThreads)
k_plan(const int32_t* __restrict__ slots, int n, int S, int maxU, int maxB, const int32_t* __restrict__ owner,
       DecodePlan* plan) {
  __shared__ int32_t scratch[2 * kMaxEntries];
  plan_body(slots, n, S, maxU, maxB, owner, plan, scratch);
}

// One decode layer's control path in one workgroup: top-K of the B logits rows, ensure, split,
// (speculative ensure + split of the next layer), the decode plan, and the host's inputs
// (host ids and x) written to host-mapped memory.
__global__ void __launch_bounds__(kThreads)
k_control(CacheState c, const float* __restrict__ logits, int B, int K, int layer, int32_t* __restrict__ ids,
          float* __restrict__ w, int32_t* __restrict__ slots, int32_t* __restrict__ cpu, int32_t* __restrict__ counts,
          const int32_t* __restrict__ spec_ids, int32_t* __restrict__ spec_slots, int32_t* __restrict__ cpu_host,
          const uint16_t* __restrict__ x, uint16_t* __restrict__ x_host, int H, int maxU, int maxB,
          DecodePlan* plan) {
  extern __shared__ uint64_t s_key[];  // victim keys; also scratch for ensure and plan
  __shared__ SplitLds L;
  __shared__ float s_sel[kThreads / 64][kMaxTopK];
  const int tid = threadIdx.x, wave = tid >> 6;
  const int n = B * K;
  for (int t = wave; t < B; t += kThreads / 64)
    wave_topk(logits + (int64_t)t * c.E, c.E, K, ids + (int64_t)t * K, w + (int64_t)t * K, s_sel[wave]);
  __syncthreads();
  for (int p = tid; p < n; p += kThreads) slots[p] = ids[p];
  // the host's copy of x travels while the control path runs (16 bytes per thread)
  for (int i = tid; i < B * H / 8; i += kThreads)
    reinterpret_cast<uint4*>(x_host)[i] = reinterpret_cast<const uint4*>(x)[i];
  __syncthreads();
  ensure_body(c, layer, slots, n, 0, reinterpret_cast<int32_t*>(s_key));
  split_body(c, slots, cpu, cpu_host, counts, L, s_key);
  if (spec_ids) {
    for (int p = tid; p < n; p += kThreads) spec_slots[p] = spec_ids[p];
    __syncthreads();
    ensure_body(c, layer + 1, spec_slots, n, 1, reinterpret_cast<int32_t*>(s_key));
    split_body(c, spec_slots, nullptr, nullptr, counts + 3, L, s_key);
  }
  plan_body(slots, n, c.S, maxU, maxB, c.owner, plan, reinterpret_cast<int32_t*>(s_key));
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
  c.sort_pow2 = sort_pow2_of(c.S);
  return c;
}

static size_t control_lds(int S) {
  const size_t keys = (size_t)sort_pow2_of(S) * sizeof(uint64_t);
  const size_t scratch = (size_t)3 * kMaxEntries * sizeof(int32_t);
  return keys > scratch ? keys : scratch;
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

hipError_t launch_plan(eff_engine* e, const int32_t* slots, int n, hipStream_t s) {
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(kThreads), 0, s, slots, n, e->cfg.num_slots, e->maxU,
                     e->cfg.max_tokens, e->d_owner, e->d_plan);
  return hipGetLastError();
}

hipError_t launch_control(eff_engine* e, int layer, const float* logits, int B, const uint16_t* x,
                          const int32_t* spec_ids, hipStream_t s) {
  const eff_config& cf = e->cfg;
  hipLaunchKernelGGL(k_control, dim3(1), dim3(kThreads), control_lds(cf.num_slots), s, state_of(e), logits, B,
                     cf.top_k, layer, e->d_ids, e->d_w, e->d_slots, e->d_cpu, e->d_counts, spec_ids,
                     e->d_spec_ids, e->h_cpu_dev, x, e->h_x_dev, cf.hidden, e->maxU, cf.max_tokens, e->d_plan);
  return hipGetLastError();
}

hipError_t split_kernel_setup(int S) {
  const int P = sort_pow2_of(S);
  hipError_t err = hipFuncSetAttribute((const void*)k_split, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)(P * sizeof(uint64_t)));
  if (err != hipSuccess) return err;
  return hipFuncSetAttribute((const void*)k_control, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)control_lds(S));
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
