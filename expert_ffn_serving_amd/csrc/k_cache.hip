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

__global__ void __launch_bounds__(kThreads)
k_ensure(int layer, int E, int32_t* __restrict__ ids, int n, int spec, const int32_t* __restrict__ table,
         int64_t* __restrict__ usage, int64_t* __restrict__ clock, Pending* __restrict__ pd,
         int32_t* __restrict__ err) {
  __shared__ int32_t s_id[kMaxEntries];
  __shared__ int32_t s_slot[kMaxEntries];
  __shared__ int32_t s_first[kMaxEntries];
  __shared__ int64_t s_step, s_floor;
  __shared__ int s_nu, s_nm;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_step = clock[0] + 1;
    s_floor = spec ? clock[1] : s_step;
    s_nu = 0;
    s_nm = 0;
  }
  for (int p = tid; p < n; p += kThreads) {
    int v = ids[p];
    if (v < 0 || v >= E) {
      atomicOr(err, 1);
      v = -1;
    }
    s_id[p] = v;
    s_slot[p] = (v >= 0) ? table[(int64_t)layer * E + v] : -1;
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
    pd->uniq[ru] = id;
    if (miss) {
      pd->miss[rm] = id;
      atomicAdd(&s_nm, 1);
    } else {
      usage[s_slot[p]] = s;  // hit: stamped as used now
    }
    atomicAdd(&s_nu, 1);
  }
  for (int p = tid; p < n; p += kThreads) {
    pd->ids[p] = s_id[p];
    ids[p] = s_slot[p];
  }
  __syncthreads();
  if (tid == 0) {
    clock[0] = s;
    pd->valid = 1;
    pd->layer = layer;
    pd->n = n;
    pd->spec = spec;
    pd->s = s;
    pd->floor_ = s_floor;
    pd->nuniq = s_nu;
    pd->nmiss = s_nm;
  }
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

__global__ void __launch_bounds__(kThreads)
k_split(int E, int S, uint32_t f, int32_t* __restrict__ ids_out, int32_t* __restrict__ cpu_out,
        int32_t* __restrict__ counts, int32_t* __restrict__ table, int32_t* __restrict__ owner,
        int64_t* __restrict__ usage, int64_t* __restrict__ recency, int64_t* __restrict__ clock,
        Pending* __restrict__ pd, FetchList* __restrict__ fl_dev, FetchList* __restrict__ fl_host,
        int64_t* __restrict__ stats, int32_t* __restrict__ err, int sort_pow2) {
  extern __shared__ uint64_t s_key[];  // [sort_pow2] victim keys (usage+1) << 14 | slot
  __shared__ int32_t s_ranked[kMaxEntries];
  __shared__ int32_t s_victim[kMaxEntries];
  __shared__ int32_t s_mid[kMaxEntries];
  __shared__ int64_t s_mrec[kMaxEntries];
  __shared__ uint64_t s_red[kThreads / 64];
  __shared__ int s_nv;
  const int tid = threadIdx.x;
  if (!pd->valid) {
    if (tid == 0) atomicOr(err, 2);
    return;
  }
  const int layer = pd->layer, n = pd->n, spec = pd->spec, m = pd->nmiss, nu = pd->nuniq;
  const int64_t s = pd->s, floor_ = pd->floor_;
  const int64_t base = (int64_t)layer * E;
  const int q = (int)qstar_dev(m, f);

  // Misses ranked by (recency desc, id asc) ([FT-deep] §4 ⑤: prefer recently active experts).
  for (int i = tid; i < m; i += kThreads) {
    int e = pd->miss[i];
    s_mid[i] = e;
    s_mrec[i] = recency[base + e];
  }
  __syncthreads();
  for (int i = tid; i < m; i += kThreads) {
    int e = s_mid[i];
    int64_t r = s_mrec[i];
    int rank = 0;
    for (int j = 0; j < m; ++j) {
      int o = s_mid[j];
      int64_t ro = s_mrec[j];
      rank += (ro > r) || (ro == r && o < e);
    }
    s_ranked[rank] = e;
  }
  // Victim keys: slots with usage below the floor, ordered by (usage, slot).
  if (tid == 0) s_nv = 0;
  __syncthreads();
  int local_nv = 0;
  for (int v = tid; v < sort_pow2; v += kThreads) {
    uint64_t key = kInfKey;
    if (v < S) {
      int64_t u = usage[v];
      if (u < floor_) {
        key = ((uint64_t)(u + 1) << 14) | (uint64_t)v;
        ++local_nv;
      }
    }
    s_key[v] = key;
  }
  if (local_nv) atomicAdd(&s_nv, local_nv);
  __syncthreads();
  const int qq = min(q, s_nv);
  if (qq > 0 && qq <= 16) {
    // few fetches: qq rounds of block-wide argmin
    for (int i = 0; i < qq; ++i) {
      uint64_t lm = kInfKey;
      for (int v = tid; v < S; v += kThreads) lm = s_key[v] < lm ? s_key[v] : lm;
      uint64_t g = block_min_u64(lm, s_red);
      int v = (int)(g & 0x3FFF);
      if (tid == 0) {
        s_victim[i] = v;
        s_key[v] = kInfKey;
      }
      __syncthreads();
    }
  } else if (qq > 16) {
    // many fetches: bitonic sort of all keys (ascending)
    for (int k = 2; k <= sort_pow2; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < sort_pow2; i += kThreads) {
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
    for (int i = tid; i < qq; i += kThreads) s_victim[i] = (int)(s_key[i] & 0x3FFF);
    __syncthreads();
  }
  // Installs: i-th ranked miss -> i-th oldest victim.
  FetchList* fl = fl_dev + (spec ? 1 : 0);
  FetchList* flh = fl_host + (spec ? 1 : 0);
  for (int i = tid; i < qq; i += kThreads) {
    int v = s_victim[i], e = s_ranked[i];
    int old = owner[v];
    if (old >= 0) table[old] = -1;
    owner[v] = (int32_t)(base + e);
    table[base + e] = v;
    usage[v] = s;
    fl->flat[i] = (int32_t)(base + e);
    fl->slot[i] = v;
    flh->flat[i] = (int32_t)(base + e);
    flh->slot[i] = v;
  }
  __syncthreads();
  // The -1 partition ([FT-deep] §4 ③): GPU owns entries with a slot, the host the rest.
  for (int p = tid; p < n; p += kThreads) {
    int id = pd->ids[p];
    int slot = (id >= 0) ? table[base + id] : -1;
    ids_out[p] = slot;
    if (cpu_out) cpu_out[p] = (!spec && slot < 0 && id >= 0) ? id : -1;
  }
  if (!spec)
    for (int u = tid; u < nu; u += kThreads) recency[base + pd->uniq[u]] = s;
  __syncthreads();
  if (tid == 0) {
    if (!spec) clock[1] = s;
    if (counts) {
      counts[0] = m;
      counts[1] = qq;
      counts[2] = spec ? 0 : m - qq;
    }
    fl->count = qq;
    flh->count = qq;
    fl->err = *err;
    flh->err = *err;
    *err = 0;
    pd->valid = 0;
    stats[ST_CALLS] += 1;
    if (spec) {
      stats[ST_SPEC_FETCHED] += qq;
    } else {
      stats[ST_HITS] += nu - m;
      stats[ST_FETCHED] += qq;
      stats[ST_HOST] += m - qq;
      stats[ST_HIST0 + (qq < 16 ? qq : 16)] += 1;
    }
  }
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

hipError_t launch_ensure(eff_engine* e, int layer, int32_t* ids, int n, int spec, hipStream_t s) {
  hipLaunchKernelGGL(k_ensure, dim3(1), dim3(kThreads), 0, s, layer, e->cfg.num_experts, ids, n, spec,
                     e->d_table, e->d_usage, e->d_clock, e->d_pending, e->d_err);
  return hipGetLastError();
}

static int sort_pow2_of(int S) {
  int p = 1024;
  while (p < S) p <<= 1;
  return p;
}

hipError_t launch_split(eff_engine* e, int32_t* ids, int32_t* cpu_ids, int32_t* counts, int which,
                        hipStream_t s) {
  (void)which;
  int P = sort_pow2_of(e->cfg.num_slots);
  hipLaunchKernelGGL(k_split, dim3(1), dim3(kThreads), (size_t)P * sizeof(uint64_t), s,
                     e->cfg.num_experts, e->cfg.num_slots, e->cfg.fetch_frac_q16, ids, cpu_ids, counts,
                     e->d_table, e->d_owner, e->d_usage, e->d_recency, e->d_clock, e->d_pending,
                     e->d_fetch, e->h_fetch_dev, e->d_stats, e->d_err, P);
  return hipGetLastError();
}

hipError_t split_kernel_setup(int S) {
  int P = sort_pow2_of(S);
  return hipFuncSetAttribute((const void*)k_split, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)(P * sizeof(uint64_t)));
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
