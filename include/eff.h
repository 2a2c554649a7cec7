/*
 * libeff — routed-expert FFN over an HBM slot cache, for AMD MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes only.  Device pointers are caller-owned HIP
 * device memory; streams are hipStream_t passed as void* (NULL = the default
 * stream).  Every call returns EFF_OK (0) or a negative EFF_E* code and never
 * aborts; eff_last_error() gives a thread-local message for the last failure.
 * Calls that take a stream only enqueue work (no allocation, no host wait)
 * unless stated otherwise.  An engine is single-threaded: do not call into one
 * engine from two threads at once.
 *
 * Sources (cited by page title and section):
 *   [FT-deep]  "FreeToken 딥다이브 — 게이밍 PC 한 대로 284B 모델을 돌리는 엔진"
 *   [FT-blog]  "FreeToken:让消费级电脑跑起 284B MoE，一次把整机当成推理集群的系统设计"
 *   [NVMe-8GB] "NVMe에서 전문가(experts)를 스트리밍하여 8GB GPU에서 133GB MoE 모델 구동하기 (11 토큰/초)"
 *   [Edge0]    "SSD 가중치층으로 35B MoE를 라우팅 예측으로 24GB 데스크톱에서 서빙한다"
 *
 * Expert records.  The full pool of L*E records lives in pinned host memory and
 * is the source of truth; HBM holds only S slots of one record each, addressed
 * by the flat id layer*E + expert ([FT-blog] §四, §七 item 3; [FT-deep] §4 ⑤).
 * Record = gate[I,H] | up[I,H] | down[H,I] payloads, then their scales in the
 * same order ([NVMe-8GB] "엔진" item 1).  Each matrix (N rows = outputs, Kd
 * columns = inputs; N % 16 == 0, Kd % 32 == 0) is stored as tiles of 16 rows x
 * 32 inputs, tile index (n/16)*(Kd/32) + k/32: the 16 rows of a row slice are one
 * contiguous run.  A tile's 256 payload bytes hold element (n, k) at byte
 * (q*16 + r)*4 + i/2 with r=n%16, q=(k%32)/8, i=k%8, even i in the low nibble.
 * Each tile has 32 scale bytes at the same index in the scale area:
 * INT4_G32_BF16 stores the bf16 scale of (n, k/32) at byte r*2 and values are
 * (u-8)*scale; NVFP4_G16_E4M3 stores the e4m3 scale of (n, k/16) at byte
 * ((k%32)/16)*16 + r and values are
 * e2m1(code)*e4m3(scale)*tensor_scale, with one fp32 tensor scale per matrix
 * kept resident in the engine (tensor_scales[(layer*E+expert)*3 + m]).
 * Record size R = 3*H*I/2 + 3*H*I/16 bytes in both formats.
 */
#ifndef EFF_H
#define EFF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct eff_engine eff_engine;
typedef void* eff_stream_t; /* hipStream_t */

enum {
  EFF_OK = 0,
  EFF_EINVAL = -1,   /* bad argument; nothing was changed */
  EFF_ENOMEM = -2,   /* device or host allocation failed; nothing was changed */
  EFF_EHIP = -3,     /* a HIP runtime call failed (message has hipGetErrorString) */
  EFF_ECAPTURE = -4, /* the call must wait on the host and the stream is being captured */
  EFF_ESTATE = -5,   /* call out of order (e.g. split without a pending ensure) */
  EFF_EDEVICE = -6,  /* a kernel reported bad input (e.g. an expert id >= E); see message */
  EFF_EREJECTED = -7 /* a rebuild was validated and refused; the engine is unchanged and usable */
};

enum { EFF_WFMT_INT4_G32_BF16 = 0, EFF_WFMT_NVFP4_G16_E4M3 = 1 };

/* eff_ensure_experts flags */
enum { EFF_SPECULATIVE = 1u };

/* eff_config.flags */
enum {
  EFF_CFG_TIMING = 1u,   /* bracket the expert kernels with HIP events on their stream; the
                            durations are summed into eff_stats (adds two event records per call) */
  EFF_CFG_SYNC_HOST = 2u /* eff_decode_layer runs the host share on the calling thread and returns
                            after enqueuing the combine (default: a worker thread runs it and the
                            combine kernel waits for it on a host-mapped word) */
};

/* Instruction sets of the host executor, best first as eff_create picks them ([FT-deep] §7:
 * AVX-512 BF16 -> AVX-512F -> AVX2 + FMA -> scalar, chosen at run time). */
enum {
  EFF_HOST_ISA_SCALAR = 0,
  EFF_HOST_ISA_AVX2 = 1,       /* AVX2 + FMA */
  EFF_HOST_ISA_AVX512F = 2,
  EFF_HOST_ISA_AVX512_BF16 = 3 /* AVX-512 F, BW, VBMI and BF16 */
};

typedef struct eff_config {
  int32_t num_layers;         /* L */
  int32_t num_experts;        /* E, <= 4096 */
  int32_t top_k;              /* K, <= 32 */
  int32_t hidden;             /* H, multiple of 64 */
  int32_t inter;              /* I, multiple of 64 */
  int32_t wformat;            /* EFF_WFMT_* */
  int32_t num_slots;          /* S, 0 <= S <= 16384 */
  int32_t max_tokens;         /* decode batch bound B, 1..32 */
  int32_t max_prefill_tokens; /* prefill chunk bound T (0: no prefill) */
  uint32_t fetch_frac_q16;    /* f = B_P/B_H * 65536, 0..65536 */
  int32_t host_threads;       /* threads of the host executor; 0: one per physical core the process
                                 may use, SMT siblings excluded, less one core left to the thread
                                 that enqueues GPU work, each pinned to its core */
  uint32_t flags;             /* EFF_CFG_* bits */
} eff_config;

/* Record size R for the config's (H, I, format); 0 if the config is invalid. */
int64_t eff_record_bytes(const eff_config* cfg);

/* Creates an engine.  Validates everything before allocating (a rejected config
 * changes nothing, [FT-deep] §4 design pattern ⑦).  host_pool: L*E*R bytes of
 * pinned host memory (hipHostMalloc), caller-owned, read-only to the library,
 * alive until eff_destroy.  tensor_scales: L*E*3 floats (NVFP4; may be NULL
 * for INT4), copied.  Allocates S*R bytes of HBM for the slots plus tables.
 * Errors: EFF_EINVAL, EFF_ENOMEM, EFF_EHIP. */
int eff_create(const eff_config* cfg, const void* host_pool, const float* tensor_scales,
               eff_engine** out);
int eff_destroy(eff_engine* e);
const char* eff_last_error(void);

/* Pinned host memory helpers (hipHostMalloc / hipHostFree) for pools and staging. */
int eff_host_alloc(size_t bytes, void** out);
int eff_host_free(void* p);

/* Router ([FT-deep] §2; [FT-blog] §二).  x: bf16 [B,H]; w_router: bf16 [E,H];
 * ids: int32 [B,K] out, ordered by (logit desc, id asc); w: fp32 [B,K] out,
 * softmax over the K selected logits.  Logits are fp32 sums in a fixed order:
 * 64 lanes, lane l adds j = 64*V*c + V*l + i (c outer, i inner; V the largest
 * of 8,4,2,1 dividing H/64), then lanes fold pairwise (l, l+o) for o =
 * 32,16,...,1.  B <= max_tokens (decode) or <= max_prefill_tokens. */
int eff_route(eff_engine* e, const void* x, const void* w_router, int B, int32_t* ids, float* w,
              eff_stream_t stream);
/* Device pointer of the engine-owned fp32 logits [B,E] (row-major) that the last
 * eff_route, or eff_decode_layer given w_router, computed; the next such call
 * overwrites them.  Diagnostics: lets a caller compare the fixed summation order
 * bit for bit.  The pointer stays valid until eff_destroy. */
int eff_last_logits(eff_engine* e, const float** logits);
/* Same top-k/softmax from precomputed fp32 logits [B,E] (routing traces). */
int eff_route_logits(eff_engine* e, const float* logits, int B, int32_t* ids, float* w,
                     eff_stream_t stream);

/* ensure ([FT-deep] §4 ③ "ensure_experts_hybrid", §4 ⑤; [FT-blog] §六):
 * ids_inout: n = B*K device int32 expert ids of `layer`, rewritten in place to
 * the resident slot or -1.  Stamps hits as used at this step; keeps the call
 * pending for eff_split_misses.  flags: EFF_SPECULATIVE for a fetch-only
 * request made one layer early ([NVMe-8GB] "시간이 실제로 소요되는 부분").
 * An id outside [0,E) is reported as EFF_EDEVICE by the next host-waiting call.
 * EFF_ESTATE while an ensure waits for its split, or while the copies of an earlier
 * split of the same kind (real or speculative) have not been issued by eff_copy_missing. */
int eff_ensure_experts(eff_engine* e, int layer, int32_t* ids_inout, int n, uint32_t flags,
                       eff_stream_t stream);

/* split ([FT-deep] §4 ② q*, ⑤ recency; [FT-blog] §六): q = q*(m, f) of the m
 * unique misses; misses ranked by (recency desc, id asc) take the q' =
 * min(q, #victims) least recently used slots (usage asc, slot asc) whose
 * usage is below the call's floor.  Rewrites ids_inout to slot-or--1, writes
 * cpu_ids (the expert id where the host computes, -1 elsewhere; all -1 for a
 * speculative call) and counts = {m, q', host}.  The fetch list is kept in the
 * engine for eff_copy_missing.  Errors: EFF_ESTATE without a pending ensure. */
int eff_split_misses(eff_engine* e, int32_t* ids_inout, int32_t* cpu_ids, int32_t* counts,
                     eff_stream_t stream);

/* q* itself: argmin over F in [0,m] of max(F*(65536-f), (m-F)*f), lowest F on
 * ties ([FT-deep] §4 ②).  Host version returns q (or -1 for bad input); the
 * batch version evaluates n pairs on the device. */
int64_t eff_qstar(int64_t m, uint32_t f);
int eff_qstar_batch(const int32_t* m, const uint32_t* f, int32_t* q, int n, eff_stream_t stream);

/* The fetch fraction from two measured rates ([FT-deep] §4 design pattern ②):
 * f = B_P / B_H * 65536 as an integer, B_P the link's expert transfer rate and
 * B_H the host's expert processing rate, in bytes/s.  The integer part, capped at
 * 65536 (B_P >= B_H fetches every miss, [FT-blog] §六); B_P = 0 gives 0, B_H = 0
 * (with B_P > 0) 65536.  Host only.  Returns 0xFFFFFFFF for a negative or NaN rate. */
uint32_t eff_frac_q16(double pcie_bytes_per_s, double host_bytes_per_s);

/* Bandwidth profile ([FT-deep] §4 ②: f comes from a profile of both paths, and
 * preferably from running them at the same time, because the link transfer and the
 * host computation compete for the host memory controller; [FT-blog] §六: measured
 * on the target machine with the real tensor shapes).  Rates are bytes of expert
 * records per second. */
typedef struct eff_bw_profile {
  double pcie_alone;       /* in-kernel record copy from the pinned pool into HBM, alone */
  double host_alone;       /* the host executor over whole experts (1 token, K per call), alone */
  double pcie_concurrent;  /* the same two, run at the same time */
  double host_concurrent;
  uint32_t frac_q16;       /* eff_frac_q16 of the concurrent rates (the one to use) */
  uint32_t frac_q16_alone; /* eff_frac_q16 of the rates measured alone */
  int64_t record_bytes;
  int32_t records;         /* records moved by each path in each measurement */
  int32_t pad;
} eff_bw_profile;

/* Measures the profile on this engine's pool, records spread over the whole pool
 * (1 <= records <= L*E).  Synchronous: waits for the device and for the host-share
 * worker first, uses the engine's host threads and a private stream and scratch
 * buffer; the slot cache, its tables and the statistics are not touched.  Not
 * during graph capture (EFF_ECAPTURE) and not while another call into the engine
 * runs.  It does not change f: pass out->frac_q16 to eff_set_fetch_frac. */
int eff_profile_bandwidth(eff_engine* e, int records, eff_bw_profile* out);

/* Sets the engine's fetch fraction (0..65536, else EFF_EINVAL) for the calls
 * enqueued after it.  A graph captured earlier keeps the value it was captured with. */
int eff_set_fetch_frac(eff_engine* e, uint32_t frac_q16);

/* Speculative fetch scheduling ([NVMe-8GB] "엔진" item 3, prefetch into the gap: a
 * few guesses of the next layer's experts, read after the layer's real reads so
 * that they do not share the link with them).
 *   max_fetch  records one speculative request may fetch at most: its q' becomes
 *              min(q', max_fetch), the first ranked misses; -1 = no budget (the
 *              default), 0 = fetch none (predicted residents are still protected).
 *   in_gap     0: eff_decode_layer's speculative copy is carried by extra
 *              workgroups of the layer's gate/up kernel, beside the layer's own
 *              fetches (the default); 1: by the layer's down kernel, after the
 *              gate/up kernel has performed those fetches.
 * Either way the next layer's kernels follow the copy in stream order, and a
 * request that can fetch nothing (max_fetch 0, or a link cap of 0) carries no
 * copy.  Applies to the calls enqueued after it (a graph captured earlier keeps
 * its values); the policy and every result other than timing are the same for
 * both values of in_gap.
 * EFF_EINVAL for max_fetch < -1 or in_gap not 0 or 1. */
int eff_set_speculation(eff_engine* e, int max_fetch, int in_gap);

/* The link's gap for speculative fetches ([NVMe-8GB] "엔진" item 3: guesses are read in the transfer
 * time the layer's real reads leave): link_records = the records the link can carry in one layer's
 * time; a speculative request then fetches at most max(0, link_records - q'), q' the records the
 * latest real split fetched (the layer's own), the first of its ranked misses.  Applies with the
 * max_fetch of eff_set_speculation (the smaller cap wins) to the calls enqueued after it; -1 (the
 * default) turns the cap off.  EFF_EINVAL below -1. */
int eff_set_speculation_link(eff_engine* e, int link_records);

/* Runtime cache rebuild ([FT-blog] §七 item 1; [FT-deep] §4 design pattern ⑦): the
 * slot cache is rebuilt with num_slots slots for a new HBM budget, without touching
 * the host pool.  Everything is checked, and the new slot arena, owner and usage
 * arrays are allocated, before anything is freed; a request that does not fit returns
 * EFF_EREJECTED and leaves the engine exactly as it was:
 *   - num_slots outside [0, 16384];
 *   - max_arena_bytes > 0 and num_slots * record bytes > max_arena_bytes;
 *   - not at a safe point: an ensure waiting for its split, a split whose copies
 *     eff_copy_missing has not issued, or a prefill layer streamed but not computed;
 *   - the new buffers cannot be allocated (the old cache is still held then).
 * On success the rebuilt cache is empty (every expert misses until fetched again);
 * the step clock, last_real and the expert recency carry over, and results are
 * unchanged because the pool is the source of truth.  Synchronous: waits for the
 * device and the host-share worker.  Not during capture (EFF_ECAPTURE).  Graphs
 * captured before a rebuild address the old arena and must not be replayed after it. */
int eff_rebuild_cache(eff_engine* e, int num_slots, uint64_t max_arena_bytes);

/* copy ([FT-deep] §4 ③ copy_missing): waits on the host for `compute` to reach
 * the last split, then enqueues one hipMemcpyAsync per fetched record (host
 * pool -> slot) on `side` and makes `compute` wait for them.  Also issues the
 * fetches of a speculative split made after it.  EFF_ECAPTURE under capture. */
int eff_copy_missing(eff_engine* e, eff_stream_t compute, eff_stream_t side);

/* GPU expert compute ([FT-deep] §4 ③ _expert_gemm; [Edge0] "어떻게 동작하나"):
 * for every entry p = t*K+k with slots[p] >= 0, y[p,:] = W_d (silu(W_g x_t) *
 * (W_u x_t)) with the record in that slot; each distinct slot's weights are
 * read once for all its tokens.  x: bf16 [B,H]; y: fp32 [B,K,H]; entries with
 * slots[p] < 0 are not written. */
int eff_expert_ffn_decode(eff_engine* e, int layer, const void* x, const int32_t* slots, int B,
                          float* y, eff_stream_t stream);

/* For callers that cannot allocate (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): eff_expert_ffn_decode with the same arguments and results, whose decode
 * plan and SwiGLU staging live in a file-scope device array of 8 MiB (its address on each device is
 * taken once, by eff_create) instead of engine buffers; it calls no hipMalloc, hipFree or other
 * allocating routine (an error message may allocate host memory).  Every call on a GPU shares that
 * array: calls that overlap on one GPU race, whatever engine they come from.  A call needs
 * 73,984 + 3 * min(B*K, units) * max_tokens * inter bytes (units = min(max_tokens*K, E));
 * beyond 8 MiB it returns EFF_EINVAL and launches nothing.  The current device must be the
 * engine's (EFF_EINVAL otherwise).  No kernel timing. */
int eff_expert_ffn_decode_noalloc(eff_engine* e, int layer, const void* x, const int32_t* slots, int B,
                                  float* y, eff_stream_t stream);

/* Host share ([FT-deep] §4 ③ decode_submit/decode_sync; [FT-blog] §三.2): the
 * same expert FFN on the host, from the pinned pool, for entries with
 * cpu_ids[p] >= 0.  Synchronous; all pointers are host memory.  y_host fp32
 * [B,K,H]; other entries are not written. */
int eff_host_ffn_decode(eff_engine* e, int layer, const void* x_host, const int32_t* cpu_ids_host,
                        int B, float* y_host);

/* Merge ([FT-deep] §4 ③ "gpu_routed + cpu_routed"): out[t,:] = bf16_rne(sum over
 * k ascending of w[t,k] * (slots[t,k] >= 0 ? y_gpu : y_host)[t,k,:]).  y_host
 * is device memory (may be NULL if no entry has slot < 0). */
int eff_combine(eff_engine* e, const float* y_gpu, const float* y_host, const int32_t* slots,
                const float* w, int B, void* out, eff_stream_t stream);

/* One decode MoE layer end to end: route (from x and w_router, or from logits if
 * w_router is NULL) -> ensure -> split -> [speculative ensure/split of layer+1
 * on spec_ids if not NULL, its copies inside this layer's expert kernels] -> GPU expert FFN -> host share
 * -> combine into out (bf16 [B,H]).  top-K, ensure, split, the speculative
 * request and the decode plan run as one single-workgroup kernel with the same
 * semantics as the separate calls ([FT-blog] §六).  Experts installed by the
 * call are read from the pinned pool by the expert kernels themselves, which
 * also write them into their slots.  The control kernel publishes the host ids
 * and x in host-mapped memory, numbers the call in device memory and publishes
 * a call word (number, layer, B, host entries) in a host-mapped ring.  The host
 * share ([FT-deep] §4 ③④) runs on an engine-owned worker thread that follows
 * that ring, and the combine kernel waits for it on a host-mapped word (a
 * bounded poll), so the call only enqueues work and returns.  Nothing of a call
 * passes through the host at enqueue time, so a sequence of calls (for example
 * all layers of one decode step) may be captured into a HIP graph on `compute`
 * and replayed (`side` is only checked for capture; nothing is enqueued on it); the inputs
 * are then read from the captured addresses at each replay ([FT-deep] §4 ④: the
 * host branch inside the graph waits on host memory).  With EFF_CFG_SYNC_HOST
 * the calling thread waits for the control kernel and runs the host share
 * itself (EFF_ECAPTURE under capture, as with EFF_CFG_TIMING).  An error of the
 * host share is reported by the next call.  ids/w/slots/cpu_ids/counts of the
 * call can be read back with eff_last_layer_info after the stream is done. */
int eff_decode_layer(eff_engine* e, int layer, const void* x, const void* w_router,
                     const float* logits, int B, const int32_t* spec_ids, void* out,
                     eff_stream_t compute, eff_stream_t side);
/* Device pointers of the engine-owned buffers used by eff_decode_layer:
 * ids int32 [B*K] (routed expert ids), w fp32 [B*K], slots int32 [B*K],
 * cpu_ids int32 [B*K], counts int32 [3] (+3 for the speculative split). */
int eff_last_layer_info(eff_engine* e, const int32_t** ids, const float** w, const int32_t** slots,
                        const int32_t** cpu_ids, const int32_t** counts);

/* Prefill streaming ([FT-deep] §4 ①; [FT-blog] §五): installs layer's E
 * experts into buffer layer%2 (slots (layer%2)*E + e) and enqueues the E
 * record copies on `side`, then records an event that the next
 * eff_expert_ffn_prefill_layer of this layer waits on.  EFF_EINVAL if S < 2E
 * (the layer then runs through the fallback inside the prefill call). */
int eff_prefill_stream_layer(eff_engine* e, int layer, eff_stream_t side);

/* Whole-layer prefill ([FT-deep] §4 ①; [NVMe-8GB] "엔진" item 5): x bf16 [T,H],
 * ids int32 [T,K] (expert ids from eff_route), w fp32 [T,K] -> out bf16 [T,H].
 * Groups the (t,k) pairs by expert and runs a grouped GEMM per expert on the
 * slot buffer of layer%2, then the weighted combine.  With S < 2E it loads the
 * routed experts on demand in groups of min(S,E) (waits on the host).  The GEMMs
 * take activations and the SwiGLU output as fp16: a value beyond 65504 is
 * reported as EFF_EDEVICE by the next host-waiting call (this one included, for
 * an earlier layer). */
int eff_expert_ffn_prefill_layer(eff_engine* e, int layer, const void* x, const int32_t* ids,
                                 const float* w, int T, void* out, eff_stream_t stream);

/* Diagnostics (wait on the host; EFF_ECAPTURE under capture).  Any pointer may
 * be NULL.  table int32 [L*E], owner int32 [S], usage int64 [S], recency int64
 * [L*E], clock int64 [2] = {step, last_real}. */
int eff_snapshot_tables(eff_engine* e, int32_t* table, int32_t* owner, int64_t* usage,
                        int64_t* recency, int64_t* clock);

/* The host executor as eff_create set it up ([FT-deep] §7 hardware requirements: one thread per
 * physical core, SMT siblings left idle because they only compete for the same load ports). */
typedef struct eff_host_info {
  int32_t isa;            /* EFF_HOST_ISA_* in use */
  int32_t isa_best;       /* the best the CPU supports */
  int32_t threads;        /* threads that run a host share (pool workers + the engine's worker) */
  int32_t pinned;         /* 1: each of them is pinned to a physical core of its own */
  int32_t physical_cores; /* physical cores the process may use (affinity mask, cgroup CPU quota) */
  int32_t pad;
} eff_host_info;
int eff_get_host_info(eff_engine* e, eff_host_info* out);
/* Selects the host executor's instruction set (EFF_HOST_ISA_*), for example a lower level than the
 * CPU's best to compare them.  Waits for the host-share worker first; not during graph capture.
 * EFF_EINVAL for an unknown level or one the CPU does not support. */
int eff_set_host_isa(eff_engine* e, int isa);

/* Kernel timing slots of eff_stats (filled with EFF_CFG_TIMING). */
enum { EFF_T_DECODE_GATEUP = 0, EFF_T_DECODE_DOWN = 1, EFF_T_PREFILL_GATEUP = 2, EFF_T_PREFILL_DOWN = 3 };

typedef struct eff_stats {
  int64_t calls, hits, fetched, host, spec_fetched; /* unique experts, summed over calls */
  int64_t bytes_fetched;  /* (fetched + spec_fetched) * record bytes */
  int64_t qstar_hist[17]; /* q' counts 0..15, 16+ */
  int64_t launches[4];    /* timed launches per EFF_T_* slot */
  double kernel_ms[4];    /* summed durations per EFF_T_* slot (HIP events) */
  double host_ms;         /* eff_decode_layer: wall time in the host executor */
  double wait_ms;         /* eff_decode_layer: wall time the host share waited for control kernels */
  int64_t host_calls;     /* eff_decode_layer calls with a host share */
  /* the EFF_T_DECODE_* slots again, counting only eff_decode_layer calls that fetched no record
   * (their kernels read HBM only; a fetch makes the gate/up kernel wait on the host link) */
  int64_t launches_nofetch[4];
  double kernel_ms_nofetch[4];
  int64_t gpu_experts_nofetch; /* distinct GPU experts summed over those calls */
} eff_stats;
/* Changes eff_config.flags of a live engine (EFF_CFG_* bits); EFF_EINVAL for unknown bits. */
int eff_set_flags(eff_engine* e, uint32_t flags);

/* Waits for the device; counters since eff_create (or the last eff_reset_stats). */
int eff_get_stats(eff_engine* e, eff_stats* out);
int eff_reset_stats(eff_engine* e);

/* Device pointer of slot s (for tests: slot bytes must equal the host record). */
int eff_slot_ptr(eff_engine* e, int slot, const void** out);

#ifdef __cplusplus
}
#endif
#endif /* EFF_H */
