// Whole-layer prefill: grouped expert GEMMs on MFMA over the layer's slot buffer.
//
// In prefill nearly every expert of a layer is routed to, so the whole layer is
// streamed into buffer layer%2 and every expert's tokens are computed together
// ([FT-deep] §4 design pattern ①; [FT-blog] §五; [NVMe-8GB] "엔진" item 5 runs a
// whole prompt through one layer so that experts are not re-read per chunk).
//
//   k_pf_sort     one workgroup: count (t,k) pairs per expert, scan, place
//   k_pf_x16      the tokens' bf16 rows to fp16 once (range-checked), for every expert that reads them
//   k_pf_gemm<2>  per (expert, 256 rows of I): [n_e x H] x [H x 256] for gate and up
//                 on v_mfma_f32_16x16x32_f16, SwiGLU in the epilogue -> fp16 a
//   k_pf_gemm<1>  per (expert, 256 rows of H): [n_e x I] x [I x 256] -> fp32 y per pair
//   k_combine     (shared with decode) out[t] = sum_k w[t,k] y[t,k]
//
// Weights stay 4-bit in HBM and are dequantized in registers straight into the
// MFMA B operand: the 4 bytes at offset (16q+r)*4 of a 16-row x 32-input tile
// (row r, inputs 8q..8q+7) are exactly the B fragment of lane 16q+r.  NVFP4:
// e2m1 -> fp16 with v_cvt_scalef32_pk_f16_fp4, times the e4m3 block scale with
// a packed fp16 multiply (e2m1 * e4m3 has at most 6 significant bits and lies
// in [2^-10, 2688], so it is exact in fp16); the fp32 tensor scale is applied
// after accumulation.  int4: fp16(1024+u) - 1032 = u - 8 exactly, then times
// the scale (exact in fp16 for scales >= 2^-14).  Activations enter the MFMA
// as fp16 (bf16 inputs convert exactly inside fp16's normal range); an input or
// SwiGLU output beyond the fp16 range sets bit 8 of the engine's device error
// word, which the next host-waiting call reports, instead of passing an inf on.
#include <hip/hip_ext.h>

#include <algorithm>

#include "eff_internal.h"
#include "lds_dma.h"

namespace eff {
namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kPfPrefetch2 = 4;  // weight prefetch depth (k-tiles) of the gate/up GEMM
constexpr int kPfPrefetch1 = 4;
constexpr int kPfGateupWPM = 4;  // gate/up: waves per matrix (64 rows each; 2, two workgroups per CU, was slower)
constexpr int kPfLead = 12, kPfPer = 3;  // VALU ops before the first MFMA of a k-tile / after each MFMA  // ... and of the down GEMM

__global__ void __launch_bounds__(1024)
k_pf_sort(const int32_t* __restrict__ ids, int n, int E, int slot_base, const int32_t* __restrict__ slot_of,
          int32_t* __restrict__ offsets, int32_t* __restrict__ rows) {
  extern __shared__ int32_t s_cnt[];  // [E] counts, then cursors
  __shared__ int32_t s_wsum[16];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += blockDim.x) s_cnt[e] = 0;
  __syncthreads();
  for (int p = tid; p < n; p += blockDim.x) {
    const int e = ids[p];
    if (e >= 0 && e < E && (slot_base >= 0 || slot_of[e] >= 0)) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();
  // exclusive scan over E counts: each thread owns a contiguous run
  const int per = (E + blockDim.x - 1) / blockDim.x;
  const int b0 = min(E, tid * per), b1 = min(E, b0 + per);
  int run = 0;
  for (int e = b0; e < b1; ++e) run += s_cnt[e];
  // inclusive scan of run across the block
  int v = run;
  const int lane = tid & 63, wave = tid >> 6;
  for (int o = 1; o < 64; o <<= 1) {
    int w = __shfl_up(v, o);
    if (lane >= o) v += w;
  }
  if (lane == 63) s_wsum[wave] = v;
  __syncthreads();
  int add = 0;
  for (int i = 0; i < wave; ++i) add += s_wsum[i];
  int excl = v + add - run;
  __syncthreads();
  for (int e = b0; e < b1; ++e) {
    const int c = s_cnt[e];
    offsets[e] = excl;
    s_cnt[e] = excl;  // becomes the placement cursor
    excl += c;
  }
  if (tid == blockDim.x - 1) offsets[E] = excl;
  __syncthreads();
  for (int p = tid; p < n; p += blockDim.x) {
    const int e = ids[p];
    if (e >= 0 && e < E && (slot_base >= 0 || slot_of[e] >= 0)) {
      const int pos = atomicAdd(&s_cnt[e], 1);
      rows[pos] = p;
    }
  }
}

// block -> (expert, chunk): the chunks of one expert go to the same XCD (block % 8),
// so its activations are fetched into that XCD's L2 once.
__device__ inline void map_block(int b, int E, int NJ, int* e, int* j) {
  if (E % 8 == 0) {
    const int rem = b % (8 * NJ);
    *j = rem / 8;
    *e = (b / (8 * NJ)) * 8 + rem % 8;
  } else {
    *e = b / NJ;
    *j = b % NJ;
  }
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr float kF16Max = 65504.f;  // activations enter the MFMA as fp16: larger ones are reported

// The tokens' bf16 rows to fp16, 8 values a thread, once per layer: each row is staged by every
// workgroup of the K experts it is routed to, which then copy it as it is.  A value beyond the fp16
// range sets bit 8 of the engine's device error word (it would become an infinity).
__global__ void __launch_bounds__(256)
k_pf_x16(const uint16_t* __restrict__ x, int64_t n8, uint16_t* __restrict__ x16, int32_t* err) {
  bool bad = false;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    const uint4 v = reinterpret_cast<const uint4*>(x)[i];
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float lo = __uint_as_float(wv[k] << 16), hi = __uint_as_float(wv[k] & 0xFFFF0000u);
      bad |= !(fabsf(lo) <= kF16Max) || !(fabsf(hi) <= kF16Max);
      o[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), f16x2_t));
    }
    reinterpret_cast<uint4*>(x16)[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
  if (err && __ballot(bad) && (threadIdx.x & 63) == 0) __hip_atomic_fetch_or(err, 8, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// two floats -> fp16 pair (round to nearest even; one v_cvt_pk_f16_f32)
__device__ inline uint32_t pk_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), f16x2_t));
}

__device__ inline uint32_t pk_mul(uint32_t a, uint32_t s2) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2_t, a) * __builtin_bit_cast(f16x2_t, s2));
}
__device__ inline uint32_t pk_fma_off(uint32_t a, uint32_t off2, uint32_t s2) {
  // (a + off) * s in fp16 pairs; both steps exact for the value ranges used here
  f16x2_t v = __builtin_bit_cast(f16x2_t, a) + __builtin_bit_cast(f16x2_t, off2);
  return __builtin_bit_cast(uint32_t, v * __builtin_bit_cast(f16x2_t, s2));
}

// 8 weights (one lane, one n-subtile) -> B fragment of 8 fp16 values in MFMA k order
template <int FMT>
__device__ inline f16x8_t dequant8(uint32_t d, uint32_t s2) {
  uint32_t o[4];
  if (FMT == EFF_WFMT_NVFP4_G16_E4M3) {
    o[0] = pk_mul(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 0)), s2);
    o[1] = pk_mul(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 1)), s2);
    o[2] = pk_mul(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 2)), s2);
    o[3] = pk_mul(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(d, 1.0f, 3)), s2);
  } else {
    // pairs (e0,e4), (e1,e5), (e2,e6), (e3,e7); the activation tile uses the same order.  A nibble
    // at bits 0-3 of a half, under exponent 2^10, reads 1024 + u; at bits 4-7, under 2^6, 64 + u
    // (mantissa weight 2^-4 * 2^6 per unit); nibbles 2 and 3 take the same two forms after one shift.
    const uint32_t d8 = d >> 8;
    o[0] = pk_fma_off((d & 0x000F000Fu) | 0x64006400u, 0xE408E408u, s2);   // -1032
    o[1] = pk_fma_off((d & 0x00F000F0u) | 0x54005400u, 0xD480D480u, s2);   // -72
    o[2] = pk_fma_off((d8 & 0x000F000Fu) | 0x64006400u, 0xE408E408u, s2);  // -1032
    o[3] = pk_fma_off((d8 & 0x00F000F0u) | 0x54005400u, 0xD480D480u, s2);  // -72
  }
  uint4 u4 = make_uint4(o[0], o[1], o[2], o[3]);
  return __builtin_bit_cast(f16x8_t, u4);
}

__device__ inline float silu(float z) { return z / (1.0f + expf(-z)); }

// fp16 pair of a raw scale (int4: bf16 bits; NVFP4: an e4m3 byte), for packed multiplies
template <int FMT>
__device__ inline uint32_t scale_pair(uint32_t raw) {
  const float f = (FMT == EFF_WFMT_NVFP4_G16_E4M3) ? __builtin_amdgcn_cvt_f32_fp8(raw, 0) : __uint_as_float(raw << 16);
  return pk_f16(f, f);
}

constexpr int kMT = 64;         // tokens per pass (4 MFMA subtiles of 16)
constexpr int kCT = 8;          // k-tiles (of 32 inputs) per staged activation chunk
constexpr int kRowU32 = 132;    // LDS row stride in dwords: 256 fp16 + 4 dwords of padding
constexpr int kGRow = 260;      // row stride (floats) of the gate results handed to the up waves
static_assert(kMT * kGRow <= 2 * kMT * kRowU32, "gate results fit the staging buffers");

// Grouped expert GEMM over the (t,k) pairs sorted by expert.  Workgroup = (expert, WPM * 64 output
// rows) with NMAT * WPM waves: wave w computes 64 rows (4 row slices of 16) of matrix w / WPM.  All
// waves share the activation rows of the expert, staged in LDS as fp16 in chunks of 8 k-tiles
// (256 inputs), double buffered with one barrier per chunk: the next chunk's global loads are
// issued before the current chunk's MFMAs.  Weights stream from the slot into registers PF
// k-tiles ahead and are dequantized into the MFMA B operand.
//   NMAT 2: gate (waves 0..WPM-1) and up (the next WPM) from x (fp16 rows of the tokens); the gate waves
//           hand g to the up waves through LDS; a = silu(g) * u -> fp16, one row per sorted pair
//   NMAT 1: down from a (fp16 sorted rows) -> y (fp32, one row per (t,k) pair)
// FULL: H and I are multiples of 256 (whole chunks, whole row blocks): no per-k-tile checks, and
// loads past the end re-read the last k-tile instead of being skipped (no branches around memory
// operations, so the compiler's wait counts stay exact and the prefetch stays in flight).
template <int NMAT>
constexpr int pf_wpm() { return NMAT == 2 ? kPfGateupWPM : 4; }
template <int NMAT>
constexpr int pf_threads() { return 64 * NMAT * pf_wpm<NMAT>(); }

template <int FMT, int NMAT, int PF, bool FULL>
__global__ void __launch_bounds__(pf_threads<NMAT>(), pf_threads<NMAT>() > 256 ? 1 : 2)
k_pf_gemm(const uint8_t* __restrict__ arena, int64_t R, const float* __restrict__ ts,
          const int32_t* __restrict__ owner, int slot_base, const int32_t* __restrict__ slot_of,
          const int32_t* __restrict__ offsets, const int32_t* __restrict__ rows, const uint16_t* __restrict__ src,
          int E, int H, int I, int K, uint16_t* __restrict__ a_out, float* __restrict__ y_out, int32_t* err) {
  constexpr int WPM = pf_wpm<NMAT>();        // waves per matrix
  constexpr int TPB = pf_threads<NMAT>();    // threads
  constexpr int SEGS = TPB / kMT;            // staging threads per row
  constexpr int SEGW = 256 / SEGS;           // inputs per staging thread per chunk
  constexpr int SV = SEGW / 8;               // 16-byte vectors per staging thread
  __shared__ uint32_t s_a[2][kMT * kRowU32];
  // FULL: each wave's scale bytes of a chunk (4 slices x 8 k-tiles x 32 bytes), double buffered
  __shared__ __attribute__((aligned(16))) uint8_t s_sc[2][NMAT * WPM][FULL ? 4 * kCT * 32 : 16];
  const int N = (NMAT == 2) ? I : H, Kd = (NMAT == 2) ? H : I;
  const int NJ = (N / 64 + WPM - 1) / WPM;
  int e, j;
  map_block(blockIdx.x, E, NJ, &e, &j);
  if (e >= E) return;
  const int off = offsets[e], ne = offsets[e + 1] - off;
  if (ne <= 0) return;
  const int slot = slot_base >= 0 ? slot_base + e : slot_of[e];
  const uint8_t* rec = arena + (int64_t)slot * R;
  const int64_t pay = (int64_t)H * I / 2, sca = (int64_t)H * I / 16;
  const int KB = Kd / 32, nchunk = (KB + kCT - 1) / kCT;
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, r = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mat = wave / WPM, wl = wave % WPM;
  const int nb = j * WPM + wl;
  // waves past the last row block only help stage (never with FULL: both dimensions are whole chunks)
  const bool active = FULL || nb < N / 64;
  const int mi = (NMAT == 2) ? mat : 2;  // gate, up | down
  // this wave's 4 row slices: tiles tstride bytes apart, k tiles 256 bytes apart.  The record is read
  // through a buffer resource: the per-lane part of each address is a constant offset register and the
  // k-tile part a scalar offset, so the weight stream costs no vector address arithmetic (a record is
  // far below 2 GiB, so 32-bit offsets suffice).
  const int tstride = KB * 256, sstride = KB * 32;
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)rec, (short)0, (int)R, 0x00020000);
  int woff[4], soff[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    woff[t] = (int)(mi * pay) + ((active ? nb : 0) * 4 + t) * tstride + lane * 4;
    soff[t] = (int)(3 * pay + mi * sca) + ((active ? nb : 0) * 4 + t) * sstride +
              (FMT == EFF_WFMT_INT4_G32_BF16 ? r * 2 : (q >> 1) * 16 + r);
  }
  float tsc = 1.f;
  if (FMT == EFF_WFMT_NVFP4_G16_E4M3) tsc = ts[(int64_t)owner[slot] * 3 + mi];
  // FULL: the scales of a slice's 8 k-tiles of a chunk are 256 contiguous bytes, so one LDS-direct
  // copy per chunk brings the wave's 4 slices (lane l: slice l/16, bytes 16(l%16)..+15) into
  // s_sc[buf][wave] = [slice][k-tile of the chunk][32 bytes], with no register held while in flight;
  // each k-tile then reads its lane's byte (int4: bf16) back.  Without FULL the scales stream
  // beside the weights in registers.
  const uint8_t* scb = rec + 3 * pay + mi * sca + (int64_t)((active ? nb : 0) * 4 + (lane >> 4)) * sstride +
                       (lane & 15) * 16;
  const uint32_t sc_lds0 = lds_address(&s_sc[0][wave][0]), sc_lds1 = lds_address(&s_sc[1][wave][0]);
  const int sc_lane = (FMT == EFF_WFMT_INT4_G32_BF16) ? r * 2 : (q >> 1) * 16 + r;
  auto sc_copy = [&](int c, int buf) {
    if constexpr (FULL) lds_copy16(scb + (int64_t)c * kCT * 32, buf ? sc_lds1 : sc_lds0);
  };
  // Staging role: row srow; piece z (8 inputs, 16 bytes) of the chunk starts at input pbase + z * pstep.
  // Every 16 (and every 8) consecutive lanes of a 16-byte LDS store hit distinct bank groups (the
  // row stride of 132 dwords advances the bank by 4 per row):
  //   NMAT 2: 8 lanes read one 128-byte line of a row (pieces interleaved); the two 8-lane halves of
  //           a 16-lane group take rows 8 apart (32 banks apart); wave w stages rows w, w+8, ..
  //   NMAT 1: each thread stages one contiguous 64-input segment; lane bits 0-2 row, 3-4 segment,
  //           5 row + 8
  const int srow = (TPB == 512) ? wave + (lane >> 3) * 8 : wave * 16 + (lane & 7) + (lane >> 5) * 8;
  const int pbase = (TPB == 512) ? (lane & 7) * 8 : ((lane >> 3) & 3) * SEGW;
  constexpr int pstep = (TPB == 512) ? 64 : 8;
  static_assert(TPB == 512 || TPB == 256, "the two staging maps");

  bool range_bad = false;  // an activation or SwiGLU output beyond the fp16 range (becomes inf)
  for (int m0 = 0; m0 < ne; m0 += kMT) {
    const int mt = min(kMT, ne - m0);
    // rows past mt stage the pass's first row again (their results are discarded)
    const int prow = off + m0 + (srow < mt ? srow : 0);
    const uint16_t* srow_ptr = (NMAT == 2) ? src + (int64_t)(rows[prow] / K) * H : src + (int64_t)prow * I;
    f32x4_t acc[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) acc[t][s2] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    uint4 stg[SV];
    auto stage_load = [&](int c) {
      const int k0 = c * kCT * 32 + pbase, kn = min(kCT, KB - c * kCT) * 32;
#pragma unroll
      for (int z = 0; z < SV; ++z) {
        if (FULL) stg[z] = *reinterpret_cast<const uint4*>(srow_ptr + k0 + z * pstep);
        else
          stg[z] = (pbase + z * pstep < kn) ? *reinterpret_cast<const uint4*>(srow_ptr + k0 + z * pstep)
                                            : make_uint4(0u, 0u, 0u, 0u);
      }
    };
    auto stage_store = [&](int buf) {
      uint32_t* dst = s_a[buf] + srow * kRowU32 + pbase / 2;
#pragma unroll
      for (int z = 0; z < SV; ++z) {
        const uint4 v = stg[z];
        uint32_t o[4];
        // fp16 rows (x converted once by k_pf_x16, or a): int4 pairs (0,4), (1,5), (2,6), (3,7)
        if (FMT == EFF_WFMT_INT4_G32_BF16) {  // fp16 halves h0..h7 -> pairs (0,4) ...
          o[0] = (v.x & 0xFFFFu) | (v.z << 16);
          o[1] = (v.x >> 16) | (v.z & 0xFFFF0000u);
          o[2] = (v.y & 0xFFFFu) | (v.w << 16);
          o[3] = (v.y >> 16) | (v.w & 0xFFFF0000u);
        } else {
          o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
        }
        *reinterpret_cast<uint4*>(dst + z * (pstep / 2)) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    };
    // weight ring: k-tile kb lives in slot kb % PF
    uint32_t wq[PF][4], sq[FULL ? 1 : PF][4];
    auto wtile = [&](int k, int ring) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        wq[ring][t] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, woff[t], k * 256, 0);
        if constexpr (!FULL)
          sq[ring][t] = (FMT == EFF_WFMT_INT4_G32_BF16)
                            ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rsrc, soff[t], k * 32, 0)
                            : (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rsrc, soff[t], k * 32, 0);
      }
    };
    auto wload = [&](int kb, int ring) {
      if (FULL) {
        wtile(min(kb, KB - 1), ring);
      } else if (active && kb < KB) {
        wtile(kb, ring);
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          wq[ring][t] = 0u;
          if constexpr (!FULL) sq[ring][t] = 0u;
        }
      }
    };
    stage_load(0);
    sc_copy(0, 0);
    if constexpr (FULL) vm_wait<0>();  // chunk 0's scales are in LDS (with the stage loads)
    stage_store(0);
#pragma unroll
    for (int p = 0; p < PF; ++p) wload(p, p);
    __syncthreads();
    for (int c = 0; c < nchunk; ++c) {
      const int buf = c & 1;
      if (c + 1 < nchunk) {
        stage_load(c + 1);
        sc_copy(c + 1, buf ^ 1);
      }
      const uint32_t* abase = s_a[buf] + r * kRowU32 + q * 4;
      const uint8_t* sbase = &s_sc[buf][wave][0] + sc_lane;
      // A fragments (all 4 subtiles; rows past mt are discarded: no branches) and, with FULL, the
      // lane's scales of the 4 slices, read one k-tile ahead
      f16x8_t an[4];
      uint32_t sn[4];
      auto aread = [&](int kk) {
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2)
          an[s2] = __builtin_bit_cast(f16x8_t, *reinterpret_cast<const uint4*>(abase + s2 * 16 * kRowU32 + kk * 16));
        if constexpr (FULL) {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            sn[t] = (FMT == EFF_WFMT_INT4_G32_BF16)
                        ? (uint32_t)*reinterpret_cast<const uint16_t*>(sbase + t * kCT * 32 + kk * 32)
                        : (uint32_t)sbase[t * kCT * 32 + kk * 32];
        }
      };
      aread(0);
#pragma unroll
      for (int kk = 0; kk < kCT; ++kk) {
        const int kb = c * kCT + kk;
        // k-tile boundary: work on ring slots of later k-tiles (their loads may still be in flight) is
        // not hoisted into this one, which would wait on the whole prefetch
        __builtin_amdgcn_sched_barrier(0);
        if (FULL || kb < KB) {  // uniform
          f16x8_t af[4];
          uint32_t sc[4];
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) af[s2] = an[s2];
#pragma unroll
          for (int t = 0; t < 4; ++t) sc[t] = FULL ? sn[t] : sq[FULL ? 0 : kk % PF][t];
          if (kk + 1 < kCT) aread(kk + 1);
          const int ring = kk % PF;  // kCT % PF == 0: static after unrolling
          uint32_t w[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) w[t] = wq[ring][t];
          wload(kb + PF, ring);  // prefetch
          __builtin_amdgcn_sched_barrier(0);  // keep the prefetch issued ahead of this k-tile's math
          if (active) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const f16x8_t bfrag = dequant8<FMT>(w[t], scale_pair<FMT>(sc[t]));
#pragma unroll
              for (int s2 = 0; s2 < 4; ++s2)
                acc[t][s2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[s2], bfrag, acc[t][s2], 0, 0, 0);
            }
            // issue pattern: the first slice's dequant, then each MFMA followed by a few VALU ops of the
            // next slice's dequant, so one wave keeps the matrix pipe fed while it dequantizes
            __builtin_amdgcn_sched_group_barrier(0x002, kPfLead, 0);
#pragma unroll
            for (int i = 0; i < 12; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, kPfPer, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          }
        }
      }
      // the next chunk's scales: their copy was issued before this chunk's 4 * kCT weight loads
      if constexpr (FULL) vm_wait<4 * kCT>();
      if (c + 1 < nchunk) stage_store(buf ^ 1);
      __syncthreads();
    }
    // epilogue: accumulator (t, s2, i) is row m0 + s2*16 + 4q + i, column nb*64 + t*16 + r
    if (NMAT == 2) {
      float* g_lds = reinterpret_cast<float*>(&s_a[0][0]);  // [64 rows][256 columns + 4 padding]
      if (mat == 0 && active) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
            for (int i = 0; i < 4; ++i) g_lds[(s2 * 16 + q * 4 + i) * kGRow + wl * 64 + t * 16 + r] = acc[t][s2][i] * tsc;
      }
      __syncthreads();
      if (mat == 1 && active) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int rr = s2 * 16 + q * 4 + i;
              if (rr < mt) {
                const float g = g_lds[rr * kGRow + wl * 64 + t * 16 + r];
                const float a = silu(g) * (acc[t][s2][i] * tsc);
                if (!(fabsf(a) <= kF16Max)) range_bad = true;
                const _Float16 av = (_Float16)a;
                a_out[(int64_t)(off + m0 + rr) * I + nb * 64 + t * 16 + r] = __builtin_bit_cast(uint16_t, av);
              }
            }
      }
      __syncthreads();  // the LDS is restaged by the next pass
    } else if (active) {
      int prow[4][4];  // output rows of this lane, loaded together before any store
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = s2 * 16 + q * 4 + i;
          prow[s2][i] = rows[off + m0 + (rr < mt ? rr : 0)];
        }
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int rr = s2 * 16 + q * 4 + i;
            if (rr < mt) y_out[(int64_t)prow[s2][i] * H + nb * 64 + t * 16 + r] = acc[t][s2][i] * tsc;
          }
    }
  }
  if (err && __ballot(range_bad) && lane == 0) __hip_atomic_fetch_or(err, 8, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

}  // namespace

hipError_t launch_prefill(eff_engine* e, int layer, const uint16_t* x, const int32_t* ids, const float* w,
                          int T, uint16_t* out, const int32_t* slot_of_expert, int slot_base, bool combine,
                          hipStream_t s) {
  (void)layer;
  const eff_config& c = e->cfg;
  const int E = c.num_experts, H = c.hidden, I = c.inter, K = c.top_k;
  const int n = T * K;
  hipLaunchKernelGGL(k_pf_sort, dim3(1), dim3(1024), (size_t)E * sizeof(int32_t), s, ids, n, E, slot_base,
                     slot_of_expert, e->d_pf_count, e->d_pf_rows);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const bool fp4 = c.wformat == EFF_WFMT_NVFP4_G16_E4M3;
  constexpr int wg = pf_wpm<2>(), wd = pf_wpm<1>();
  const int nbx1 = ((E + 7) / 8) * 8 * ((I / 64 + wg - 1) / wg);
  const int nbx2 = ((E + 7) / 8) * 8 * ((H / 64 + wd - 1) / wd);
  // timed outside a capture: each GEMM sets its own start and end events (its own duration)
  const bool own = (c.flags & EFF_CFG_TIMING) && !stream_capturing(s);
  const int ts = timing_begin(e, EFF_T_PREFILL_GATEUP, s, !own);
  hipEvent_t t0 = own ? timing_event(e, ts, 0) : nullptr, t1 = own ? timing_event(e, ts, 1) : nullptr;
  const bool full = H % 256 == 0 && I % 256 == 0;
#define EFF_PF_LAUNCH(F, NM, PFD, FU, GRID, SRC, AO, YO)                                                        \
  hipExtLaunchKernelGGL((k_pf_gemm<F, NM, PFD, FU>), dim3(GRID), dim3(pf_threads<NM>()), 0, s, t0, t1, 0, e->d_arena, e->R, \
                        e->d_ts, e->d_owner, slot_base, slot_of_expert, (const int32_t*)e->d_pf_count,          \
                        (const int32_t*)e->d_pf_rows, (const uint16_t*)(SRC), E, H, I, K, AO, YO, e->h_err_dev)
#define EFF_PF_PICK(NM, PFD, FU, GRID, SRC, AO, YO)                                           \
  do {                                                                                        \
    if (fp4) {                                                                                \
      if (FU) EFF_PF_LAUNCH(EFF_WFMT_NVFP4_G16_E4M3, NM, PFD, true, GRID, SRC, AO, YO);       \
      else EFF_PF_LAUNCH(EFF_WFMT_NVFP4_G16_E4M3, NM, PFD, false, GRID, SRC, AO, YO);         \
    } else {                                                                                  \
      if (FU) EFF_PF_LAUNCH(EFF_WFMT_INT4_G32_BF16, NM, PFD, true, GRID, SRC, AO, YO);        \
      else EFF_PF_LAUNCH(EFF_WFMT_INT4_G32_BF16, NM, PFD, false, GRID, SRC, AO, YO);          \
    }                                                                                         \
  } while (0)
  // the tokens' rows to fp16 once; timed, the gate/up interval starts at this kernel
  const int64_t n8 = (int64_t)T * H / 8;
  const int xg = (int)std::min<int64_t>((n8 + 255) / 256, 2048);
  if (own)
    hipExtLaunchKernelGGL(k_pf_x16, dim3(xg), dim3(256), 0, s, t0, nullptr, 0, x, n8, e->d_pf_x, e->h_err_dev);
  else
    hipLaunchKernelGGL(k_pf_x16, dim3(xg), dim3(256), 0, s, x, n8, e->d_pf_x, e->h_err_dev);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  t0 = nullptr;
  EFF_PF_PICK(2, kPfPrefetch2, full, nbx1, e->d_pf_x, e->d_pf_a, (float*)nullptr);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (!own) {
    timing_mark(e, ts, 1, s);
    timing_mark(e, ts, 2, s);
  }
  t0 = own ? timing_event(e, ts, 2) : nullptr;
  t1 = own ? timing_event(e, ts, 3) : nullptr;
  EFF_PF_PICK(1, kPfPrefetch1, full, nbx2, e->d_pf_a, (uint16_t*)nullptr, e->d_pf_y);
#undef EFF_PF_PICK
#undef EFF_PF_LAUNCH
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (!own) timing_mark(e, ts, 3, s);
  if (!combine) return hipSuccess;
  return launch_combine(e->d_pf_y, nullptr, nullptr, w, T, K, H, out, s);
}

}  // namespace eff
