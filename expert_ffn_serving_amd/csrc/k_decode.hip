// Decode expert FFN: y = W_d (silu(W_g x) * (W_u x)) per GPU-owned (token, k) entry,
// straight from the slot bytes, with weights dequantized in registers.
//
// The step is bound by HBM bandwidth: every routed expert's weights are read in
// full per step ([FT-blog] §三.2).  Each distinct slot's record is read once for
// all tokens routed to it.  Work is split three ways:
//   (plan)      distinct GPU slots of the call and their entries, one record per slot,
//               made by the control kernels (k_plan or the fused k_control)
//   k_gateup    gate and up rows of one 16-row slice over all of H, both matrices
//               at once, reduced inside the workgroup, SwiGLU applied; the result is
//               written as fp16 in the order k_down reads it, scaled per (token, slice)
//               by a power of two into [2^14, 2^15), with the scale and (int4) the sum
//               of every 8-group beside it
//   k_down      one 16-row slice of the down matrix over all of I
// No workgroup depends on another inside a kernel, so no device-scope fence is
// needed (on this multi-die part such a fence writes back and invalidates a whole
// L2 per wave).
//   k_combine   out[t] = sum over k of w[t,k] * y[t,k] (fixed k order), bf16 RNE
// Every reduction has a fixed order (no float atomics): results are bitwise
// reproducible from run to run.
//
// Register dequantization:
//   int4   nibble u -> bf16(128 + u) by OR-ing it under 0x4300; a 2-wide bf16 dot
//          then gives sum (128+u) x, and sum (u-8) x = that - 136 * sum x.  In the
//          down projection the activations are fp16 and the base is fp16(1024+u).
//   e2m1   v_cvt_scalef32_pk_{bf16,f16}_fp4 with scale 1.0 (the instruction uses
//          only the exponent of its scale operand, so the e4m3 block scale is
//          applied afterwards in fp32); e4m3 via v_cvt_f32_fp8 (OCP E4M3FN).
#include <hip/hip_ext.h>

#include <mutex>

#include "eff_internal.h"
#include "lds_dma.h"

namespace eff {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

constexpr int kWG = 256;  // 4 waves

// Workgroup wg of nwg (kWG threads) copies its share of a fetch list's records from the pinned host
// pool into their slots: 16 KiB chunks in turn, 16 bytes per thread; entries outside the pool or the
// arena are skipped.
__device__ void copy_fetch_list(const uint8_t* __restrict__ pool, uint8_t* __restrict__ arena, int64_t R,
                                int64_t n_flat, int S, const FetchList* __restrict__ fl, int wg, int nwg) {
  constexpr int64_t kChunk = 16384;
  const int n = min(fl->count, kMaxEntries);
  const int64_t chunks = (R + kChunk - 1) / kChunk;
  for (int64_t c = wg; c < (int64_t)n * chunks; c += nwg) {
    const int i = (int)(c / chunks);
    const int64_t off = (c % chunks) * kChunk, len = min(kChunk, R - off);
    const int flat = fl->flat[i], slot = fl->slot[i];
    if (flat < 0 || flat >= n_flat || slot < 0 || slot >= S) continue;
    const uint4* src = reinterpret_cast<const uint4*>(pool + (int64_t)flat * R + off);
    uint4* dst = reinterpret_cast<uint4*>(arena + (int64_t)slot * R + off);
    for (int64_t b = threadIdx.x; b < len / 16; b += kWG) dst[b] = src[b];
  }
}

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ inline float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b),
                                         c, false);
}
__device__ inline float dot2_f16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c, false);
}

template <int SEL>
__device__ inline uint32_t fp4_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL));
}
template <int SEL>
__device__ inline uint32_t fp4_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL));
}

__device__ inline float silu(float z) { return z / (1.0f + expf(-z)); }

// ---------------------------------------------------------------------------- gate / up
// A matrix is stored as 16-row x 32-input tiles, row slices outer: the 16 rows of slice sl are
// one contiguous run of (Kd/32) tiles of 256 payload bytes (and 32 scale bytes).  Inside a tile,
// the dword at byte 4*(q*16 + r) holds row r, inputs 8q..8q+7.
//
// A wave reads a slice in 1 KiB runs of 4 consecutive tiles, one 16-byte load per lane.  Lane l
// gets bytes 16l..16l+15 of the run: tile t = l/16 of the run, rows 4g..4g+3 (g = l%4), inputs
// 8q..8q+7 of the tile (q = (l/4)%4), one dword per row.  Its scales are one aligned word of the
// tile's scale bytes (NVFP4: the 4 e4m3 bytes of its rows in group q/2; int4: the 4 bf16 of its
// rows), and the 8 inputs it needs, x[128*run + 8*(l/4) ...], are shared by its 4 rows.  The partial
// sums of row 4g+j end in the 16 lanes with l%4 = g and are added by a fixed butterfly.

// Copies n bytes (n % 16 == 0, both ends 16-byte aligned) with the whole workgroup, 16 bytes per
// thread and four loads in flight per thread.
__device__ inline void wg_copy(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t n) {
  const uint4* s4 = reinterpret_cast<const uint4*>(src);
  uint4* d4 = reinterpret_cast<uint4*>(dst);
  const int64_t n4 = n / 16;
  int64_t i = threadIdx.x;
  for (; i + 3 * kWG < n4; i += 4 * kWG) {
    const uint4 a = s4[i], b = s4[i + kWG], c = s4[i + 2 * kWG], d = s4[i + 3 * kWG];
    d4[i] = a;
    d4[i + kWG] = b;
    d4[i + 2 * kWG] = c;
    d4[i + 3 * kWG] = d;
  }
  for (; i < n4; i += kWG) d4[i] = s4[i];
}

// the lane's scale word inside a tile's 32 scale bytes (NVFP4: 4 bytes; int4: 8 bytes)
template <int FMT>
__device__ inline int lane_scale_off(int q, int g) {
  return FMT == EFF_WFMT_INT4_G32_BF16 ? 8 * g : 16 * (q >> 1) + 4 * g;
}
struct Scales4 {
  uint32_t a, b;  // NVFP4: a = e4m3 of rows 4g..4g+3 (byte j = row 4g+j); int4: a, b = bf16 pairs
};
template <int FMT>
__device__ inline Scales4 load_scales4(const uint8_t* p) {
  Scales4 s;
  if (FMT == EFF_WFMT_INT4_G32_BF16) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    s.a = v.x;
    s.b = v.y;
  } else {
    s.a = *reinterpret_cast<const uint32_t*>(p);
    s.b = 0;
  }
  return s;
}
template <int FMT>
__device__ inline void scale_values(const Scales4& s, float (&v)[4]) {
  if (FMT == EFF_WFMT_INT4_G32_BF16) {
    v[0] = bf16_lo(s.a);
    v[1] = bf16_hi(s.a);
    v[2] = bf16_lo(s.b);
    v[3] = bf16_hi(s.b);
  } else {
    v[0] = __builtin_amdgcn_cvt_f32_fp8(s.a, 0);
    v[1] = __builtin_amdgcn_cvt_f32_fp8(s.a, 1);
    v[2] = __builtin_amdgcn_cvt_f32_fp8(s.a, 2);
    v[3] = __builtin_amdgcn_cvt_f32_fp8(s.a, 3);
  }
}

// 8 bf16 activations -> the 4 pairs that meet the weight pairs of one dword
template <int FMT>
__device__ inline void x_pairs(const uint4 v, uint32_t* xw) {
  if (FMT == EFF_WFMT_INT4_G32_BF16) {
    // pairs (x0,x4), (x1,x5), (x2,x6), (x3,x7) meet the nibble pairs (e0,e4) ...
    xw[0] = (v.x & 0xFFFFu) | (v.z << 16);
    xw[1] = (v.x >> 16) | (v.z & 0xFFFF0000u);
    xw[2] = (v.y & 0xFFFFu) | (v.w << 16);
    xw[3] = (v.y >> 16) | (v.w & 0xFFFF0000u);
  } else {
    xw[0] = v.x; xw[1] = v.y; xw[2] = v.z; xw[3] = v.w;
  }
}

// one weight dword (8 inputs of one row) as 4 bf16 pairs that meet the paired activations: int4
// nibble u becomes bf16(128 + u) (OR-ed under 0x4300), e2m1 is converted exactly
template <int FMT>
__device__ inline void dequant_bf16(uint32_t d, uint32_t (&p)[4]) {
  if (FMT == EFF_WFMT_INT4_G32_BF16) {
    p[0] = (d & 0x000F000Fu) | 0x43004300u;
    p[1] = ((d >> 4) & 0x000F000Fu) | 0x43004300u;
    p[2] = ((d >> 8) & 0x000F000Fu) | 0x43004300u;
    p[3] = ((d >> 12) & 0x000F000Fu) | 0x43004300u;
  } else {
    p[0] = fp4_to_bf16x2<0>(d); p[1] = fp4_to_bf16x2<1>(d);
    p[2] = fp4_to_bf16x2<2>(d); p[3] = fp4_to_bf16x2<3>(d);
  }
}

// The lane's 4 rows of one matrix in one run against `nt` tokens (paired activations xw, and for
// int4 the sum of each token's 8 inputs, which takes off the 128 + u encoding and the -8 offset:
// sum (u - 8) x = sum (128 + u) x - 136 sum x).  Each row's dword is dequantized once for all tokens.
template <int FMT, int NT>
__device__ inline void matrix_run(const uint4 w, const Scales4& rs, const uint32_t (&xw)[NT][4], const float (&xs)[NT],
                                  int nt, float (&acc)[4][NT]) {
  float s[4];
  scale_values<FMT>(rs, s);
  const uint32_t d4[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    uint32_t p[4];
    dequant_bf16<FMT>(d4[r], p);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if (NT > 1 && j >= nt) break;
      float raw = dot2_bf16(p[3], xw[j][3], dot2_bf16(p[2], xw[j][2], dot2_bf16(p[1], xw[j][1],
                  dot2_bf16(p[0], xw[j][0], 0.f))));
      if (FMT == EFF_WFMT_INT4_G32_BF16) raw = fmaf(-136.f, xs[j], raw);
      acc[r][j] = fmaf(s[r], raw, acc[r][j]);
    }
  }
}

// the lane's share of one run of one matrix against `nt` tokens (nt uniform per wave, NT > 1 stops there)
template <int FMT, int NT>
__device__ inline void run_tokens(const uint4 w, const Scales4& rs, const uint4* xv, int nt, float (&acc)[4][NT]) {
  uint32_t xw[NT][4];
  float xs[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    if (NT > 1 && j >= nt) break;
    x_pairs<FMT>(xv[j], xw[j]);
    xs[j] = 0.f;
    if (FMT == EFF_WFMT_INT4_G32_BF16)
      xs[j] = dot2_bf16(xw[j][3], 0x3F803F80u, dot2_bf16(xw[j][2], 0x3F803F80u,
                        dot2_bf16(xw[j][1], 0x3F803F80u, dot2_bf16(xw[j][0], 0x3F803F80u, 0.f))));
  }
  matrix_run<FMT, NT>(w, rs, xw, xs, nt, acc);
}

// The same for NT > 1 tokens whose 8 inputs are read from LDS (token j at sx[j * stride]): the 4 rows
// are dequantized first and each token's activations read only when they meet them, so the
// registers hold one token's activations at a time (same operations, same order as run_tokens).
template <int FMT, int NT>
__device__ inline void run_tokens_lds(const uint4 w, const Scales4& rs, const uint4* sx, int stride, int nt,
                                      float (&acc)[4][NT]) {
  float s[4];
  scale_values<FMT>(rs, s);
  const uint32_t d4[4] = {w.x, w.y, w.z, w.w};
  uint32_t p[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) dequant_bf16<FMT>(d4[r], p[r]);
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    if (j >= nt) break;
    uint32_t xw[4];
    x_pairs<FMT>(sx[j * stride], xw);
    float xs = 0.f;
    if (FMT == EFF_WFMT_INT4_G32_BF16)
      xs = dot2_bf16(xw[3], 0x3F803F80u, dot2_bf16(xw[2], 0x3F803F80u,
                     dot2_bf16(xw[1], 0x3F803F80u, dot2_bf16(xw[0], 0x3F803F80u, 0.f))));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float raw = dot2_bf16(p[r][3], xw[3], dot2_bf16(p[r][2], xw[2], dot2_bf16(p[r][1], xw[1],
                  dot2_bf16(p[r][0], xw[0], 0.f))));
      if (FMT == EFF_WFMT_INT4_G32_BF16) raw = fmaf(-136.f, xs, raw);
      acc[r][j] = fmaf(s[r], raw, acc[r][j]);
    }
  }
}

// Lane moves without LDS round trips: DPP inside rows of 16 lanes (CTRL: 0x120 + n rotates a row by n,
// 0x104 reads the lane 4 above in the row, 0xB1 / 0x4E swap neighbours / pairs in each quad).
template <int CTRL>
__device__ inline float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Adds v over the 16 lanes with the same l % 4 (l the lane id) in a fixed order: rotations by 4 and 8
// inside each row of 16 lanes, then gfx950's row swaps bring row 1 onto row 0 (and 3 onto 2) and rows
// 2-3 onto rows 0-1.  The sum is complete in lanes 0..15 only.
__device__ inline float sum16(float v) {
  v += dpp_f32<0x124>(v);
  v += dpp_f32<0x128>(v);
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  v += __builtin_bit_cast(float, (uint32_t)__builtin_amdgcn_permlane16_swap(b, b, false, false)[1]);
  const uint32_t c = __builtin_bit_cast(uint32_t, v);
  v += __builtin_bit_cast(float, (uint32_t)__builtin_amdgcn_permlane32_swap(c, c, false, false)[1]);
  return v;
}

// grid: (u2 * nch + maxU - u2) * (I/16) * P / 2 workgroups of 256 threads, one per (plan unit, token
// chunk, group of 2/P consecutive 16-row slices of I).  A slice takes 2P waves: P for its gate rows and P for its up rows, each wave
// every P-th run of its matrix; everything reduces inside the workgroup (the SwiGLU meets gate and
// up in LDS), so no workgroup ever waits for another.  A unit installed by this call (fetch) first
// copies its workgroup's gate and up slices from the pinned host pool into the slot (16-byte loads)
// and, once its rows are done, the same share of the down matrix: the whole record crosses the link
// inside this kernel, and k_down finds it resident.
template <int FMT, int NT, int P>
__global__ void __launch_bounds__(kWG, (FMT == EFF_WFMT_NVFP4_G16_E4M3 || NT < 8) ? 3 : 2)
k_gateup(uint8_t* arena, const uint8_t* __restrict__ pool, int64_t R, SpecCopy sc,
         const float* __restrict__ ts, const DecodePlan* __restrict__ plan, const uint16_t* __restrict__ x, int H,
         int I, int K, int maxB, int nch, int u2, uint16_t* __restrict__ a16, float2* __restrict__ ag) {
  static_assert(P == 1 || P == 2, "1 or 2 waves per matrix of a slice");
  constexpr int SPW = 2 / P;                      // slices per workgroup
  constexpr int UNR = NT == 1 ? 4 : NT == 2 ? 8 : NT == 4 ? 5 : 4;  // runs in flight per wave (NT = 4: 4 waves per SIMD)
  extern __shared__ uint4 s_x[];                  // NT > 1: [NT][H/8] token rows of the chunk, 1 KiB slack
  __shared__ float s_red[4][16][NT];
  if ((int)blockIdx.x < sc.nwg) {  // the front of the grid carries a speculative copy
    copy_fetch_list(pool, arena, R, sc.n_flat, sc.S, sc.fl, blockIdx.x, sc.nwg);
    return;
  }
  const int bid = blockIdx.x - sc.nwg;
  const int NS = I / 16, NG = NS / SPW, KB = H / 32, NRF = KB / 4;
  // Only the first u2 units (busiest first; no later unit can hold more than NT tokens) have nch
  // chunk blocks; the others one, which takes all their tokens.
  // Workgroups go to the 8 dies (XCDs) in turn by block number, and each die has its own L2.  The
  // slice groups of a unit's later chunks are rotated by their block's offset mod 8, so that most
  // of them run on the die that reads the same slices for chunk 0 (about the same time: the chunks
  // are adjacent in the grid) and find them in its L2 instead of reading the weights again.
  const int nA = u2 * nch * NG;
  const int nchu = bid < nA ? nch : 1;
  const int u = bid < nA ? bid / (NG * nch) : u2 + (bid - nA) / NG;
  const int ch = bid < nA ? (bid / NG) % nch : 0;
  const int sgp = ((bid < nA ? bid : bid - nA) % NG + (ch * NG) % 8) % NG;
  const DecodeUnit* un = &plan->unit[u];
  // The entries of chunk ch (lane l: entry ch*NT + l % NT), read at once rather than after the unit's
  // fields: they are the workgroup's first chunk unless a fetched unit takes all its chunks.  A
  // relaxed atomic load, which the compiler issues here instead of moving it behind the branch that
  // waits for those fields.  Lanes past the chunk's tokens read entries that are not used.
  const int e_first = __hip_atomic_load(const_cast<int32_t*>(&un->entry[min(ch * NT + (int)(threadIdx.x & 63) % NT,
                                                                               kMaxTokens - 1)]),
                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  const int cnt = un->count;
  // A resident unit's token chunks run in workgroups of their own (chunk ch: tokens ch*NT ..), so the
  // busiest experts do not run their chunks one after the other.  A unit installed by this call is
  // copied by its chunk-0 workgroups, which then take every chunk themselves.
  const int c_begin = un->fetch ? 0 : ch * NT;
  const int c_end = (un->fetch || ch == nchu - 1) ? cnt : min(cnt, (ch + 1) * NT);
  if (c_begin >= c_end || (un->fetch && ch > 0)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ss = wave / (2 * P), mat = (wave / P) & 1, wp = wave % P, sl = sgp * SPW + ss;
  const int t4 = lane >> 4, g = lane & 3, q = (lane >> 2) & 3;
  const int64_t pay = (int64_t)H * I / 2, sca = (int64_t)H * I / 16;
  uint8_t* rec = arena + (int64_t)un->slot * R;
  // NVFP4 tensor scales, read now: in the epilogue their load would be one more round trip to wait for
  float tsg = 1.f, tsu = 1.f;
  if (FMT == EFF_WFMT_NVFP4_G16_E4M3) {
    tsg = ts[(int64_t)un->flat * 3 + 0];
    tsu = ts[(int64_t)un->flat * 3 + 1];
  }
  if (un->fetch) {
    // installed by this call: copy this workgroup's gate and up slices (payload and scales) from
    // the pool into the slot, then read them back like any resident record
    const uint8_t* src = pool + (int64_t)un->flat * R;
    const int64_t po = (int64_t)sgp * SPW * KB * 256, so = 3 * pay + (int64_t)sgp * SPW * KB * 32;
    wg_copy(src + po, rec + po, (int64_t)SPW * KB * 256);
    wg_copy(src + pay + po, rec + pay + po, (int64_t)SPW * KB * 256);
    wg_copy(src + so, rec + so, (int64_t)SPW * KB * 32);
    wg_copy(src + sca + so, rec + sca + so, (int64_t)SPW * KB * 32);
    __syncthreads();
  }
  // run r of the wave's matrix slice: payload at +r*1024 (+16 lane), the lane's scale word at +(4r + t4)*32 + off
  const uint8_t* wp8 = rec + mat * pay + (int64_t)sl * KB * 256 + lane * 16;
  const uint8_t* sp8 = rec + 3 * pay + mat * sca + (int64_t)sl * KB * 32 + t4 * 32 + lane_scale_off<FMT>(q, g);
  const int xo = 8 * (lane >> 2);           // the lane's inputs in a run: 128 r + xo .. +7
  const bool tail = (KB & 3) != 0;          // a last run of 1..3 tiles (H % 128 != 0)
  const bool tail_lane = 4 * NRF + t4 < KB; // the lane's tile exists in that run
  const int H8 = H / 8;
  // the wave's runs are wp, wp + P, ...: nr of them; past the last one (and where there is none) a
  // load takes the last (or first) run again, so every load below is unconditional and the compiler
  // keeps UNR of them in flight (a load behind a branch makes it wait for all of them at the join)
  const int nr = NRF > wp ? (NRF - wp + P - 1) / P : 0;
  const int rlast = wp + P * max(nr - 1, 0);
  for (int c0 = c_begin; c0 < c_end; c0 += NT) {
    const int nt = min(NT, c_end - c0);
    float acc[4][NT];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[r][j] = 0.f;
    uint4 wv[UNR], xg[NT == 1 ? UNR : 1];
    Scales4 rs[UNR];
    // NT == 1: the token's row
    const uint16_t* xr = x + (int64_t)(__builtin_amdgcn_readfirstlane(c0 == ch * NT ? e_first : un->entry[c0]) / K) * H;
    const uint16_t* xt = xr + xo;
    // NT > 1: the chunk's token rows go to LDS straight from memory (no registers), 1 KiB per copy over
    // the rows laid end to end: lane l of copy c fills place 64 c + l of row (64 c + l) / (H/8); past the
    // last row it loads the last row's end into the slack behind s_x.  Every place is written by one
    // lane.  Issued before the weights' loads, and waited for below while those are still in flight.
    // The chunk's row numbers are read once (lane j holds token c0 + j's, lanes past nt repeat the
    // last): a load inside the copy loop would make every pass wait for all copies issued before it.
    if constexpr (NT > 1) {
      const int rowj = (c0 == ch * NT ? e_first : un->entry[c0 + min(lane % NT, nt - 1)]) / K;
      const uint32_t lds0 = lds_address(s_x);
      const int n = nt * H8;
      for (int c = wave; c < (n + 63) / 64; c += kWG / 64) {
        const int pl = min(c * 64 + lane, n - 1), j = pl / H8;
        const uint16_t* row = x + (int64_t)__shfl(rowj, j) * H;
        lds_copy16(row + (pl - j * H8) * 8, lds0 + c * 1024);
      }
    }
    auto load_run = [&](int z, int r) {
      wv[z] = *reinterpret_cast<const uint4*>(wp8 + (int64_t)r * 1024);
      rs[z] = load_scales4<FMT>(sp8 + r * 128);
      if constexpr (NT == 1) xg[z] = *reinterpret_cast<const uint4*>(xr + min(r * 128 + xo, H - 8));  // in the row
    };
#pragma unroll
    for (int z = 0; z < UNR; ++z) load_run(z, min(wp + P * z, rlast));
    if constexpr (NT > 1) {
      // the row copies are complete once at most the weights' 2 * UNR loads (issued after them) remain
      vm_wait<2 * UNR>();
      __syncthreads();
    }
    // a rolling pipeline: UNR register slots, each refilled with the run UNR ahead once it is used.
    // An iteration takes UNR runs, one per slot, and every path through it issues the same refills
    // (past the wave's last run only the arithmetic is skipped), so the loop head is reached with the
    // same loads in flight from before the loop and from its end, and the compiler's wait there
    // covers just the next run (a loop left from inside made it wait for every load in flight).
    for (int i0 = 0; i0 < nr; i0 += UNR) {
#pragma unroll
      for (int z = 0; z < UNR; ++z) {
        const int r = wp + P * (i0 + z);
        if (i0 + z < nr) {  // uniform
          if constexpr (NT == 1) {
            run_tokens<FMT, NT>(wv[z], rs[z], &xg[z], 1, acc);
          } else {
            run_tokens_lds<FMT, NT>(wv[z], rs[z], s_x + r * 16 + (lane >> 2), H8, nt, acc);
          }
        }
        load_run(z, min(r + P * UNR, rlast));
      }
    }
    if (tail && wp == NRF % P && tail_lane) {  // the last, partial run
      const int r = NRF;
      const uint4 w1 = *reinterpret_cast<const uint4*>(wp8 + (int64_t)r * 1024);
      const Scales4 s1 = load_scales4<FMT>(sp8 + r * 128);
      if constexpr (NT == 1) {
        const uint4 xv = *reinterpret_cast<const uint4*>(xt + r * 128);
        run_tokens<FMT, NT>(w1, s1, &xv, 1, acc);
      } else {
        run_tokens_lds<FMT, NT>(w1, s1, s_x + r * 16 + (lane >> 2), H8, nt, acc);
      }
    }
    // rows 4g+r: the 16 lanes with the same g, then the matrix's waves in order (through LDS)
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < NT; ++j)
        if (NT == 1 || j < nt) acc[r][j] = sum16(acc[r][j]);
    if (lane < 4) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < NT; ++j) s_red[wave][4 * lane + r][j] = acc[r][j];
    }
    __syncthreads();
    // 16 consecutive lanes per (slice, token), row = idx % 16; a whole 16-lane group is in or out of
    // each pass (kWG and the total are multiples of 16), so the group reductions below see all its rows
    for (int idx = tid; idx < SPW * 16 * nt; idx += kWG) {
      const int s2 = idx / (16 * nt), j = (idx / 16) % nt, row = idx & 15;
      const int wg0 = s2 * 2 * P, wu0 = wg0 + P;   // the slice's gate waves, then its up waves
      float gv = s_red[wg0][row][j], uv = s_red[wu0][row][j];
#pragma unroll
      for (int w2 = 1; w2 < P; ++w2) {
        gv += s_red[wg0 + w2][row][j];
        uv += s_red[wu0 + w2][row][j];
      }
      if (FMT == EFF_WFMT_NVFP4_G16_E4M3) {
        gv *= tsg;
        uv *= tsu;
      }
      const float a = silu(gv) * uv;
      // the slice's power-of-two scale: max |a| over its 16 rows lands in [2^14, 2^15)
      float mx = fabsf(a);  // over the group's 16 lanes, one DPP row
      mx = fmaxf(mx, dpp_f32<0x128>(mx));
      mx = fmaxf(mx, dpp_f32<0x124>(mx));
      mx = fmaxf(mx, dpp_f32<0x122>(mx));
      mx = fmaxf(mx, dpp_f32<0x121>(mx));
      int sh = 0;
      if (mx > 0.f) {
        int ex;
        frexpf(mx, &ex);  // mx < 2^ex
        sh = min(15 - ex, 100);
      }
      const _Float16 h = (_Float16)ldexpf(a, sh);
      float gsum = (float)h;  // sum of the 8-group (rows 8*(row/8) ..), complete in its first lane; int4 only
      gsum += dpp_f32<0xB1>(gsum);
      gsum += dpp_f32<0x4E>(gsum);
      gsum += dpp_f32<0x104>(gsum);
      // int4: the pairs (a_m, a_m+4) of each 8-group meet the nibble pairs of a weight dword
      const int pos = FMT == EFF_WFMT_INT4_G32_BF16 ? (row & 8) | ((row & 3) << 1) | ((row >> 2) & 1) : row;
      const int slice = sgp * SPW + s2;
      const int64_t tok = (int64_t)u * maxB + c0 + j;
      a16[tok * I + slice * 16 + pos] = __builtin_bit_cast(uint16_t, h);
      if ((row & 7) == 0) ag[tok * (I / 8) + slice * 2 + (row >> 3)] = make_float2(ldexpf(1.f, -sh), gsum);
    }
    __syncthreads();
  }
  if (un->fetch) {  // this workgroup's share of the down payload and scales
    const uint8_t* src = pool + (int64_t)un->flat * R;
    const int64_t dpo = 2 * pay + (int64_t)sgp * (pay / NG), dso = 3 * pay + 2 * sca + (int64_t)sgp * (sca / NG);
    wg_copy(src + dpo, rec + dpo, pay / NG);
    wg_copy(src + dso, rec + dso, sca / NG);
  }
}

// ---------------------------------------------------------------------------- down
// The lane's share of one run of the down matrix against `nt` tokens: its 8 inputs of the SwiGLU
// output are fp16 (already scaled per (token, 16-row slice of I) by k_gateup; int4 pairs them like
// the nibbles), with that 8-group's (2^-shift, sum) pair.
template <int FMT, int NT>
__device__ inline void down_run(const uint4 wd, const Scales4& rd, const uint4* s_a4, const float2* s_ag, int idx,
                                int nt, int I8, float (&acc)[4][NT]) {
  float sd[4];
  scale_values<FMT>(rd, sd);
  const uint32_t d4[4] = {wd.x, wd.y, wd.z, wd.w};
  uint32_t p[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t d = d4[r];
    if (FMT == EFF_WFMT_INT4_G32_BF16) {
      p[r][0] = (d & 0x000F000Fu) | 0x64006400u;
      p[r][1] = ((d >> 4) & 0x000F000Fu) | 0x64006400u;
      p[r][2] = ((d >> 8) & 0x000F000Fu) | 0x64006400u;
      p[r][3] = ((d >> 12) & 0x000F000Fu) | 0x64006400u;
    } else {
      p[r][0] = fp4_to_f16x2<0>(d); p[r][1] = fp4_to_f16x2<1>(d);
      p[r][2] = fp4_to_f16x2<2>(d); p[r][3] = fp4_to_f16x2<3>(d);
    }
  }
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    if (NT > 1 && j >= nt) break;
    const uint4 av = s_a4[j * I8 + idx];
    const float2 sg = s_ag[j * I8 + idx];  // (2^-shift of the slice, sum of the 8-group)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float raw = dot2_f16(p[r][3], av.w, dot2_f16(p[r][2], av.z, dot2_f16(p[r][1], av.y, dot2_f16(p[r][0], av.x, 0.f))));
      if (FMT == EFF_WFMT_INT4_G32_BF16) raw = fmaf(-1032.f, sg.y, raw);
      acc[r][j] = fmaf(sd[r], raw * sg.x, acc[r][j]);
    }
  }
}

// Tokens of a unit whose activations the down kernel stages into LDS at once (a multiple of NT): as
// many of the call's maxB as fit kDownLds bytes beside the 1 KiB slacks, never fewer than NT.
constexpr int kDownLds = 38 * 1024;  // 4 workgroups per CU (the kernel's register bound) within 160 KiB
inline int down_span(int NT, int maxB, int I) {
  const int fit = (kDownLds - 2048) / ((I / 8) * 24) / NT * NT;
  return std::max(NT, std::min(maxB, fit));
}
inline int down_lds_bytes(int NT, int maxB, int I) { return down_span(NT, maxB, I) * (I / 8) * 24 + 2048; }

// grid: maxU * (H/16) / (4/WPS) workgroups, one per (plan unit, group of 4/WPS consecutive 16-row
// slices of H); WPS waves share a slice.  The workgroup takes all of its unit's tokens, NT at a time.
// Their SwiGLU activations (already fp16 from k_gateup) and per-group (scale, sum) pairs are rows
// u * maxB + j of a16 and ag, contiguous for a unit: they go to LDS by direct copies, `span` tokens
// per pass (all of them unless the unit has more), with one barrier per pass.  When a wave's runs all
// fit its UNR register slots (KEEP) the weights are loaded once and stay in registers for every chunk.
template <int NT>
constexpr int down_unr() { return NT <= 2 ? 4 : 5; }  // runs in flight per wave (NVFP4 NT = 4 fits 128 VGPRs: 4 waves per SIMD)
template <int FMT, int NT, int WPS, bool KEEP>
__global__ void __launch_bounds__(kWG)
k_down(uint8_t* arena, const uint8_t* __restrict__ pool, int64_t R, SpecCopy sc,
       const float* __restrict__ ts, const DecodePlan* __restrict__ plan, const uint16_t* __restrict__ a16,
       const float2* __restrict__ ag, int H, int I, int maxB, int span, float* __restrict__ y) {
  static_assert(WPS == 1 || WPS == 2 || WPS == 4, "1, 2 or 4 waves per slice");
  constexpr int SPW = 4 / WPS;
  constexpr int UNR = down_unr<NT>();
  extern __shared__ uint4 s_a4[];               // [span][I/8] groups of 8 fp16, 1 KiB slack, [span][I/8] float2, 1 KiB slack
  __shared__ float s_red[4][16][NT];
  __shared__ int s_p[kMaxTokens];               // the pass's entries (rows of y)
  if ((int)blockIdx.x < sc.nwg) {  // the front of the grid carries a speculative copy
    copy_fetch_list(pool, arena, R, sc.n_flat, sc.S, sc.fl, blockIdx.x, sc.nwg);
    return;
  }
  const int bid = blockIdx.x - sc.nwg;
  const int NSH = H / 16, NG = NSH / SPW, KB = I / 32, NRF = KB / 4, I8 = I / 8;
  const int u = bid / NG, sgp = bid % NG;
  const DecodeUnit* un = &plan->unit[u];
  const int cnt = un->count;
  if (cnt <= 0) return;
  const int64_t pay = (int64_t)H * I / 2, sca = (int64_t)H * I / 16;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ss = wave / WPS, wp = wave % WPS, sl = sgp * SPW + ss;
  const int t4 = lane >> 4, g = lane & 3, q = (lane >> 2) & 3;
  // a record installed by this call was copied whole by k_gateup, the previous kernel on the stream
  const uint8_t* rec = arena + (int64_t)un->slot * R;
  // the NVFP4 tensor scale is read before the weights, not in the epilogue, where the load would be
  // one more round trip to wait for
  const float tsd = FMT == EFF_WFMT_NVFP4_G16_E4M3 ? ts[(int64_t)un->flat * 3 + 2] : 1.f;
  const int SL = span * I8;                     // 16-byte places of a pass's activations
  float2* s_ag = reinterpret_cast<float2*>(s_a4 + SL + 64);
  const uint32_t ldsA = lds_address(s_a4), ldsG = ldsA + (uint32_t)(SL + 64) * 16;
  const uint8_t* dp = rec + 2 * pay + (int64_t)sl * KB * 256 + lane * 16;
  const uint8_t* ds = rec + 3 * pay + 2 * sca + (int64_t)sl * KB * 32 + t4 * 32 + lane_scale_off<FMT>(q, g);
  const int ai = lane >> 2;                     // the lane's 8-group in a run: 16 r + ai
  const bool tail = (KB & 3) != 0;
  const bool tail_lane = 4 * NRF + t4 < KB;

  // the wave's runs are wp, wp + WPS, ...: nr of them; as in k_gateup every load below is unconditional
  // (past the last run a load takes it again) so that the compiler keeps them in flight
  const int nr = NRF > wp ? (NRF - wp + WPS - 1) / WPS : 0;
  const int rlast = wp + WPS * max(nr - 1, 0);
  uint4 wd[UNR];
  Scales4 rd[UNR];
  auto load_run = [&](int z, int r) {
    wd[z] = *reinterpret_cast<const uint4*>(dp + (int64_t)r * 1024);
    rd[z] = load_scales4<FMT>(ds + r * 128);
  };
  // a pass's rows, 1 KiB per copy laid end to end: lane l of copy c fills place 64 c + l; past the
  // last place it loads the last one again into the slack.  Every place is written by one lane.  (I
  // is a multiple of 32, so a pass's float2 pairs fill whole 16-byte places.)  Returns the entry of
  // the pass's token tid (rows of y).
  auto stage = [&](int p0, int np) {
    const uint16_t* asrc = a16 + ((int64_t)u * maxB + p0) * I;
    const float2* gsrc = ag + ((int64_t)u * maxB + p0) * I8;
    const int na = np * I8, ng = np * I8 / 2;
    for (int c = wave; c < (na + 63) / 64; c += kWG / 64) lds_copy16(asrc + (int64_t)min(c * 64 + lane, na - 1) * 8, ldsA + c * 1024);
    for (int c = wave; c < (ng + 63) / 64; c += kWG / 64) lds_copy16(gsrc + 2 * min(c * 64 + lane, ng - 1), ldsG + c * 1024);
    return tid < np ? un->entry[p0 + tid] : 0;
  };
  // the first pass's copies go out first, then (KEEP) the wave's runs, once for all passes
  int pe = stage(0, min(span, cnt));
  if constexpr (KEEP) {
#pragma unroll
    for (int z = 0; z < UNR; ++z) load_run(z, min(wp + WPS * z, rlast));
  }
#pragma nounroll
  for (int p0 = 0; p0 < cnt; p0 += span) {
    const int np = min(span, cnt - p0);
    if (p0 > 0) pe = stage(p0, np);
    if constexpr (KEEP) {
      // the copies are complete once at most the runs' 2 * UNR loads, issued after them, remain
      if (p0 == 0) vm_wait<2 * UNR>(); else vm_wait<0>();
    } else {
      // the pass's first runs, issued after the copies: the copies are complete once at most these
      // 2 * UNR loads remain
#pragma unroll
      for (int z = 0; z < UNR; ++z) load_run(z, min(wp + WPS * z, rlast));
      vm_wait<2 * UNR>();
    }
    if (tid < np) s_p[tid] = pe;
    __syncthreads();
#pragma nounroll
    for (int c0 = p0; c0 < p0 + np; c0 += NT) {
      const int nt = min(NT, p0 + np - c0);
      const uint4* sa = s_a4 + (c0 - p0) * I8;
      const float2* sg = s_ag + (c0 - p0) * I8;
      float acc[4][NT];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[r][j] = 0.f;
      if constexpr (KEEP) {  // nr <= UNR
#pragma unroll
        for (int z = 0; z < UNR; ++z) {
          if (z >= nr) break;  // uniform
          down_run<FMT, NT>(wd[z], rd[z], sa, sg, (wp + WPS * z) * 16 + ai, nt, I8, acc);
        }
      } else {
        // a rolling pipeline of UNR slots, each refilled with the run UNR ahead once used; a later
        // chunk of the pass loads its first runs again (from L2)
        if (c0 > p0) {
#pragma unroll
          for (int z = 0; z < UNR; ++z) load_run(z, min(wp + WPS * z, rlast));
        }
        constexpr int RB = 2 * UNR;  // runs unrolled whole per block (no loop back-edge inside)
        for (int i0 = 0; i0 < nr; i0 += RB) {
#pragma unroll
          for (int k = 0; k < RB; ++k) {
            const int i = i0 + k, z = k % UNR, r = wp + WPS * i;
            if (i >= nr) break;  // uniform
            down_run<FMT, NT>(wd[z], rd[z], sa, sg, r * 16 + ai, nt, I8, acc);
            load_run(z, min(r + WPS * UNR, rlast));
          }
        }
      }
      if (tail && wp == NRF % WPS && tail_lane) {
        const int r = NRF;
        const uint4 w1 = *reinterpret_cast<const uint4*>(dp + (int64_t)r * 1024);
        const Scales4 s1 = load_scales4<FMT>(ds + r * 128);
        down_run<FMT, NT>(w1, s1, sa, sg, r * 16 + ai, nt, I8, acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          if (NT == 1 || j < nt) acc[r][j] = sum16(acc[r][j]);
      if (lane < 4) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int j = 0; j < NT; ++j) s_red[wave][4 * lane + r][j] = acc[r][j];
      }
      __syncthreads();
      for (int idx = tid; idx < 16 * SPW * nt; idx += kWG) {
        const int j = idx % nt, rr = idx / nt, s2 = rr / 16, row = rr % 16;
        float v = s_red[s2 * WPS][row][j];  // the slice's waves in order
#pragma unroll
        for (int w2 = 1; w2 < WPS; ++w2) v += s_red[s2 * WPS + w2][row][j];
        if (FMT == EFF_WFMT_NVFP4_G16_E4M3) v *= tsd;
        const int p = s_p[c0 - p0 + j];
        y[(int64_t)p * H + (sgp * SPW + s2) * 16 + row] = v;
      }
      __syncthreads();
      if constexpr (KEEP) {
        // the kept runs count as rewritten here (no code): otherwise the compiler would keep every
        // run's dequantized values live across the chunks instead of the packed weights
#pragma unroll
        for (int z = 0; z < UNR; ++z) {
          asm volatile("" : "+v"(wd[z].x), "+v"(wd[z].y), "+v"(wd[z].z), "+v"(wd[z].w), "+v"(rd[z].a));
          if constexpr (FMT == EFF_WFMT_INT4_G32_BF16) asm volatile("" : "+v"(rd[z].b));
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------- combine
// out[t, h] = sum over k (ascending) of w[t,k] * y[t,k,h], y from the GPU or the host buffer by the
// entry's slot (slots == nullptr: all from yg; yh may be host-mapped memory).
// With `done` (host-mapped), the kernel first waits until *done >= *seq (the number the control
// kernel gave this call, in device memory): the host share of the call is in yh (or it had none).  One thread per workgroup polls with a bounded spin; past the
// bound it sets bit 4 of *err and combines anyway, so the kernel always ends.
template <int KMAX>
__global__ void __launch_bounds__(256)
k_combine(const float* __restrict__ yg, const float* __restrict__ yh, const int32_t* __restrict__ slots,
          const float* __restrict__ w, int K, int H, uint16_t* __restrict__ out, const uint64_t* done,
          const uint64_t* seq_dev, int32_t* err) {
  if (done) {
    if (threadIdx.x == 0) {
      const uint64_t seq = *seq_dev;
      for (uint32_t spin = 0; __hip_atomic_load(done, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_SYSTEM) < seq; ++spin) {
        if (spin >= kCombineSpinLimit) {
          atomicOr(err, 4);
          break;
        }
        __builtin_amdgcn_s_sleep(8);
      }
    }
    __syncthreads();
  }
  const int t = blockIdx.y;
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= H) return;
  float v[KMAX], wk[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (k < K) {
      const int64_t p = (int64_t)t * K + k;
      wk[k] = w[p];
      const bool gpu = slots == nullptr || slots[p] >= 0;  // the same for every thread of the token
      v[k] = (gpu ? yg : yh)[p * H + h];
    }
  }
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < KMAX; ++k)
    if (k < K) acc = fmaf(wk[k], v[k], acc);
  uint32_t b = __float_as_uint(acc);
  b += 0x7FFFu + ((b >> 16) & 1u);  // round to nearest even
  out[(int64_t)t * H + h] = (uint16_t)(b >> 16);
}

// The link rate of the in-kernel fetch path, for the bandwidth profile: n records (flat ids first,
// first + stride, ... modulo the pool) copied from the pinned host pool with 16-byte loads, like
// the fetch units of k_gateup, into two record-sized device buffers used in turn.
__global__ void __launch_bounds__(256)
k_bw_copy(const uint8_t* __restrict__ pool, int64_t R, int64_t n_flat, int64_t first, int64_t stride, int n,
          uint8_t* __restrict__ dst) {
  const int64_t per = R / 16, total = per * n;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / per, c = i % per;
    const int64_t flat = (first + r * stride) % n_flat;
    reinterpret_cast<uint4*>(dst + (r & 1) * R)[c] = reinterpret_cast<const uint4*>(pool + flat * R)[c];
  }
}

// Waves per 16-row slice of a matrix (the rest of a 4-wave workgroup takes further slices).  A
// launch wants a few thousand waves to keep every CU streaming, and a wave enough 1 KiB runs to make
// its reduction worth it: with many slices each wave takes a whole slice of one matrix, with few the
// slice's runs are split over more waves.
int gateup_waves_per_matrix(int slices) { return slices >= 1024 ? 1 : 2; }
int down_wps(int slices, int runs) {
  if (slices >= 2048 || runs <= 8) return 1;
  return slices >= 1024 ? 2 : 4;
}

// With events (t0, t1) the launch sets them at the kernel's own start and end (hipExtLaunchKernelGGL):
// the timing then covers the kernel alone, as a profiler's kernel trace does.
template <int FMT, int NT, int P>
hipError_t launch_gateup_t(eff_engine* e, const DecodePlan* plan, const uint16_t* x, int units, int nch, int u2,
                           hipStream_t s, uint16_t* a16, float2* ag, hipEvent_t t0, hipEvent_t t1, SpecCopy sc) {
  const eff_config& c = e->cfg;
  const int H = c.hidden, I = c.inter;
  if (!sc.fl) sc.nwg = 0;
  const dim3 grid(sc.nwg + (u2 * nch + (units - u2)) * (I / 16) * P / 2), block(kWG);
  const uint32_t lds = NT > 1 ? NT * H * 2 + 1024 : 0;  // token rows and the copies' slack
  if (t0)
    hipExtLaunchKernelGGL((k_gateup<FMT, NT, P>), grid, block, lds, s, t0, t1, 0, e->d_arena, e->pool_dev, e->R, sc,
                          e->d_ts, plan, x, H, I, c.top_k, c.max_tokens, nch, u2, a16, ag);
  else
    hipLaunchKernelGGL((k_gateup<FMT, NT, P>), grid, block, lds, s, e->d_arena, e->pool_dev, e->R, sc, e->d_ts, plan,
                       x, H, I, c.top_k, c.max_tokens, nch, u2, a16, ag);
  return hipGetLastError();
}

template <int FMT, int NT, int WPS, bool KEEP>
hipError_t launch_down_t(eff_engine* e, const DecodePlan* plan, int units, hipStream_t s, const uint16_t* a16,
                         const float2* ag, float* y, hipEvent_t t0, hipEvent_t t1, SpecCopy sc) {
  const eff_config& c = e->cfg;
  const int H = c.hidden, I = c.inter;
  if (!sc.fl) sc.nwg = 0;
  const int span = down_span(NT, c.max_tokens, I);
  const uint32_t lds = (uint32_t)down_lds_bytes(NT, c.max_tokens, I);
  const dim3 grid(sc.nwg + units * (H / 16) * WPS / 4), block(kWG);
  if (t0)
    hipExtLaunchKernelGGL((k_down<FMT, NT, WPS, KEEP>), grid, block, lds, s, t0, t1, 0, e->d_arena, e->pool_dev, e->R, sc,
                          e->d_ts, plan, a16, ag, H, I, c.max_tokens, span, y);
  else
    hipLaunchKernelGGL((k_down<FMT, NT, WPS, KEEP>), grid, block, lds, s, e->d_arena, e->pool_dev, e->R, sc, e->d_ts, plan,
                       a16, ag, H, I, c.max_tokens, span, y);
  return hipGetLastError();
}

// Token chunk widths (tokens a workgroup takes at once) by the call's batch, measured at the
// qwen3.8-flash-next expert shape: gate/up is the longer sweep, where 8-token chunks pay at B = 16
// (61.6 against 67.8 us with 4) and 4-token chunks at B = 8 (36.0 against 48.0 us with 8); the down
// rows are short, and 4-token chunks are faster there at both (B = 16: 35.7 against 45.5 us).
int gateup_nt(int B) { return B >= 16 ? 8 : B >= 4 ? 4 : B >= 2 ? 2 : 1; }
// (N * I <= 8192 keeps a pass of N tokens within 26 KiB of LDS whatever I)
int down_nt(int B, int I) {
  int n = B >= 4 ? 4 : B >= 2 ? 2 : 1;
  while (n > 1 && n * I > 8192) n /= 2;
  return n;
}

template <int FMT, int NT>
hipError_t launch_gateup_p(eff_engine* e, const DecodePlan* plan, const uint16_t* x, int units, int B, hipStream_t s,
                           uint16_t* a16, float2* ag, hipEvent_t t0, hipEvent_t t1, SpecCopy sc) {
  const int nch = (B + NT - 1) / NT;  // token chunks a unit can have (a unit holds at most one entry per token)
  // units that can hold more than NT tokens: each has NT + 1 of the call's B * K entries or more, and
  // the plan lists them first (busiest first); the grid gives only those nch chunk blocks
  const int u2 = nch > 1 ? std::min(units, B * e->cfg.top_k / (NT + 1)) : units;
  if (gateup_waves_per_matrix(units * (e->cfg.inter / 16)) == 1)
    return launch_gateup_t<FMT, NT, 1>(e, plan, x, units, nch, u2, s, a16, ag, t0, t1, sc);
  return launch_gateup_t<FMT, NT, 2>(e, plan, x, units, nch, u2, s, a16, ag, t0, t1, sc);
}

// the weights stay in registers when every wave's runs, (I/128 + WPS - 1) / WPS at most, fit its slots
inline bool down_keep(int I, int WPS, int unr) { return (I / 128 + WPS - 1) / WPS <= unr; }
template <int FMT, int NT, int WPS>
hipError_t launch_down_k(eff_engine* e, const DecodePlan* plan, int units, hipStream_t s, const uint16_t* a16,
                         const float2* ag, float* y, hipEvent_t t0, hipEvent_t t1, SpecCopy sc) {
  if (down_keep(e->cfg.inter, WPS, down_unr<NT>()))
    return launch_down_t<FMT, NT, WPS, true>(e, plan, units, s, a16, ag, y, t0, t1, sc);
  return launch_down_t<FMT, NT, WPS, false>(e, plan, units, s, a16, ag, y, t0, t1, sc);
}

template <int FMT, int NT>
hipError_t launch_down_w(eff_engine* e, const DecodePlan* plan, int units, hipStream_t s, const uint16_t* a16,
                         const float2* ag, float* y, hipEvent_t t0, hipEvent_t t1, SpecCopy sc) {
  // the down kernel takes a unit's chunks in turn: its rows are short (I inputs), so a second wave of
  // workgroups per unit costs more than the chunks' arithmetic it would spread
  switch (down_wps(units * (e->cfg.hidden / 16), e->cfg.inter / 128)) {
    case 1: return launch_down_k<FMT, NT, 1>(e, plan, units, s, a16, ag, y, t0, t1, sc);
    case 2: return launch_down_k<FMT, NT, 2>(e, plan, units, s, a16, ag, y, t0, t1, sc);
    default: return launch_down_k<FMT, NT, 4>(e, plan, units, s, a16, ag, y, t0, t1, sc);
  }
}

// The two expert kernels of one call on the plan `plan`; a16 holds units * max_tokens * I fp16
// activations (a unit's token j is row u * max_tokens + j whatever the chunk widths) and ag one
// (scale, sum) pair per 8 of them.  `timed`: bracket the kernels with the engine's timing events.
// `spec`: a speculative copy carried by the gate/up kernel, or by the down kernel when in_down.
template <int FMT>
hipError_t launch_ffn_t(eff_engine* e, const DecodePlan* plan, uint16_t* a16, float2* ag, const uint16_t* x, float* y,
                        int units, int B, hipStream_t s, SpecCopy spec, bool in_down, bool timed) {
  const SpecCopy none, sg = in_down ? none : spec, sd = in_down ? spec : none;
  // timed outside a capture: each kernel sets its own start and end events; inside a capture the
  // events are recorded on the stream around the launches
  const bool own = timed && !stream_capturing(s);
  const int ts = timed ? timing_begin(e, EFF_T_DECODE_GATEUP, s, !own) : -1;
  hipEvent_t g0 = own ? timing_event(e, ts, 0) : nullptr, g1 = own ? timing_event(e, ts, 1) : nullptr;
  hipEvent_t d0 = own ? timing_event(e, ts, 2) : nullptr, d1 = own ? timing_event(e, ts, 3) : nullptr;
  hipError_t err;
  switch (gateup_nt(B)) {
    case 1: err = launch_gateup_p<FMT, 1>(e, plan, x, units, B, s, a16, ag, g0, g1, sg); break;
    case 2: err = launch_gateup_p<FMT, 2>(e, plan, x, units, B, s, a16, ag, g0, g1, sg); break;
    case 4: err = launch_gateup_p<FMT, 4>(e, plan, x, units, B, s, a16, ag, g0, g1, sg); break;
    default: err = launch_gateup_p<FMT, 8>(e, plan, x, units, B, s, a16, ag, g0, g1, sg); break;
  }
  if (err != hipSuccess) return err;
  if (!own) {
    timing_mark(e, ts, 1, s);
    timing_mark(e, ts, 2, s);
  }
  switch (down_nt(B, e->cfg.inter)) {
    case 1: err = launch_down_w<FMT, 1>(e, plan, units, s, a16, ag, y, d0, d1, sd); break;
    case 2: err = launch_down_w<FMT, 2>(e, plan, units, s, a16, ag, y, d0, d1, sd); break;
    default: err = launch_down_w<FMT, 4>(e, plan, units, s, a16, ag, y, d0, d1, sd); break;
  }
  if (!own) timing_mark(e, ts, 3, s);
  return err;
}

}  // namespace

hipError_t decode_kernels_setup(int fmt, int maxB, int H, int I) {
  // allow N * H * 2 bytes of dynamic LDS for the gate/up kernel and N * I * 3 for the down kernel,
  // for every token width N a call can take
  const int NG = gateup_nt(maxB), ND = down_nt(maxB, I);
  hipError_t err = hipSuccess;
  auto set = [&](const void* fn, int bytes) {
    if (err == hipSuccess) err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  };
#define SETUP_G(F, N)                                                       \
  if (fmt == F && N <= NG) {                                                \
    set((const void*)k_gateup<F, N, 1>, N * H * 2 + 1024);                  \
    set((const void*)k_gateup<F, N, 2>, N * H * 2 + 1024);                  \
  }
#define SETUP_D(F, N)                                                       \
  if (fmt == F && N <= ND) {                                                \
    set((const void*)k_down<F, N, 1, true>, down_lds_bytes(N, maxB, I));    \
    set((const void*)k_down<F, N, 1, false>, down_lds_bytes(N, maxB, I));   \
    set((const void*)k_down<F, N, 2, true>, down_lds_bytes(N, maxB, I));    \
    set((const void*)k_down<F, N, 2, false>, down_lds_bytes(N, maxB, I));   \
    set((const void*)k_down<F, N, 4, true>, down_lds_bytes(N, maxB, I));    \
    set((const void*)k_down<F, N, 4, false>, down_lds_bytes(N, maxB, I));   \
  }
  SETUP_G(EFF_WFMT_INT4_G32_BF16, 1) SETUP_G(EFF_WFMT_INT4_G32_BF16, 2) SETUP_G(EFF_WFMT_INT4_G32_BF16, 4)
  SETUP_G(EFF_WFMT_INT4_G32_BF16, 8) SETUP_G(EFF_WFMT_NVFP4_G16_E4M3, 1) SETUP_G(EFF_WFMT_NVFP4_G16_E4M3, 2)
  SETUP_G(EFF_WFMT_NVFP4_G16_E4M3, 4) SETUP_G(EFF_WFMT_NVFP4_G16_E4M3, 8)
  SETUP_D(EFF_WFMT_INT4_G32_BF16, 1) SETUP_D(EFF_WFMT_INT4_G32_BF16, 2) SETUP_D(EFF_WFMT_INT4_G32_BF16, 4)
  SETUP_D(EFF_WFMT_NVFP4_G16_E4M3, 1) SETUP_D(EFF_WFMT_NVFP4_G16_E4M3, 2) SETUP_D(EFF_WFMT_NVFP4_G16_E4M3, 4)
#undef SETUP_G
#undef SETUP_D
  return err;
}

hipError_t launch_ffn_decode(eff_engine* e, int layer, const uint16_t* x, const int32_t* slots, int B,
                             float* y, hipStream_t s, bool plan_ready, SpecCopy spec, bool in_down) {
  (void)layer;
  if (!plan_ready) {
    hipError_t err = launch_plan(e, slots, B * e->cfg.top_k, s, e->d_plan, e->maxU);
    if (err != hipSuccess) return err;
  }
  // the token widths follow the call's batch (a unit holds at most one entry per token): a B = 1 call
  // takes the one-token kernels whatever max_tokens is
  const int units = std::min(e->maxU, B * e->cfg.top_k);  // plan units a call of B tokens can have
  uint16_t* a16 = reinterpret_cast<uint16_t*>(e->d_a);
  float2* ag = reinterpret_cast<float2*>(a16 + (size_t)e->maxU * e->cfg.max_tokens * e->cfg.inter);
  if (e->cfg.wformat == EFF_WFMT_NVFP4_G16_E4M3)
    return launch_ffn_t<EFF_WFMT_NVFP4_G16_E4M3>(e, e->d_plan, a16, ag, x, y, units, B, s, spec, in_down, true);
  return launch_ffn_t<EFF_WFMT_INT4_G32_BF16>(e, e->d_plan, a16, ag, x, y, units, B, s, spec, in_down, true);
}

// ---------------------------------------------------------------------------- static scratch
// The scratch of eff_expert_ffn_decode_noalloc, for callers that cannot allocate (graph capture,
// tight serving loops): the decode plan, then the SwiGLU activations (fp16) and their (scale, sum)
// pairs, in one file-scope device array.  Each GPU holds its own copy until the process ends.  Host
// code never passes the array's name to a kernel (on the host it is only a stand-in): the address of
// each device's copy comes from hipGetSymbolAddress, taken once per device with that device current,
// and kernels get that address.  Every call on a GPU shares its copy, so calls that overlap on one
// GPU race; nothing in it needs to start at zero (the plan kernel writes every unit the expert
// kernels read, and they write the activations before reading them).
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
constexpr size_t kPlanBytes = (sizeof(DecodePlan) + 255) / 256 * 256;
}  // namespace

hipError_t noalloc_setup(int device) {
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  if (g_scratch_ptr[device]) return hipSuccess;
  void* p = nullptr;
  const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (err != hipSuccess) return err;
  if (!p) return hipErrorInvalidSymbol;
  g_scratch_ptr[device] = p;
  return hipSuccess;
}

size_t noalloc_need(const eff_engine* e, int B) {
  const size_t units = (size_t)std::min(e->maxU, B * e->cfg.top_k);
  // fp16 activations (2 bytes) and one 8-byte pair per 8 of them: 3 bytes per activation
  return kPlanBytes + units * (size_t)e->cfg.max_tokens * (size_t)e->cfg.inter * 3;
}

hipError_t launch_ffn_decode_noalloc(eff_engine* e, const uint16_t* x, const int32_t* slots, int B, float* y,
                                     hipStream_t s) {
  void* base = nullptr;
  {
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (e->device >= 0 && e->device < kMaxDevices) base = g_scratch_ptr[e->device];
  }
  if (!base) return hipErrorNotInitialized;
  const int units = std::min(e->maxU, B * e->cfg.top_k);
  DecodePlan* plan = reinterpret_cast<DecodePlan*>(base);
  uint16_t* a16 = reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(base) + kPlanBytes);
  float2* ag = reinterpret_cast<float2*>(a16 + (size_t)units * e->cfg.max_tokens * e->cfg.inter);
  hipError_t err = launch_plan(e, slots, B * e->cfg.top_k, s, plan, units);
  if (err != hipSuccess) return err;
  if (e->cfg.wformat == EFF_WFMT_NVFP4_G16_E4M3)
    return launch_ffn_t<EFF_WFMT_NVFP4_G16_E4M3>(e, plan, a16, ag, x, y, units, B, s, SpecCopy(), false, false);
  return launch_ffn_t<EFF_WFMT_INT4_G32_BF16>(e, plan, a16, ag, x, y, units, B, s, SpecCopy(), false, false);
}

hipError_t launch_bw_copy(eff_engine* e, int64_t first, int64_t stride, int n, uint8_t* dst, hipStream_t s) {
  const eff_config& c = e->cfg;
  hipLaunchKernelGGL(k_bw_copy, dim3(1024), dim3(256), 0, s, e->pool_dev, e->R,
                     (int64_t)c.num_layers * c.num_experts, first, stride, n, dst);
  return hipGetLastError();
}

hipError_t launch_combine(const float* ygpu, const float* yhost, const int32_t* slots, const float* w,
                          int B, int K, int H, uint16_t* out, hipStream_t s, const uint64_t* done, const uint64_t* seq,
                          int32_t* err) {
  dim3 g((H + 255) / 256, B);
  if (!slots) yhost = nullptr;
  if (K <= 8)
    hipLaunchKernelGGL(k_combine<8>, g, dim3(256), 0, s, ygpu, yhost, slots, w, K, H, out, done, seq, err);
  else if (K <= 16)
    hipLaunchKernelGGL(k_combine<16>, g, dim3(256), 0, s, ygpu, yhost, slots, w, K, H, out, done, seq, err);
  else
    hipLaunchKernelGGL(k_combine<kMaxTopK>, g, dim3(256), 0, s, ygpu, yhost, slots, w, K, H, out, done, seq, err);
  return hipGetLastError();
}

}  // namespace eff
