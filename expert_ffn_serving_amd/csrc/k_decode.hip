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
#include "eff_internal.h"

namespace eff {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

constexpr int kWG = 256;  // 4 waves

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
// one contiguous run of (Kd/32) tiles of 256 payload bytes (and 32 scale bytes).  Lane
// (q = lane/16, r = lane%16) reads the dword at byte lane*4 of a tile: row r, inputs 8q..8q+7.

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

// per-lane scale offset inside a tile's 32 scale bytes
template <int FMT>
__device__ inline uint32_t scale_lane_off(int q, int r) {
  return FMT == EFF_WFMT_INT4_G32_BF16 ? (uint32_t)r * 2u : (uint32_t)((q >> 1) * 16 + r);
}
// raw scale bits of one lane (int4: a bf16; NVFP4: an e4m3 byte) and their value
template <int FMT>
__device__ inline uint32_t load_scale_raw(const uint8_t* p) {
  if (FMT == EFF_WFMT_INT4_G32_BF16) return (uint32_t)*reinterpret_cast<const uint16_t*>(p);
  return (uint32_t)*p;
}
template <int FMT>
__device__ inline float scale_value(uint32_t raw) {
  if (FMT == EFF_WFMT_INT4_G32_BF16) return __uint_as_float(raw << 16);
  return __builtin_amdgcn_cvt_f32_fp8(raw, 0);
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

// sum over the 8 inputs of one dword of weights against the paired activations (unscaled)
template <int FMT>
__device__ inline float dword_dot_bf16(uint32_t d, const uint32_t* xw, float xs) {
  uint32_t p0, p1, p2, p3;
  if (FMT == EFF_WFMT_INT4_G32_BF16) {
    p0 = (d & 0x000F000Fu) | 0x43004300u;
    p1 = ((d >> 4) & 0x000F000Fu) | 0x43004300u;
    p2 = ((d >> 8) & 0x000F000Fu) | 0x43004300u;
    p3 = ((d >> 12) & 0x000F000Fu) | 0x43004300u;
  } else {
    p0 = fp4_to_bf16x2<0>(d); p1 = fp4_to_bf16x2<1>(d);
    p2 = fp4_to_bf16x2<2>(d); p3 = fp4_to_bf16x2<3>(d);
  }
  float raw = dot2_bf16(p3, xw[3], dot2_bf16(p2, xw[2], dot2_bf16(p1, xw[1], dot2_bf16(p0, xw[0], 0.f))));
  if (FMT == EFF_WFMT_INT4_G32_BF16) raw = fmaf(-136.f, xs, raw);
  return raw;
}

// tokens j >= nt (a unit's last chunk holds fewer than NT) are skipped: nt is uniform per workgroup
template <int FMT, int NT>
__device__ inline void gateup_tile(uint32_t wg, uint32_t wu, uint32_t rg, uint32_t ru, const uint4* xv, int nt,
                                   float (&acc)[2][NT]) {
  const float sg = scale_value<FMT>(rg), su = scale_value<FMT>(ru);
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    if (NT > 1 && j >= nt) break;
    uint32_t xw[4];
    x_pairs<FMT>(xv[j], xw);
    float xs = 0.f;
    if (FMT == EFF_WFMT_INT4_G32_BF16)
      xs = dot2_bf16(xw[3], 0x3F803F80u, dot2_bf16(xw[2], 0x3F803F80u,
                     dot2_bf16(xw[1], 0x3F803F80u, dot2_bf16(xw[0], 0x3F803F80u, 0.f))));
    acc[0][j] = fmaf(sg, dword_dot_bf16<FMT>(wg, xw, xs), acc[0][j]);
    acc[1][j] = fmaf(su, dword_dot_bf16<FMT>(wu, xw, xs), acc[1][j]);
  }
}

// grid: maxU * (I/16) workgroups of 256 threads, one per (plan unit, 16-row slice of I).  Wave w
// takes tiles w, w+4, ... of the slice (the 4 waves together sweep 1 KiB runs), gate and up at
// once; everything reduces inside the workgroup, so no workgroup ever waits for another.
// A unit installed by this call (fetch) first copies its gate and up slices from the pinned host
// pool into the slot (16-byte loads) and, once its rows are done, a 1/(I/16) share of the down
// matrix: the whole record crosses the link inside this kernel, and k_down finds it resident.
template <int FMT, int NT>
__global__ void __launch_bounds__(kWG)
k_gateup(uint8_t* arena, const uint8_t* __restrict__ pool, int64_t R,
         const float* __restrict__ ts, const DecodePlan* __restrict__ plan, const uint16_t* __restrict__ x, int H,
         int I, int K, int maxB, uint16_t* __restrict__ a16, float2* __restrict__ ag) {
  extern __shared__ uint4 s_x[];  // NT > 1: [NT][H/8], the token rows of the current chunk
  __shared__ float s_red[4][2][16][NT];
  const int NS = I / 16, KB = H / 32;
  const int u = blockIdx.x / NS, sl = blockIdx.x % NS;
  const DecodeUnit* un = &plan->unit[u];
  const int cnt = un->count;
  if (cnt <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, r = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t pay = (int64_t)H * I / 2, sca = (int64_t)H * I / 16;
  uint8_t* rec = arena + (int64_t)un->slot * R;
  if (un->fetch) {
    // installed by this call: copy this workgroup's gate and up slices (payload and scales) from
    // the pool into the slot, then read them back like any resident record
    const uint8_t* src = pool + (int64_t)un->flat * R;
    const int64_t po = (int64_t)sl * KB * 256, so = 3 * pay + (int64_t)sl * KB * 32;
    wg_copy(src + po, rec + po, (int64_t)KB * 256);
    wg_copy(src + pay + po, rec + pay + po, (int64_t)KB * 256);
    wg_copy(src + so, rec + so, (int64_t)KB * 32);
    wg_copy(src + sca + so, rec + sca + so, (int64_t)KB * 32);
    __syncthreads();
  }
  const uint8_t* gp = rec + (int64_t)sl * KB * 256 + lane * 4;
  const uint8_t* up = gp + pay;
  const uint8_t* gs = rec + 3 * pay + (int64_t)sl * KB * 32 + scale_lane_off<FMT>(q, r);
  const uint8_t* us = gs + sca;
  const int H8 = H / 8;
  for (int c0 = 0; c0 < cnt; c0 += NT) {
    const int nt = min(NT, cnt - c0);
    float acc[2][NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[0][j] = acc[1][j] = 0.f;
    if constexpr (NT == 1) {
      // one token: its activations ride with the weight loads, straight from global memory (an
      // LDS stage and its barrier cost more than they free at this width)
      constexpr int UNR = 8;  // tiles in flight per wave
      const uint16_t* xt = x + q * 8 + (int64_t)(un->entry[c0] / K) * H;
      int kb = wave;
      for (; kb + 4 * (UNR - 1) < KB; kb += 4 * UNR) {  // full rounds: every load first
        uint32_t wg[UNR], wu[UNR], rg[UNR], ru[UNR];
        uint4 xv[UNR][1];
#pragma unroll
        for (int z = 0; z < UNR; ++z) {
          const int k = kb + 4 * z;
          wg[z] = *reinterpret_cast<const uint32_t*>(gp + k * 256);
          wu[z] = *reinterpret_cast<const uint32_t*>(up + k * 256);
          rg[z] = load_scale_raw<FMT>(gs + k * 32);
          ru[z] = load_scale_raw<FMT>(us + k * 32);
          xv[z][0] = *reinterpret_cast<const uint4*>(xt + k * 32);
        }
        __builtin_amdgcn_sched_barrier(0);  // every load of the round is in flight before any use
#pragma unroll
        for (int z = 0; z < UNR; ++z) gateup_tile<FMT, NT>(wg[z], wu[z], rg[z], ru[z], xv[z], 1, acc);
      }
      if (kb < KB) {  // the last, partial round (H / 32 not a multiple of 4 * UNR): its loads together too
        uint32_t wg[UNR], wu[UNR], rg[UNR], ru[UNR];
        uint4 xv[UNR][1];
#pragma unroll
        for (int z = 0; z < UNR; ++z) {
          const int k = kb + 4 * z;
          const bool in = k < KB;  // uniform per wave
          wg[z] = in ? *reinterpret_cast<const uint32_t*>(gp + k * 256) : 0u;
          wu[z] = in ? *reinterpret_cast<const uint32_t*>(up + k * 256) : 0u;
          rg[z] = in ? load_scale_raw<FMT>(gs + k * 32) : 0u;
          ru[z] = in ? load_scale_raw<FMT>(us + k * 32) : 0u;
          xv[z][0] = in ? *reinterpret_cast<const uint4*>(xt + k * 32) : make_uint4(0, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int z = 0; z < UNR; ++z)
          if (kb + 4 * z < KB) gateup_tile<FMT, NT>(wg[z], wu[z], rg[z], ru[z], xv[z], 1, acc);
      }
    } else {
      // several tokens: the first round of weight loads, then the chunk's token rows into LDS (the
      // weights do not wait for them); the registers then hold weights only
      constexpr int UNR = NT >= 4 ? 4 : 8;  // tiles in flight per wave
      uint32_t wg[UNR], wu[UNR], rg[UNR], ru[UNR];
      int kb = wave;
#pragma unroll
      for (int z = 0; z < UNR; ++z) {
        const int k = kb + 4 * z;
        const bool in = k < KB;
        wg[z] = in ? *reinterpret_cast<const uint32_t*>(gp + k * 256) : 0u;
        wu[z] = in ? *reinterpret_cast<const uint32_t*>(up + k * 256) : 0u;
        rg[z] = in ? load_scale_raw<FMT>(gs + k * 32) : 0u;
        ru[z] = in ? load_scale_raw<FMT>(us + k * 32) : 0u;
      }
      for (int i = tid; i < nt * H8; i += kWG) {
        const int j = i / H8, g = i % H8;
        s_x[i] = *reinterpret_cast<const uint4*>(x + (int64_t)(un->entry[c0 + j] / K) * H + g * 8);
      }
      __syncthreads();
      for (;;) {
#pragma unroll
        for (int z = 0; z < UNR; ++z) {
          const int k = kb + 4 * z;
          if (k < KB) {  // uniform per wave
            uint4 xv[NT];
#pragma unroll
            for (int j = 0; j < NT; ++j) xv[j] = j < nt ? s_x[j * H8 + k * 4 + q] : make_uint4(0, 0, 0, 0);  // read only below nt
            gateup_tile<FMT, NT>(wg[z], wu[z], rg[z], ru[z], xv, nt, acc);
          }
        }
        kb += 4 * UNR;
        if (kb >= KB) break;
#pragma unroll
        for (int z = 0; z < UNR; ++z) {  // the next round
          const int k = kb + 4 * z;
          const bool in = k < KB;
          wg[z] = in ? *reinterpret_cast<const uint32_t*>(gp + k * 256) : 0u;
          wu[z] = in ? *reinterpret_cast<const uint32_t*>(up + k * 256) : 0u;
          rg[z] = in ? load_scale_raw<FMT>(gs + k * 32) : 0u;
          ru[z] = in ? load_scale_raw<FMT>(us + k * 32) : 0u;
        }
      }
    }
    // reduce over q (lanes r, r+16, r+32, r+48), then over the 4 waves in order
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        float v = acc[m][j];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        acc[m][j] = v;
      }
    if (lane < 16) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int j = 0; j < NT; ++j) s_red[wave][m][r][j] = acc[m][j];
    }
    __syncthreads();
    if (tid < 16 * nt) {  // 16 consecutive lanes per token: j = tid / 16, row = tid % 16
      const int j = tid >> 4, row = tid & 15;
      float g = s_red[0][0][row][j] + s_red[1][0][row][j];
      g += s_red[2][0][row][j];
      g += s_red[3][0][row][j];
      float v = s_red[0][1][row][j] + s_red[1][1][row][j];
      v += s_red[2][1][row][j];
      v += s_red[3][1][row][j];
      if (FMT == EFF_WFMT_NVFP4_G16_E4M3) {
        g *= ts[(int64_t)un->flat * 3 + 0];
        v *= ts[(int64_t)un->flat * 3 + 1];
      }
      const float a = silu(g) * v;
      // the slice's power-of-two scale: max |a| over its 16 rows lands in [2^14, 2^15)
      float mx = fabsf(a);
      mx = fmaxf(mx, __shfl_xor(mx, 8));
      mx = fmaxf(mx, __shfl_xor(mx, 4));
      mx = fmaxf(mx, __shfl_xor(mx, 2));
      mx = fmaxf(mx, __shfl_xor(mx, 1));
      int sh = 0;
      if (mx > 0.f) {
        int ex;
        frexpf(mx, &ex);  // mx < 2^ex
        sh = min(15 - ex, 100);
      }
      const _Float16 h = (_Float16)ldexpf(a, sh);
      float gs = (float)h;  // sum of the 8-group (rows 8*(row/8) ..), int4 only
      gs += __shfl_xor(gs, 4);
      gs += __shfl_xor(gs, 2);
      gs += __shfl_xor(gs, 1);
      // int4: the pairs (a_m, a_m+4) of each 8-group meet the nibble pairs of a weight dword
      const int pos = FMT == EFF_WFMT_INT4_G32_BF16 ? (row & 8) | ((row & 3) << 1) | ((row >> 2) & 1) : row;
      const int64_t tok = (int64_t)u * maxB + c0 + j;
      a16[tok * I + sl * 16 + pos] = __builtin_bit_cast(uint16_t, h);
      if ((row & 7) == 0) ag[tok * (I / 8) + sl * 2 + (row >> 3)] = make_float2(ldexpf(1.f, -sh), gs);
    }
    __syncthreads();
  }
  if (un->fetch) {  // this workgroup's share of the down payload and scales
    const uint8_t* src = pool + (int64_t)un->flat * R;
    const int64_t dpo = 2 * pay + (int64_t)sl * (pay / NS), dso = 3 * pay + 2 * sca + (int64_t)sl * (sca / NS);
    wg_copy(src + dpo, rec + dpo, pay / NS);
    wg_copy(src + dso, rec + dso, sca / NS);
  }
}

// ---------------------------------------------------------------------------- down
template <int FMT, int NT>
__device__ inline void down_tile(uint32_t d, uint32_t rd, const uint4* s_a4, const float2* s_ag, int kb, int q,
                                 int nt, int I8, float (&acc)[NT]) {
  const float sd = scale_value<FMT>(rd);
  uint32_t p0, p1, p2, p3;
  if (FMT == EFF_WFMT_INT4_G32_BF16) {
    p0 = (d & 0x000F000Fu) | 0x64006400u;
    p1 = ((d >> 4) & 0x000F000Fu) | 0x64006400u;
    p2 = ((d >> 8) & 0x000F000Fu) | 0x64006400u;
    p3 = ((d >> 12) & 0x000F000Fu) | 0x64006400u;
  } else {
    p0 = fp4_to_f16x2<0>(d); p1 = fp4_to_f16x2<1>(d);
    p2 = fp4_to_f16x2<2>(d); p3 = fp4_to_f16x2<3>(d);
  }
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    if (j < nt) {
      const uint4 av = s_a4[j * I8 + kb * 4 + q];
      const float2 sg = s_ag[j * I8 + kb * 4 + q];  // (2^-shift of the slice, sum of the 8-group)
      float raw = dot2_f16(p3, av.w, dot2_f16(p2, av.z, dot2_f16(p1, av.y, dot2_f16(p0, av.x, 0.f))));
      if (FMT == EFF_WFMT_INT4_G32_BF16) raw = fmaf(-1032.f, sg.y, raw);
      acc[j] = fmaf(sd, raw * sg.x, acc[j]);
    }
  }
}

// grid: maxU * (H/(16*RS)) workgroups, one per (plan unit, RS 16-row slices of H); 4/RS waves
// share a slice.  The unit's SwiGLU activations, already fp16 from k_gateup, are copied into LDS
// with their per-group scales and sums before the sweep, once for the RS slices.
template <int FMT, int NT, int RS>
__global__ void __launch_bounds__(kWG)
k_down(uint8_t* arena, const uint8_t* __restrict__ pool, int64_t R,
       const float* __restrict__ ts, const DecodePlan* __restrict__ plan, const uint16_t* __restrict__ a16,
       const float2* __restrict__ ag, int H, int I, int maxB, float* __restrict__ y) {
  extern __shared__ uint4 s_a4[];            // [NT][I/8] groups of 8 fp16, then [NT][I/8] float2
  __shared__ float s_red[4][16][NT];
  constexpr int UNR = NT >= 4 ? 4 : 8;  // tiles in flight per wave
  constexpr int NW = 4 / RS;            // waves per slice
  static_assert(RS == 1 || RS == 2 || RS == 4, "1, 2 or 4 slices per workgroup");
  const int NG = H / (16 * RS), KB = I / 32, I8 = I / 8;
  const int u = blockIdx.x / NG, sg = blockIdx.x % NG;
  const DecodeUnit* un = &plan->unit[u];
  const int cnt = un->count;
  if (cnt <= 0) return;
  const int64_t pay = (int64_t)H * I / 2, sca = (int64_t)H * I / 16;
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, r = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ss = wave % RS, sw = wave / RS, sl = sg * RS + ss;  // this wave's slice, its place in it
  // a record installed by this call was copied whole by k_gateup, the previous kernel on the stream
  const uint8_t* rec = arena + (int64_t)un->slot * R;
  float2* s_ag = reinterpret_cast<float2*>(s_a4 + NT * I8);
  const uint8_t* dp = rec + 2 * pay + (int64_t)sl * KB * 256 + lane * 4;
  const uint8_t* ds = rec + 3 * pay + 2 * sca + (int64_t)sl * KB * 32 + scale_lane_off<FMT>(q, r);

  for (int c0 = 0; c0 < cnt; c0 += NT) {
    const int nt = min(NT, cnt - c0);
    // the weights do not depend on the activations: start their loads first
    uint32_t wd[UNR], rd[UNR];
#pragma unroll
    for (int z = 0; z < UNR; ++z) {
      const int k = sw + NW * z;
      wd[z] = k < KB ? *reinterpret_cast<const uint32_t*>(dp + k * 256) : 0u;
      rd[z] = k < KB ? load_scale_raw<FMT>(ds + k * 32) : 0u;
    }
    // the tokens' activations (16 B per 8-group) and their (scale, sum) pairs into LDS
    for (int i = tid; i < nt * I8; i += kWG) {
      const int j = i / I8, g = i % I8;
      const int64_t tok = (int64_t)u * maxB + c0 + j;
      s_a4[j * I8 + g] = *reinterpret_cast<const uint4*>(a16 + tok * I + g * 8);
      s_ag[j * I8 + g] = ag[tok * I8 + g];
    }
    __syncthreads();
    float acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = 0.f;
#pragma unroll
    for (int z = 0; z < UNR; ++z)
      if (sw + NW * z < KB) down_tile<FMT, NT>(wd[z], rd[z], s_a4, s_ag, sw + NW * z, q, nt, I8, acc);
    for (int kb0 = sw + NW * UNR; kb0 < KB; kb0 += NW * UNR) {
#pragma unroll
      for (int z = 0; z < UNR; ++z) {
        const int k = kb0 + NW * z;
        wd[z] = k < KB ? *reinterpret_cast<const uint32_t*>(dp + k * 256) : 0u;
        rd[z] = k < KB ? load_scale_raw<FMT>(ds + k * 32) : 0u;
      }
#pragma unroll
      for (int z = 0; z < UNR; ++z)
        if (kb0 + NW * z < KB) down_tile<FMT, NT>(wd[z], rd[z], s_a4, s_ag, kb0 + NW * z, q, nt, I8, acc);
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      float v = acc[j];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      acc[j] = v;
    }
    if (lane < 16) {
#pragma unroll
      for (int j = 0; j < NT; ++j) s_red[wave][r][j] = acc[j];
    }
    __syncthreads();
    for (int idx = tid; idx < 16 * RS * nt; idx += kWG) {
      const int j = idx % nt, rr = idx / nt, s2 = rr / 16, row = rr % 16;
      // the slice's waves in order (RS = 1: waves 0, 1, 2, 3)
      float v = s_red[s2][row][j];
#pragma unroll
      for (int w2 = 1; w2 < NW; ++w2) v += s_red[w2 * RS + s2][row][j];
      if (FMT == EFF_WFMT_NVFP4_G16_E4M3) v *= ts[(int64_t)un->flat * 3 + 2];
      const int p = un->entry[c0 + j];
      y[(int64_t)p * H + (sg * RS + s2) * 16 + row] = v;
    }
    __syncthreads();
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

// ---------------------------------------------------------------------------- fetch copy
// Copies the records of a fetch list from the pinned host pool into their slots (16 KiB chunks,
// 16 bytes per thread); entries outside the pool or the arena are skipped.
__global__ void __launch_bounds__(256)
k_fetch_copy(const uint8_t* __restrict__ pool, uint8_t* __restrict__ arena, int64_t R, int64_t n_flat, int S,
             const FetchList* __restrict__ fl) {
  constexpr int64_t kChunk = 16384;
  const int n = min(fl->count, kMaxEntries);
  const int64_t chunks = (R + kChunk - 1) / kChunk;
  for (int64_t c = blockIdx.x; c < (int64_t)n * chunks; c += gridDim.x) {
    const int i = (int)(c / chunks);
    const int64_t off = (c % chunks) * kChunk, len = min(kChunk, R - off);
    const int flat = fl->flat[i], slot = fl->slot[i];
    if (flat < 0 || flat >= n_flat || slot < 0 || slot >= S) continue;
    const uint4* src = reinterpret_cast<const uint4*>(pool + (int64_t)flat * R + off);
    uint4* dst = reinterpret_cast<uint4*>(arena + (int64_t)slot * R + off);
    for (int64_t b = threadIdx.x; b < len / 16; b += 256) dst[b] = src[b];
  }
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

// 16-row slices per down workgroup (measured): 4 when a launch would otherwise have 8192 or more
// small workgroups (qwen3.8-flash-next shape, B = 8 and 16: 47 -> 34 us and 80 -> 58 us); 2 for
// long rows (I >= 1024: the activation stage is shared by enough tiles per wave); else 1 (the
// 35b-a3b shape at B = 1, where fewer, longer workgroups are slower)
int down_slices(int units, int H, int I) {
  if (units * (H / 16) >= 8192 && H % 64 == 0) return 4;
  if (I >= 1024 && H % 32 == 0) return 2;
  return 1;
}

template <int FMT, int NT>
hipError_t launch_ffn_t(eff_engine* e, const uint16_t* x, float* y, int units, hipStream_t s, hipEvent_t after_gateup) {
  const eff_config& c = e->cfg;
  const int H = c.hidden, I = c.inter;
  const int ts = timing_begin(e, EFF_T_DECODE_GATEUP, s);
  // d_a holds 4 bytes per activation: the fp16 values, then one (scale, sum) pair per 8 of them
  uint16_t* a16 = reinterpret_cast<uint16_t*>(e->d_a);
  float2* ag = reinterpret_cast<float2*>(a16 + (size_t)e->maxU * c.max_tokens * I);
  hipLaunchKernelGGL((k_gateup<FMT, NT>), dim3(units * (I / 16)), dim3(kWG), (size_t)(NT > 1 ? NT * H * 2 : 0), s, e->d_arena,
                     e->pool_dev, e->R,
                     e->d_ts, e->d_plan, x, H, I, c.top_k, c.max_tokens, a16, ag);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (after_gateup && (err = hipEventRecord(after_gateup, s)) != hipSuccess) return err;
  timing_mark(e, ts, 1, s);
  timing_mark(e, ts, 2, s);
  size_t lds = (size_t)NT * (I / 8) * (sizeof(uint4) + sizeof(float2));
  const int rs = down_slices(units, H, I);
  if (rs == 4)
    hipLaunchKernelGGL((k_down<FMT, NT, 4>), dim3(units * (H / 64)), dim3(kWG), lds, s, e->d_arena, e->pool_dev, e->R,
                       e->d_ts, e->d_plan, a16, ag, H, I, c.max_tokens, y);
  else if (rs == 2)
    hipLaunchKernelGGL((k_down<FMT, NT, 2>), dim3(units * (H / 32)), dim3(kWG), lds, s, e->d_arena, e->pool_dev, e->R,
                       e->d_ts, e->d_plan, a16, ag, H, I, c.max_tokens, y);
  else
    hipLaunchKernelGGL((k_down<FMT, NT, 1>), dim3(units * (H / 16)), dim3(kWG), lds, s, e->d_arena, e->pool_dev, e->R,
                       e->d_ts, e->d_plan, a16, ag, H, I, c.max_tokens, y);
  err = hipGetLastError();
  timing_mark(e, ts, 3, s);
  return err;
}

}  // namespace

int decode_nt(int maxB) { return maxB >= 8 ? 8 : maxB >= 4 ? 4 : maxB >= 2 ? 2 : 1; }

hipError_t decode_kernels_setup(int fmt, int maxB, int H, int I) {
  // allow N * H * 2 bytes of dynamic LDS for the gate/up kernel and N * I * 3 for the down kernel,
  // for every token width N a call can take
  const int NT = decode_nt(maxB);
  hipError_t err = hipSuccess;
#define SETUP(F, N)                                                                                    \
  if (fmt == F && N <= NT && err == hipSuccess)                                                         \
    err = hipFuncSetAttribute((const void*)k_down<F, N, 1>, hipFuncAttributeMaxDynamicSharedMemorySize, \
                              N * (I / 8) * 24);                                                        \
  if (fmt == F && N <= NT && err == hipSuccess)                                                         \
    err = hipFuncSetAttribute((const void*)k_down<F, N, 2>, hipFuncAttributeMaxDynamicSharedMemorySize, \
                              N * (I / 8) * 24);                                                        \
  if (fmt == F && N <= NT && err == hipSuccess)                                                         \
    err = hipFuncSetAttribute((const void*)k_down<F, N, 4>, hipFuncAttributeMaxDynamicSharedMemorySize, \
                              N * (I / 8) * 24);                                                        \
  if (fmt == F && N <= NT && err == hipSuccess)                                                         \
    err = hipFuncSetAttribute((const void*)k_gateup<F, N>, hipFuncAttributeMaxDynamicSharedMemorySize,  \
                              N * H * 2);
  SETUP(EFF_WFMT_INT4_G32_BF16, 1) SETUP(EFF_WFMT_INT4_G32_BF16, 2) SETUP(EFF_WFMT_INT4_G32_BF16, 4)
  SETUP(EFF_WFMT_INT4_G32_BF16, 8) SETUP(EFF_WFMT_NVFP4_G16_E4M3, 1) SETUP(EFF_WFMT_NVFP4_G16_E4M3, 2)
  SETUP(EFF_WFMT_NVFP4_G16_E4M3, 4) SETUP(EFF_WFMT_NVFP4_G16_E4M3, 8)
#undef SETUP
  return err;
}

hipError_t launch_ffn_decode(eff_engine* e, int layer, const uint16_t* x, const int32_t* slots, int B,
                             float* y, hipStream_t s, bool plan_ready, hipEvent_t after_gateup) {
  (void)layer;
  if (!plan_ready) {
    hipError_t err = launch_plan(e, slots, B * e->cfg.top_k, s);
    if (err != hipSuccess) return err;
  }
  // the token width follows the call's batch (a unit holds at most one entry per token): a B = 1 call
  // takes the widest weight prefetch whatever max_tokens is
  const int NT = decode_nt(B);
  const int units = std::min(e->maxU, B * e->cfg.top_k);  // plan units a call of B tokens can have
  const bool fp4 = e->cfg.wformat == EFF_WFMT_NVFP4_G16_E4M3;
  switch (NT) {
    case 1: return fp4 ? launch_ffn_t<EFF_WFMT_NVFP4_G16_E4M3, 1>(e, x, y, units, s, after_gateup)
                       : launch_ffn_t<EFF_WFMT_INT4_G32_BF16, 1>(e, x, y, units, s, after_gateup);
    case 2: return fp4 ? launch_ffn_t<EFF_WFMT_NVFP4_G16_E4M3, 2>(e, x, y, units, s, after_gateup)
                       : launch_ffn_t<EFF_WFMT_INT4_G32_BF16, 2>(e, x, y, units, s, after_gateup);
    case 4: return fp4 ? launch_ffn_t<EFF_WFMT_NVFP4_G16_E4M3, 4>(e, x, y, units, s, after_gateup)
                       : launch_ffn_t<EFF_WFMT_INT4_G32_BF16, 4>(e, x, y, units, s, after_gateup);
    default: return fp4 ? launch_ffn_t<EFF_WFMT_NVFP4_G16_E4M3, 8>(e, x, y, units, s, after_gateup)
                        : launch_ffn_t<EFF_WFMT_INT4_G32_BF16, 8>(e, x, y, units, s, after_gateup);
  }
}

hipError_t launch_bw_copy(eff_engine* e, int64_t first, int64_t stride, int n, uint8_t* dst, hipStream_t s) {
  const eff_config& c = e->cfg;
  hipLaunchKernelGGL(k_bw_copy, dim3(1024), dim3(256), 0, s, e->pool_dev, e->R,
                     (int64_t)c.num_layers * c.num_experts, first, stride, n, dst);
  return hipGetLastError();
}

hipError_t launch_fetch_copy(eff_engine* e, int which, hipStream_t s) {
  const eff_config& c = e->cfg;
  hipLaunchKernelGGL(k_fetch_copy, dim3(256), dim3(256), 0, s, e->pool_dev, e->d_arena, e->R,
                     (int64_t)c.num_layers * c.num_experts, c.num_slots, e->d_fetch + which);
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
