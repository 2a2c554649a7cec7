// Whole-layer prefill: grouped expert GEMMs on MFMA over the layer's slot buffer.
//
// In prefill nearly every expert of a layer is routed to, so the whole layer is
// streamed into buffer layer%2 and every expert's tokens are computed together
// ([FT-deep] §4 design pattern ①; [FT-blog] §五; [NVMe-8GB] "엔진" item 5 runs a
// whole prompt through one layer so that experts are not re-read per chunk).
//
//   k_pf_sort     one workgroup: count (t,k) pairs per expert, scan, place
//   k_pf_gateup   per (expert, 256 rows of I): [n_e x H] x [H x 256] for gate and up
//                 on v_mfma_f32_16x16x32_f16, SwiGLU in the epilogue -> fp16 a
//   k_pf_down     per (expert, 256 rows of H): [n_e x I] x [I x 256] -> fp32 y per pair
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
// as fp16 (bf16 inputs convert exactly inside fp16's normal range).
#include "eff_internal.h"

namespace eff {
namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMT = 64;       // tokens per M pass (4 subtiles of 16)

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

__device__ inline uint32_t pk_f16(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
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
    // pairs (e0,e4), (e1,e5), (e2,e6), (e3,e7); the activation tile uses the same order
    const uint32_t off = 0xE408E408u;  // fp16(-1032) in both halves
    o[0] = pk_fma_off((d & 0x000F000Fu) | 0x64006400u, off, s2);
    o[1] = pk_fma_off(((d >> 4) & 0x000F000Fu) | 0x64006400u, off, s2);
    o[2] = pk_fma_off(((d >> 8) & 0x000F000Fu) | 0x64006400u, off, s2);
    o[3] = pk_fma_off(((d >> 12) & 0x000F000Fu) | 0x64006400u, off, s2);
  }
  uint4 u4 = make_uint4(o[0], o[1], o[2], o[3]);
  return __builtin_bit_cast(f16x8_t, u4);
}

// 4 scales of one lane for the tiles of 4 consecutive row slices (tiles tstride apart, scale
// areas tstride/8 apart) as fp16 pairs
template <int FMT>
__device__ inline void load_scales(const uint8_t* sp, int64_t sstride, uint32_t* s2) {
  float f[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if (FMT == EFF_WFMT_NVFP4_G16_E4M3)
      f[t] = __builtin_amdgcn_cvt_f32_fp8((uint32_t)sp[t * sstride], 0);
    else
      f[t] = __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t*>(sp + t * sstride) << 16);
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) s2[t] = pk_f16(f[t], f[t]);
}

// Stage a 64 x 32 activation tile into LDS as fp16 (row-major, 64 B per row).  src_bf16: rows
// of a bf16 matrix (x, row index t = entry / K); src_f16: rows of an fp16 matrix indexed by
// sorted position.  Rows >= mt are zero.  int4 permutes each group of 8 as 0,4,1,5,2,6,3,7.
template <int FMT, bool BF16_SRC>
__device__ inline void stage_tile(uint32_t* s_tile, const void* src, int ld, const int32_t* rows, int off,
                                  int m0, int mt, int K, int k0) {
  const int tid = threadIdx.x;
  const int row = tid >> 2, ch = tid & 3;  // 64 rows x 4 chunks of 8
  uint32_t o[4] = {0u, 0u, 0u, 0u};
  if (row < mt) {
    uint4 v;
    if (BF16_SRC) {
      const int t = rows[off + m0 + row] / K;
      v = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(src) + (int64_t)t * ld + k0 + ch * 8);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      float f[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
      if (FMT == EFF_WFMT_INT4_G32_BF16) {
        o[0] = pk_f16(f[0], f[4]); o[1] = pk_f16(f[1], f[5]); o[2] = pk_f16(f[2], f[6]); o[3] = pk_f16(f[3], f[7]);
      } else {
        o[0] = pk_f16(f[0], f[1]); o[1] = pk_f16(f[2], f[3]); o[2] = pk_f16(f[4], f[5]); o[3] = pk_f16(f[6], f[7]);
      }
    } else {
      v = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(src) + (int64_t)(off + m0 + row) * ld +
                                          k0 + ch * 8);
      if (FMT == EFF_WFMT_INT4_G32_BF16) {
        // halves h0..h7 in v.x = h0|h1, v.y = h2|h3, v.z = h4|h5, v.w = h6|h7
        o[0] = (v.x & 0xFFFFu) | (v.z << 16);
        o[1] = (v.x >> 16) | (v.z & 0xFFFF0000u);
        o[2] = (v.y & 0xFFFFu) | (v.w << 16);
        o[3] = (v.y >> 16) | (v.w & 0xFFFF0000u);
      } else {
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
      }
    }
  }
  *reinterpret_cast<uint4*>(s_tile + row * 16 + ch * 4) = make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ inline float silu(float z) { return z / (1.0f + expf(-z)); }

// The 4 bytes of this lane in the same k tile of 4 consecutive row slices (tstride bytes apart).
__device__ inline uint4 load_block(const uint8_t* p, int64_t tstride) {
  return make_uint4(*reinterpret_cast<const uint32_t*>(p), *reinterpret_cast<const uint32_t*>(p + tstride),
                    *reinterpret_cast<const uint32_t*>(p + 2 * tstride),
                    *reinterpret_cast<const uint32_t*>(p + 3 * tstride));
}

// grid: E * (I / 256); 4 waves, wave w owns row block nb = j*4 + w of gate and up
template <int FMT>
__global__ void __launch_bounds__(256)
k_pf_gateup(const uint8_t* __restrict__ arena, int64_t R, const float* __restrict__ ts,
            const int32_t* __restrict__ owner, int slot_base, const int32_t* __restrict__ slot_of,
            const int32_t* __restrict__ offsets, const int32_t* __restrict__ rows,
            const uint16_t* __restrict__ x, int E, int H, int I, int K, uint16_t* __restrict__ a_out) {
  __shared__ uint32_t s_tile[kMT * 16];  // 64 rows x 32 fp16
  const int NJ = (I / 64 + 3) / 4;
  int e, j;
  map_block(blockIdx.x, E, NJ, &e, &j);
  if (e >= E) return;
  const int off = offsets[e], ne = offsets[e + 1] - off;
  if (ne <= 0) return;
  const int slot = slot_base >= 0 ? slot_base + e : slot_of[e];
  const uint8_t* rec = arena + (int64_t)slot * R;
  const int64_t pay = (int64_t)H * I / 2, sca = (int64_t)H * I / 16;
  const int NB = I / 64, KB = H / 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, q = lane >> 4, r = lane & 15;
  const int nb = j * 4 + wave;
  const bool active = nb < NB;  // waves past the last row block only help stage tiles
  // this wave's 64 rows are row slices 4nb..4nb+3: tiles KB*256 bytes apart, k tiles 256 apart
  const int64_t tstride = (int64_t)KB * 256, sstride = (int64_t)KB * 32;
  const uint8_t* gp = rec + (int64_t)nb * 4 * tstride + lane * 4;
  const uint8_t* gs = rec + 3 * pay + (int64_t)nb * 4 * sstride +
                      (FMT == EFF_WFMT_INT4_G32_BF16 ? r * 2 : (q >> 1) * 16 + r);
  float tsg = 1.f, tsu = 1.f;
  if (FMT == EFF_WFMT_NVFP4_G16_E4M3) {
    const int fl = owner[slot];
    tsg = ts[(int64_t)fl * 3];
    tsu = ts[(int64_t)fl * 3 + 1];
  }
  for (int m0 = 0; m0 < ne; m0 += kMT) {
    const int mt = min(kMT, ne - m0), msub = (mt + 15) / 16;
    f32x4_t acc[2][4][4];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[m][t][s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    uint4 wn[2] = {make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u)};
    uint32_t sn[2][4] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
    if (active) {
      wn[0] = load_block(gp, tstride);
      wn[1] = load_block(gp + pay, tstride);
      load_scales<FMT>(gs, sstride, sn[0]);
      load_scales<FMT>(gs + sca, sstride, sn[1]);
    }
    for (int kb = 0; kb < KB; ++kb) {
      const uint4 wc[2] = {wn[0], wn[1]};
      uint32_t sc[2][4];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int t = 0; t < 4; ++t) sc[m][t] = sn[m][t];
      if (active && kb + 1 < KB) {  // prefetch the next k tile
        wn[0] = load_block(gp + (kb + 1) * 256, tstride);
        wn[1] = load_block(gp + pay + (kb + 1) * 256, tstride);
        load_scales<FMT>(gs + (kb + 1) * 32, sstride, sn[0]);
        load_scales<FMT>(gs + sca + (kb + 1) * 32, sstride, sn[1]);
      }
      __syncthreads();
      stage_tile<FMT, true>(s_tile, x, H, rows, off, m0, mt, K, kb * 32);
      __syncthreads();
      if (!active) continue;
      f16x8_t af[4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if (s < msub) af[s] = __builtin_bit_cast(f16x8_t, *reinterpret_cast<const uint4*>(s_tile + (s * 16 + r) * 16 + q * 4));
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const uint32_t dw[4] = {wc[m].x, wc[m].y, wc[m].z, wc[m].w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const f16x8_t bfrag = dequant8<FMT>(dw[t], sc[m][t]);
#pragma unroll
          for (int s = 0; s < 4; ++s)
            if (s < msub) acc[m][t][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[s], bfrag, acc[m][t][s], 0, 0, 0);
        }
      }
    }
    // epilogue: a = silu(g) * u, rows m0 + s*16 + 4*q + i, column nb*64 + t*16 + r
    if (!active) continue;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = s * 16 + q * 4 + i;
          if (rr < mt) {
            const float g = acc[0][t][s][i] * tsg, u = acc[1][t][s][i] * tsu;
            const _Float16 av = (_Float16)(silu(g) * u);
            a_out[(int64_t)(off + m0 + rr) * I + nb * 64 + t * 16 + r] = __builtin_bit_cast(uint16_t, av);
          }
        }
  }
}

// grid: E * (H / 256); wave w owns row block nb = j*4 + w of down
template <int FMT>
__global__ void __launch_bounds__(256)
k_pf_down(const uint8_t* __restrict__ arena, int64_t R, const float* __restrict__ ts,
          const int32_t* __restrict__ owner, int slot_base, const int32_t* __restrict__ slot_of,
          const int32_t* __restrict__ offsets, const int32_t* __restrict__ rows,
          const uint16_t* __restrict__ a_in, int E, int H, int I, float* __restrict__ y) {
  __shared__ uint32_t s_tile[kMT * 16];
  const int NJ = (H / 64 + 3) / 4;
  int e, j;
  map_block(blockIdx.x, E, NJ, &e, &j);
  if (e >= E) return;
  const int off = offsets[e], ne = offsets[e + 1] - off;
  if (ne <= 0) return;
  const int slot = slot_base >= 0 ? slot_base + e : slot_of[e];
  const uint8_t* rec = arena + (int64_t)slot * R;
  const int64_t pay = (int64_t)H * I / 2, sca = (int64_t)H * I / 16;
  const int NB = H / 64, KB = I / 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, q = lane >> 4, r = lane & 15;
  const int nb = j * 4 + wave;
  const bool active = nb < NB;
  const int64_t tstride = (int64_t)KB * 256, sstride = (int64_t)KB * 32;
  const uint8_t* dp = rec + 2 * pay + (int64_t)nb * 4 * tstride + lane * 4;
  const uint8_t* ds = rec + 3 * pay + 2 * sca + (int64_t)nb * 4 * sstride +
                      (FMT == EFF_WFMT_INT4_G32_BF16 ? r * 2 : (q >> 1) * 16 + r);
  float tsd = 1.f;
  if (FMT == EFF_WFMT_NVFP4_G16_E4M3) tsd = ts[(int64_t)owner[slot] * 3 + 2];
  for (int m0 = 0; m0 < ne; m0 += kMT) {
    const int mt = min(kMT, ne - m0), msub = (mt + 15) / 16;
    f32x4_t acc[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int s = 0; s < 4; ++s) acc[t][s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    uint4 wn = make_uint4(0u, 0u, 0u, 0u);
    uint32_t sn[4] = {0u, 0u, 0u, 0u};
    if (active) {
      wn = load_block(dp, tstride);
      load_scales<FMT>(ds, sstride, sn);
    }
    for (int kb = 0; kb < KB; ++kb) {
      const uint4 wc = wn;
      uint32_t sc[4] = {sn[0], sn[1], sn[2], sn[3]};
      if (active && kb + 1 < KB) {
        wn = load_block(dp + (kb + 1) * 256, tstride);
        load_scales<FMT>(ds + (kb + 1) * 32, sstride, sn);
      }
      __syncthreads();
      stage_tile<FMT, false>(s_tile, a_in, I, rows, off, m0, mt, 0, kb * 32);
      __syncthreads();
      if (!active) continue;
      f16x8_t af[4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if (s < msub) af[s] = __builtin_bit_cast(f16x8_t, *reinterpret_cast<const uint4*>(s_tile + (s * 16 + r) * 16 + q * 4));
      const uint32_t dw[4] = {wc.x, wc.y, wc.z, wc.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const f16x8_t bfrag = dequant8<FMT>(dw[t], sc[t]);
#pragma unroll
        for (int s = 0; s < 4; ++s)
          if (s < msub) acc[t][s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[s], bfrag, acc[t][s], 0, 0, 0);
      }
    }
    if (!active) continue;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = s * 16 + q * 4 + i;
          if (rr < mt) {
            const int p = rows[off + m0 + rr];
            y[(int64_t)p * H + nb * 64 + t * 16 + r] = acc[t][s][i] * tsd;
          }
        }
  }
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
  const int nbx1 = ((E + 7) / 8) * 8 * ((I / 64 + 3) / 4);
  const int nbx2 = ((E + 7) / 8) * 8 * ((H / 64 + 3) / 4);
  const int ts = timing_begin(e, EFF_T_PREFILL_GATEUP, s);
  if (fp4)
    hipLaunchKernelGGL(k_pf_gateup<EFF_WFMT_NVFP4_G16_E4M3>, dim3(nbx1), dim3(256), 0, s, e->d_arena, e->R,
                       e->d_ts, e->d_owner, slot_base, slot_of_expert, e->d_pf_count, e->d_pf_rows, x, E, H, I,
                       K, e->d_pf_a);
  else
    hipLaunchKernelGGL(k_pf_gateup<EFF_WFMT_INT4_G32_BF16>, dim3(nbx1), dim3(256), 0, s, e->d_arena, e->R,
                       e->d_ts, e->d_owner, slot_base, slot_of_expert, e->d_pf_count, e->d_pf_rows, x, E, H, I,
                       K, e->d_pf_a);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  timing_mark(e, ts, 1, s);
  timing_mark(e, ts, 2, s);
  if (fp4)
    hipLaunchKernelGGL(k_pf_down<EFF_WFMT_NVFP4_G16_E4M3>, dim3(nbx2), dim3(256), 0, s, e->d_arena, e->R,
                       e->d_ts, e->d_owner, slot_base, slot_of_expert, e->d_pf_count, e->d_pf_rows, e->d_pf_a,
                       E, H, I, e->d_pf_y);
  else
    hipLaunchKernelGGL(k_pf_down<EFF_WFMT_INT4_G32_BF16>, dim3(nbx2), dim3(256), 0, s, e->d_arena, e->R,
                       e->d_ts, e->d_owner, slot_base, slot_of_expert, e->d_pf_count, e->d_pf_rows, e->d_pf_a,
                       E, H, I, e->d_pf_y);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  timing_mark(e, ts, 3, s);
  if (!combine) return hipSuccess;
  return launch_combine(e->d_pf_y, nullptr, nullptr, w, T, K, H, out, s);
}

}  // namespace eff
