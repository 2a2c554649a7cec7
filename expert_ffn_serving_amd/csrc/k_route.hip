// Router: fp32 logits in a fixed summation order, then top-K and softmax over the K.
//
// Routing is computed exactly and the model is left untouched ([FT-deep] §2);
// the router runs on the GPU ahead of the hit/miss split ([FT-blog] §二).  The
// expert ids must be reproducible bit for bit, so the fp32 order is fixed:
// lane l of a wave adds x[j]*w[j] for j = 64*V*c + V*l + i (c outer, i inner;
// V = 8, 4, 2 or 1, the largest with H % (64*V) == 0), then the 64 lane sums are
// folded pairwise (l, l^o) for o = 32, 16, ..., 1.  A product of two bf16 values
// is exact in fp32, so a fused multiply-add equals the separate add.
#include "eff_internal.h"

namespace eff {
namespace {

template <int V>
struct Vec;
template <>
struct Vec<8> { typedef uint4 T; };
template <>
struct Vec<4> { typedef uint2 T; };
template <>
struct Vec<2> { typedef uint32_t T; };
template <>
struct Vec<1> { typedef uint16_t T; };

template <int V>
__device__ inline void unpack(const typename Vec<V>::T& v, float* out);
template <>
__device__ inline void unpack<8>(const uint4& v, float* o) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
template <>
__device__ inline void unpack<4>(const uint2& v, float* o) {
  o[0] = __uint_as_float(v.x << 16);
  o[1] = __uint_as_float(v.x & 0xFFFF0000u);
  o[2] = __uint_as_float(v.y << 16);
  o[3] = __uint_as_float(v.y & 0xFFFF0000u);
}
template <>
__device__ inline void unpack<2>(const uint32_t& v, float* o) {
  o[0] = __uint_as_float(v << 16);
  o[1] = __uint_as_float(v & 0xFFFF0000u);
}
template <>
__device__ inline void unpack<1>(const uint16_t& v, float* o) {
  o[0] = __uint_as_float((uint32_t)v << 16);
}

// grid: (ceil(E / (4*EPW)), ceil(B / TB)); wave w handles experts bx*4*EPW + w*EPW + [0, EPW)
// for the tokens of tile by.
template <int V, int EPW>
__global__ void __launch_bounds__(256)
k_logits(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int B, int E, int H, int TB,
         float* __restrict__ logits) {
  typedef typename Vec<V>::T VT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e0 = (blockIdx.x * 4 + wave) * EPW;
  if (e0 >= E) return;
  const int t0 = blockIdx.y * TB, t1 = min(B, t0 + TB);
  const int rounds = H / (64 * V);
  for (int t = t0; t < t1; ++t) {
    float acc[EPW];
#pragma unroll
    for (int q = 0; q < EPW; ++q) acc[q] = 0.f;
    for (int c = 0; c < rounds; ++c) {
      const int j0 = 64 * V * c + V * lane;
      float xv[V];
      unpack<V>(*reinterpret_cast<const VT*>(x + (int64_t)t * H + j0), xv);
#pragma unroll
      for (int q = 0; q < EPW; ++q) {
        if (e0 + q < E) {
          float wv[V];
          unpack<V>(*reinterpret_cast<const VT*>(wr + (int64_t)(e0 + q) * H + j0), wv);
#pragma unroll
          for (int i = 0; i < V; ++i) acc[q] = fmaf(xv[i], wv[i], acc[q]);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < EPW; ++q) {
      float v = acc[q];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) v = v + __shfl_xor(v, o);
      if (lane == 0 && e0 + q < E) logits[(int64_t)t * E + e0 + q] = v;
    }
  }
}

__device__ inline bool better(float a, int ia, float b, int ib) { return a > b || (a == b && ia < ib); }

// one workgroup per token: K rounds of block argmax over E logits by (logit desc, id asc)
__global__ void __launch_bounds__(256)
k_topk(const float* __restrict__ logits, int E, int K, int32_t* __restrict__ ids, float* __restrict__ w) {
  extern __shared__ float s_l[];            // [E]
  __shared__ int32_t s_taken[kMaxExperts / 32];
  __shared__ float s_bv[4];
  __shared__ int s_bi[4];
  __shared__ float s_sel[kMaxTopK];
  __shared__ int s_selid[kMaxTopK];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += blockDim.x) s_l[e] = logits[(int64_t)t * E + e];
  for (int i = tid; i < (E + 31) / 32; i += blockDim.x) s_taken[i] = 0;
  __syncthreads();
  for (int k = 0; k < K; ++k) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int e = tid; e < E; e += blockDim.x) {
      if ((s_taken[e >> 5] >> (e & 31)) & 1) continue;
      float v = s_l[e];
      if (bi == 0x7FFFFFFF || better(v, e, bv, bi)) {
        bv = v;
        bi = e;
      }
    }
    for (int o = 32; o >= 1; o >>= 1) {
      float ov = __shfl_xor(bv, o);
      int oi = __shfl_xor(bi, o);
      if (oi != 0x7FFFFFFF && (bi == 0x7FFFFFFF || better(ov, oi, bv, bi))) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == 0) {
      s_bv[wave] = bv;
      s_bi[wave] = bi;
    }
    __syncthreads();
    if (tid == 0) {
      float v = s_bv[0];
      int i = s_bi[0];
      for (int q = 1; q < 4; ++q)
        if (s_bi[q] != 0x7FFFFFFF && (i == 0x7FFFFFFF || better(s_bv[q], s_bi[q], v, i))) {
          v = s_bv[q];
          i = s_bi[q];
        }
      s_sel[k] = v;
      s_selid[k] = i;
      s_taken[i >> 5] |= 1 << (i & 31);
    }
    __syncthreads();
  }
  if (tid == 0) {
    // softmax over the K selected logits, relative to the largest
    float sum = 0.f;
    for (int k = 0; k < K; ++k) sum += expf(s_sel[k] - s_sel[0]);
    for (int k = 0; k < K; ++k) {
      ids[(int64_t)t * K + k] = s_selid[k];
      w[(int64_t)t * K + k] = expf(s_sel[k] - s_sel[0]) / sum;
    }
  }
}

template <int V>
hipError_t launch_logits_v(const uint16_t* x, const uint16_t* wr, int B, int E, int H, float* lg,
                           hipStream_t s) {
  if (B <= 32) {
    dim3 g((E + 3) / 4, 1);
    hipLaunchKernelGGL((k_logits<V, 1>), g, dim3(256), 0, s, x, wr, B, E, H, B, lg);
  } else {
    const int TB = 64;
    dim3 g((E + 15) / 16, (B + TB - 1) / TB);
    hipLaunchKernelGGL((k_logits<V, 4>), g, dim3(256), 0, s, x, wr, B, E, H, TB, lg);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route_logits(const uint16_t* x, const uint16_t* wr, int B, int E, int H, float* logits,
                               hipStream_t s) {
  if (H % 512 == 0) return launch_logits_v<8>(x, wr, B, E, H, logits, s);
  if (H % 256 == 0) return launch_logits_v<4>(x, wr, B, E, H, logits, s);
  if (H % 128 == 0) return launch_logits_v<2>(x, wr, B, E, H, logits, s);
  return launch_logits_v<1>(x, wr, B, E, H, logits, s);
}

hipError_t launch_topk(const float* logits, int B, int E, int K, int32_t* ids, float* w, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_topk, dim3(B), dim3(256), (size_t)E * sizeof(float), s, logits, E, K, ids, w);
  return hipGetLastError();
}

}  // namespace eff
