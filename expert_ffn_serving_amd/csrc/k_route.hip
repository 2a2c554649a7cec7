// Router logits: fp32 sums in a fixed order (top-K and softmax are in k_cache.hip).
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

// grid: (ceil(E / (4*EE)), ceil(B / TT)).  Wave w of workgroup (bx, by) computes the logits of
// tokens by*TT .. +TT-1 against experts (bx*4 + w)*EE .. +EE-1; every (token, expert) sum keeps
// the fixed lane order, the tile only shares the loads.
template <int V, int TT, int EE>
__global__ void __launch_bounds__(256)
k_logits(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int B, int E, int H,
         float* __restrict__ logits) {
  typedef typename Vec<V>::T VT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e0 = (blockIdx.x * 4 + wave) * EE;
  if (e0 >= E) return;
  const int t0 = blockIdx.y * TT;
  const int rounds = H / (64 * V);
  float acc[TT][EE];
#pragma unroll
  for (int a = 0; a < TT; ++a)
#pragma unroll
    for (int b = 0; b < EE; ++b) acc[a][b] = 0.f;
  for (int c = 0; c < rounds; ++c) {
    const int j0 = 64 * V * c + V * lane;
    float xv[TT][V];
#pragma unroll
    for (int a = 0; a < TT; ++a) {
      if (t0 + a < B) {
        unpack<V>(*reinterpret_cast<const VT*>(x + (int64_t)(t0 + a) * H + j0), xv[a]);
      } else {
#pragma unroll
        for (int i = 0; i < V; ++i) xv[a][i] = 0.f;
      }
    }
#pragma unroll
    for (int b = 0; b < EE; ++b) {
      if (e0 + b < E) {
        float wv[V];
        unpack<V>(*reinterpret_cast<const VT*>(wr + (int64_t)(e0 + b) * H + j0), wv);
#pragma unroll
        for (int a = 0; a < TT; ++a)
#pragma unroll
          for (int i = 0; i < V; ++i) acc[a][b] = fmaf(xv[a][i], wv[i], acc[a][b]);
      }
    }
  }
#pragma unroll
  for (int a = 0; a < TT; ++a)
#pragma unroll
    for (int b = 0; b < EE; ++b) {
      float v = acc[a][b];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) v = v + __shfl_xor(v, o);
      if (lane == 0 && t0 + a < B && e0 + b < E) logits[(int64_t)(t0 + a) * E + e0 + b] = v;
    }
}

template <int V, int TT, int EE>
hipError_t launch_logits_t(const uint16_t* x, const uint16_t* wr, int B, int E, int H, float* lg, hipStream_t s) {
  dim3 g((E + 4 * EE - 1) / (4 * EE), (B + TT - 1) / TT);
  hipLaunchKernelGGL((k_logits<V, TT, EE>), g, dim3(256), 0, s, x, wr, B, E, H, lg);
  return hipGetLastError();
}

template <int V>
hipError_t launch_logits_v(const uint16_t* x, const uint16_t* wr, int B, int E, int H, float* lg,
                           hipStream_t s) {
  if (B <= 2) return launch_logits_t<V, 1, 1>(x, wr, B, E, H, lg, s);
  if (B <= 32) return launch_logits_t<V, 4, 2>(x, wr, B, E, H, lg, s);
  return launch_logits_t<V, 8, 4>(x, wr, B, E, H, lg, s);
}

}  // namespace

hipError_t launch_route_logits(const uint16_t* x, const uint16_t* wr, int B, int E, int H, float* logits,
                               hipStream_t s) {
  if (H % 512 == 0) return launch_logits_v<8>(x, wr, B, E, H, logits, s);
  if (H % 256 == 0) return launch_logits_v<4>(x, wr, B, E, H, logits, s);
  if (H % 128 == 0) return launch_logits_v<2>(x, wr, B, E, H, logits, s);
  return launch_logits_v<1>(x, wr, B, E, H, logits, s);
}

}  // namespace eff
