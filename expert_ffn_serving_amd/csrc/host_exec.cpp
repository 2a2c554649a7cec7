// Host share of a decode step: the same SwiGLU expert on the CPU, straight from
// the pinned pool, for the entries the split left to the host.
//
// [FT-deep] §4 design pattern ③: the host executor receives the routed ids with
// -1 wherever the GPU owns the entry and skips those; §7: it runs one thread per
// physical core because decode on the host is bound by memory bandwidth
// ([FT-blog] §三.2).  fp32 accumulation, fixed order per output row.
#include <immintrin.h>
#include <pthread.h>
#include <sched.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <set>
#include <utility>
#include <vector>

#include "eff_internal.h"

namespace eff {

namespace {

struct Tables {
  float e4m3[256];
  float e2m1[16];
  Tables() {
    for (int c = 0; c < 256; ++c) {
      int s = (c >> 7) & 1, ex = (c >> 3) & 15, m = c & 7;
      float v = (ex == 0) ? std::ldexp((float)m, -9) : std::ldexp(1.0f + m / 8.0f, ex - 7);
      if (ex == 15 && m == 7) v = NAN;
      e4m3[c] = s ? -v : v;
    }
    static const float mag[8] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};
    for (int c = 0; c < 16; ++c) e2m1[c] = (c & 8) ? -mag[c & 7] : mag[c & 7];
  }
};
const Tables& tables() {
  static Tables t;
  return t;
}

inline float bf16f(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}
inline uint16_t f2bf_trunc(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}
inline uint16_t f2bf_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// The slice kernels: rows 16*sl .. 16*sl+15 of one matrix (KB tiles of 16 rows x 32 inputs, the
// slice's tiles contiguous at pay + (sl*KB + kb)*256, scales at sca + (sl*KB + kb)*32) against
// `nrows` bf16 input rows; row i accumulates into token i % nt (so a value can come as a hi + lo
// pair of rows).  out[r * nt + j] = tscale * sum_k W[16*sl + r][k] * x_j[k], fp32.
// AVX2 + FMA: per row, 8-wide fp32 FMAs over the row's 32 inputs of each tile, reduced at the end.
// The 4 bytes of row r, inputs 8q..8q+7 of a tile are its dword (q*16 + r).
__attribute__((target("avx2,fma"))) void slice_avx2(const uint8_t* pay, const uint8_t* sca, int KB, int sl, int fmt,
                                                   const uint16_t* const* xr, int nrows, int nt, float tscale,
                                                   float* out) {
  const __m256i shifts = _mm256_setr_epi32(0, 4, 8, 12, 16, 20, 24, 28);
  const __m256i m15 = _mm256_set1_epi32(15), m7 = _mm256_set1_epi32(7), m8 = _mm256_set1_epi32(8);
  const __m256 eight = _mm256_set1_ps(8.f);
  const __m256 mag = _mm256_setr_ps(0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f);
  const Tables& T = tables();
  __m256 acc[16 * kMaxTokens];
  for (int i = 0; i < 16 * nt; ++i) acc[i] = _mm256_setzero_ps();
  for (int kb = 0; kb < KB; ++kb) {
    const int64_t tile = (int64_t)sl * KB + kb;
    const uint32_t* sp = reinterpret_cast<const uint32_t*>(pay + tile * 256);
    const uint8_t* sb = sca + tile * 32;
    __m256 xv[2 * kMaxTokens][4];
    for (int i = 0; i < nrows; ++i)
      for (int q = 0; q < 4; ++q) {
        const __m128i b = _mm_loadu_si128(reinterpret_cast<const __m128i*>(xr[i] + kb * 32 + q * 8));
        xv[i][q] = _mm256_castsi256_ps(_mm256_slli_epi32(_mm256_cvtepu16_epi32(b), 16));
      }
    for (int r = 0; r < 16; ++r) {
      __m256 w[4];
      for (int q = 0; q < 4; ++q) {
        const __m256i c = _mm256_and_si256(_mm256_srlv_epi32(_mm256_set1_epi32((int)sp[q * 16 + r]), shifts), m15);
        if (fmt == EFF_WFMT_INT4_G32_BF16) {
          w[q] = _mm256_sub_ps(_mm256_cvtepi32_ps(c), eight);
        } else {
          const __m256 v = _mm256_permutevar8x32_ps(mag, _mm256_and_si256(c, m7));
          const __m256i sgn = _mm256_slli_epi32(_mm256_and_si256(c, m8), 28);
          w[q] = _mm256_xor_ps(v, _mm256_castsi256_ps(sgn));
        }
      }
      float s0, s1;
      if (fmt == EFF_WFMT_INT4_G32_BF16) {
        uint16_t sbits;
        std::memcpy(&sbits, sb + r * 2, 2);
        s0 = s1 = bf16f(sbits);
      } else {
        s0 = T.e4m3[sb[r]];
        s1 = T.e4m3[sb[16 + r]];
      }
      const __m256 vs0 = _mm256_set1_ps(s0), vs1 = _mm256_set1_ps(s1);
      for (int i = 0; i < nrows; ++i) {
        __m256 h0 = _mm256_mul_ps(w[0], xv[i][0]);
        h0 = _mm256_fmadd_ps(w[1], xv[i][1], h0);
        __m256 h1 = _mm256_mul_ps(w[2], xv[i][2]);
        h1 = _mm256_fmadd_ps(w[3], xv[i][3], h1);
        __m256& a = acc[(size_t)r * nt + (i % nt)];
        a = _mm256_fmadd_ps(h0, vs0, a);
        a = _mm256_fmadd_ps(h1, vs1, a);
      }
    }
  }
  for (int r = 0; r < 16; ++r)
    for (int j = 0; j < nt; ++j) {
      alignas(32) float v[8];
      _mm256_store_ps(v, acc[(size_t)r * nt + j]);
      out[r * nt + j] = (((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]))) * tscale;
    }
}

// AVX-512 BF16: the 16 rows of a tile are the 16 dword lanes of a zmm.  Shifting a row's dword
// (inputs 8q..8q+7, input 8q+e in nibble e) right by 4m and masking with 0x000F000F leaves the
// codes of inputs 8q+m and 8q+m+4 in the two 16-bit halves of each lane; vpermw maps them to
// bf16 weights (exact for int4 and e2m1), and vdpbf16ps multiplies them with the broadcast bf16
// pair (x[8q+m], x[8q+m+4]): products exact, fp32 accumulation.  The inputs therefore come in
// "paired" order (pair_pos), prepared once per call.  Scales per (row, group) are applied per
// half tile in fp32; the fp32 tensor scale at the end.
struct MatRef {
  const uint8_t* pay;  // payload of the matrix (tiles of 16 rows x 32 inputs)
  const uint8_t* sca;  // its scale bytes
  float tscale;        // NVFP4 tensor scale, 1 for int4
  float* out;          // out[r * nt + j] for the slice's 16 rows
};

// bf16 bit patterns of the 16 codes, indexed by code (entries 16..31 unused)
struct CodeTables {
  alignas(64) uint16_t int4[32];
  alignas(64) uint16_t e2m1[32];
  CodeTables() {
    for (int u = 0; u < 32; ++u) {
      int4[u] = u < 16 ? f2bf_trunc((float)(u - 8)) : 0;  // exact
      e2m1[u] = u < 16 ? f2bf_trunc(tables().e2m1[u]) : 0;
    }
  }
};
const CodeTables& code_tables() {
  static CodeTables t;
  return t;
}

template <int NM, bool FP4>
__attribute__((target("avx512f,avx512bw,avx512bf16"))) void slices_avx512(const MatRef* mat, int KB, int sl,
                                                                          const uint16_t* const* xr, int nrows,
                                                                          int nt) {
  const __m512i table = _mm512_load_si512(FP4 ? code_tables().e2m1 : code_tables().int4);
  const __m512i lo4 = _mm512_set1_epi32(0x000F000F);
  __m512 tot[NM][kMaxTokens];
  for (int mi = 0; mi < NM; ++mi)
    for (int j = 0; j < nt; ++j) tot[mi][j] = _mm512_setzero_ps();
  for (int kb = 0; kb < KB; ++kb) {
    const int64_t tile = (int64_t)sl * KB + kb;
    __m512 sc[NM][2];
    for (int mi = 0; mi < NM; ++mi) {
      const uint8_t* sp = mat[mi].sca + tile * 32;
      if (!FP4) {
        const __m256i b = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(sp));
        sc[mi][0] = sc[mi][1] = _mm512_castsi512_ps(_mm512_slli_epi32(_mm512_cvtepu16_epi32(b), 16));
      } else {
        // e4m3 -> fp32: magnitude bits placed under the fp32 exponent/mantissa, times 2^120
        // (normals and subnormals alike), then the sign
        const __m512 k120 = _mm512_set1_ps(1.329227995784916e36f);  // 2^120
        const __m512i x7f = _mm512_set1_epi32(0x7F), x80 = _mm512_set1_epi32(0x80);
        for (int h = 0; h < 2; ++h) {
          const __m512i c = _mm512_cvtepu8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(sp + 16 * h)));
          const __m512 m = _mm512_mul_ps(_mm512_castsi512_ps(_mm512_slli_epi32(_mm512_and_si512(c, x7f), 20)), k120);
          sc[mi][h] = _mm512_castsi512_ps(
              _mm512_or_si512(_mm512_castps_si512(m), _mm512_slli_epi32(_mm512_and_si512(c, x80), 24)));
        }
      }
    }
    for (int h = 0; h < 2; ++h) {  // inputs 16h .. 16h+15 of the tile (one scale group for NVFP4)
      __m512i w[NM][8];
      for (int mi = 0; mi < NM; ++mi)
        for (int qq = 0; qq < 2; ++qq) {
          const __m512i d = _mm512_loadu_si512(mat[mi].pay + tile * 256 + 64 * (2 * h + qq));
          w[mi][4 * qq + 0] = _mm512_permutexvar_epi16(_mm512_and_si512(d, lo4), table);
          w[mi][4 * qq + 1] = _mm512_permutexvar_epi16(_mm512_and_si512(_mm512_srli_epi32(d, 4), lo4), table);
          w[mi][4 * qq + 2] = _mm512_permutexvar_epi16(_mm512_and_si512(_mm512_srli_epi32(d, 8), lo4), table);
          w[mi][4 * qq + 3] = _mm512_permutexvar_epi16(_mm512_and_si512(_mm512_srli_epi32(d, 12), lo4), table);
        }
      for (int i = 0; i < nrows; ++i) {
        const int32_t* xk = reinterpret_cast<const int32_t*>(xr[i] + kb * 32 + 16 * h);  // 8 bf16 pairs
        __m512 a[NM], b[NM];  // two accumulation chains per matrix (even and odd pairs)
        for (int mi = 0; mi < NM; ++mi) a[mi] = b[mi] = _mm512_setzero_ps();
        for (int z = 0; z < 8; z += 2) {
          const __m512bh bx0 = (__m512bh)_mm512_set1_epi32(xk[z]), bx1 = (__m512bh)_mm512_set1_epi32(xk[z + 1]);
          for (int mi = 0; mi < NM; ++mi) {
            a[mi] = _mm512_dpbf16_ps(a[mi], (__m512bh)w[mi][z], bx0);
            b[mi] = _mm512_dpbf16_ps(b[mi], (__m512bh)w[mi][z + 1], bx1);
          }
        }
        for (int mi = 0; mi < NM; ++mi) a[mi] = _mm512_add_ps(a[mi], b[mi]);
        const int j = i < nt ? i : i - nt;
        for (int mi = 0; mi < NM; ++mi) tot[mi][j] = _mm512_fmadd_ps(sc[mi][h], a[mi], tot[mi][j]);
      }
    }
  }
  for (int mi = 0; mi < NM; ++mi) {
    const __m512 ts = _mm512_set1_ps(mat[mi].tscale);
    for (int j = 0; j < nt; ++j) {
      alignas(64) float v[16];
      _mm512_store_ps(v, _mm512_mul_ps(tot[mi][j], ts));
      for (int r = 0; r < 16; ++r) mat[mi].out[r * nt + j] = v[r];
    }
  }
}

// AVX-512F (no BF16 dot product): the 16 rows of a tile are the 16 dword lanes of a zmm as above;
// shifting a row dword right by 4m and masking leaves the code of input 8q+m in each lane, and one
// vpermps maps the 16 codes to fp32 weights (exact).  Each weight vector meets the broadcast fp32
// input of its column; the half-tile sums get the (row, group) scales, the tensor scale comes last.
// Inputs in natural order.
template <int NM, bool FP4>
__attribute__((target("avx512f"))) void slices_avx512f(const MatRef* mat, int KB, int sl, const uint16_t* const* xr,
                                                      int nrows, int nt) {
  alignas(64) float tab[16];
  for (int c = 0; c < 16; ++c) tab[c] = FP4 ? tables().e2m1[c] : (float)(c - 8);
  const __m512 table = _mm512_load_ps(tab);
  const __m512i m15 = _mm512_set1_epi32(15);
  __m512 tot[NM][kMaxTokens];
  for (int mi = 0; mi < NM; ++mi)
    for (int j = 0; j < nt; ++j) tot[mi][j] = _mm512_setzero_ps();
  alignas(64) float xf[2 * kMaxTokens][32];
  for (int kb = 0; kb < KB; ++kb) {
    const int64_t tile = (int64_t)sl * KB + kb;
    for (int i = 0; i < nrows; ++i)
      for (int h = 0; h < 2; ++h) {
        const __m256i b = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(xr[i] + kb * 32 + 16 * h));
        _mm512_store_ps(&xf[i][16 * h], _mm512_castsi512_ps(_mm512_slli_epi32(_mm512_cvtepu16_epi32(b), 16)));
      }
    __m512 sc[NM][2];
    for (int mi = 0; mi < NM; ++mi) {
      const uint8_t* sp = mat[mi].sca + tile * 32;
      if (!FP4) {
        const __m256i b = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(sp));
        sc[mi][0] = sc[mi][1] = _mm512_castsi512_ps(_mm512_slli_epi32(_mm512_cvtepu16_epi32(b), 16));
      } else {
        const __m512 k120 = _mm512_set1_ps(1.329227995784916e36f);  // 2^120, as in the BF16 kernel
        const __m512i x7f = _mm512_set1_epi32(0x7F), x80 = _mm512_set1_epi32(0x80);
        for (int h = 0; h < 2; ++h) {
          const __m512i c = _mm512_cvtepu8_epi32(_mm_loadu_si128(reinterpret_cast<const __m128i*>(sp + 16 * h)));
          const __m512 m = _mm512_mul_ps(_mm512_castsi512_ps(_mm512_slli_epi32(_mm512_and_si512(c, x7f), 20)), k120);
          sc[mi][h] = _mm512_castsi512_ps(
              _mm512_or_si512(_mm512_castps_si512(m), _mm512_slli_epi32(_mm512_and_si512(c, x80), 24)));
        }
      }
    }
    for (int h = 0; h < 2; ++h) {  // inputs 16h .. 16h+15: dwords q = 2h, 2h+1 of every row
      __m512 w[NM][16];
      for (int mi = 0; mi < NM; ++mi)
        for (int qq = 0; qq < 2; ++qq) {
          const __m512i d = _mm512_loadu_si512(mat[mi].pay + tile * 256 + 64 * (2 * h + qq));
          for (int m = 0; m < 8; ++m)
            w[mi][8 * qq + m] = _mm512_permutexvar_ps(_mm512_and_si512(_mm512_srli_epi32(d, 4 * m), m15), table);
        }
      for (int i = 0; i < nrows; ++i) {
        const int j = i < nt ? i : i - nt;
        for (int mi = 0; mi < NM; ++mi) {
          __m512 a = _mm512_mul_ps(w[mi][0], _mm512_set1_ps(xf[i][16 * h]));
          for (int z = 1; z < 16; ++z) a = _mm512_fmadd_ps(w[mi][z], _mm512_set1_ps(xf[i][16 * h + z]), a);
          tot[mi][j] = _mm512_fmadd_ps(sc[mi][h], a, tot[mi][j]);
        }
      }
    }
  }
  for (int mi = 0; mi < NM; ++mi) {
    const __m512 ts = _mm512_set1_ps(mat[mi].tscale);
    for (int j = 0; j < nt; ++j) {
      alignas(64) float v[16];
      _mm512_store_ps(v, _mm512_mul_ps(tot[mi][j], ts));
      for (int r = 0; r < 16; ++r) mat[mi].out[r * nt + j] = v[r];
    }
  }
}

// Scalar: the same sums one row and one input at a time (any x86-64 host).  Per row and token, the
// half-tile sums get the (row, group) scale, the tensor scale comes last.  Inputs in natural order.
void slices_scalar(const MatRef* mat, int nm, int fmt, int KB, int sl, const uint16_t* const* xr, int nrows,
                   int nt) {
  const Tables& T = tables();
  const bool fp4 = fmt == EFF_WFMT_NVFP4_G16_E4M3;
  for (int mi = 0; mi < nm; ++mi)
    for (int r = 0; r < 16; ++r) {
      float tot[kMaxTokens];
      for (int j = 0; j < nt; ++j) tot[j] = 0.f;
      for (int kb = 0; kb < KB; ++kb) {
        const int64_t tile = (int64_t)sl * KB + kb;
        const uint8_t* pay = mat[mi].pay + tile * 256;
        const uint8_t* sp = mat[mi].sca + tile * 32;
        for (int h = 0; h < 2; ++h) {
          float s;
          if (fp4) {
            s = T.e4m3[sp[16 * h + r]];
          } else {
            uint16_t sb;
            std::memcpy(&sb, sp + 2 * r, 2);
            s = bf16f(sb);
          }
          float w[16];
          for (int qq = 0; qq < 2; ++qq) {
            uint32_t d;
            std::memcpy(&d, pay + 4 * ((2 * h + qq) * 16 + r), 4);
            for (int m = 0; m < 8; ++m) {
              const uint32_t c = (d >> (4 * m)) & 15u;
              w[8 * qq + m] = fp4 ? T.e2m1[c] : (float)((int)c - 8);
            }
          }
          for (int i = 0; i < nrows; ++i) {
            const uint16_t* x = xr[i] + kb * 32 + 16 * h;
            float a = 0.f;
            for (int z = 0; z < 16; ++z) a = std::fma(w[z], bf16f(x[z]), a);
            float& t = tot[i < nt ? i : i - nt];
            t = std::fma(s, a, t);
          }
        }
      }
      for (int j = 0; j < nt; ++j) mat[mi].out[r * nt + j] = tot[j] * mat[mi].tscale;
    }
}

// position of input i in the paired order: inside each group of 8, input e goes to 2*(e%4) + e/4
inline int pair_pos(int i) { return (i & ~7) | ((i & 3) << 1) | ((i >> 2) & 1); }

// rows 16*sl.. of NM matrices (1 or 2, same shape) against the same input rows, with the kernel of
// the engine's instruction set (only the AVX-512 BF16 kernel takes its inputs in paired order)
void run_slices(int isa, int fmt, int nm, const MatRef* m, int KB, int sl, const uint16_t* const* xr, int nrows,
                int nt) {
  const bool fp4 = fmt == EFF_WFMT_NVFP4_G16_E4M3;
  switch (isa) {
    case EFF_HOST_ISA_AVX512_BF16:
      if (nm == 2)
        fp4 ? slices_avx512<2, true>(m, KB, sl, xr, nrows, nt) : slices_avx512<2, false>(m, KB, sl, xr, nrows, nt);
      else
        fp4 ? slices_avx512<1, true>(m, KB, sl, xr, nrows, nt) : slices_avx512<1, false>(m, KB, sl, xr, nrows, nt);
      return;
    case EFF_HOST_ISA_AVX512F:
      if (nm == 2)
        fp4 ? slices_avx512f<2, true>(m, KB, sl, xr, nrows, nt) : slices_avx512f<2, false>(m, KB, sl, xr, nrows, nt);
      else
        fp4 ? slices_avx512f<1, true>(m, KB, sl, xr, nrows, nt) : slices_avx512f<1, false>(m, KB, sl, xr, nrows, nt);
      return;
    case EFF_HOST_ISA_AVX2:
      for (int mi = 0; mi < nm; ++mi)
        slice_avx2(m[mi].pay, m[mi].sca, KB, sl, fmt, xr, nrows, nt, m[mi].tscale, m[mi].out);
      return;
    default:
      slices_scalar(m, nm, fmt, KB, sl, xr, nrows, nt);
  }
}

}  // namespace

// The best host instruction set of the running CPU: AVX-512 BF16 (with BW and VBMI) ->
// AVX-512F -> AVX2 + FMA -> scalar ([FT-deep] §7: the host executor picks the best of these at
// run time).
int host_isa_best() {
  __builtin_cpu_init();
  if (__builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
      __builtin_cpu_supports("avx512vbmi") && __builtin_cpu_supports("avx512bf16"))
    return EFF_HOST_ISA_AVX512_BF16;
  if (__builtin_cpu_supports("avx512f")) return EFF_HOST_ISA_AVX512F;
  if (__builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma")) return EFF_HOST_ISA_AVX2;
  return EFF_HOST_ISA_SCALAR;
}

// Host share of one call: entries with cpu_ids[p] >= 0 get y[p] = W_d (silu(W_g x) * (W_u x)) of
// expert cpu_ids[p] of `layer`, x the entry's token row (bf16).
//
// The work is 16-row slices: U*SI of gate+up (both matrices in one sweep over the shared inputs,
// SwiGLU applied) and U*SH of down.  With C pool threads it runs as 2C ordered tasks: task c < C
// takes a contiguous range of the gate/up slices, task C + c a contiguous range of the down
// slices, so each thread streams contiguous memory and the claiming costs 2C atomic operations
// per call instead of one per slice (on the 16-core host this was measured 1.6x faster than one
// task per slice, and faster than three ranges per thread).  A down range first waits until every gate/up slice of the
// experts it touches is done; tasks are claimed in order, so every gate/up range has been taken
// by a running thread by then and the wait always ends.  The down input a = silu(g)*u goes in as
// a bf16 hi + lo pair (error ~2^-16).  The AVX-512 kernel takes its inputs in paired order: the
// token rows are permuted once per call and a is written that way.
void host_ffn(eff_engine* e, int layer, const uint16_t* x, const int32_t* cpu_ids, int B, float* y) {
  const eff_config& c = e->cfg;
  const int K = c.top_k, H = c.hidden, I = c.inter, E = c.num_experts;
  HostScratch& hs = e->hscratch;
  // unique host experts, ascending, and their entries (at most one per token)
  int U = 0;
  for (int p = 0; p < B * K; ++p) {
    const int id = cpu_ids[p];
    if (id < 0 || id >= E) continue;
    int u = 0;
    while (u < U && hs.uexp[u] < id) ++u;
    if (u < U && hs.uexp[u] == id) {
      if (hs.ucnt[u] < kMaxTokens) hs.uent[u][hs.ucnt[u]++] = p;
      continue;
    }
    for (int v = U; v > u; --v) {
      hs.uexp[v] = hs.uexp[v - 1];
      hs.ucnt[v] = hs.ucnt[v - 1];
      std::memcpy(hs.uent[v], hs.uent[v - 1], sizeof(hs.uent[v]));
    }
    hs.uexp[u] = id;
    hs.ucnt[u] = 1;
    hs.uent[u][0] = p;
    ++U;
  }
  if (U == 0) return;
  const int isa = e->host_isa;
  // the token rows as the slice kernel reads them
  const uint16_t* xin = x;
  if (isa == EFF_HOST_ISA_AVX512_BF16) {
    if (hs.xp.size() < (size_t)B * H) hs.xp.resize((size_t)B * H);
    for (int t = 0; t < B; ++t)
      for (int i = 0; i < H; ++i) hs.xp[(size_t)t * H + pair_pos(i)] = x[(size_t)t * H + i];
    xin = hs.xp.data();
  }
  // SwiGLU activations (hi and lo bf16 rows) per (expert, token)
  int off[kMaxEntries + 1];
  off[0] = 0;
  for (int u = 0; u < U; ++u) off[u + 1] = off[u] + hs.ucnt[u];
  const size_t need = (size_t)off[U] * I * 2;
  if (hs.a.size() < need) hs.a.resize(need);
  for (int u = 0; u < U; ++u) hs.done[u].v.store(0, std::memory_order_relaxed);
  const int64_t pay = (int64_t)H * I / 2, sca = (int64_t)H * I / 16;
  const int SI = I / 16, SH = H / 16;
  const int NG = U * SI, ND = U * SH;
  const int C = e->pool_threads->size();
  auto gate_up = [&](int u, int sl) {  // 16 rows of a
    const int nt = hs.ucnt[u];
    const int64_t flat = (int64_t)layer * E + hs.uexp[u];
    const uint8_t* rec = e->pool + flat * e->R;
    const uint16_t* xr[kMaxTokens];
    for (int j = 0; j < nt; ++j) xr[j] = xin + (size_t)(hs.uent[u][j] / K) * H;
    float g[16 * kMaxTokens], v[16 * kMaxTokens];
    const MatRef m[2] = {{rec, rec + 3 * pay, e->h_ts[flat * 3 + 0], g},
                         {rec + pay, rec + 3 * pay + sca, e->h_ts[flat * 3 + 1], v}};
    run_slices(isa, c.wformat, 2, m, H / 32, sl, xr, nt, nt);
    uint16_t* ahi = hs.a.data() + (size_t)off[u] * I * 2;
    for (int r = 0; r < 16; ++r) {
      const int col = isa == EFF_HOST_ISA_AVX512_BF16 ? pair_pos(sl * 16 + r) : sl * 16 + r;
      for (int j = 0; j < nt; ++j) {
        const float gg = g[r * nt + j], uu = v[r * nt + j];
        const float a = gg / (1.f + std::exp(-gg)) * uu;
        const uint16_t hi = f2bf_trunc(a);
        ahi[(size_t)j * I + col] = hi;                                   // row j
        ahi[(size_t)(nt + j) * I + col] = f2bf_rne(a - bf16f(hi));      // row nt + j
      }
    }
  };
  auto down = [&](int u, int sl) {  // 16 rows of y
    const int nt = hs.ucnt[u];
    const int64_t flat = (int64_t)layer * E + hs.uexp[u];
    const uint8_t* rec = e->pool + flat * e->R;
    const uint16_t* ar[2 * kMaxTokens];
    const uint16_t* abase = hs.a.data() + (size_t)off[u] * I * 2;
    for (int i = 0; i < 2 * nt; ++i) ar[i] = abase + (size_t)i * I;
    float out[16 * kMaxTokens];
    const MatRef m = {rec + 2 * pay, rec + 3 * pay + 2 * sca, e->h_ts[flat * 3 + 2], out};
    run_slices(isa, c.wformat, 1, &m, I / 32, sl, ar, 2 * nt, nt);
    for (int r = 0; r < 16; ++r)
      for (int j = 0; j < nt; ++j) y[(int64_t)hs.uent[u][j] * H + sl * 16 + r] = out[r * nt + j];
  };
  e->pool_threads->parallel_for(2 * C, [&](int task) {
    if (task < C) {  // gate/up slices [b, f) in (expert, slice) order
      const int b = (int)((int64_t)NG * task / C), f = (int)((int64_t)NG * (task + 1) / C);
      int run = 0;
      for (int i = b; i < f; ++i) {
        gate_up(i / SI, i % SI);
        ++run;
        if (i + 1 == f || (i + 1) % SI == 0) {  // end of this expert's share of the range
          hs.done[i / SI].v.fetch_add(run, std::memory_order_release);
          run = 0;
        }
      }
      return;
    }
    const int b = (int)((int64_t)ND * (task - C) / C), f = (int)((int64_t)ND * (task - C + 1) / C);
    int ready = -1;
    for (int i = b; i < f; ++i) {
      const int u = i / SH;
      if (u != ready) {
        while (hs.done[u].v.load(std::memory_order_acquire) < SI) _mm_pause();
        ready = u;
      }
      down(u, i % SH);
    }
  });
}

// ------------------------------------------------------------------------------- topology
namespace {
int read_int(const char* path, int fallback) {
  FILE* f = std::fopen(path, "r");
  if (!f) return fallback;
  int v = fallback;
  if (std::fscanf(f, "%d", &v) != 1) v = fallback;
  std::fclose(f);
  return v;
}

// CPUs the cgroup's quota allows (cgroup v2 cpu.max, else v1 cfs quota / period); 0 = no limit
int cgroup_cpu_limit() {
  if (FILE* f = std::fopen("/sys/fs/cgroup/cpu.max", "r")) {
    char q[32] = {0};
    long long period = 0;
    const int n = std::fscanf(f, "%31s %lld", q, &period);
    std::fclose(f);
    if (n == 2 && std::strcmp(q, "max") != 0 && period > 0) {
      const long long quota = std::atoll(q);
      if (quota > 0) return (int)std::max(1LL, (quota + period - 1) / period);
    }
    return 0;
  }
  const int quota = read_int("/sys/fs/cgroup/cpu/cpu.cfs_quota_us", -1);
  const int period = read_int("/sys/fs/cgroup/cpu/cpu.cfs_period_us", -1);
  if (quota > 0 && period > 0) return std::max(1, (quota + period - 1) / period);
  return 0;
}
}  // namespace

std::vector<int> physical_core_cpus() {
  std::vector<int> out;
  cpu_set_t set;
  CPU_ZERO(&set);
  if (sched_getaffinity(0, sizeof(set), &set) != 0) return out;
  std::set<std::pair<int, int>> seen;  // (package, core)
  for (int cpu = 0; cpu < CPU_SETSIZE; ++cpu) {
    if (!CPU_ISSET(cpu, &set)) continue;
    char path[128];
    std::snprintf(path, sizeof(path), "/sys/devices/system/cpu/cpu%d/topology/core_id", cpu);
    const int core = read_int(path, -1 - cpu);  // unknown topology: every CPU its own core
    std::snprintf(path, sizeof(path), "/sys/devices/system/cpu/cpu%d/topology/physical_package_id", cpu);
    const int pkg = read_int(path, 0);
    if (seen.insert({pkg, core}).second) out.push_back(cpu);
  }
  const int lim = cgroup_cpu_limit();
  if (lim > 0 && (int)out.size() > lim) out.resize(lim);
  return out;
}

bool pin_this_thread(int cpu) {
  if (cpu < 0 || cpu >= CPU_SETSIZE) return false;
  cpu_set_t set;
  CPU_ZERO(&set);
  CPU_SET(cpu, &set);
  return pthread_setaffinity_np(pthread_self(), sizeof(set), &set) == 0;
}

// ----------------------------------------------------------------------------------- pool
ThreadPool::ThreadPool(int n, const std::vector<int>* pin) {
  for (int i = 0; i < n - 1; ++i) {
    const int cpu = (pin && i + 1 < (int)pin->size()) ? (*pin)[i + 1] : -1;
    workers_.emplace_back([this, cpu] {
      if (cpu >= 0 && pin_this_thread(cpu)) pinned_.fetch_add(1);
      loop();
    });
  }
}

ThreadPool::~ThreadPool() {
  {
    std::lock_guard<std::mutex> g(mu_);
    stop_.store(true);
  }
  cv_.notify_all();
  for (auto& t : workers_) t.join();
}

void ThreadPool::run_tasks(uint64_t g, const std::function<void(int)>* fn, int n) {
  const uint64_t tag = (g & 0xFFFFFFFFull) << 32;
  for (;;) {
    uint64_t v = next_.load(std::memory_order_acquire);
    if ((v & ~0xFFFFFFFFull) != tag || (int64_t)(v & 0xFFFFFFFFull) >= n) return;
    if (!next_.compare_exchange_weak(v, v + 1, std::memory_order_acq_rel)) continue;
    (*fn)((int)(v & 0xFFFFFFFFull));
    done_.fetch_add(1, std::memory_order_release);
  }
}

void ThreadPool::loop() {
  uint64_t seen = gen_.load(std::memory_order_acquire);
  while (!stop_.load(std::memory_order_relaxed)) {
    uint64_t g = seen;
    const auto t0 = std::chrono::steady_clock::now();
    for (int it = 0;; ++it) {
      g = gen_.load(std::memory_order_acquire);
      if (g != seen || stop_.load(std::memory_order_relaxed)) break;
      _mm_pause();
      if ((it & 1023) == 1023 && std::chrono::steady_clock::now() - t0 > std::chrono::milliseconds(2)) break;
    }
    if (g == seen) {  // idle: sleep until a new job or shutdown
      std::unique_lock<std::mutex> lk(mu_);
      sleepers_.fetch_add(1);
      cv_.wait(lk, [&] { return stop_.load() || gen_.load() != seen; });
      sleepers_.fetch_sub(1);
      continue;
    }
    seen = g;
    run_tasks(g, fn_.load(std::memory_order_acquire), n_.load(std::memory_order_acquire));
  }
}

void ThreadPool::parallel_for(int n, const std::function<void(int)>& fn) {
  if (n <= 0) return;
  const uint64_t g = gen_.load(std::memory_order_relaxed) + 1;
  fn_.store(&fn, std::memory_order_relaxed);
  n_.store(n, std::memory_order_relaxed);
  done_.store(0, std::memory_order_relaxed);
  next_.store((g & 0xFFFFFFFFull) << 32, std::memory_order_relaxed);
  gen_.store(g, std::memory_order_release);
  if (sleepers_.load() > 0) {
    std::lock_guard<std::mutex> lk(mu_);
    cv_.notify_all();
  }
  run_tasks(g, &fn, n);
  while (done_.load(std::memory_order_acquire) < n) _mm_pause();
}

}  // namespace eff
