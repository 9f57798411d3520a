// Elementwise max and min of a page's valid key rows by one wavefront, shared
// by the metadata kernel and the page score that refreshes the last page.
// ("Don't read the haystack", section "Part two: the skipping": a page is
// summarised by the elementwise min and max of its keys.)
#pragma once

#include "ps_device.h"

namespace ps {

// The page's 16 rows are read with coalesced 16-byte loads, lane = (row
// group r0, column vector c); every row is read (all are inside the page) and
// rows at or past cnt do not count. Max/min are folded over the lane's rows in
// order, then across row groups with xor shuffles; afterwards every lane of
// column vector c holds the max and min of columns c*V .. c*V+V-1. Min and
// max select stored values, so the result is exact in either dtype.
template <typename T, int D>
struct PageFold {
  using L = RowLayout<T, D>;
  static constexpr int V = L::kVec;
  static constexpr int NT = L::kLoadsPerPage;
  uint4 rows[NT];

  __device__ __forceinline__ void load(const T* __restrict__ page, int lane) {
    const int r0 = lane / L::kLanesPerRow;
    const int c = lane % L::kLanesPerRow;
#pragma unroll
    for (int i = 0; i < NT; ++i) rows[i] = ld16(page + (r0 + i * L::kRowsPerLoad) * D + c * V);
  }

  __device__ __forceinline__ void fold(int cnt, int lane, float (&mx)[V], float (&mn)[V]) const {
    const int r0 = lane / L::kLanesPerRow;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      mx[j] = -INFINITY;
      mn[j] = INFINITY;
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const bool valid = r0 + i * L::kRowsPerLoad < cnt;
      float f[V];
      unpack(rows[i], f);
#pragma unroll
      for (int j = 0; j < V; ++j) {
        mx[j] = fmax_(mx[j], valid ? f[j] : -INFINITY);
        mn[j] = fmin_(mn[j], valid ? f[j] : INFINITY);
      }
    }
#pragma unroll
    for (int off = L::kLanesPerRow; off < kWave; off <<= 1) {
#pragma unroll
      for (int j = 0; j < V; ++j) {
        mx[j] = fmax_(mx[j], __shfl_xor(mx[j], off));
        mn[j] = fmin_(mn[j], __shfl_xor(mn[j], off));
      }
    }
  }
};

// 8-bit metadata. ("Faster Than Flash: Exploiting Attention Sparsity for
// Efficient Long-Context Decoding", section "Methodology", item 1: the scan
// that picks the blocks to read runs on a low-bit copy; here that copy is
// the page metadata, rounded so the page bound stays an upper bound.)
// Format: OCP E4M3 without infinities (sign, 4 exponent bits with bias 7, 3
// mantissa bits; exponent 0 = subnormals m * 2^-9; largest finite 448). kmax
// is rounded up and kmin down; a zero result is code 0x00; magnitudes past
// 448 saturate to 448.
//
// Code of a finite x rounded toward +inf (up) or -inf (!up). The magnitude
// is truncated from the fp32 bits (exponent rebiased, top 3 mantissa bits, or
// x * 2^9 for the subnormal range, an exact scaling); when bits were dropped
// and the rounding direction points away from zero the magnitude code is
// incremented, which is the next larger magnitude because codes order like
// magnitudes (a mantissa carry moves into the exponent).
__device__ __forceinline__ uint32_t fp8_e4m3_directed(float x, bool up) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = u >> 31;
  const float a = __uint_as_float(u & 0x7fffffffu);
  uint32_t mag;
  bool inexact;
  if (a >= 0.015625f) {  // 2^-6: normal E4M3 range
    const int e = (int)((u >> 23) & 0xffu) - 127 + 7;
    mag = e > 15 ? 0x7fu : ((uint32_t)e << 3) | ((u >> 20) & 7u);
    inexact = e > 15 || (u & 0xfffffu) != 0u;
  } else {
    const float t = a * 512.0f;  // exact: a power-of-two scaling
    mag = (uint32_t)t;           // 0..7, truncated
    inexact = (float)mag != t;
  }
  const bool away = (sign == 0u) == up;
  mag += (away && inexact) ? 1u : 0u;
  mag = mag >= 0x7fu ? 0x7eu : mag;  // 0x7f is NaN: saturate at 448
  return mag == 0u ? 0u : (sign << 7) | mag;
}

// Eight codes (kmax rounded up when up, else kmin rounded down), two words.
__device__ __forceinline__ uint2 fp8_pack8(const float (&f)[8], bool up) {
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) w[j / 4] |= fp8_e4m3_directed(f[j], up) << (8 * (j % 4));
  return make_uint2(w[0], w[1]);
}

// Four codes, one word (code j in byte j).
__device__ __forceinline__ uint32_t fp8_pack4(const float (&f)[4], bool up) {
  uint32_t w = 0u;
#pragma unroll
  for (int j = 0; j < 4; ++j) w |= fp8_e4m3_directed(f[j], up) << (8 * j);
  return w;
}

// Four codes (one word, code j in byte j) widened exactly to fp32.
__device__ __forceinline__ void fp8x4_to_f32x4(uint32_t w, float (&f)[4]) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);  // codes 0, 1
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);   // codes 2, 3
  f[0] = lo[0];
  f[1] = lo[1];
  f[2] = hi[0];
  f[3] = hi[1];
}

// Four E4M3 codes (one word, code j in byte j) widened to four bf16 (two
// words, value j in half j): every E4M3 value is a bf16 value, so the
// hardware conversion to fp32 followed by keeping the high halves is exact.
__device__ __forceinline__ uint2 fp8x4_to_bf16x4(uint32_t w) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);  // codes 0, 1
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);   // codes 2, 3
  // v_perm: bytes 2,3 of the first value then bytes 2,3 of the second
  const uint32_t b01 = __builtin_amdgcn_perm(__float_as_uint(lo[1]), __float_as_uint(lo[0]),
                                             0x07060302u);
  const uint32_t b23 = __builtin_amdgcn_perm(__float_as_uint(hi[1]), __float_as_uint(hi[0]),
                                             0x07060302u);
  return make_uint2(b01, b23);
}

// Eight codes (two words) widened to eight bf16 (one 16-byte vector).
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  const uint2 a = fp8x4_to_bf16x4(w0), b = fp8x4_to_bf16x4(w1);
  return make_uint4(a.x, a.y, b.x, b.y);
}

}  // namespace ps
