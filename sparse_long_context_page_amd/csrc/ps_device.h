// Device-side helpers shared by the pagesparse kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ps {

constexpr int kPage = 16;   // tokens per page
constexpr int kWave = 64;   // CDNA wavefront width

// Storage element of the K/V pools and metadata: bf16 is carried as its raw
// 16-bit pattern, fp32 as float.
using bf16_t = uint16_t;

template <typename T>
struct Elem;
template <>
struct Elem<bf16_t> {
  static constexpr int kBytes = 2;
  static constexpr int kPerVec = 8;  // elements per 16-byte vector
};
template <>
struct Elem<float> {
  static constexpr int kBytes = 4;
  static constexpr int kPerVec = 4;
};

// Lane geometry of a row of D elements read with one 16-byte vector per lane.
template <typename T, int D>
struct RowLayout {
  static constexpr int kVec = Elem<T>::kPerVec;           // values per lane-vector
  static constexpr int kLanesPerRow = D / kVec;           // lanes covering one row
  static constexpr int kRowsPerLoad = kWave / kLanesPerRow;  // rows one wave-load covers
  static constexpr int kLoadsPerPage = kPage / kRowsPerLoad; // wave-loads per 16-row page
  static_assert(kLanesPerRow >= 8 && kLanesPerRow <= 32, "row layout");
  static_assert(kPage % kRowsPerLoad == 0, "row layout");
};

__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ void st16(void* p, const uint4& v) {
  *reinterpret_cast<uint4*>(p) = v;
}

// Widen one 16-byte vector to floats (bf16 -> fp32 is exact).
__device__ __forceinline__ void unpack(const uint4& v, float (&f)[8]) {
  f[0] = __uint_as_float(v.x << 16);
  f[1] = __uint_as_float(v.x & 0xffff0000u);
  f[2] = __uint_as_float(v.y << 16);
  f[3] = __uint_as_float(v.y & 0xffff0000u);
  f[4] = __uint_as_float(v.z << 16);
  f[5] = __uint_as_float(v.z & 0xffff0000u);
  f[6] = __uint_as_float(v.w << 16);
  f[7] = __uint_as_float(v.w & 0xffff0000u);
}

__device__ __forceinline__ void unpack(const uint4& v, float (&f)[4]) {
  f[0] = __uint_as_float(v.x);
  f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z);
  f[3] = __uint_as_float(v.w);
}

// Narrow floats that hold exact bf16 values back to a 16-byte vector.
__device__ __forceinline__ uint4 pack(const float (&f)[8]) {
  uint4 v;
  v.x = (__float_as_uint(f[0]) >> 16) | (__float_as_uint(f[1]) & 0xffff0000u);
  v.y = (__float_as_uint(f[2]) >> 16) | (__float_as_uint(f[3]) & 0xffff0000u);
  v.z = (__float_as_uint(f[4]) >> 16) | (__float_as_uint(f[5]) & 0xffff0000u);
  v.w = (__float_as_uint(f[6]) >> 16) | (__float_as_uint(f[7]) & 0xffff0000u);
  return v;
}

__device__ __forceinline__ uint4 pack(const float (&f)[4]) {
  uint4 v;
  v.x = __float_as_uint(f[0]);
  v.y = __float_as_uint(f[1]);
  v.z = __float_as_uint(f[2]);
  v.w = __float_as_uint(f[3]);
  return v;
}

// DPP lane permutations inside a 16-lane row.
enum : int {
  kDppXor1 = 0xB1,        // quad_perm [1,0,3,2]
  kDppXor2 = 0x4E,        // quad_perm [2,3,0,1]
  kDppHalfMirror = 0x141, // lane i <-> 7-i within each 8-lane half-row
  kDppMirror = 0x140,     // lane i <-> 15-i within each 16-lane row
};

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over groups of N adjacent lanes (N in {8, 16, 32}); every lane of the
// group receives the same bits (each step adds two equal-order operands).
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 8 || N == 16 || N == 32, "group size");
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  if constexpr (N >= 16) v += dpp<kDppMirror>(v);
  if constexpr (N >= 32) v += __shfl_xor(v, 16);
  return v;
}

__device__ __forceinline__ float fmax_(float a, float b) { return a > b ? a : b; }
__device__ __forceinline__ float fmin_(float a, float b) { return a < b ? a : b; }

// 2^x via the hardware transcendental; exact 0 for -inf.
__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace ps
