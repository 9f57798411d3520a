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

// A 16-byte load marked non-temporal (data read once).
__device__ __forceinline__ uint4 ld16nt(const void* p) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
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

// Whole-wavefront reductions and scans on DPP lane moves (a few cycles each,
// against an LDS round trip per step for __shfl). Results are uniform.
enum : int {
  kDppRowShr1 = 0x111,
  kDppRowShr2 = 0x112,
  kDppRowShr4 = 0x114,
  kDppRowShr8 = 0x118,
  kDppRowBcast15 = 0x142,  // lane 15 of each row to the next row
  kDppRowBcast31 = 0x143,  // lane 31 to the rows above it
};

template <int CTRL>
__device__ __forceinline__ uint32_t dppu(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dppu<kDppXor1>(v));
  v = min(v, dppu<kDppXor2>(v));
  v = min(v, dppu<kDppHalfMirror>(v));
  v = min(v, dppu<kDppMirror>(v));  // every lane of a row holds the row's min
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return min(min(a, b), min(c, d));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dppu<kDppXor1>(v));
  v = max(v, dppu<kDppXor2>(v));
  v = max(v, dppu<kDppHalfMirror>(v));
  v = max(v, dppu<kDppMirror>(v));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(a, b), max(c, d));
}

// Sum over the 64 lanes (uniform result).
__device__ __forceinline__ int wave_sum_i32(int v) {
  v += (int)dppu<kDppXor1>((uint32_t)v);
  v += (int)dppu<kDppXor2>((uint32_t)v);
  v += (int)dppu<kDppHalfMirror>((uint32_t)v);
  v += (int)dppu<kDppMirror>((uint32_t)v);  // every lane of a row holds the row's sum
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
         __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

// Inclusive prefix sum over the 64 lanes in lane order: shifts of 1, 2, 4
// and 8 within each 16-lane row (lanes shifted in from outside the row add
// 0), then each row adds the total of the rows below it.
__device__ __forceinline__ int wave_prefix_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr2, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr4, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr8, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast15, 0xA, 0xF, false);  // rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast31, 0xC, 0xF, false);  // rows 2, 3
  return v;
}

__device__ __forceinline__ float fmax_(float a, float b) { return a > b ? a : b; }
__device__ __forceinline__ float fmin_(float a, float b) { return a < b ? a : b; }

// 2^x via the hardware transcendental; exact 0 for -inf.
__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// bf16 bits of a finite float, rounded to nearest even.
__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) { return __uint_as_float(b << 16); }

// Exact three-term bf16 split of a finite fp32 value: x == hi + mid + lo with
// every term a bf16 (each residual is exact in fp32 and has at most 16, then
// 8, significant bits), barring underflow below 2^-100.
__device__ __forceinline__ void bf16_split3(float x, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = bf16_rne_bits(x);
  const float r1 = x - bf16_bits_to_float(hi);
  mid = bf16_rne_bits(r1);
  const float r2 = r1 - bf16_bits_to_float(mid);
  lo = bf16_rne_bits(r2);
}

// Matrix-core fragments of v_mfma_f32_16x16x32_bf16: A and B are 8 bf16 per
// lane (A: row = lane % 16; B: column = lane % 16; the same 8 contraction
// indices for a given lane / 16), C and D 4 floats per lane
// (row = 4 * (lane / 16) + i, column = lane % 16).
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

__device__ __forceinline__ f32x4_t mfma_bf16_16x16x32(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// v_mfma_f32_16x16x16_bf16: A and B are 4 bf16 per lane (A: row = lane % 16,
// B: column = lane % 16; contraction indices 4 * (lane / 16) + i), C and D as
// for the 16x16x32 form.
typedef __attribute__((ext_vector_type(4))) short i16x4_t;

__device__ __forceinline__ f32x4_t mfma_bf16_16x16x16(const uint2& a, const uint2& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                   __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane 4a+e receives
// element e of the 4-element (8-byte) chunks addressed by lanes a, a+4, a+8
// and a+12 of its group, in that order. With lane L of group k addressing
// row 4k + L/4, columns c0 + 4(L%4) .. +3 of a row-major bf16 tile, lane
// 16k + j receives rows 4k..4k+3 of column c0 + j: the B operand of
// v_mfma_f32_16x16x16_bf16 with k = row and column = c0 + j.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

}  // namespace ps
