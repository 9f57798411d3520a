// Log-sum-exp merge of split partials, with an optional learned sink that
// joins only the denominator.
// ("Don't read the haystack", section "Part one: hitting the wall on
// purpose"; "Attention: Undivided & Uncompressed", section "Traffic";
// "Training-free sparse attention for long-context LLM decode", section
// "Strongest signals", item 1.)
//
// One wavefront per (request, query head): lanes stride over the splits for
// the max and the normaliser (wave reductions); each lane computes the weight
// of one split, and the weighted sum of accumulators runs over the head
// dimension with the weights broadcast by shuffles, splits in order.
#include "ps_device.h"
#include "ps_launch.h"

namespace ps {

constexpr int kCombineWaves = 4;

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) v = fmax_(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) v += __shfl_xor(v, off);
  return v;
}

__global__ __launch_bounds__(kCombineWaves * kWave) void combine_kernel(
    const float* __restrict__ part_acc, const float* __restrict__ part_ml, int n_splits, int d_,
    int hq, int64_t rows, const float* __restrict__ sink, float* __restrict__ out,
    float* __restrict__ lse) {
  const int64_t row = (int64_t)blockIdx.x * kCombineWaves + threadIdx.x / kWave;  // b * hq + h
  const int lane = threadIdx.x % kWave;
  if (row >= rows) return;  // uniform per wavefront
  const int h = (int)(row % hq);
  const float* ml = part_ml + row * n_splits * 2;
  const float* acc = part_acc + row * n_splits * d_;
  const float sig = sink ? sink[h] : -INFINITY;

  float mx = -INFINITY;
  for (int s = lane; s < n_splits; s += kWave) mx = fmax_(mx, ml[2 * s]);
  mx = fmax_(wave_max(mx), sig);
  float* o = out + row * d_;
  if (mx == -INFINITY) {
    for (int d = lane; d < d_; d += kWave) o[d] = 0.0f;
    if (lse && lane == 0) lse[row] = -INFINITY;
    return;
  }
  // Normaliser: lanes stride over the splits, then a wave sum.
  float l = 0.0f;
  for (int s = lane; s < n_splits; s += kWave) {
    const float ms = ml[2 * s];
    if (ms != -INFINITY) l = __builtin_fmaf(expf(ms - mx), ml[2 * s + 1], l);
  }
  l = wave_sum(l);
  if (sig != -INFINITY) l += expf(sig - mx);
  const float inv = 1.0f / l;

  // Weighted sum of accumulators, splits in order; a chunk of up to 64 split
  // weights is held one per lane and broadcast with shuffles, and the
  // accumulator rows of 8 splits are loaded before they are used.
  constexpr int kDPerLane = 2;  // head_dim <= 128
  constexpr int kBatch = 8;
  float a[kDPerLane] = {0.0f, 0.0f};
  for (int s0 = 0; s0 < n_splits; s0 += kWave) {
    const int sl = s0 + lane;
    float w = 0.0f;
    if (sl < n_splits) {
      const float ms = ml[2 * sl];
      w = ms == -INFINITY ? 0.0f : expf(ms - mx);
    }
    const int cnt = min(kWave, n_splits - s0);
    for (int j0 = 0; j0 < cnt; j0 += kBatch) {
      float v[kBatch][kDPerLane];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const float* src = acc + (int64_t)(s0 + j0 + j) * d_;
#pragma unroll
        for (int k = 0; k < kDPerLane; ++k) {
          const int d = lane + k * kWave;
          v[j][k] = (j0 + j < cnt && d < d_) ? src[d] : 0.0f;
        }
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const float wj = __shfl(w, (j0 + j) & (kWave - 1));
        if (j0 + j < cnt) {
#pragma unroll
          for (int k = 0; k < kDPerLane; ++k) a[k] = __builtin_fmaf(wj, v[j][k], a[k]);
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kDPerLane; ++k) {
    const int d = lane + k * kWave;
    if (d < d_) o[d] = a[k] * inv;
  }
  if (lse && lane == 0) lse[row] = mx + logf(l);
}

hipError_t launch_combine(const Shape& s, const float* part_acc, const float* part_ml,
                          int n_splits, const float* sink, float* out, float* lse,
                          hipStream_t st) {
  const int64_t rows = (int64_t)s.batch * s.hq;
  const int64_t blocks = (rows + kCombineWaves - 1) / kCombineWaves;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(kCombineWaves * kWave), 0, st,
                     part_acc, part_ml, n_splits, s.head_dim, s.hq, rows, sink, out, lse);
  return hipGetLastError();
}

}  // namespace ps
