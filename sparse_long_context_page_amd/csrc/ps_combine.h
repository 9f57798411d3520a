// Log-sum-exp merge of one (request, query head)'s split partials by one
// wavefront, shared by the merge kernel and the decode that merges its own
// splits. ("Attention: Undivided & Uncompressed", section "Traffic": partial
// softmaxes merge by rescaling with exp of the difference of their maxima;
// "Training-free sparse attention for long-context LLM decode", section
// "Strongest signals", item 1: a learned sink joins only the denominator.)
#pragma once

#include "ps_device.h"

namespace ps {

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) v = fmax_(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) v += __shfl_xor(v, off);
  return v;
}

// A partial's value; COHERENT: an agent-scope load, which reads past any
// chiplet cache (partials written by workgroups of the same launch).
template <bool COHERENT>
__device__ __forceinline__ float load_partial(const float* p) {
  if constexpr (COHERENT)
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    return *p;
}

// Lanes stride over the splits for the max and the normaliser (wave
// reductions); each lane computes the weight of one split, and the weighted
// sum of accumulators runs over the head dimension with the weights
// broadcast by shuffles, splits in order. ml = [n_splits, 2] (max in natural
// log units, normaliser), acc = [n_splits, d_], sig = the sink logit or -inf.
// COHERENT selects the loads only; the arithmetic is the same.
template <bool COHERENT = false>
__device__ __forceinline__ void combine_row(const float* __restrict__ acc,
                                            const float* __restrict__ ml, int n_splits, int d_,
                                            float sig, float* __restrict__ o, float* lse_out) {
  auto ld = [](const float* p) { return load_partial<COHERENT>(p); };
  const int lane = threadIdx.x % kWave;
  constexpr int kDPerLane = 2;  // head_dim <= 128
  constexpr int kBatch = 8;
  if (n_splits <= kBatch) {
    // Few splits (the merge inside the decode launch): every partial is
    // requested at once, one round trip instead of one per stage below; the
    // arithmetic is the general path's, operation for operation.
    float ms = -INFINITY, ls = 0.0f;
    if (lane < n_splits) {
      ms = ld(ml + 2 * lane);
      ls = ld(ml + 2 * lane + 1);
    }
    float v[kBatch][kDPerLane];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
#pragma unroll
      for (int k = 0; k < kDPerLane; ++k) {
        const int d = lane + k * kWave;
        v[j][k] = (j < n_splits && d < d_) ? ld(acc + (int64_t)j * d_ + d) : 0.0f;
      }
    }
    float mx = fmax_(wave_max_f32(ms), sig);
    if (mx == -INFINITY) {
      for (int d = lane; d < d_; d += kWave) o[d] = 0.0f;
      if (lse_out && lane == 0) *lse_out = -INFINITY;
      return;
    }
    float l = (lane < n_splits && ms != -INFINITY) ? __builtin_fmaf(expf(ms - mx), ls, 0.0f)
                                                   : 0.0f;
    l = wave_sum_f32(l);
    if (sig != -INFINITY) l += expf(sig - mx);
    const float inv = 1.0f / l;
    const float w = (lane < n_splits && ms != -INFINITY) ? expf(ms - mx) : 0.0f;
    float a[kDPerLane] = {0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const float wj = __shfl(w, j);
      if (j < n_splits) {
#pragma unroll
        for (int k = 0; k < kDPerLane; ++k) a[k] = __builtin_fmaf(wj, v[j][k], a[k]);
      }
    }
#pragma unroll
    for (int k = 0; k < kDPerLane; ++k) {
      const int d = lane + k * kWave;
      if (d < d_) o[d] = a[k] * inv;
    }
    if (lse_out && lane == 0) *lse_out = mx + logf(l);
    return;
  }
  float mx = -INFINITY;
  for (int s = lane; s < n_splits; s += kWave) mx = fmax_(mx, ld(ml + 2 * s));
  mx = fmax_(wave_max_f32(mx), sig);
  if (mx == -INFINITY) {
    for (int d = lane; d < d_; d += kWave) o[d] = 0.0f;
    if (lse_out && lane == 0) *lse_out = -INFINITY;
    return;
  }
  float l = 0.0f;
  for (int s = lane; s < n_splits; s += kWave) {
    const float ms = ld(ml + 2 * s);
    if (ms != -INFINITY) l = __builtin_fmaf(expf(ms - mx), ld(ml + 2 * s + 1), l);
  }
  l = wave_sum_f32(l);
  if (sig != -INFINITY) l += expf(sig - mx);
  const float inv = 1.0f / l;

  // a chunk of up to 64 split weights is held one per lane and broadcast with
  // shuffles; the accumulator rows of 8 splits are loaded before they are used
  float a[kDPerLane] = {0.0f, 0.0f};
  for (int s0 = 0; s0 < n_splits; s0 += kWave) {
    const int sl = s0 + lane;
    float w = 0.0f;
    if (sl < n_splits) {
      const float ms = ld(ml + 2 * sl);
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
          v[j][k] = (j0 + j < cnt && d < d_) ? ld(src + d) : 0.0f;
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
  if (lse_out && lane == 0) *lse_out = mx + logf(l);
}

}  // namespace ps
