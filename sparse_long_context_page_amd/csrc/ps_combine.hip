// Log-sum-exp merge of split partials, with an optional learned sink that
// joins only the denominator.
// ("Don't read the haystack", section "Part one: hitting the wall on
// purpose"; "Attention: Undivided & Uncompressed", section "Traffic";
// "Training-free sparse attention for long-context LLM decode", section
// "Strongest signals", item 1.)
//
// One wavefront per (request, query head) runs combine_row.
#include "ps_combine.h"
#include "ps_launch.h"

namespace ps {

constexpr int kCombineWaves = 4;

__global__ __launch_bounds__(kCombineWaves * kWave) void combine_kernel(
    const float* __restrict__ part_acc, const float* __restrict__ part_ml, int n_splits, int d_,
    int hq, int64_t rows, const float* __restrict__ sink, float* __restrict__ out,
    float* __restrict__ lse) {
  const int64_t row = (int64_t)blockIdx.x * kCombineWaves + threadIdx.x / kWave;  // b * hq + h
  if (row >= rows) return;  // uniform per wavefront
  const int h = (int)(row % hq);
  combine_row(part_acc + row * n_splits * d_, part_ml + row * n_splits * 2, n_splits, d_,
              sink ? sink[h] : -INFINITY, out + row * d_, lse ? lse + row : nullptr);
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
