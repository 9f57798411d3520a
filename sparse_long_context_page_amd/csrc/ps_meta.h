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

}  // namespace ps
