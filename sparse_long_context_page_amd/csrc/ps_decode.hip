// Split-KV decode over a page list (sparse) or over every page (dense):
// per split, the running max, normaliser and unnormalised accumulator of the
// softmax of scale*q.k for every query head of one KV head.
// ("Don't read the haystack", sections "Part one: hitting the wall on
// purpose" and "Part two: the skipping"; "Attention: Undivided &
// Uncompressed", section "Traffic", for the rescaling merge.)
//
// One workgroup of 4 wavefronts per (request, KV head, split). The split's
// pages are dealt round-robin to the wavefronts, two pages in flight per
// wavefront. A page's 16 K rows and 16 V rows are read with coalesced
// 16-byte loads, lane = (row group, column vector); the page table (and the
// page list) is read per page, so physical pages may be anywhere and in any
// order. Each lane keeps a private softmax state over its own tokens (all G
// heads), rescaling lazily only when a page raises its running max by more
// than 8 (log2 units), so the common path has no cross-lane max and no
// rescale; the true max is tracked alongside and restored as the state's
// reference at the end, so each written max is the split's. States are merged
// across row groups with shuffles and across wavefronts through LDS, then
// written as fp32 partials (max in natural-log units).
#include "ps_device.h"
#include "ps_launch.h"

namespace ps {

constexpr int kDecWaves = 4;
constexpr float kLazyRescale = 8.0f;  // log2 headroom before the running max is raised
constexpr float kLn2 = 0.69314718055994530942f;

template <typename T, int D, int G>
struct DecodeState {
  using L = RowLayout<T, D>;
  static constexpr int V = L::kVec;
  static constexpr int NT = L::kLoadsPerPage;  // tokens per lane per page
  // m: reference max of the state (at most kLazyRescale below the true max);
  // mt: true running max, restored as the reference before the state leaves.
  float m[G], mt[G], l[G], acc[G][V];
};

template <typename T, int D, int G>
__device__ __forceinline__ void load_page(const T* __restrict__ k_pool, const T* __restrict__ v_pool,
                                          int64_t base, int cnt, int r0,
                                          uint4 (&kv)[DecodeState<T, D, G>::NT],
                                          uint4 (&vv)[DecodeState<T, D, G>::NT]) {
  using L = RowLayout<T, D>;
#pragma unroll
  for (int i = 0; i < L::kLoadsPerPage; ++i) {
    const int t = r0 + i * L::kRowsPerLoad;
    if (t < cnt) {
      kv[i] = ld16(k_pool + base + (int64_t)t * D);
      vv[i] = ld16(v_pool + base + (int64_t)t * D);
    } else {
      kv[i] = make_uint4(0, 0, 0, 0);
      vv[i] = make_uint4(0, 0, 0, 0);
    }
  }
}

template <typename T, int D, int G>
__device__ __forceinline__ void attend_page(DecodeState<T, D, G>& st,
                                            const float (&qs)[G][DecodeState<T, D, G>::V],
                                            const uint4 (&kv)[DecodeState<T, D, G>::NT],
                                            const uint4 (&vv)[DecodeState<T, D, G>::NT], int cnt,
                                            int r0) {
  using L = RowLayout<T, D>;
  constexpr int V = L::kVec;
  constexpr int NT = L::kLoadsPerPage;
  float x[NT][G];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    float kf[V];
    unpack(kv[i], kf);
    const bool valid = r0 + i * L::kRowsPerLoad < cnt;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float d = 0.0f;
#pragma unroll
      for (int j = 0; j < V; ++j) d = __builtin_fmaf(qs[h][j], kf[j], d);
      d = group_sum<L::kLanesPerRow>(d);
      x[i][h] = valid ? d : -INFINITY;
    }
  }
  float vf[NT][V];
#pragma unroll
  for (int i = 0; i < NT; ++i) unpack(vv[i], vf[i]);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mp = x[0][h];
#pragma unroll
    for (int i = 1; i < NT; ++i) mp = fmax_(mp, x[i][h]);
    st.mt[h] = fmax_(st.mt[h], mp);
    if (mp > st.m[h] + kLazyRescale) {  // also taken when the state is empty (-inf)
      const float a = exp2_(st.m[h] - mp);
      st.l[h] *= a;
#pragma unroll
      for (int j = 0; j < V; ++j) st.acc[h][j] *= a;
      st.m[h] = mp;
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const float pr = x[i][h] == -INFINITY ? 0.0f : exp2_(x[i][h] - st.m[h]);
      st.l[h] += pr;
#pragma unroll
      for (int j = 0; j < V; ++j) st.acc[h][j] = __builtin_fmaf(pr, vf[i][j], st.acc[h][j]);
    }
  }
}

// Merge two softmax states (log2 units); an empty state has m = -inf, l = 0.
__device__ __forceinline__ void merge_weights(float m1, float m2, float& mo, float& a1,
                                              float& a2) {
  mo = fmax_(m1, m2);
  a1 = m1 == -INFINITY ? 0.0f : exp2_(m1 - mo);
  a2 = m2 == -INFINITY ? 0.0f : exp2_(m2 - mo);
}

template <typename T, int D, int G, bool SPARSE>
__global__ __launch_bounds__(kDecWaves * kWave) void decode_kernel(
    const float* __restrict__ q, const T* __restrict__ k_pool, const T* __restrict__ v_pool,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ sel_count, int budget, int hkv,
    int max_pages, int n_splits, float qscale, float* __restrict__ part_acc,
    float* __restrict__ part_ml) {
  using L = RowLayout<T, D>;
  using S = DecodeState<T, D, G>;
  constexpr int V = L::kVec;
  constexpr int LPR = L::kLanesPerRow;
  constexpr int NT = S::NT;
  __shared__ float sm_m[kDecWaves][G];
  __shared__ float sm_l[kDecWaves][G];
  __shared__ float sm_acc[kDecWaves][G][D];

  const int split = blockIdx.x % n_splits;
  const int unit = blockIdx.x / n_splits;  // b * hkv + g
  const int b = unit / hkv;
  const int g = unit % hkv;
  const int len = seq_lens[b];
  const int np = ceil_div(len, kPage);
  int lo, hi;
  if constexpr (SPARSE) {
    const int per = ceil_div(budget, n_splits);
    const int cnt = min(sel_count[unit], budget);
    lo = min(split * per, cnt);
    hi = min(split * per + per, cnt);
  } else {
    const int per = ceil_div(np, n_splits);
    lo = min(split * per, np);
    hi = min(split * per + per, np);
  }
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int r0 = lane / LPR;
  const int c = lane % LPR;

  float qs[G][V];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float* qh = q + ((int64_t)b * hkv * G + g * G + h) * D + c * V;
#pragma unroll
    for (int j = 0; j < V; j += 4) {
      const float4 v4 = *reinterpret_cast<const float4*>(qh + j);
      qs[h][j + 0] = v4.x * qscale;
      qs[h][j + 1] = v4.y * qscale;
      qs[h][j + 2] = v4.z * qscale;
      qs[h][j + 3] = v4.w * qscale;
    }
  }
  S st;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.m[h] = -INFINITY;
    st.mt[h] = -INFINITY;
    st.l[h] = 0.0f;
#pragma unroll
    for (int j = 0; j < V; ++j) st.acc[h][j] = 0.0f;
  }

  const int32_t* list = SPARSE ? sel + (int64_t)unit * budget : nullptr;
  const int32_t* row = page_table + (int64_t)b * max_pages;
  const int64_t head_off = (int64_t)g * kPage * D + c * V;
  for (int it = lo + wave; it < hi; it += 2 * kDecWaves) {
    const int pa = SPARSE ? list[it] : it;
    const bool has_b = it + kDecWaves < hi;
    const int pb = has_b ? (SPARSE ? list[it + kDecWaves] : it + kDecWaves) : pa;
    const int cnt_a = min(kPage, len - pa * kPage);
    const int cnt_b = has_b ? min(kPage, len - pb * kPage) : 0;
    const int64_t base_a = (int64_t)row[pa] * hkv * kPage * D + head_off;
    const int64_t base_b = (int64_t)row[pb] * hkv * kPage * D + head_off;
    uint4 ka[NT], va[NT], kb[NT], vb[NT];
    load_page<T, D, G>(k_pool, v_pool, base_a, cnt_a, r0, ka, va);
    load_page<T, D, G>(k_pool, v_pool, base_b, cnt_b, r0, kb, vb);
    attend_page<T, D, G>(st, qs, ka, va, cnt_a, r0);
    if (has_b) attend_page<T, D, G>(st, qs, kb, vb, cnt_b, r0);
  }

  // Re-reference each state to its true max, so the written max is exact.
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (st.mt[h] > st.m[h]) {
      const float a = exp2_(st.m[h] - st.mt[h]);
      st.l[h] *= a;
#pragma unroll
      for (int j = 0; j < V; ++j) st.acc[h][j] *= a;
      st.m[h] = st.mt[h];
    }
  }
  // Merge the row groups of this wavefront (lanes sharing a column vector).
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float m2 = __shfl_xor(st.m[h], off);
      const float l2 = __shfl_xor(st.l[h], off);
      float mo, a1, a2;
      merge_weights(st.m[h], m2, mo, a1, a2);
      st.l[h] = st.l[h] * a1 + l2 * a2;
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const float o2 = __shfl_xor(st.acc[h][j], off);
        st.acc[h][j] = st.acc[h][j] * a1 + o2 * a2;
      }
      st.m[h] = mo;
    }
  }
  if (r0 == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int j = 0; j < V; ++j) sm_acc[wave][h][c * V + j] = st.acc[h][j];
      if (c == 0) {
        sm_m[wave][h] = st.m[h];
        sm_l[wave][h] = st.l[h];
      }
    }
  }
  __syncthreads();

  // Merge the wavefronts and write this split's partials.
  const int hq = hkv * G;
  for (int idx = threadIdx.x; idx < G * D; idx += kDecWaves * kWave) {
    const int h = idx / D;
    const int d = idx % D;
    float mo = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) mo = fmax_(mo, sm_m[w][h]);
    float a = 0.0f, lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float mw = sm_m[w][h];
      const float wt = mw == -INFINITY ? 0.0f : exp2_(mw - mo);
      a = __builtin_fmaf(wt, sm_acc[w][h][d], a);
      lsum = __builtin_fmaf(wt, sm_l[w][h], lsum);
    }
    const int64_t ph = ((int64_t)b * hq + g * G + h) * n_splits + split;
    part_acc[ph * D + d] = a;
    if (d == 0) {
      part_ml[ph * 2 + 0] = mo == -INFINITY ? -INFINITY : mo * kLn2;
      part_ml[ph * 2 + 1] = lsum;
    }
  }
}

hipError_t launch_decode(const Shape& s, bool sparse, const float* q, const void* k_pool,
                         const void* v_pool, const int32_t* page_table, const int32_t* seq_lens,
                         const int32_t* sel, const int32_t* sel_count, int budget, float scale,
                         int n_splits, float* part_acc, float* part_ml, hipStream_t st) {
  const int64_t blocks = (int64_t)s.batch * s.hkv * n_splits;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks), block(kDecWaves * kWave);
  const float qscale = scale * 1.44269504088896340736f;  // log2(e)
  PS_WITH_KV(s.kv_bf16, s.head_dim, {
    PS_WITH_GROUP(s.group, {
      if (sparse) {
        hipLaunchKernelGGL((decode_kernel<TElem, kD, kG, true>), grid, block, 0, st, q,
                           static_cast<const TElem*>(k_pool), static_cast<const TElem*>(v_pool),
                           page_table, seq_lens, sel, sel_count, budget, s.hkv, s.max_pages,
                           n_splits, qscale, part_acc, part_ml);
      } else {
        hipLaunchKernelGGL((decode_kernel<TElem, kD, kG, false>), grid, block, 0, st, q,
                           static_cast<const TElem*>(k_pool), static_cast<const TElem*>(v_pool),
                           page_table, seq_lens, nullptr, nullptr, 0, s.hkv, s.max_pages,
                           n_splits, qscale, part_acc, part_ml);
      }
    });
  });
  return hipGetLastError();
}

}  // namespace ps
