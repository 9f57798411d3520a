// Selection: forced sink/local pages plus the top-scoring remaining pages,
// per (request, KV head), emitted in ascending logical order.
// ("Don't read the haystack", section "Part two: the skipping";
// "perf(core): fused sparse-attention decode via page indirection - #1005",
// section "The reduction, and why it needed no kernel change": the kept count
// depends only on the context length, so nothing is read back.)
// One workgroup of eight wavefronts per (request, KV head) runs select_unit.
#include "ps_launch.h"
#include "ps_select.h"

namespace ps {

constexpr int kSelWaves = 8;
constexpr int kSelThreads = kSelWaves * kWave;
static_assert(kSelectMaxPages == kSelThreads * 128, "largest register tile");
template <int C>
__global__ __launch_bounds__(kSelThreads) void select_topk_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens, int hkv,
    int max_pages, int budget, int n_sink, int n_local, int32_t* __restrict__ sel,
    int32_t* __restrict__ sel_count) {
  __shared__ SelectLds<kSelWaves> sh;
  const int unit = blockIdx.x;  // b * hkv + g
  const int n = ceil_div(seq_lens[unit / hkv], kPage);
  int32_t* dst = sel + (int64_t)unit * budget;
  const int kept = select_unit<kSelWaves, C, false, false>(
      scores + (int64_t)unit * max_pages, n, budget, n_sink, n_local, sh, nullptr,
      [&](int o, int p, int) { dst[o] = p; });
  for (int i = kept + (int)threadIdx.x; i < budget; i += kSelThreads) dst[i] = -1;
  if (threadIdx.x == 0) sel_count[unit] = kept;
}

// Top-delta selection ("Faster Than Flash: Exploiting Attention Sparsity for
// Efficient Long-Context Decoding", section "Methodology", item 2, eq. (1)-(3)
// and "Pseudo-Max Robustness as Fail-Safe"): the pseudo-max of each query
// head is its largest scale * q.k over the valid tokens of the forced pages;
// the unit's threshold is the smallest of its heads' pseudo-maxima minus
// delta; select_unit keeps the forced pages and the best-scoring pages with
// scale * score >= threshold, at most budget of them in all. The logits are
// formed in fp64 (every fp32 * bf16 or fp32 * fp32 product is exact there),
// one (token, head) pair per thread with the key row in registers and the
// queries in LDS, then reduced per head across the workgroup.
template <typename T, int C, int D>
__global__ __launch_bounds__(kSelThreads) void select_topdelta_kernel(
    const float* __restrict__ q, const T* __restrict__ k_pool,
    const int32_t* __restrict__ page_table, const float* __restrict__ scores,
    const int32_t* __restrict__ seq_lens, int hkv, int group, int max_pages, int budget,
    int n_sink, int n_local, float scale, float delta, int32_t* __restrict__ sel,
    int32_t* __restrict__ sel_count) {
  using L = RowLayout<T, D>;
  constexpr int V = L::kVec;
  __shared__ SelectLds<kSelWaves> sh;
  __shared__ double sm_max[kSelWaves][8];
  __shared__ __align__(16) float sm_q[8][D];
  const int unit = blockIdx.x;  // b * hkv + g
  const int b = unit / hkv;
  const int g = unit % hkv;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int len = seq_lens[b];
  const int n = ceil_div(len, kPage);

  // pseudo-max and threshold, evaluated inside select_unit once the scores
  // are requested
  auto threshold = [&]() -> double {
    if (budget >= n || n_sink + n_local == 0) return -INFINITY;  // uniform
    // the group's queries, staged once in LDS (fp32; widened per product)
    const float* qg = q + ((int64_t)b * hkv * group + g * group) * D;
    for (int i = threadIdx.x; i < group * D / 4; i += kSelThreads)
      reinterpret_cast<float4*>(sm_q)[i] = reinterpret_cast<const float4*>(qg)[i];
    const int n_s = min(n_sink, n);
    const int l0 = max(n - n_local, n_s);  // local pages [l0, n), after the sink pages
    const int items = (n_s + n - l0) * kPage * group;  // (forced page, token, head)
    double mx[8];
#pragma unroll
    for (int h = 0; h < 8; ++h) mx[h] = -INFINITY;
    __syncthreads();  // sm_q complete
    for (int it = threadIdx.x; it < items; it += kSelThreads) {
      const int h = it % group;
      const int tok = it / group;
      const int fp = tok / kPage, t = tok % kPage;
      const int p = fp < n_s ? fp : l0 + (fp - n_s);
      if (p * kPage + t >= len) continue;  // unused slot of a partial page
      const int phys = page_table[(int64_t)b * max_pages + p];
      const T* krow = k_pool + (((int64_t)phys * hkv + g) * kPage + t) * D;
      uint4 kv[D / V];
#pragma unroll
      for (int i = 0; i < D / V; ++i) kv[i] = ld16(krow + i * V);
      // four partial sums over interleaved coordinates, then a fixed order
      double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int i = 0; i < D / V; ++i) {
        float kf[V];
        unpack(kv[i], kf);
#pragma unroll
        for (int j = 0; j < V; ++j)
          acc[j % 4] = __builtin_fma((double)sm_q[h][i * V + j], (double)kf[j], acc[j % 4]);
      }
      const double s = (double)scale * ((acc[0] + acc[1]) + (acc[2] + acc[3]));
#pragma unroll
      for (int hh = 0; hh < 8; ++hh) mx[hh] = hh == h ? fmax(mx[hh], s) : mx[hh];
    }
#pragma unroll
    for (int hh = 0; hh < 8; ++hh) {
      double v = mx[hh];
      for (int off = kWave / 2; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off));
      if (lane == 0) sm_max[wave][hh] = v;
    }
    __syncthreads();
    double m_min = INFINITY;
    for (int hh = 0; hh < group; ++hh) {
      double m = -INFINITY;
#pragma unroll
      for (int w = 0; w < kSelWaves; ++w) m = fmax(m, sm_max[w][hh]);
      m_min = fmin(m_min, m);
    }
    return m_min - (double)delta;
  };
  int32_t* dst = sel + (int64_t)unit * budget;
  const int kept = select_unit<kSelWaves, C, false, true>(
      scores + (int64_t)unit * max_pages, n, budget, n_sink, n_local, sh, nullptr,
      [&](int o, int p, int) { dst[o] = p; }, (double)scale, threshold);
  for (int i = kept + (int)threadIdx.x; i < budget; i += kSelThreads) dst[i] = -1;
  if (threadIdx.x == 0) sel_count[unit] = kept;
}

hipError_t launch_select_topdelta(const Shape& s, const float* q, const void* k_pool,
                                  const int32_t* page_table, const float* scores,
                                  const int32_t* seq_lens, int budget, int n_sink, int n_local,
                                  float scale, float delta, int32_t* sel, int32_t* sel_count,
                                  hipStream_t st) {
  const int64_t units = (int64_t)s.batch * s.hkv;
  if (units > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (s.max_pages > kSelectMaxPages || s.group > 8) return hipErrorInvalidValue;
  const dim3 grid((unsigned)units), block(kSelThreads);
  const int per_lane = (s.max_pages + kSelThreads - 1) / kSelThreads;
#define PS_TOPDELTA(TT, CC, DD)                                                               \
  hipLaunchKernelGGL((select_topdelta_kernel<TT, CC, DD>), grid, block, 0, st, q,             \
                     static_cast<const TT*>(k_pool), page_table, scores, seq_lens, s.hkv,     \
                     s.group, s.max_pages, budget, n_sink, n_local, scale, delta, sel,       \
                     sel_count)
#define PS_TOPDELTA_C(TT, DD)                          \
  do {                                                 \
    if (per_lane <= 2) PS_TOPDELTA(TT, 2, DD);         \
    else if (per_lane <= 8) PS_TOPDELTA(TT, 8, DD);    \
    else if (per_lane <= 32) PS_TOPDELTA(TT, 32, DD);  \
    else PS_TOPDELTA(TT, 128, DD);                     \
  } while (0)
  PS_WITH_KV(s.kv_bf16, s.head_dim, { PS_TOPDELTA_C(TElem, kD); });
#undef PS_TOPDELTA_C
#undef PS_TOPDELTA
  return hipGetLastError();
}

hipError_t launch_select_topk(const Shape& s, const float* scores, const int32_t* seq_lens,
                              int budget, int n_sink, int n_local, int32_t* sel,
                              int32_t* sel_count, hipStream_t st) {
  const int64_t units = (int64_t)s.batch * s.hkv;
  if (units > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (s.max_pages > kSelectMaxPages) return hipErrorInvalidValue;
  const dim3 grid((unsigned)units), block(kSelThreads);
#define PS_SELECT_LAUNCH(CC)                                                              \
  hipLaunchKernelGGL(select_topk_kernel<CC>, grid, block, 0, st, scores, seq_lens, s.hkv, \
                     s.max_pages, budget, n_sink, n_local, sel, sel_count)
  const int per_lane = (s.max_pages + kSelThreads - 1) / kSelThreads;
  if (per_lane <= 1) PS_SELECT_LAUNCH(1);
  else if (per_lane <= 2) PS_SELECT_LAUNCH(2);
  else if (per_lane <= 4) PS_SELECT_LAUNCH(4);
  else if (per_lane <= 8) PS_SELECT_LAUNCH(8);
  else if (per_lane <= 16) PS_SELECT_LAUNCH(16);
  else if (per_lane <= 32) PS_SELECT_LAUNCH(32);
  else if (per_lane <= 64) PS_SELECT_LAUNCH(64);
  else PS_SELECT_LAUNCH(128);
#undef PS_SELECT_LAUNCH
  return hipGetLastError();
}

}  // namespace ps
