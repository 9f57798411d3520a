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

// Top-delta selection: select_unit keeps the forced pages and the
// best-scoring pages with scale * score >= topdelta_threshold (compared in
// fp64), at most budget of them in all.
template <typename T, int C, int D>
__global__ __launch_bounds__(kSelThreads) void select_topdelta_kernel(
    const float* __restrict__ q, const T* __restrict__ k_pool,
    const int32_t* __restrict__ page_table, const float* __restrict__ scores,
    const int32_t* __restrict__ seq_lens, int hkv, int group, int max_pages, int budget,
    int n_sink, int n_local, float scale, float delta, int32_t* __restrict__ sel,
    int32_t* __restrict__ sel_count) {
  __shared__ SelectLds<kSelWaves> sh;
  __shared__ TopDeltaLds<kSelWaves, D> td;
  const int unit = blockIdx.x;  // b * hkv + g
  const int b = unit / hkv;
  const int g = unit % hkv;
  const int len = seq_lens[b];
  const int n = ceil_div(len, kPage);
  const int32_t* table = page_table + (int64_t)b * max_pages;
  // evaluated inside select_unit, its loads issued before the scores'
  TopDeltaThreshold<T, D, kSelWaves> threshold{
      q + ((int64_t)b * hkv * group + g * group) * D, k_pool, table, g, hkv, len, n, group,
      budget, n_sink, n_local, scale, delta, &td};
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
