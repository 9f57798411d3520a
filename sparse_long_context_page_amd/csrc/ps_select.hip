// Selection: forced sink/local pages plus the top-scoring remaining pages,
// per (request, KV head), emitted in ascending logical order.
// ("Don't read the haystack", section "Part two: the skipping";
// "perf(core): fused sparse-attention decode via page indirection - #1005",
// section "The reduction, and why it needed no kernel change": the kept count
// depends only on the context length, so nothing is read back.)
//
// One workgroup of eight wavefronts per (request, KV head); every score stays
// in registers. Wavefront w owns the pages [w*64*C, (w+1)*64*C), lane l the
// pages w*64*C + j*64 + l for j < C, so every load is coalesced and the
// output can be compacted in page order with ballots. Scores become
// order-preserving 32-bit keys (a larger float gives a larger key; -0 is
// folded onto +0). The candidates' keys share every bit above the highest bit
// where their min and max differ; an MSB-first radix select with 8-bit digits
// starts below those bits. A pass histograms, in LDS, the digit of every key
// still on the threshold path; after one barrier each wavefront scans the 256
// bins itself (no second barrier), so all agree on the threshold digit.
// Passes stop once the threshold bin holds exactly as many keys as slots are
// left, or once every bit is decided (the bin's keys are then equal and the
// lowest pages among them win). Three histogram buffers rotate so that the
// one cleared during a pass was last read two passes before.
#include "ps_device.h"
#include "ps_launch.h"

namespace ps {

constexpr int kSelWaves = 8;
constexpr int kSelThreads = kSelWaves * kWave;
constexpr int kDigitBits = 8;
constexpr int kBins = 1 << kDigitBits;
static_assert(kSelectMaxPages == kSelThreads * 128, "largest register tile");

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

template <int C>
__global__ __launch_bounds__(kSelThreads) void select_topk_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens, int hkv,
    int max_pages, int budget, int n_sink, int n_local, int32_t* __restrict__ sel,
    int32_t* __restrict__ sel_count) {
  __shared__ int hist[3][kBins];
  __shared__ uint32_t wave_min[kSelWaves], wave_max[kSelWaves];
  __shared__ int wave_cnt[2][kSelWaves];

  const int unit = blockIdx.x;  // b * hkv + g
  const int b = unit / hkv;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n = ceil_div(seq_lens[b], kPage);
  int32_t* dst = sel + (int64_t)unit * budget;

  if (budget >= n) {  // dense: every page, ascending
    for (int i = tid; i < budget; i += kSelThreads) dst[i] = i < n ? i : -1;
    if (tid == 0) sel_count[unit] = n;
    return;
  }

  const int lo = n_sink;  // candidates are the pages [lo, hi)
  const int hi = n - n_local;
  const int r = budget - n_sink - n_local;  // candidates to keep (hi - lo > r)
  const int seg = wave * kWave * C;
  auto page = [&](int j) { return seg + j * kWave + lane; };
  auto is_cand = [&](int p) { return p >= lo && p < hi; };

  // Keys (pages past the request re-read its last score and never count).
  const float* row = scores + (int64_t)unit * max_pages;
  uint32_t key[C];
#pragma unroll
  for (int j = 0; j < C; ++j) key[j] = order_key(row[min(page(j), n - 1)]);
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const bool c = is_cand(page(j));
    kmin = c ? min(kmin, key[j]) : kmin;
    kmax = c ? max(kmax, key[j]) : kmax;
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, off));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, off));
  }
  if (lane == 0) {
    wave_min[wave] = kmin;
    wave_max[wave] = kmax;
  }
  if (tid < 2 * kBins) hist[tid / kBins][tid % kBins] = 0;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    kmin = min(kmin, wave_min[w]);
    kmax = max(kmax, wave_max[w]);
  }

  // Radix passes. Invariant: candidates with (k & pmask) > prefix are kept,
  // those with (k & pmask) < prefix are dropped, and `remaining` of the
  // `in_bin` candidates with (k & pmask) == prefix are kept.
  const uint32_t diff = kmin ^ kmax;
  int top = diff ? 32 - __clz(diff) : 0;  // undecided low bits
  uint32_t pmask = top == 32 ? 0u : ~((1u << top) - 1u);
  uint32_t prefix = kmin & pmask;
  int remaining = r;
  int in_bin = hi - lo;
  int pass = 0;
#pragma unroll 1
  while (remaining > 0 && in_bin > remaining && top > 0) {
    const int width = top < kDigitBits ? top : kDigitBits;
    const int shift = top - width;
    int* h = hist[pass % 3];
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const uint32_t k = key[j];
      if (is_cand(page(j)) && (k & pmask) == prefix) atomicAdd(&h[(k >> shift) & (kBins - 1)], 1);
    }
    if (tid < kBins) hist[(pass + 1) % 3][tid] = 0;
    __syncthreads();
    // Lane l holds bins 4l..4l+3. The threshold bin d holds the remaining-th
    // largest key: keys in bins above d < remaining <= keys from d up.
    int hb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) hb[i] = h[4 * lane + i];
    const int mine = hb[0] + hb[1] + hb[2] + hb[3];
    int suffix = mine;  // sum over lanes >= lane
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_down(suffix, off);
      suffix += lane + off < kWave ? y : 0;
    }
    int acc = suffix - mine;  // keys in bins above this lane's
    int found_d = -1, found_rem = 0, found_bin = 0;
#pragma unroll
    for (int i = 3; i >= 0; --i) {
      if (found_d < 0 && acc < remaining && acc + hb[i] >= remaining) {
        found_d = 4 * lane + i;
        found_rem = remaining - acc;
        found_bin = hb[i];
      }
      acc += hb[i];
    }
    const uint64_t fm = __ballot(found_d >= 0);
    const int src = (int)__builtin_ctzll(fm);
    const int d = __shfl(found_d, src);
    remaining = __shfl(found_rem, src);
    in_bin = __shfl(found_bin, src);
    prefix |= (uint32_t)d << shift;
    pmask |= ((1u << width) - 1u) << shift;
    top = shift;
    ++pass;
  }

  // Class of a page: 2 = kept, 1 = tie on the threshold key (the lowest
  // `remaining` of them are kept), 0 = dropped or past the request.
  auto page_class = [&](int j) -> int {
    const int p = page(j);
    if (p >= n) return 0;
    if (!is_cand(p)) return 2;
    if (remaining == 0) return 0;
    const uint32_t km = key[j] & pmask;
    return km > prefix ? 2 : (km == prefix ? 1 : 0);
  };
  int cnt_keep = 0, cnt_tie = 0;
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int c = page_class(j);
    cnt_keep += __popcll(__ballot(c == 2));
    cnt_tie += __popcll(__ballot(c == 1));
  }
  if (lane == 0) {
    wave_cnt[0][wave] = cnt_keep;
    wave_cnt[1][wave] = cnt_tie;
  }
  __syncthreads();
  int keep_before = 0, tie_before = 0, keep_all = 0, tie_all = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    keep_before += w < wave ? wave_cnt[0][w] : 0;
    tie_before += w < wave ? wave_cnt[1][w] : 0;
    keep_all += wave_cnt[0][w];
    tie_all += wave_cnt[1][w];
  }
  const int kept_total = keep_all + min(tie_all, remaining);
  int slot = keep_before + min(tie_before, remaining);
  int tie_rank = tie_before;
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int c = page_class(j);
    const uint64_t tm = __ballot(c == 1);
    const bool keep = c == 2 || (c == 1 && tie_rank + lanes_below(tm) < remaining);
    const uint64_t km = __ballot(keep);
    const int o = slot + lanes_below(km);
    if (keep && o < budget) dst[o] = page(j);
    slot += __popcll(km);
    tie_rank += __popcll(tm);
  }
  for (int i = kept_total + tid; i < budget; i += kSelThreads) dst[i] = -1;
  if (tid == 0) sel_count[unit] = kept_total < budget ? kept_total : budget;
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
