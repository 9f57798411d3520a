// Selection: forced sink/local pages plus the top-scoring remaining pages,
// per (request, KV head), emitted in ascending logical order.
// ("Don't read the haystack", section "Part two: the skipping";
// "perf(core): fused sparse-attention decode via page indirection - #1005",
// section "The reduction, and why it needed no kernel change": the kept count
// depends only on the context length, so nothing is read back.)
//
// One workgroup per (request, KV head). Scores are mapped to order-preserving
// 32-bit keys (a larger float gives a larger key; -0 is folded onto +0) and
// staged in LDS while the block finds their min and max. Every key shares the
// bits above the highest bit where min and max differ, so an MSB-first radix
// select with 12-bit digits and LDS histograms starts there (scores of one
// request sit in a narrow range; a digit over the shared bits would put every
// key into one bin). After a pass, keys whose decided bits beat the threshold
// path are kept, keys below it are dropped, and the keys in the threshold bin
// compete for the remaining slots: when that bin holds at most 64 keys, one
// wavefront ranks them exactly by (key descending, page ascending); otherwise
// another pass narrows it, and once every bit is decided the bin's keys are
// equal and the lowest pages win. The ordered output is a ballot/mbcnt
// compaction: each wavefront owns a contiguous run of pages, and one exchange
// of per-wavefront counts gives every kept page its slot, ascending.
#include "ps_device.h"
#include "ps_launch.h"

namespace ps {

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kSelCap = 16384;  // candidates staged in LDS; more are re-read from memory
constexpr int kDigitBits = 12;
constexpr int kBins = 1 << kDigitBits;
constexpr int kRankMax = kWave;  // threshold-bin size ranked directly by one wavefront

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Block-wide exclusive prefix sum in thread order; *total receives the sum.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_sums, int* total) {
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  int x = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) wave_sums[wave] = x;
  __syncthreads();
  int base = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int ws = wave_sums[w];
    base += w < wave ? ws : 0;
    all += ws;
  }
  __syncthreads();  // wave_sums may be reused by the next scan
  *total = all;
  return base + x - v;
}

__global__ __launch_bounds__(kSelThreads) void select_topk_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ seq_lens, int hkv,
    int max_pages, int budget, int n_sink, int n_local, int32_t* __restrict__ sel,
    int32_t* __restrict__ sel_count) {
  __shared__ uint32_t keys[kSelCap];
  __shared__ int hist[kBins];
  __shared__ uint32_t bin_key[kRankMax];  // threshold-bin keys, their candidate indices
  __shared__ int bin_idx[kRankMax];       // and whether the ranking keeps them
  __shared__ int bin_keep[kRankMax];
  __shared__ int wave_sums[kSelWaves];
  __shared__ int wave_cnt[2][kSelWaves];
  __shared__ uint32_t wave_min[kSelWaves], wave_max[kSelWaves];
  __shared__ int sh_digit, sh_rem, sh_bin, sh_fill;

  const int unit = blockIdx.x;  // b * hkv + g
  const int b = unit / hkv;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int n = ceil_div(seq_lens[b], kPage);
  int32_t* dst = sel + (int64_t)unit * budget;

  if (budget >= n) {  // dense: every page, ascending
    for (int i = tid; i < budget; i += kSelThreads) dst[i] = i < n ? i : -1;
    if (tid == 0) sel_count[unit] = n;
    return;
  }

  const int lo = n_sink;  // candidates are the pages [lo, hi)
  const int hi = n - n_local;
  const int m = hi - lo;
  const int r = budget - n_sink - n_local;  // candidates to keep
  const float* sc = scores + (int64_t)unit * max_pages + lo;
  const bool staged = m <= kSelCap;

  // Stage keys and reduce their min and max.
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  for (int i = tid; i < m; i += kSelThreads) {
    const uint32_t k = order_key(sc[i]);
    if (staged) keys[i] = k;
    kmin = min(kmin, k);
    kmax = max(kmax, k);
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
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    kmin = min(kmin, wave_min[w]);
    kmax = max(kmax, wave_max[w]);
  }

  // Radix passes. Invariant: keys with (k & pmask) > prefix are kept, keys
  // with (k & pmask) < prefix are dropped, and `remaining` of the `in_bin`
  // keys with (k & pmask) == prefix are kept.
  const uint32_t diff = kmin ^ kmax;
  int top = diff ? 32 - __clz(diff) : 0;  // undecided low bits
  const uint32_t low = top == 32 ? 0xffffffffu : ((1u << top) - 1u);
  uint32_t prefix = kmin & ~low;
  uint32_t pmask = ~low;
  int remaining = r;
  int in_bin = m;
  bool ranked = false;  // threshold bin resolved by direct ranking
#pragma unroll 1
  while (r > 0 && top > 0 && in_bin > kRankMax) {
    const int width = top < kDigitBits ? top : kDigitBits;
    const int shift = top - width;
    const uint32_t dmask = (1u << width) - 1u;
    for (int i = tid; i < kBins; i += kSelThreads) hist[i] = 0;
    if (tid == 0) {
      sh_digit = 0;
      sh_rem = remaining;
      sh_bin = in_bin;
    }
    __syncthreads();
    for (int i = tid; i < m; i += kSelThreads) {
      const uint32_t k = staged ? keys[i] : order_key(sc[i]);
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & dmask], 1);
    }
    __syncthreads();
    // Thread t owns bins [kPer*t, kPer*t + kPer). The threshold bin holds the
    // remaining-th largest key: keys strictly above it < remaining <= keys
    // from it up.
    constexpr int kPer = kBins / kSelThreads;
    int local = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) local += hist[tid * kPer + j];
    int total;
    const int before = block_exclusive_scan(local, wave_sums, &total);
    const int above = total - before - local;
    if (above < remaining && above + local >= remaining) {
      int acc = above;
      for (int j = kPer - 1; j >= 0; --j) {
        const int hc = hist[tid * kPer + j];
        if (acc + hc >= remaining) {
          sh_digit = tid * kPer + j;
          sh_rem = remaining - acc;
          sh_bin = hc;
          break;
        }
        acc += hc;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sh_digit << shift;
    pmask |= dmask << shift;
    remaining = sh_rem;
    in_bin = sh_bin;
    top = shift;
  }

  if (r > 0 && in_bin <= kRankMax && in_bin > remaining) {
    // Rank the threshold bin directly: gather its keys, one wavefront counts
    // for each how many bin keys precede it (key descending, page ascending).
    if (tid == 0) sh_fill = 0;
    __syncthreads();
    for (int i = tid; i < m; i += kSelThreads) {
      const uint32_t k = staged ? keys[i] : order_key(sc[i]);
      if ((k & pmask) == prefix) {
        const int slot = atomicAdd(&sh_fill, 1);
        bin_key[slot] = k;
        bin_idx[slot] = i;
      }
    }
    __syncthreads();
    if (wave == 0) {
      const bool mine = lane < in_bin;
      const uint32_t k = mine ? bin_key[lane] : 0u;
      const int idx = mine ? bin_idx[lane] : 0x7fffffff;
      int rank = 0;
      for (int j = 0; j < in_bin; ++j) {
        const uint32_t kj = (uint32_t)__shfl((int)k, j);
        const int ij = __shfl(idx, j);
        rank += (kj > k || (kj == k && ij < idx)) ? 1 : 0;
      }
      if (mine) bin_keep[lane] = rank < remaining ? 1 : 0;
    }
    ranked = true;
    __syncthreads();
  }

  // Ordered output by ballot compaction. Wavefront w owns pages
  // [w*seg, (w+1)*seg); pass 1 counts kept pages (and threshold-bin pages for
  // the equal-key case), pass 2 writes them at their slots.
  const int seg = ceil_div(ceil_div(n, kSelWaves), kWave) * kWave;
  const int pbeg = wave * seg;
  const int pend = min(n, pbeg + seg);
  // class of page p: 2 = kept outright, 1 = in the threshold bin, 0 = dropped
  auto page_class = [&](int p) -> int {
    if (p < lo || p >= hi) return 2;
    if (r == 0) return 0;
    const int i = p - lo;
    const uint32_t k = (staged ? keys[i] : order_key(sc[i])) & pmask;
    if (k > prefix) return 2;
    if (k < prefix) return 0;
    if (in_bin <= remaining) return 2;  // the whole bin is kept
    if (ranked) {
      for (int j = 0; j < in_bin; ++j)
        if (bin_idx[j] == i) return bin_keep[j] ? 2 : 0;
      return 0;
    }
    return 1;  // equal keys: the lowest pages of the bin are kept
  };
  int cnt_keep = 0, cnt_bin = 0;
  for (int p0 = pbeg; p0 < pend; p0 += kWave) {
    const int p = p0 + lane;
    const int c = p < pend ? page_class(p) : 0;
    cnt_keep += __popcll(__ballot(c == 2));
    cnt_bin += __popcll(__ballot(c == 1));
  }
  if (lane == 0) {
    wave_cnt[0][wave] = cnt_keep;
    wave_cnt[1][wave] = cnt_bin;
  }
  __syncthreads();
  // Bin pages taken by wavefront v: those whose bin rank (bin pages of
  // earlier wavefronts plus earlier lanes) is below `remaining`.
  int base_keep = 0, base_bin = 0, kept_total = 0, bin_before = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int bk = wave_cnt[1][w];
    const int taken = max(0, min(bk, remaining - bin_before));
    if (w < wave) {
      base_keep += wave_cnt[0][w] + taken;
      base_bin += bk;
    }
    kept_total += wave_cnt[0][w] + taken;
    bin_before += bk;
  }
  int slot = base_keep, bin_rank = base_bin;
  for (int p0 = pbeg; p0 < pend; p0 += kWave) {
    const int p = p0 + lane;
    const int c = p < pend ? page_class(p) : 0;
    const uint64_t bin_mask = __ballot(c == 1);
    const bool keep = c == 2 || (c == 1 && bin_rank + lanes_below(bin_mask) < remaining);
    const uint64_t keep_mask = __ballot(keep);
    const int o = slot + lanes_below(keep_mask);
    if (keep && o < budget) dst[o] = p;
    slot += __popcll(keep_mask);
    bin_rank += __popcll(bin_mask);
  }
  for (int i = kept_total + tid; i < budget; i += kSelThreads) dst[i] = -1;
  if (tid == 0) sel_count[unit] = kept_total < budget ? kept_total : budget;
}

hipError_t launch_select_topk(const Shape& s, const float* scores, const int32_t* seq_lens,
                              int budget, int n_sink, int n_local, int32_t* sel,
                              int32_t* sel_count, hipStream_t st) {
  const int64_t units = (int64_t)s.batch * s.hkv;
  if (units > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(select_topk_kernel, dim3((unsigned)units), dim3(kSelThreads), 0, st, scores,
                     seq_lens, s.hkv, s.max_pages, budget, n_sink, n_local, sel, sel_count);
  return hipGetLastError();
}

}  // namespace ps
