// Selection: forced sink/local pages plus the top-scoring remaining pages,
// per (request, KV head), emitted in ascending logical order.
// ("Don't read the haystack", section "Part two: the skipping";
// "perf(core): fused sparse-attention decode via page indirection - #1005",
// section "The reduction, and why it needed no kernel change": the kept count
// depends only on the context length, so nothing is read back.)
//
// One workgroup per (request, KV head). Scores are mapped to order-preserving
// 32-bit keys (a larger float gives a larger key; -0 is folded onto +0) and
// staged in LDS. A three-pass MSB-first radix select (11, 11, 10 bits) with
// LDS histograms finds the key T of the R-th kept candidate and how many
// candidates equal to T are kept. A final ordered pass (each thread owns a
// contiguous run of pages, block-wide scans give ranks) keeps every forced
// page, every candidate above T and the lowest-index candidates equal to T,
// and writes their ids ascending.
#include "ps_device.h"
#include "ps_launch.h"

namespace ps {

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kSelCap = 16384;  // candidates staged in LDS; more are re-read from memory
constexpr int kBins = 2048;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
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
  __shared__ int wave_sums[kSelWaves];
  __shared__ int sh_digit, sh_rem;

  const int unit = blockIdx.x;  // b * hkv + g
  const int b = unit / hkv;
  const int tid = threadIdx.x;
  const int n = ceil_div(seq_lens[b], kPage);
  int32_t* dst = sel + (int64_t)unit * budget;

  if (budget >= n) {  // dense: every page, ascending
    for (int i = tid; i < budget; i += kSelThreads) dst[i] = i < n ? i : -1;
    if (tid == 0) sel_count[unit] = n;
    return;
  }

  const int lo = n_sink;          // candidates are the pages [lo, hi)
  const int hi = n - n_local;
  const int m = hi - lo;
  const int r = budget - n_sink - n_local;  // candidates to keep
  const float* sc = scores + (int64_t)unit * max_pages + lo;
  const bool staged = m <= kSelCap;
  if (staged) {
    for (int i = tid; i < m; i += kSelThreads) keys[i] = order_key(sc[i]);
  }
  __syncthreads();

  uint32_t prefix = 0u, pmask = 0u;
  int remaining = r;
  if (r > 0) {
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const uint32_t dmask = pass == 2 ? 0x3ffu : 0x7ffu;
      for (int i = tid; i < kBins; i += kSelThreads) hist[i] = 0;
      __syncthreads();
      for (int i = tid; i < m; i += kSelThreads) {
        const uint32_t k = staged ? keys[i] : order_key(sc[i]);
        if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & dmask], 1);
      }
      __syncthreads();
      // Thread t owns bins [4t, 4t+4). Find the bin holding the remaining-th
      // largest key: counts strictly above it < remaining <= counts from it up.
      constexpr int kPer = kBins / kSelThreads;
      int local = 0;
#pragma unroll
      for (int j = 0; j < kPer; ++j) local += hist[tid * kPer + j];
      int total;
      const int before = block_exclusive_scan(local, wave_sums, &total);
      const int above = total - before - local;  // keys in bins above this thread's
      if (above < remaining && above + local >= remaining) {
        int acc = above;
        for (int j = kPer - 1; j >= 0; --j) {
          const int hc = hist[tid * kPer + j];
          if (acc + hc >= remaining) {
            sh_digit = tid * kPer + j;
            sh_rem = remaining - acc;
            break;
          }
          acc += hc;
        }
      }
      __syncthreads();
      prefix |= (uint32_t)sh_digit << shift;
      pmask |= dmask << shift;
      remaining = sh_rem;
      __syncthreads();
    }
  }
  // Kept candidates: key > prefix, or key == prefix and among the first
  // `remaining` such candidates by page index. (With r == 0 nothing is kept.)
  const uint32_t thr = prefix;
  const int take_eq = r > 0 ? remaining : 0;
  const bool any = r > 0;

  const int per = ceil_div(n, kSelThreads);
  const int beg = min(n, tid * per);
  const int end = min(n, beg + per);

  int eq_local = 0;
  for (int p = beg; p < end; ++p) {
    if (p >= lo && p < hi) {
      const uint32_t k = staged ? keys[p - lo] : order_key(sc[p - lo]);
      eq_local += (any && k == thr) ? 1 : 0;
    }
  }
  int dummy;
  int eq_rank = block_exclusive_scan(eq_local, wave_sums, &dummy);

  int kept_local = 0;
  {
    int er = eq_rank;
    for (int p = beg; p < end; ++p) {
      bool keep;
      if (p < lo || p >= hi) {
        keep = true;
      } else {
        const uint32_t k = staged ? keys[p - lo] : order_key(sc[p - lo]);
        keep = any && (k > thr || (k == thr && er < take_eq));
        er += (any && k == thr) ? 1 : 0;
      }
      kept_local += keep ? 1 : 0;
    }
  }
  int kept_total;
  const int out_base = block_exclusive_scan(kept_local, wave_sums, &kept_total);
  {
    int er = eq_rank, o = out_base;
    for (int p = beg; p < end; ++p) {
      bool keep;
      if (p < lo || p >= hi) {
        keep = true;
      } else {
        const uint32_t k = staged ? keys[p - lo] : order_key(sc[p - lo]);
        keep = any && (k > thr || (k == thr && er < take_eq));
        er += (any && k == thr) ? 1 : 0;
      }
      if (keep && o < budget) dst[o++] = p;
    }
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
