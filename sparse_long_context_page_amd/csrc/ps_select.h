// Top-k page selection of one (request, KV head) by one workgroup, shared by
// the selection kernel and the decode kernel that selects its own pages.
// ("Don't read the haystack", section "Part two: the skipping": the kept set
// is the sink pages, the last local pages and the best-scoring others.)
//
// Every score stays in registers: wavefront w owns the pages
// [w*64*C, (w+1)*64*C), lane l the pages w*64*C + j*64 + l for j < C, so
// every load is coalesced and the output can be compacted in page order with
// ballots. Scores become order-preserving 32-bit keys (a larger float gives a
// larger key; -0 is folded onto +0). The candidates' keys share every bit
// above the highest bit where their min and max differ; an MSB-first radix
// select with 8-bit digits starts below those bits. A pass histograms, in
// LDS, the digit of every key still on the threshold path; after one barrier
// each wavefront scans the 256 bins itself (no second barrier), so all agree
// on the threshold digit. Passes stop once the threshold bin holds exactly as
// many keys as slots are left, or once every bit is decided (the bin's keys
// are then equal and the lowest pages among them win). Three histogram
// buffers rotate so that the one cleared during a pass was last read two
// passes before.
#pragma once

#include "ps_device.h"

namespace ps {

constexpr int kSelDigitBits = 8;
constexpr int kSelBins = 1 << kSelDigitBits;

template <int WAVES>
struct SelectLds {
  int hist[3][kSelBins];
  uint32_t wave_min[WAVES], wave_max[WAVES];
  int wave_cnt[2][WAVES];
};

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Selects the kept pages of one unit whose n pages have the scores row[0..n).
// Called by all WAVES*64 threads of the workgroup with the same arguments;
// requires n <= WAVES*64*C and n_sink + n_local <= budget. Calls
// emit(slot, page) once per kept page, slots 0..kept-1 in ascending page
// order, and returns kept = min(budget, n). Ends with the workgroup's LDS
// free for reuse only after a barrier of the caller.
template <int WAVES, int C, typename Emit>
__device__ __forceinline__ int select_unit(const float* __restrict__ row, int n, int budget,
                                           int n_sink, int n_local, SelectLds<WAVES>& sh,
                                           Emit emit) {
  constexpr int kThreads = WAVES * kWave;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);

  if (budget >= n) {  // dense: every page, ascending
    for (int i = tid; i < n; i += kThreads) emit(i, i);
    return n;
  }

  const int lo = n_sink;  // candidates are the pages [lo, hi)
  const int hi = n - n_local;
  const int r = budget - n_sink - n_local;  // candidates to keep (hi - lo > r)
  const int seg = wave * kWave * C;
  auto page = [&](int j) { return seg + j * kWave + lane; };
  auto is_cand = [&](int p) { return p >= lo && p < hi; };

  // Keys (pages past the request re-read its last score and never count).
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
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  if (lane == 0) {
    sh.wave_min[wave] = kmin;
    sh.wave_max[wave] = kmax;
  }
  for (int i = tid; i < 2 * kSelBins; i += kThreads) sh.hist[i / kSelBins][i % kSelBins] = 0;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < WAVES; ++w) {
    kmin = min(kmin, sh.wave_min[w]);
    kmax = max(kmax, sh.wave_max[w]);
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
    const int width = top < kSelDigitBits ? top : kSelDigitBits;
    const int shift = top - width;
    int* h = sh.hist[pass % 3];
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const uint32_t k = key[j];
      if (is_cand(page(j)) && (k & pmask) == prefix)
        atomicAdd(&h[(k >> shift) & (kSelBins - 1)], 1);
    }
    for (int i = tid; i < kSelBins; i += kThreads) sh.hist[(pass + 1) % 3][i] = 0;
    __syncthreads();
    // Lane l holds bins 4l..4l+3. The threshold bin d holds the remaining-th
    // largest key: keys in bins above d < remaining <= keys from d up.
    int hb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) hb[i] = h[4 * lane + i];
    const int mine = hb[0] + hb[1] + hb[2] + hb[3];
    const int incl = wave_prefix_sum(mine);  // keys in bins 0 .. 4*lane+3
    int acc = __builtin_amdgcn_readlane(incl, kWave - 1) - incl;  // keys in bins above
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
    const int src = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(fm));
    const int d = __builtin_amdgcn_readlane(found_d, src);
    remaining = __builtin_amdgcn_readlane(found_rem, src);
    in_bin = __builtin_amdgcn_readlane(found_bin, src);
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
    sh.wave_cnt[0][wave] = cnt_keep;
    sh.wave_cnt[1][wave] = cnt_tie;
  }
  __syncthreads();
  int keep_before = 0, tie_before = 0, keep_all = 0, tie_all = 0;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) {
    keep_before += w < wave ? sh.wave_cnt[0][w] : 0;
    tie_before += w < wave ? sh.wave_cnt[1][w] : 0;
    keep_all += sh.wave_cnt[0][w];
    tie_all += sh.wave_cnt[1][w];
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
    if (keep && o < budget) emit(o, page(j));
    slot += __popcll(km);
    tie_rank += __popcll(tm);
  }
  return kept_total < budget ? kept_total : budget;
}

}  // namespace ps
