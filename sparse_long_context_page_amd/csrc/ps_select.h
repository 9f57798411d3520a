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
constexpr int kBpl = kSelBins / kWave;  // histogram bins per lane in the scan
static_assert(kBpl >= 1 && kSelBins % kWave == 0, "bins per lane");
constexpr int kSelRankMax = kWave;  // threshold bins up to this size are ranked directly

template <int WAVES>
struct SelectLds {
  int hist[3][kSelBins];
  uint32_t wave_min[WAVES], wave_max[WAVES];
  int wave_cnt[WAVES];
  uint64_t bin_val[kSelRankMax];  // the threshold bin as (key, ~page) values
  uint64_t cut;  // kept: every candidate at or above this value
};

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The score of a key (a negative zero comes back as +0, which compares the
// same).
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Selects the kept pages of one unit whose n pages have the scores row[0..n).
// Called by all WAVES*64 threads of the workgroup with the same arguments;
// requires n <= WAVES*64*C and n_sink + n_local <= budget. Calls
// emit(slot, page, phys) once per kept page, slots 0..kept-1 in ascending
// page order, with phys = table[page] read next to the scores when a table
// row is given (else -1), and returns kept = min(budget, n). Ends with the
// workgroup's LDS free for reuse only after a barrier of the caller.
//
// FILTER (top-delta selection, "Faster Than Flash: Exploiting Attention
// Sparsity for Efficient Long-Context Decoding", section "Methodology", item
// 2): only pages with scale * score >= tau (compared in fp64) are kept, at
// most budget - |forced| of them, the best. The passing pages are a prefix
// of the (score descending, page ascending) order, so these are the best
// budget - |forced| candidates of all with the failing ones dropped: the
// radix passes run on every candidate and tau is applied at the end. Every
// thread calls tau_fn.issue() before the scores are requested and
// tau_fn.prefetch() after (the threshold's loads: table entries, then key
// rows), and tau = tau_fn() once the cut is known, so the threshold's round
// trips overlap the passes (it may hold barriers; at least one workgroup
// barrier separates prefetch() from it, so LDS written in prefetch() is
// visible to every thread there).
//
// The kept candidates are the r best in the order (key descending, page
// ascending). Radix passes narrow the r-th key's bits; once its bin holds at
// most 64 keys and more than two passes would still be needed, those keys are
// gathered and wavefront 0 ranks them directly, which fixes the cut exactly as
// (key, page); when every bit is decided first, the bin's keys are equal and
// the cut is the remaining-th lowest page among them.
struct NoThreshold {
  __device__ void issue() const {}
  __device__ void prefetch() const {}
  __device__ double operator()() const { return 0.0; }
};

template <int WAVES, int C, bool PHYS, bool FILTER, typename Emit, typename TauFn = NoThreshold>
__device__ __forceinline__ int select_unit(const float* __restrict__ row, int n, int budget,
                                           int n_sink, int n_local, SelectLds<WAVES>& sh,
                                           const int32_t* __restrict__ table, Emit emit,
                                           double scale = 0.0, TauFn tau_fn = TauFn()) {
  constexpr int kThreads = WAVES * kWave;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);

  if (budget >= n) {  // dense: every page, ascending
    for (int i = tid; i < n; i += kThreads) emit(i, i, PHYS ? table[i] : -1);
    return n;
  }

  const int lo = n_sink;  // candidates are the pages [lo, hi)
  const int hi = n - n_local;
  const int seg = wave * kWave * C;
  auto page = [&](int j) { return seg + j * kWave + lane; };
  auto in_range = [&](int p) { return p >= lo && p < hi; };

  // Keys (pages past the request re-read its last score and never count).
  uint32_t key[C];
  int phys[PHYS ? C : 1];
  if constexpr (FILTER) tau_fn.issue();
  float sc[C];
#pragma unroll
  for (int j = 0; j < C; ++j) {
    sc[j] = row[min(page(j), n - 1)];
    if constexpr (PHYS) phys[j] = table[min(page(j), n - 1)];
  }
  if constexpr (FILTER) tau_fn.prefetch();
#pragma unroll
  for (int j = 0; j < C; ++j) key[j] = order_key(sc[j]);
  auto cand_j = [&](int j) { return in_range(page(j)); };
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const bool c = cand_j(j);
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
  const int cands = hi - lo;  // candidates: every scored page that is not forced
#pragma unroll
  for (int w = 0; w < WAVES; ++w) {
    kmin = min(kmin, sh.wave_min[w]);
    kmax = max(kmax, sh.wave_max[w]);
  }
  const int r = min(budget - n_sink - n_local, cands);  // candidates to keep

  // Radix passes. Invariant: candidates with (k & pmask) > prefix are kept,
  // those with (k & pmask) < prefix are dropped, and `remaining` of the
  // `in_bin` candidates with (k & pmask) == prefix are kept. A pass costs one
  // barrier and ranking the bin three, so passes continue while at most two
  // more would decide every bit, even when the bin is small enough to rank
  // (one pass usually leaves exactly the keys still needed).
  const uint32_t diff = kmin ^ kmax;
  int top = diff ? 32 - __clz(diff) : 0;  // undecided low bits
  uint32_t pmask = top == 32 ? 0u : ~((1u << top) - 1u);
  uint32_t prefix = kmin & pmask;
  int remaining = r;
  int in_bin = cands;
  int pass = 0;
#pragma unroll 1
  while (remaining > 0 && in_bin > remaining && top > 0 &&
         (in_bin > kSelRankMax || top <= 2 * kSelDigitBits)) {
    const int width = top < kSelDigitBits ? top : kSelDigitBits;
    const int shift = top - width;
    int* h = sh.hist[pass % 3];
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const uint32_t k = key[j];
      if (cand_j(j) && (k & pmask) == prefix)
        atomicAdd(&h[(k >> shift) & (kSelBins - 1)], 1);
    }
    for (int i = tid; i < kSelBins; i += kThreads) sh.hist[(pass + 1) % 3][i] = 0;
    __syncthreads();
    // Lane l holds bins kBpl*l .. kBpl*l + kBpl - 1. The threshold bin d holds
    // the remaining-th largest key: keys in bins above d < remaining <= keys
    // from d up.
    int hb[kBpl];
#pragma unroll
    for (int i = 0; i < kBpl; ++i) hb[i] = h[kBpl * lane + i];
    int mine = 0;
#pragma unroll
    for (int i = 0; i < kBpl; ++i) mine += hb[i];
    const int incl = wave_prefix_sum(mine);  // keys in bins 0 .. kBpl*lane+kBpl-1
    int acc = __builtin_amdgcn_readlane(incl, kWave - 1) - incl;  // keys in bins above
    int found_d = -1, found_rem = 0, found_bin = 0;
#pragma unroll
    for (int i = kBpl - 1; i >= 0; --i) {
      if (found_d < 0 && acc < remaining && acc + hb[i] >= remaining) {
        found_d = kBpl * lane + i;
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

  // The cut. Default: every candidate above the bin is kept and the bin's
  // lowest `remaining` pages (all of it when it holds exactly that many;
  // equal keys when every bit is decided). Candidates compare as one 64-bit
  // value, key high and complemented page low, so (key descending, page
  // ascending) order is plain unsigned order.
  auto order64 = [](uint32_t k, int p) {
    return ((uint64_t)k << 32) | (uint64_t)(0xffffffffu - (uint32_t)p);
  };
  bool ranked = false;
  uint64_t cut = 0;
  if (remaining > 0 && in_bin > remaining && top > 0) {
    // 64 or fewer keys in the bin: gather them (slots from per-wavefront
    // ballot counts); wavefront 0 ranks them in vector registers, reading
    // the gathered values as LDS broadcasts
    auto in_bin_key = [&](int j) { return cand_j(j) && (key[j] & pmask) == prefix; };
    int mine_cnt = 0;
#pragma unroll
    for (int j = 0; j < C; ++j) mine_cnt += __popcll(__ballot(in_bin_key(j)));
    if (lane == 0) sh.wave_cnt[wave] = mine_cnt;
    __syncthreads();
    int slot = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) slot += w < wave ? sh.wave_cnt[w] : 0;
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const bool on = in_bin_key(j);
      const uint64_t m = __ballot(on);
      if (on) sh.bin_val[slot + lanes_below(m)] = order64(key[j], page(j));
      slot += __popcll(m);
    }
    __syncthreads();
    if (wave == 0) {
      const uint64_t v = lane < in_bin ? sh.bin_val[lane] : 0;
      int rank = 0;  // bin values above this one
#pragma unroll
      for (int j0 = 0; j0 < kSelRankMax; j0 += 8) {
        if (j0 >= in_bin) break;  // uniform
        uint64_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = sh.bin_val[j0 + i];
#pragma unroll
        for (int i = 0; i < 8; ++i) rank += (j0 + i < in_bin && w[i] > v) ? 1 : 0;
      }
      if (lane < in_bin && rank == remaining - 1) sh.cut = v;
    }
    __syncthreads();
    ranked = true;
    cut = sh.cut;
  }

  // FILTER: kept candidates below the threshold are dropped (ties in the bin
  // have equal scores and pass or fail together)
  double tau = 0.0;
  if constexpr (FILTER) tau = tau_fn();
  auto passes = [&](uint32_t k) { return !FILTER || scale * (double)key_value(k) >= tau; };

  // Class of each page, 2 bits per page: 2 = kept, 1 = tie in the bin (the
  // lowest `remaining` of them are kept), 0 = dropped or past the request.
  uint32_t cls[(C + 15) / 16];
#pragma unroll
  for (int i = 0; i < (C + 15) / 16; ++i) cls[i] = 0;
  int cnt_keep = 0, cnt_tie = 0;
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int p = page(j);
    const uint32_t k = key[j];
    const uint32_t km = k & pmask;
    const bool above = ranked ? order64(k, p) >= cut : km > prefix;
    const bool tie = !ranked && km == prefix;
    const int cc = above ? 2 : (tie ? 1 : 0);
    // out of range = forced (kept); in range but below the threshold: dropped
    const int c = p >= n ? 0 : (!in_range(p) ? 2 : (remaining == 0 || !passes(k) ? 0 : cc));
    cls[j / 16] |= (uint32_t)c << (2 * (j % 16));
    cnt_keep += c == 2 ? 1 : 0;
    cnt_tie += c == 1 ? 1 : 0;
  }
  const int wave_counts = wave_sum_i32((cnt_keep << 16) | cnt_tie);
  if (lane == 0) sh.wave_cnt[wave] = wave_counts;
  __syncthreads();
  int keep_before = 0, tie_before = 0, keep_all = 0, tie_all = 0;
#pragma unroll
  for (int w = 0; w < WAVES; ++w) {
    const int kc = sh.wave_cnt[w] >> 16, tc = sh.wave_cnt[w] & 0xffff;
    keep_before += w < wave ? kc : 0;
    tie_before += w < wave ? tc : 0;
    keep_all += kc;
    tie_all += tc;
  }
  const int kept_total = keep_all + min(tie_all, remaining);
  int slot = keep_before + min(tie_before, remaining);
  if (tie_all <= remaining) {  // every tie is kept (the usual case)
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const bool keep = ((cls[j / 16] >> (2 * (j % 16))) & 3) != 0;
      const uint64_t km = __ballot(keep);
      const int o = slot + lanes_below(km);
      if (keep && o < budget) emit(o, page(j), PHYS ? phys[PHYS ? j : 0] : -1);
      slot += __popcll(km);
    }
  } else {  // equal keys: the lowest `remaining` tied pages are kept
    int tie_rank = tie_before;
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const int c = (cls[j / 16] >> (2 * (j % 16))) & 3;
      const uint64_t tm = __ballot(c == 1);
      const bool keep = c == 2 || (c == 1 && tie_rank + lanes_below(tm) < remaining);
      const uint64_t km = __ballot(keep);
      const int o = slot + lanes_below(km);
      if (keep && o < budget) emit(o, page(j), PHYS ? phys[PHYS ? j : 0] : -1);
      slot += __popcll(km);
      tie_rank += __popcll(tm);
    }
  }
  return kept_total < budget ? kept_total : budget;
}

// Top-delta threshold ("Faster Than Flash: Exploiting Attention Sparsity for
// Efficient Long-Context Decoding", section "Methodology", item 2, eq. (1)-(3)
// and "Pseudo-Max Robustness as Fail-Safe"): the pseudo-max of each query
// head is its largest scale * q.k over the valid tokens of the forced pages
// (sink pages, then local pages after them); the unit's threshold is the
// smallest of its heads' pseudo-maxima minus delta; -inf when the budget
// covers the request or no page is forced (every page is then a candidate).
// The logits are formed in fp64 (every fp32 * bf16 or fp32 * fp32 product is
// exact there): the queries are widened once into LDS; eight consecutive
// threads share a forced token, each takes an eighth of the coordinates,
// widens its key values once and accumulates them in order for one head after
// another; the eighths are added pairwise, ((e0 + e1) + (e2 + e3)) + ((e4 +
// e5) + (e6 + e7)). The maximum per head across the workgroup is exact in any
// order.
// issue() requests the page-table entries of the first forced tokens and the
// queries (called before the selection requests its scores); prefetch()
// requests those tokens' key rows and widens the queries into LDS (called
// after the scores are requested); operator()() computes and returns the
// threshold once the selection's passes are done (after at least one of its
// barriers). All three are called by every thread of the workgroup;
// operator()() holds one barrier.
// DPP lane move of a double (both 32-bit halves), and the max over the 64
// lanes (uniform result; exact in any order).
template <int CTRL>
__device__ __forceinline__ double dppd(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint64_t lo = dppu<CTRL>((uint32_t)u);
  const uint64_t hi = dppu<CTRL>((uint32_t)(u >> 32));
  return __longlong_as_double((long long)((hi << 32) | lo));
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
  return __longlong_as_double((long long)((hi << 32) | lo));
}

__device__ __forceinline__ double wave_max_f64(double v) {
  v = fmax(v, dppd<kDppXor1>(v));
  v = fmax(v, dppd<kDppXor2>(v));
  v = fmax(v, dppd<kDppHalfMirror>(v));
  v = fmax(v, dppd<kDppMirror>(v));  // every lane of a row holds the row's max
  return fmax(fmax(readlane_f64(v, 0), readlane_f64(v, 16)),
              fmax(readlane_f64(v, 32), readlane_f64(v, 48)));
}

// GL: query rows held (the group size, or 8 when it is known only at run
// time). A row holds the 8 segments of D/8 coordinates that the 8 threads of
// a forced token read, each segment followed by 2 unused doubles: without
// them the 8 segments start 128 bytes apart and every read of the 8 threads
// falls on the same two LDS banks (top-delta selection 11.3 -> 9.9 us at 32 x
// 64k tokens, 9.3 -> 7.9 us at 8 x 16k).
constexpr int kTdSegPad = 2;
template <int WAVES, int D, int GL = 8>
struct TopDeltaLds {
  double wave_max[WAVES][GL];
  __align__(16) double q[GL][D + 8 * kTdSegPad];
};

// G: the group size when known at compile time, else 0 (the group member).
template <typename T, int D, int WAVES, int G = 0>
struct TopDeltaThreshold {
  static constexpr int kG = G ? G : 8;  // heads computed (those past the group skipped)
  static constexpr int kThreads = WAVES * kWave;
  static constexpr int kParts = 8;                // threads per forced token
  static constexpr int kTokens = kThreads / kParts;  // forced tokens per round
  static constexpr int kCoords = D / kParts;      // coordinates per thread
  static constexpr int kVec = Elem<T>::kPerVec;
  static constexpr int kLoads = kCoords / kVec;   // 16-byte key loads per thread
  static_assert(kLoads >= 1 && kCoords % kVec == 0, "key row split");
  static_assert(kParts == 8 && kCoords % 4 == 0,
                "8 padded query segments, 4 coordinates per write");
  static_assert(kWave % kParts == 0, "a token's eight threads are lanes 8i..8i+7 of a wavefront");
  static_assert(kG * D / 4 <= kThreads, "one float4 of the queries per thread");

  const float* qg;     // the group's queries [group, D]
  const T* k_pool;
  const int32_t* table;  // the request's page-table row
  int g, hkv, len, n, group, budget, n_sink, n_local;
  float scale, delta;
  TopDeltaLds<WAVES, D, kG>* sh;
  int phys0 = 0;  // page of this thread's first-round token
  float4 qv = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  uint4 kv0[kLoads];  // this thread's share of its first-round key row

  __device__ int ng() const { return G ? G : group; }
  __device__ bool active() const { return budget < n && n_sink + n_local > 0; }
  __device__ int n_s() const { return min(n_sink, n); }
  __device__ int l0() const { return max(n - n_local, n_s()); }  // first local page
  __device__ int tokens() const { return (n_s() + n - l0()) * kPage; }
  // logical page of forced token index ft: sink pages, then local pages
  __device__ int page_of(int ft) const {
    const int fp = ft / kPage;
    return fp < n_s() ? fp : l0() + (fp - n_s());
  }

  __device__ void issue() {
    if (!active()) return;  // uniform
    const int t = threadIdx.x;
    if (t < ng() * D / 4) qv = reinterpret_cast<const float4*>(qg)[t];
    const int ft = t / kParts;
    phys0 = ft < tokens() ? table[page_of(ft)] : 0;
  }

  // The first round's key rows, requested as soon as their table entries
  // (issue) have arrived; later loads need not complete first.
  __device__ void prefetch() {
    if (!active()) return;  // uniform
    const int t = threadIdx.x;
    const int ft = t / kParts;
    const int tt = ft < tokens() ? ft % kPage : 0;
    const T* krow = k_pool + (((int64_t)phys0 * hkv + g) * kPage + tt) * D + (t % kParts) * kCoords;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) kv0[i] = ld16(krow + i * kVec);
    // the queries, widened into LDS here (their load was issued before the
    // table entries waited for above): the selection's barriers before the
    // threshold is evaluated publish them, so the evaluation needs no
    // barrier of its own
    if (t < ng() * D / 4) {  // coordinates 4t .. 4t+3, within one segment
      const int qh = (4 * t) / D, qd = (4 * t) % D;
      double* dq = &sh->q[qh][(qd / kCoords) * (kCoords + kTdSegPad) + qd % kCoords];
      dq[0] = (double)qv.x;
      dq[1] = (double)qv.y;
      dq[2] = (double)qv.z;
      dq[3] = (double)qv.w;
    }
  }

  __device__ double operator()() {
    if (!active()) return -INFINITY;  // uniform
    const int t = threadIdx.x;
    const int lane = t % kWave;
    const int wave = t / kWave;
    const int part = t % kParts;
    const int n_tok = tokens();
    double mx[kG];
#pragma unroll
    for (int h = 0; h < kG; ++h) mx[h] = -INFINITY;
    for (int base = 0; base < n_tok; base += kTokens) {  // uniform trip count
      const int ft = base + t / kParts;
      const int p = ft < n_tok ? page_of(ft) : 0;
      const int tt = ft % kPage;
      const bool valid = ft < n_tok && p * kPage + tt < len;
      // rows past the forced tokens read row 0 of physical page 0 (in the
      // pool) and are not counted; the first round's rows were prefetched
      uint4 kv[kLoads];
      if (base == 0) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) kv[i] = kv0[i];
      } else {
        const int phys = ft < n_tok ? table[p] : 0;
        const T* krow = k_pool + (((int64_t)phys * hkv + g) * kPage + (ft < n_tok ? tt : 0)) * D +
                        part * kCoords;
#pragma unroll
        for (int i = 0; i < kLoads; ++i) kv[i] = ld16(krow + i * kVec);
      }
      double k64[kCoords];
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        float kf[kVec];
        unpack(kv[i], kf);
#pragma unroll
        for (int j = 0; j < kVec; ++j) k64[i * kVec + j] = (double)kf[j];
      }
      const double* qp = &sh->q[0][0] + part * (kCoords + kTdSegPad);
#pragma unroll
      for (int h = 0; h < kG; ++h) {
        if (!G && h >= group) break;  // uniform
        __builtin_amdgcn_sched_barrier(0);  // one head's query values live at a time
        double acc = 0.0;
#pragma unroll
        for (int c = 0; c < kCoords; ++c)
          acc = __builtin_fma(qp[h * (D + 8 * kTdSegPad) + c], k64[c], acc);
        // ((e0 + e1) + (e2 + e3)) + ((e4 + e5) + (e6 + e7)) in every lane of
        // the eight (DPP: the neighbour, the other pair of the quad, the
        // mirrored lane of the other quad, which holds that quad's sum)
        {
          const double o = dppd<kDppXor1>(acc);
          acc = (part & 1) ? o + acc : acc + o;
        }
        {
          const double o = dppd<kDppXor2>(acc);
          acc = (part & 2) ? o + acc : acc + o;
        }
        {
          const double o = dppd<kDppHalfMirror>(acc);
          acc = (part & 4) ? o + acc : acc + o;
        }
        const double sv = (double)scale * acc;
        mx[h] = valid ? fmax(mx[h], sv) : mx[h];
      }
    }
#pragma unroll
    for (int hh = 0; hh < kG; ++hh) {
      if (!G && hh >= group) break;  // uniform
      const double v = wave_max_f64(mx[hh]);
      if (lane == 0) sh->wave_max[wave][hh] = v;
    }
    __syncthreads();
    double m_min = INFINITY;
    for (int hh = 0; hh < ng(); ++hh) {
      double m = -INFINITY;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) m = fmax(m, sh->wave_max[w][hh]);
      m_min = fmin(m_min, m);
    }
    return m_min - (double)delta;
  }
};

}  // namespace ps
