// Split-KV decode over every page (dense), a page list (sparse), or the
// pages the workgroup selects itself (top-k or top-delta): per split, the
// running max, normaliser and unnormalised accumulator of the softmax of
// scale*q.k for every query head of one KV head; optionally the merged
// output (with one split, or with several in the selecting modes, where the
// last split of a unit to finish merges). ("Don't read the haystack",
// sections "Part one: hitting the wall on purpose" and "Part two: the
// skipping"; "Attention: Undivided & Uncompressed", section "Traffic", for
// the rescaling merge.) Two kernels:
// decode_kernel (fp32 pools, vector ALUs, described here) and
// decode_mfma_kernel (bf16 pools, matrix cores, described at its definition).
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
#pragma once

#include "ps_combine.h"
#include "ps_device.h"
#include "ps_launch.h"
#include "ps_select.h"

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

// Where a workgroup's pages come from: every page of the request (dense), a
// page list (sparse), or a selection the workgroup makes itself from the page
// scores (sparse, fused with the selection: every split of a (request, KV
// head) runs the same selection and keeps its share of the list), by top-k
// (kSelect) or by the top-delta threshold (kSelectDelta).
enum DecodeMode : int { kDense = 0, kList = 1, kSelect = 2, kSelectDelta = 3 };

// Selection inputs and outputs of the selecting modes, and the merged output
// (with one split, or with more and the arrival counters).
struct SelectArgs {
  const float* scores;  // [B, Hkv, max_pages]
  int n_sink, n_local;
  int32_t* sel;        // [B, Hkv, budget] or null
  int32_t* sel_count;  // [B, Hkv] or null
  const float* sink;   // [Hq] or null; with out
  float* out;          // [B, Hq, D] or null: merged output written
  float* lse;          // [B, Hq] or null
  float scale, delta;  // kSelectDelta: the softmax scale and delta
  int32_t* arrivals;   // [B, Hkv], all zero, or null: with out and more than one
                       // split, the last split of a unit to finish merges
};

// The selection of a selecting workgroup (W wavefronts): every split of a
// (request, KV head) makes the same selection, with the physical page of
// each kept page read next to its score, so the pages' K and V can be
// requested right after it. This split keeps list slots [first, first +
// per) in LDS (pages, phys) and writes them, and the padding among them, to
// the page list output; split 0 writes the count. Returns the kept count.
template <int W, int C, int MODE, typename T, int D, int G, typename TdLds>
__device__ __forceinline__ int decode_select(const SelectArgs& sa, const float* qg,
                                             const T* k_pool, const int32_t* row, int unit,
                                             int g, int hkv, int len, int budget,
                                             int max_pages, int split, int first, int per,
                                             SelectLds<W>& ssel, TdLds& td, int* pages,
                                             int* phys) {
  const int np = ceil_div(len, kPage);
  int32_t* dst = sa.sel ? sa.sel + (int64_t)unit * budget : nullptr;
  auto emit = [&](int o, int p, int ph) {
    if (o >= first && o < first + per) {
      pages[o - first] = p;
      phys[o - first] = ph;
      if (dst) dst[o] = p;
    }
  };
  const float* row_scores = sa.scores + (int64_t)unit * max_pages;
  int kept;
  if constexpr (MODE == kSelectDelta) {
    TopDeltaThreshold<T, D, W, G> threshold{qg, k_pool, row, g, hkv, len, np, G, budget,
                                            sa.n_sink, sa.n_local, sa.scale, sa.delta, &td};
    kept = select_unit<W, C, true, true>(row_scores, np, budget, sa.n_sink, sa.n_local, ssel,
                                         row, emit, (double)sa.scale, threshold);
  } else {
    kept = select_unit<W, C, true, false>(row_scores, np, budget, sa.n_sink, sa.n_local, ssel,
                                          row, emit);
  }
  __syncthreads();  // pages complete
  if (dst)
    for (int o = max(kept, first) + (int)threadIdx.x; o < min(first + per, budget);
         o += W * kWave)
      dst[o] = -1;
  if (sa.sel_count && split == 0 && threadIdx.x == 0) sa.sel_count[unit] = kept;
  return kept;
}

// One split: the merge of ps_combine over that single partial (max m_nat in
// natural-log units, normaliser lsum, accumulator a at coordinate d of query
// head `row`), with the same operations (sink in the denominator only).
__device__ __forceinline__ void write_merged(const SelectArgs& sa, int64_t row, int hq_index,
                                             int d, int dim, float m_nat, float lsum, float a) {
  const float sig = sa.sink ? sa.sink[hq_index] : -INFINITY;
  const float mx = fmax_(m_nat, sig);
  if (mx == -INFINITY) {
    sa.out[row * dim + d] = 0.0f;
    if (sa.lse && d == 0) sa.lse[row] = -INFINITY;
    return;
  }
  float l = m_nat != -INFINITY ? __builtin_fmaf(expf(m_nat - mx), lsum, 0.0f) : 0.0f;
  if (sig != -INFINITY) l += expf(sig - mx);
  const float inv = 1.0f / l;
  const float wgt = m_nat == -INFINITY ? 0.0f : expf(m_nat - mx);
  sa.out[row * dim + d] = __builtin_fmaf(wgt, a, 0.0f) * inv;
  if (sa.lse && d == 0) sa.lse[row] = mx + logf(l);
}

// More than one split and a merged output: after writing its partials a
// split counts itself in at its (request, KV head), and the split that
// arrives last merges every split's partials of the group's query heads with
// the merge kernel's row merge (so bitwise as ps_combine), then re-arms the
// counter to zero for the next launch. No workgroup waits for another.
// An agent-scope fence writes back or invalidates a whole chiplet cache, so
// none is used: the partials are written with agent-scope stores (through
// the chiplet cache), every wavefront waits until its stores are
// acknowledged before the count is taken, and the merging workgroup reads
// the partials with agent-scope loads (past the chiplet cache). These are
// the instructions of the agent-scope release and acquire without their
// whole-cache write-back and invalidation, which only ordinary stores and
// loads need.
__device__ __forceinline__ void store_partial(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int W, int G>
__device__ __forceinline__ void merge_if_last(const SelectArgs& sa, int b, int g, int hkv,
                                              int unit, int n_splits, int dim,
                                              const float* part_acc, const float* part_ml) {
  __shared__ int last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = __hip_atomic_fetch_add(sa.arrivals + unit, 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
    last = prev == n_splits - 1;
    if (last) __hip_atomic_store(sa.arrivals + unit, 0, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!last) return;
  const int hq = hkv * G;
  for (int h = (int)(threadIdx.x / kWave); h < G; h += W) {
    const int64_t row = (int64_t)b * hq + g * G + h;
    combine_row<true>(part_acc + row * n_splits * dim, part_ml + row * n_splits * 2, n_splits,
                      dim, sa.sink ? sa.sink[g * G + h] : -INFINITY, sa.out + row * dim,
                      sa.lse ? sa.lse + row : nullptr);
  }
}

template <typename T, int D, int G, int MODE, int C>
__global__ __launch_bounds__(kDecWaves * kWave) void decode_kernel(
    const float* __restrict__ q, const T* __restrict__ k_pool, const T* __restrict__ v_pool,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ sel_count, int budget, int hkv,
    int max_pages, int n_splits, float qscale, float* __restrict__ part_acc,
    float* __restrict__ part_ml, SelectArgs sa) {
  constexpr bool SPARSE = MODE != kDense;
  using L = RowLayout<T, D>;
  using S = DecodeState<T, D, G>;
  constexpr int V = L::kVec;
  constexpr int LPR = L::kLanesPerRow;
  constexpr int NT = S::NT;
  __shared__ float sm_m[kDecWaves][G];
  __shared__ float sm_l[kDecWaves][G];
  __shared__ float sm_acc[kDecWaves][G][D];
  // selecting modes: the selection's workspace and this split's share of the
  // list
  constexpr bool SEL = MODE >= kSelect;
  __shared__ SelectLds<SEL ? kDecWaves : 1> ssel;
  __shared__ TopDeltaLds<MODE == kSelectDelta ? kDecWaves : 1, MODE == kSelectDelta ? D : 4, G>
      td;
  __shared__ int spages[SEL ? kMaxSplitPages : 1];
  __shared__ int sphys[SEL ? kMaxSplitPages : 1];

  const int split = blockIdx.x % n_splits;
  const int unit = blockIdx.x / n_splits;  // b * hkv + g
  const int b = unit / hkv;
  const int g = unit % hkv;
  const int len = seq_lens[b];
  const int np = ceil_div(len, kPage);
  const int32_t* row = page_table + (int64_t)b * max_pages;
  int lo, hi;
  if constexpr (SEL) {
    const int per = ceil_div(budget, n_splits);
    lo = split * per;
    const int kept = decode_select<kDecWaves, C, MODE, T, D, G>(
        sa, q + ((int64_t)b * hkv * G + g * G) * D, k_pool, row, unit, g, hkv, len, budget,
        max_pages, split, lo, per, ssel, td, spages, sphys);
    hi = min(lo + per, kept);
  } else if constexpr (SPARSE) {
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

  const int32_t* list = MODE == kList ? sel + (int64_t)unit * budget : nullptr;
  const int64_t head_off = (int64_t)g * kPage * D + c * V;
  // logical and physical page of item i of the split (i in [lo, hi))
  auto logical = [&](int i) {
    if constexpr (SEL) return spages[i - lo];
    else return MODE == kList ? list[i] : i;
  };
  auto physical = [&](int i, int p) {
    if constexpr (SEL) return sphys[i - lo];
    else return row[p];
  };
  for (int it = lo + wave; it < hi; it += 2 * kDecWaves) {
    const int pa = logical(it);
    const bool has_b = it + kDecWaves < hi;
    const int ib = has_b ? it + kDecWaves : it;
    const int pb = logical(ib);
    const int cnt_a = min(kPage, len - pa * kPage);
    const int cnt_b = has_b ? min(kPage, len - pb * kPage) : 0;
    const int64_t base_a = (int64_t)physical(it, pa) * hkv * kPage * D + head_off;
    const int64_t base_b = (int64_t)physical(ib, pb) * hkv * kPage * D + head_off;
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
    const float m_nat = mo == -INFINITY ? -INFINITY : mo * kLn2;
    if (SEL && sa.out && n_splits == 1) {
      write_merged(sa, (int64_t)b * hq + g * G + h, g * G + h, d, D, m_nat, lsum, a);
      continue;
    }
    const int64_t ph = ((int64_t)b * hq + g * G + h) * n_splits + split;
    if (SEL && sa.out) {  // merged in this launch: through the chiplet cache
      store_partial(part_acc + ph * D + d, a);
      if (d == 0) {
        store_partial(part_ml + ph * 2 + 0, m_nat);
        store_partial(part_ml + ph * 2 + 1, lsum);
      }
      continue;
    }
    part_acc[ph * D + d] = a;
    if (d == 0) {
      part_ml[ph * 2 + 0] = m_nat;
      part_ml[ph * 2 + 1] = lsum;
    }
  }
  if constexpr (SEL) {
    if (sa.out && n_splits > 1)
      merge_if_last<kDecWaves, G>(sa, b, g, hkv, unit, n_splits, D, part_acc, part_ml);
  }
}

// bf16 K/V: q.k on the matrix cores. A page (16 tokens) is one
// v_mfma_f32_16x16x32_bf16 row block: A = K (row = token, the 8 contraction
// coordinates of a lane are 8 consecutive d of one 16-byte load straight from
// the pool), B = the group's queries scaled by scale*log2(e) (column = head,
// padded to 16 with zeros), split exactly into hi + mid + lo bf16 terms in
// LDS once per workgroup and read from there as each product is issued. Lane
// (token group, head) then holds 4 logits of one head; the page max per head
// is a 2-step shuffle, the running max is uniform per head and raised lazily
// (by more than 8 in log2 units), and p = 2^(x - m) stays in the lane as the
// A operand of P.V on the matrix cores (v_mfma_f32_16x16x16_bf16, p split
// into hi + lo bf16; B = V staged in LDS and read transposed, 16 columns per
// product). The queries are requested first; each wavefront resolves its page
// ids (list entry, then table entry) two blocks of P pages ahead, keeps the
// next block's K and V in flight while the current one is attended, and
// leaves its state in LDS for the workgroup merge.
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// A page as the decode sees it: valid token count (0 = none) and its
// physical page.
struct PageRef {
  int cnt;
  int phys;
};



// Wavefronts per workgroup: 8 when the launch has at most one workgroup per
// compute unit (256), else 4.
inline int decode_waves(int64_t blocks) { return blocks <= 256 ? 8 : 4; }

// P: pages in flight per wavefront (its K and V rows held in registers).
template <int D, int G, int MODE, int C, int W, int P>
__global__ __launch_bounds__(W * kWave,
                             W == 8 ? 1
                                    : (((MODE >= kSelect && D == 128) ||
                                        (MODE == kSelectDelta && C == 32)) ? 2 : 3))
void decode_mfma_kernel(
    const float* __restrict__ q, const bf16_t* __restrict__ k_pool,
    const bf16_t* __restrict__ v_pool, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ sel_count, int budget, int hkv, int max_pages, int n_splits,
    float qscale, float* __restrict__ part_acc, float* __restrict__ part_ml, SelectArgs sa) {
  using L = RowLayout<bf16_t, D>;  // V row layout
  constexpr int KB = D / 32;
  constexpr int LPR = L::kLanesPerRow;
  constexpr int RPL = L::kRowsPerLoad;
  constexpr int NT = L::kLoadsPerPage;  // V rows per lane per page
  constexpr int NB = D / 16;            // 16-column blocks of the output
  static_assert(G <= 8, "group size");
  // Rows padded against LDS bank conflicts: unpadded, rows sit a multiple of
  // 256 bytes apart, so the query rows of the group's heads (one per B
  // column) and the 16 V rows of a transposed read all fall on the same
  // banks (select+decode 24.3 -> 23.9 us at 32 x 64k tokens, 16.9 -> 16.4 us
  // at 8 x 16k).
  __shared__ __align__(16) uint16_t qsp[3][8][D + 32];  // split scaled queries
  __shared__ __align__(16) uint16_t vt[W][16][D + 8];   // V page of each wavefront
  __shared__ float sm_m[W][G], sm_mt[W][G], sm_l[W][G];
  // rows padded by 4: the heads 4 apart that one store writes then fall on
  // different banks
  __shared__ float sm_acc[W][G][D + 4];
  // selecting modes: the selection's workspace and this split's share of the
  // list
  constexpr bool SEL = MODE >= kSelect;
  __shared__ SelectLds<SEL ? W : 1> ssel;
  __shared__ int spages[SEL ? kMaxSplitPages : 1];
  __shared__ int sphys[SEL ? kMaxSplitPages : 1];
  // kSelectDelta: the threshold's queries and maxima live in the V staging
  // buffer, unused until the selection has ended (and at a low LDS address,
  // so its reads take immediate offsets)
  using TdLds = TopDeltaLds<W, D, G>;
  static_assert(sizeof(TdLds) <= sizeof(vt), "threshold workspace fits the V staging buffer");
  TdLds& td = *reinterpret_cast<TdLds*>(&vt[0][0][0]);

  const int split = blockIdx.x % n_splits;
  const int unit = blockIdx.x / n_splits;  // b * hkv + g
  const int b = unit / hkv;
  const int g = unit % hkv;
  // Uniform per wavefront, so page ids below are scalar loads: they are
  // counted apart from the vector loads of K and V and never make a wait for
  // one page's K/V drain the loads of the pages behind it.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int col = lane % 16;   // token row of A / head column of B
  const int kgrp = lane / 16;  // which 8 of each 32 coordinates; token group of D
  const int rg = lane / LPR;   // V row group
  const int vc = lane % LPR;   // V column vector

  // The queries are requested first: their split is the first thing waited
  // for after the page ids, and vector loads complete in order.
  const float* qg = q + ((int64_t)b * hkv * G + g * G) * D;
  constexpr int kQPer = (G * D + W * kWave - 1) / (W * kWave);
  float qv[kQPer];
#pragma unroll
  for (int i = 0; i < kQPer; ++i) {
    const int e = threadIdx.x + i * W * kWave;
    qv[i] = e < G * D ? qg[e] : 0.0f;
  }

  const int32_t* list = MODE == kList ? sel + (int64_t)unit * budget : nullptr;
  const int32_t* row = page_table + (int64_t)b * max_pages;
  const int len = seq_lens[b];
  int first, hi;
  if constexpr (SEL) {
    const int per = ceil_div(budget, n_splits);
    first = split * per;
    const int kept = decode_select<W, C, MODE, bf16_t, D, G>(
        sa, qg, k_pool, row, unit, g, hkv, len, budget, max_pages, split, first, per, ssel, td,
        spages, sphys);
    hi = min(first + per, kept);
  } else if constexpr (MODE == kList) {
    const int per = ceil_div(budget, n_splits);
    first = split * per;
    hi = min(first + per, min(sel_count[unit], budget));
  } else {
    const int np = ceil_div(len, kPage);
    const int per = ceil_div(np, n_splits);
    first = min(split * per, np);
    hi = min(split * per + per, np);
  }
  // Wavefront `wave` takes the split's items first + wave + W*k.
  const int n_items = hi > first + wave ? ceil_div(hi - first - wave, W) : 0;


  // Page ids of a block of P items (list entry, then table entry). Every
  // read is in bounds: list slots are clamped to the row, and items past the
  // wavefront's last one read logical page 0 and get no tokens.
  auto resolve_block = [&](int blk, PageRef (&refs)[P]) {
    int pg[P];
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const int item = first + wave + (blk * P + j) * W;
      if constexpr (SEL)
        pg[j] = spages[min(item - first, kMaxSplitPages - 1)];
      else
        pg[j] = MODE == kList ? list[min(item, budget - 1)] : item;
    }
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const bool ok = blk * P + j < n_items;
      const int pc = ok ? pg[j] : 0;
      if constexpr (SEL) {  // physical pages came with the selection
        const int item = first + wave + (blk * P + j) * W;
        refs[j].phys = ok ? sphys[min(item - first, kMaxSplitPages - 1)] : 0;
      } else {
        refs[j].phys = row[pc];
      }
      refs[j].cnt = ok ? min(kPage, len - pc * kPage) : 0;
    }
  };
  // All 16 rows of a (page, KV head) block are read (they are in bounds);
  // rows past the valid count are zeroed in V and masked in the logits.
  // K/V rows are read once per step; at D = 128 they are loaded
  // non-temporal (default steps: ragged 64 x 4k-128k tokens 172.2 -> 166.0
  // us, 32 x 64k 51.9 -> 51.3 us, 8 x 16k unchanged within 0.15 us); at
  // D = 64 that measured slower (16 x 32k with 8 KV heads: 34.0-34.7 -> 35.3).
  auto kv16 = [](const bf16_t* p) {
    if constexpr (D == 128)
      return ld16nt(p);
    else
      return ld16(p);
  };
  auto load = [&](const PageRef& r, uint4 (&kf)[KB], uint4 (&vf)[NT]) {
    const int64_t off = ((int64_t)r.phys * hkv + g) * kPage * D;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) kf[kb] = kv16(k_pool + off + col * D + kb * 32 + kgrp * 8);
#pragma unroll
    for (int i = 0; i < NT; ++i) vf[i] = kv16(v_pool + off + (rg + i * RPL) * D + vc * 8);
  };

  // Page ids are resolved two blocks of P ahead of their use.
  PageRef ids[P], nxt[P];
  resolve_block(0, ids);
  resolve_block(1, nxt);

  // Split of the scaled queries, once per workgroup (the table reads above
  // are in flight meanwhile).
#pragma unroll
  for (int i = 0; i < kQPer; ++i) {
    const int e = threadIdx.x + i * W * kWave;
    if (e < G * D) {
      uint32_t hi_, mid_, lo_;
      bf16_split3(qv[i] * qscale, hi_, mid_, lo_);
      const int h = e / D, d = e % D;
      qsp[0][h][d] = (uint16_t)hi_;
      qsp[1][h][d] = (uint16_t)mid_;
      qsp[2][h][d] = (uint16_t)lo_;
    }
  }

  // P pages in flight before the barrier.
  uint4 kbuf[P][KB], vbuf[P][NT];
#pragma unroll
  for (int j = 0; j < P; ++j) load(ids[j], kbuf[j], vbuf[j]);
  __syncthreads();
  const bool live = col < G;  // lanes of real heads in the B operand

  float m_run = -INFINITY, m_true = -INFINITY, l_part = 0.0f;  // head `col`
  // P.V accumulators: acc[nb][i] = output of head 4*kgrp+i, column 16*nb+col.
  f32x4_t acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const int trow = 4 * kgrp + (col >> 2);  // V row this lane hands to the transposed read
  const int tcol = 4 * (col & 3);          // and its 4-column offset within a 16-column block

  auto attend = [&](const PageRef& r, const uint4 (&kf)[KB], const uint4 (&vf)[NT]) {
    f32x4_t s[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s[kb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 2; k >= 0; --k)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const uint4 bq = live ? *reinterpret_cast<const uint4*>(&qsp[k][col][kb * 32 + kgrp * 8])
                              : make_uint4(0, 0, 0, 0);
        s[kb] = mfma_bf16_16x16x32(kf[kb], bq, s[kb]);
      }
    float x[4];
    {
      f32x4_t t = s[0];
#pragma unroll
      for (int kb = 1; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i] += s[kb][i];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = 4 * kgrp + i < r.cnt ? t[i] : -INFINITY;
    }
    float mp = fmax_(fmax_(x[0], x[1]), fmax_(x[2], x[3]));
    mp = fmax_(mp, __shfl_xor(mp, 16));
    mp = fmax_(mp, __shfl_xor(mp, 32));
    m_true = fmax_(m_true, mp);
    const bool resc = mp > m_run + kLazyRescale;
    float alpha = 1.0f;
    if (resc) {
      alpha = exp2_(m_run - mp);
      m_run = mp;
      l_part *= alpha;
    }
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[i] = x[i] == -INFINITY ? 0.0f : exp2_(x[i] - m_run);
    l_part += (pr[0] + pr[1]) + (pr[2] + pr[3]);
    // Weights as the A operand of P.V (row = head `col`, k = token 4*kgrp+i),
    // split into hi + lo bf16 so the product keeps ~16 bits of each weight.
    uint32_t whi[4], wlo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      whi[i] = bf16_rne_bits(pr[i]);
      wlo[i] = bf16_rne_bits(pr[i] - bf16_bits_to_float(whi[i]));
    }
    const uint2 aph = make_uint2(whi[0] | (whi[1] << 16), whi[2] | (whi[3] << 16));
    const uint2 apl = make_uint2(wlo[0] | (wlo[1] << 16), wlo[2] | (wlo[3] << 16));
    if (__any(resc && live)) {
      // accumulator rows are heads 4*kgrp+i; their factors live in lanes 4*kgrp+i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(alpha, 4 * kgrp + i);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb][i] *= ai;
      }
    }
    // Stage V (rows past the valid count as zeros), then P.V per 16 columns
    // with the B operand read transposed from LDS.
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int t = rg + i * RPL;
      *reinterpret_cast<uint4*>(&vt[wave][t][vc * 8]) = t < r.cnt ? vf[i] : make_uint4(0, 0, 0, 0);
    }
    wave_sync_lds();
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint2 bv = lds_read_tr16(&vt[wave][trow][nb * 16 + tcol]);
      acc[nb] = mfma_bf16_16x16x16(apl, bv, acc[nb]);
      acc[nb] = mfma_bf16_16x16x16(aph, bv, acc[nb]);
    }
    wave_sync_lds();  // V is read before the next page overwrites it
  };

  // Pipeline: while page j of a block is attended, the loads of the pages of
  // the next block are in flight; each buffer is refilled as soon as its
  // page is attended (every load in the loop unconditional, so the number in
  // flight is the same on every path). The last block is attended after the
  // loop and requests nothing more.
  int base = 0;
  for (; base + P < n_items; base += P) {
    PageRef nn[P];
    resolve_block(base / P + 2, nn);
#pragma unroll
    for (int j = 0; j < P; ++j) {
      attend(ids[j], kbuf[j], vbuf[j]);
      load(nxt[j], kbuf[j], vbuf[j]);
    }
#pragma unroll
    for (int j = 0; j < P; ++j) {
      ids[j] = nxt[j];
      nxt[j] = nn[j];
    }
  }
#pragma unroll
  for (int j = 0; j < P; ++j)
    if (base + j < n_items) attend(ids[j], kbuf[j], vbuf[j]);  // uniform per wavefront

  // Per wavefront: normaliser over token groups; each (head, column) of the
  // accumulators is owned by one lane.
  l_part += __shfl_xor(l_part, 16);
  l_part += __shfl_xor(l_part, 32);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * kgrp + i;
    if (h < G) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) sm_acc[wave][h][nb * 16 + col] = acc[nb][i];
    }
  }
  if (kgrp == 0 && live) {
    sm_m[wave][col] = m_run;
    sm_mt[wave][col] = m_true;
    sm_l[wave][col] = l_part;
  }
  __syncthreads();

  // Merge against the split's true max; write the partials.
  const int hq = hkv * G;
  for (int idx = threadIdx.x; idx < G * D; idx += W * kWave) {
    const int h = idx / D;
    const int d = idx % D;
    float mo = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) mo = fmax_(mo, sm_mt[w][h]);
    float a = 0.0f, lsum = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float mw = sm_m[w][h];
      const float wt = mw == -INFINITY ? 0.0f : exp2_(mw - mo);
      a = __builtin_fmaf(wt, sm_acc[w][h][d], a);
      lsum = __builtin_fmaf(wt, sm_l[w][h], lsum);
    }
    const float m_nat = mo == -INFINITY ? -INFINITY : mo * kLn2;
    if (sa.out && n_splits == 1) {
      write_merged(sa, (int64_t)b * hq + g * G + h, g * G + h, d, D, m_nat, lsum, a);
      continue;
    }
    const int64_t ph = ((int64_t)b * hq + g * G + h) * n_splits + split;
    if (SEL && sa.out) {  // merged in this launch: through the chiplet cache
      store_partial(part_acc + ph * D + d, a);
      if (d == 0) {
        store_partial(part_ml + ph * 2 + 0, m_nat);
        store_partial(part_ml + ph * 2 + 1, lsum);
      }
      continue;
    }
    part_acc[ph * D + d] = a;
    if (d == 0) {
      part_ml[ph * 2 + 0] = m_nat;
      part_ml[ph * 2 + 1] = lsum;
    }
  }
  if constexpr (SEL) {
    if (sa.out && n_splits > 1)
      merge_if_last<W, G>(sa, b, g, hkv, unit, n_splits, D, part_acc, part_ml);
  }
}

// The launch of a selecting decode (MODE = kSelect or kSelectDelta), each
// instantiated in a source file of its own.
template <int MODE>
hipError_t launch_selecting_decode(const Shape& s, const float* q, const void* k_pool,
                                   const void* v_pool, const int32_t* page_table,
                                   const int32_t* seq_lens, int budget, float scale,
                                   int n_splits, float* part_acc, float* part_ml,
                                   const SelectArgs& sa, hipStream_t st) {
  const int64_t blocks = (int64_t)s.batch * s.hkv * n_splits;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (s.max_pages > kSelectDecodeMaxPages ||
      (budget + n_splits - 1) / n_splits > kMaxSplitPages ||
      (sa.out && n_splits != 1 && !sa.arrivals))
    return hipErrorInvalidValue;
  const float qscale = scale * 1.44269504088896340736f;  // log2(e)
  if (!s.kv_bf16) {  // fp32 K/V: the vector-ALU decode, 4 wavefronts
    const dim3 grid((unsigned)blocks), block(kDecWaves * kWave);
    const int per_lane = (s.max_pages + kDecWaves * kWave - 1) / (kDecWaves * kWave);
#define PS_SELECT_DECODE_F32(DD, CC)                                                         \
  hipLaunchKernelGGL((decode_kernel<float, DD, kG, MODE, CC>), grid, block, 0, st, q,     \
                     static_cast<const float*>(k_pool), static_cast<const float*>(v_pool),  \
                     page_table, seq_lens, nullptr, nullptr, budget, s.hkv, s.max_pages,    \
                     n_splits, qscale, part_acc, part_ml, sa)
#define PS_SELECT_DECODE_F32_C(DD)                          \
  do {                                                      \
    if (per_lane <= 2) PS_SELECT_DECODE_F32(DD, 2);         \
    else if (per_lane <= 8) PS_SELECT_DECODE_F32(DD, 8);    \
    else PS_SELECT_DECODE_F32(DD, 32);                      \
  } while (0)
    PS_WITH_GROUP(s.group, {
      if (s.head_dim == 64)
        PS_SELECT_DECODE_F32_C(64);
      else
        PS_SELECT_DECODE_F32_C(128);
    });
#undef PS_SELECT_DECODE_F32_C
#undef PS_SELECT_DECODE_F32
    return hipGetLastError();
  }
  const int waves = decode_waves(blocks);
  const dim3 grid((unsigned)blocks), block(waves * kWave);
  const int per_lane = (s.max_pages + waves * kWave - 1) / (waves * kWave);
#define PS_SELECT_DECODE(DD, CC, WW)                                                          \
  hipLaunchKernelGGL((decode_mfma_kernel<DD, kG, MODE, CC, WW, 2>), grid,                   \
                     block, 0, st, q,                                                         \
                     static_cast<const bf16_t*>(k_pool), static_cast<const bf16_t*>(v_pool),  \
                     page_table, seq_lens, nullptr, nullptr, budget, s.hkv, s.max_pages,      \
                     n_splits, qscale, part_acc, part_ml, sa)
#define PS_SELECT_DECODE_C(DD)                                                   \
  do {                                                                           \
    if (waves == 8) {                                                            \
      if (per_lane <= 8) PS_SELECT_DECODE(DD, 8, 8);                             \
      else PS_SELECT_DECODE(DD, 16, 8);                                          \
    } else {                                                                     \
      if (per_lane <= 16) PS_SELECT_DECODE(DD, 16, 4);                           \
      else PS_SELECT_DECODE(DD, 32, 4);                                          \
    }                                                                            \
  } while (0)
  PS_WITH_GROUP(s.group, {
    if (s.head_dim == 64)
      PS_SELECT_DECODE_C(64);
    else
      PS_SELECT_DECODE_C(128);
  });
#undef PS_SELECT_DECODE_C
#undef PS_SELECT_DECODE
  return hipGetLastError();
}

}  // namespace ps
