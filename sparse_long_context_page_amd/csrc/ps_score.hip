// Page score: the min/max upper bound of q.k per page, max over the GQA group.
// ("Don't read the haystack", section "Part two: the skipping".)
//
// The bound sum_d max(q_d*kmin_d, q_d*kmax_d) is evaluated as the contraction
// [max(q,0), min(q,0)] . [kmax; kmin]: for each coordinate exactly one of the
// two products is non-zero and it is the larger one. Each product of an fp32
// query and a stored (bf16 or fp32) bound is formed inside an fma, so the
// only roundings are the fma accumulations: V sequential terms per lane, then
// a fixed butterfly over the row's lanes. The order is fixed, so results are
// bitwise reproducible.
//
// Two kernels: bf16 metadata goes to the matrix cores (below); fp32 metadata
// uses the vector ALUs: a workgroup of 4 wavefronts covers a chunk of
// consecutive logical pages of one (request, KV head); within a wavefront,
// lane = (page slot, column vector); a page's kmax and kmin rows are read as
// coalesced 16-byte vectors, several pages per wave-load, and all loads of a
// wavefront's pages are issued before any arithmetic. In its refresh variant
// the wavefront holding a request's last page also reads that page's keys,
// folds them with the lane layout of the scoring (lane = (row, column
// vector)), writes the page's metadata and scores the page from the folded
// registers.
//
// LOGICAL: the metadata sit in the request's logical page order
// ([B, Hkv, max_pages, 2, D]), so a page's metadata are read at an address
// known from the page index alone; only a refresh reads the page table (for
// the last page's keys).
#include <algorithm>
#include <type_traits>

#include "ps_device.h"
#include "ps_launch.h"
#include "ps_meta.h"

namespace ps {

constexpr int kScoreWaves = 4;
constexpr int kScoreIters = 4;  // wave-loads per wavefront

template <typename T, int D>
struct ScoreCfg {
  using L = RowLayout<T, D>;
  static constexpr int kPagesPerLoad = L::kRowsPerLoad;  // one meta row per page slot
  static constexpr int kPagesPerWave = kPagesPerLoad * kScoreIters;
  static constexpr int kPagesPerBlock = kPagesPerWave * kScoreWaves;
};

// META8: the metadata are 8-bit codes (4 per lane and bound), widened
// exactly to fp32. meta is not restrict-qualified: a refresh writes the last
// pages' metadata through meta_out, which is the same buffer.
template <typename T, int D, int G, bool REFRESH, bool META8, bool LOGICAL>
__global__ __launch_bounds__(kScoreWaves * kWave) void score_pages_kernel(
    const float* __restrict__ q, const void* meta,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens, int hkv,
    int max_pages, int chunks_per_unit, float* __restrict__ scores,
    const T* __restrict__ k_pool, void* meta_out) {
  using C = ScoreCfg<T, D>;
  using L = typename C::L;
  constexpr int V = L::kVec;
  constexpr int LPR = L::kLanesPerRow;
  static_assert(!META8 || V == 4, "8-bit codes: four per lane and bound");
  using MV = std::conditional_t<META8, uint32_t, uint4>;  // one lane's bound values
  constexpr int EB = META8 ? 1 : (int)sizeof(T);          // bytes per metadata element

  // Consecutive workgroups go to the 8 XCDs in turn; rotating the chunk
  // index by the request spreads the leading chunks of short requests (the
  // only ones with pages) over every XCD instead of the first few, and keeps
  // a request's KV heads (interleaved in the metadata) on the same XCDs.
  const int unit = blockIdx.x / chunks_per_unit;  // b * hkv + g
  const int chunk = (blockIdx.x % chunks_per_unit + unit / hkv) % chunks_per_unit;
  const int b = unit / hkv;
  const int g = unit % hkv;
  const int len = seq_lens[b];
  const int np = ceil_div(len, kPage);
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int p0 = chunk * C::kPagesPerBlock + wave * C::kPagesPerWave;
  if (p0 >= np) return;  // uniform per wavefront
  const int slot = lane / LPR;
  const int c = lane % LPR;

  // The last page's keys, read (and folded below) by every wavefront of a
  // refresh launch: the one holding the page (p0 <= np - 1 here) its own,
  // the others page 0 of this KV head, before the metadata and with no branch
  // around the loads (a branch made the compiler wait for every load in
  // flight at the join).
  const int tail = np - 1;
  const bool has_tail = REFRESH && tail < p0 + C::kPagesPerWave;  // uniform
  // page-table entries first (the tail's and this wavefront's pages')
  int tp = 0;
  if constexpr (REFRESH) tp = page_table[(int64_t)b * max_pages + tail];
  int phys_it[kScoreIters];
#pragma unroll
  for (int it = 0; it < kScoreIters; ++it) {
    const int p = p0 + it * C::kPagesPerLoad + slot;
    phys_it[it] = LOGICAL ? 0 : page_table[(int64_t)b * max_pages + min(p, np - 1)];
  }
  PageFold<T, D> tail_keys;
  int64_t tail_base = g;
  if constexpr (REFRESH) {
    tail_base = (int64_t)(has_tail ? tp : 0) * hkv + g;
    tail_keys.load(k_pool + tail_base * kPage * D, lane);
  }

  // Then every metadata load of this wavefront, unconditionally (a slot past
  // the request re-reads the last page's metadata and its score is not
  // written): a conditional load made the compiler wait after each one.
  MV vmax[kScoreIters], vmin[kScoreIters];
#pragma unroll
  for (int it = 0; it < kScoreIters; ++it) {
    const int64_t mslot =
        LOGICAL ? (int64_t)unit * max_pages + min(p0 + it * C::kPagesPerLoad + slot, np - 1)
                : (int64_t)phys_it[it] * hkv + g;
    const uint8_t* src = static_cast<const uint8_t*>(meta) + (mslot * 2 * D + c * V) * EB;
    vmax[it] = *reinterpret_cast<const MV*>(src);
    vmin[it] = *reinterpret_cast<const MV*>(src + D * EB);
  }

  // Split query coordinates by sign: qp = max(q, 0) multiplies kmax,
  // qn = min(q, 0) multiplies kmin.
  float qp[G][V], qn[G][V];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float* qh = q + ((int64_t)b * hkv * G + g * G + h) * D + c * V;
#pragma unroll
    for (int j = 0; j < V; j += 4) {
      const float4 v4 = *reinterpret_cast<const float4*>(qh + j);
      const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qp[h][j + e] = vv[e] > 0.0f ? vv[e] : 0.0f;
        qn[h][j + e] = vv[e] < 0.0f ? vv[e] : 0.0f;
      }
    }
  }

  // The last page's metadata, folded from its keys: lane (row r0, column
  // vector c) ends with columns c of both bounds, the columns it scores
  // (8-bit: the codes written, widened back).
  float tx[V], tn[V];
  if constexpr (REFRESH) {
    tail_keys.fold(len - tail * kPage, lane, tx, tn);
    const int64_t tslot = LOGICAL ? (int64_t)unit * max_pages + tail : tail_base;
    uint8_t* dst = static_cast<uint8_t*>(meta_out) + (tslot * 2 * D + slot * D + c * V) * EB;
    if constexpr (META8) {
      const uint32_t cx = fp8_pack4(tx, true), cn = fp8_pack4(tn, false);
      if (has_tail && slot < 2) *reinterpret_cast<uint32_t*>(dst) = slot == 0 ? cx : cn;
      fp8x4_to_f32x4(cx, tx);
      fp8x4_to_f32x4(cn, tn);
    } else {
      if (has_tail && slot < 2) st16(dst, slot == 0 ? pack(tx) : pack(tn));
    }
  }

  float* out = scores + (int64_t)unit * max_pages;
#pragma unroll
  for (int it = 0; it < kScoreIters; ++it) {
    const int p = p0 + it * C::kPagesPerLoad + slot;
    float kx[V], kn[V];
    if constexpr (META8) {
      fp8x4_to_f32x4(vmax[it], kx);
      fp8x4_to_f32x4(vmin[it], kn);
    } else {
      unpack(vmax[it], kx);
      unpack(vmin[it], kn);
    }
    if (has_tail && p == tail) {
#pragma unroll
      for (int j = 0; j < V; ++j) {
        kx[j] = tx[j];
        kn[j] = tn[j];
      }
    }
    float best = -INFINITY;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < V; ++j) {
        acc = __builtin_fmaf(qp[h][j], kx[j], acc);
        acc = __builtin_fmaf(qn[h][j], kn[j], acc);
      }
      acc = group_sum<LPR>(acc);
      best = fmax_(best, acc);
    }
    if (c == 0 && p < np) out[p] = best;
  }
}

// bf16 metadata: the contraction on the matrix cores. A 16-page tile is one
// v_mfma_f32_16x16x32_bf16 column block: B = metadata (column = page, the
// 8 contraction coordinates of a lane are 8 consecutive d of one 16-byte
// load), A = the group's queries (row = head, padded to 16 with zeros). The
// fp32 queries are split exactly into hi + mid + lo bf16 terms and the signs
// separated (max(q,0) against kmax, min(q,0) against kmin), so every product
// is exact; each (sign, 32-coordinate block) has its own accumulator (lo, mid,
// then hi added), and the 2*D/32 accumulators are summed in a fixed tree.
// Each wavefront streams tiles of one (request, KV head), every w_u-th tile
// of the request (w_u = the request's wavefronts): it splits
// its own slice of the queries in registers (no LDS, no barrier), reads its
// table entries once up front, and keeps the metadata of the next two tiles
// in flight while the current tile is scored.
// LOGICAL: the tiles' metadata are read at the request's logical slots, with
// no page table in front of them; a refresh then folds the last page after
// the wavefront's other tiles (its keys' physical page is the only table
// entry read), so the first tile waits for one memory round trip, not two.
// META8: the metadata are 8-bit codes, widened exactly to bf16 in registers
// before the same contraction. Each lane then takes one contiguous quarter
// of the page's coordinates (block kb of lane group kgrp holds coordinates
// kgrp*D/4 + kb*8 .. +8, the queries use the same assignment), so a lane
// reads D/4 contiguous bytes per bound instead of 16-byte pieces D/4 apart.
template <int N>
__device__ __forceinline__ f32x4_t tree_sum(const f32x4_t (&a)[N]) {
  if constexpr (N == 1) {
    return a[0];
  } else {
    f32x4_t lo[N / 2], hi[N / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      lo[i] = a[i];
      hi[i] = a[N / 2 + i];
    }
    const f32x4_t x = tree_sum<N / 2>(lo);
    const f32x4_t y = tree_sum<N / 2>(hi);
    f32x4_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = x[i] + y[i];
    return r;
  }
}


constexpr int kMfmaWaves = 4;
constexpr int kMaxTiles = 16;  // 16-page tiles one wavefront streams at most
// tiles in flight per wavefront with 8-bit metadata (bf16 metadata: 2); an
// 8-bit tile is half the bytes of a bf16 one
constexpr int kMeta8InFlight = 3;

// REFRESH: the wavefront holding a request's last page first rebuilds that
// page's metadata from its keys (the page a decode step appends to), writes
// it to meta_out and scores the page with it. NF: tiles of metadata in flight
// per wavefront.
// meta is not restrict-qualified: meta_out (a refresh) is the same buffer.
template <int D, int G, bool REFRESH, bool META8, bool LOGICAL, int NF>
__global__ __launch_bounds__(kMfmaWaves * kWave, 2) void score_pages_mfma_kernel(
    const float* __restrict__ q, const void* meta,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens, int hkv,
    int max_pages, int last_phys, int chunks_per_unit, int tiles_per_wave,
    float* __restrict__ scores, const bf16_t* __restrict__ k_pool, void* meta_out) {
  constexpr int KB = D / 32;  // 32-coordinate blocks
  constexpr int ML = META8 ? KB / 2 : KB;  // 16-byte metadata loads per bound per tile
  constexpr int EB = META8 ? 1 : 2;        // bytes per metadata element
  // first coordinate of the 8 a lane of group kgrp holds in block kb
  auto coord = [](int kgrp_, int kb) { return META8 ? kgrp_ * (D / 4) + kb * 8 : kb * 32 + kgrp_ * 8; };
  static_assert(G <= 8, "group size");
  // the refreshed last page: kmax, kmin (one wavefront of a workgroup at most
  // holds a request's last page)
  __shared__ __align__(16) uint16_t tail_lds[2][REFRESH ? D : 8];

  // Consecutive workgroups go to the 8 XCDs in turn; rotating the chunk
  // index by the request spreads the leading chunks of short requests (the
  // only ones with pages) over every XCD instead of the first few, and keeps
  // a request's KV heads (interleaved in the metadata) on the same XCDs.
  const int unit = blockIdx.x / chunks_per_unit;  // b * hkv + g
  const int chunk = (blockIdx.x % chunks_per_unit + unit / hkv) % chunks_per_unit;
  const int b = unit / hkv;
  const int g = unit % hkv;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int col = lane % 16;   // page of the tile (B column), head of A (row)
  const int kgrp = lane / 16;  // which 8 of each 32 coordinates
  const bool live = col < G;   // A rows G..15 are zero
  // The unit's tiles are dealt to its wavefronts round-robin (wavefront wu
  // takes tiles wu, wu + w_u, wu + 2 w_u, ...), so every wavefront reads
  // from all over the unit's metadata rather than one contiguous run; the
  // wavefronts then finish closer together.
  const int wu = chunk * kMfmaWaves + wave;      // wavefront within the unit
  const int w_u = chunks_per_unit * kMfmaWaves;  // wavefronts per unit
  auto tile_page = [&](int t) { return ((int64_t)wu + (int64_t)t * w_u) * 16; };

  // 1. Everything that does not depend on the request length is requested at
  // once: the length, the A-operand slice of the queries (8 consecutive
  // coordinates per 32-block), and the table entries of the wavefront's tiles.
  // Every load is unconditional and in bounds (padding lanes re-read head
  // G-1, entries past the run re-read the row's last one): a conditional load
  // makes later waits cover it, and an early exit lets the compiler sink the
  // loads behind the length, a round trip more.
  const int len = seq_lens[b];
  __builtin_amdgcn_sched_barrier(0);
  // table entries first: vector loads complete in order, and the first
  // metadata requests wait only for the entries of the first tiles
  const int32_t* row = page_table + (int64_t)b * max_pages;
  int phys[kMaxTiles];
#pragma unroll
  for (int t = 0; t < kMaxTiles; ++t)
    phys[t] = LOGICAL ? 0 : row[min(tile_page(t) + col, (int64_t)max_pages - 1)];
  __builtin_amdgcn_sched_barrier(0);
  const float* qh = q + ((int64_t)b * hkv * G + g * G + min(col, G - 1)) * D;
  float4 qv[KB][2];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    qv[kb][0] = *reinterpret_cast<const float4*>(qh + coord(kgrp, kb));
    qv[kb][1] = *reinterpret_cast<const float4*>(qh + coord(kgrp, kb) + 4);
  }
  __builtin_amdgcn_sched_barrier(0);  // issue all of the above first

  const int np = ceil_div(len, kPage);
  // tiles of this wavefront that hold pages of the request
  const int n_all = ceil_div(np, 16);  // tiles of the request
  const int n_tiles = wu < n_all ? min(tiles_per_wave, ceil_div(n_all - wu, w_u)) : 0;
  // A page past the request reads the metadata of physical page 0 (shared by
  // all such lanes, so it stays in cache) and its score is not written; an
  // entry of a live page is clamped into the pool. Logical layout: such a
  // page reads its own slot (in the buffer, contents unused: a B column only
  // reaches its own page's output).
#pragma unroll
  for (int t = 0; t < kMaxTiles; ++t)
    phys[t] = tile_page(t) + col < np ? min(max(phys[t], 0), last_phys) : 0;
  auto load = [&](int t, uint4 (&bx)[ML], uint4 (&bn)[ML]) {
    const int64_t mslot =
        LOGICAL ? (int64_t)unit * max_pages + min(tile_page(t) + col, (int64_t)max_pages - 1)
                : (int64_t)phys[t] * hkv + g;
    const uint8_t* src = static_cast<const uint8_t*>(meta) + (mslot * 2 * D + coord(kgrp, 0)) * EB;
#pragma unroll
    for (int i = 0; i < ML; ++i) {
      // bf16: block i's 8 coordinates; 8-bit: blocks 2i and 2i+1
      const int off = (META8 ? i * 16 : i * 32) * EB;
      bx[i] = ld16(src + off);
      bn[i] = ld16(src + D * EB + off);
    }
  };
  // Physical layout: the last page's keys are read by every wavefront of a
  // refresh launch, the one holding the page reading its own, the others
  // page 0 of this KV head (the same rows for all, so they stay in cache).
  // Requested before the metadata tiles, so waiting for them waits for no
  // tile, and with no branch around the loads or the fold (a branch made the
  // first tile wait for every load in flight: the compiler could not tell
  // whether the key registers, reused after the fold, still had loads
  // pending).
  const int tail = np - 1;
  const bool has_tail = REFRESH && n_tiles > 0 && (tail / 16) % w_u == wu;
  const int col_tail = tail % 16;
  PageFold<bf16_t, D> tail_keys;
  int phys_tail = 0;
  if constexpr (REFRESH && LOGICAL) {
    // the last page's physical page, for its keys (read before the last tile)
    phys_tail = has_tail ? min(max(row[max(tail, 0)], 0), last_phys) : 0;
  } else if constexpr (REFRESH) {
    int pt = phys[0];
#pragma unroll
    for (int t = 1; t < kMaxTiles; ++t) pt = t == (tail / 16) / w_u ? phys[t] : pt;
    phys_tail = has_tail ? __builtin_amdgcn_readlane(pt, col_tail) : 0;
    tail_keys.load(k_pool + ((int64_t)phys_tail * hkv + g) * kPage * D, lane);
  }
  // NF tiles of metadata in flight, requested whatever the run's length.
  static_assert(NF >= 2 && NF <= 8, "tiles in flight");
  uint4 xs[NF][ML], ns[NF][ML];
#pragma unroll
  for (int f = 0; f < NF; ++f) load(f, xs[f], ns[f]);
  __builtin_amdgcn_sched_barrier(0);  // the split below overlaps these loads
  // 2. exact split of the queries, by sign, straight into A fragments:
  // a[sign][part][kb], sign 0 = max(q,0), 1 = min(q,0); part 0 = hi, 1 = mid,
  // 2 = lo; 8 bf16 per lane
  uint4 a[2][3][KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    float v[8] = {qv[kb][0].x, qv[kb][0].y, qv[kb][0].z, qv[kb][0].w,
                  qv[kb][1].x, qv[kb][1].y, qv[kb][1].z, qv[kb][1].w};
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = live ? v[j] : 0.0f;
    uint32_t part[3][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) bf16_split3(v[j], part[0][j], part[1][j], part[2][j]);
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      uint32_t pw[4], nw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = part[k][2 * j], hi = part[k][2 * j + 1];
        const bool plo = v[2 * j] > 0.0f, phi = v[2 * j + 1] > 0.0f;
        pw[j] = (plo ? lo : 0u) | ((phi ? hi : 0u) << 16);
        nw[j] = (plo ? 0u : lo) | ((phi ? 0u : hi) << 16);
      }
      a[0][k][kb] = make_uint4(pw[0], pw[1], pw[2], pw[3]);
      a[1][k][kb] = make_uint4(nw[0], nw[1], nw[2], nw[3]);
    }
  }

  // The last page's metadata: folded from its keys, written out and kept in
  // LDS for the last tile by the wavefront holding the page.
  const int64_t tail_slot =
      LOGICAL ? (int64_t)unit * max_pages + tail : (int64_t)phys_tail * hkv + g;
  auto publish_tail = [&](const float (&mx)[8], const float (&mn)[8]) {
    using LP = RowLayout<bf16_t, D>;
    const int r0 = lane / LP::kLanesPerRow;
    const int c = lane % LP::kLanesPerRow;
    if (has_tail && r0 < 2) {
      const int64_t off = tail_slot * 2 * D + r0 * D + c * 8;
      if constexpr (META8) {
        const uint2 codes = r0 == 0 ? fp8_pack8(mx, true) : fp8_pack8(mn, false);
        *reinterpret_cast<uint2*>(static_cast<uint8_t*>(meta_out) + off) = codes;
        *reinterpret_cast<uint4*>(&tail_lds[r0][c * 8]) = fp8x8_to_bf16x8(codes.x, codes.y);
      } else {
        const uint4 v = r0 == 0 ? pack(mx) : pack(mn);
        st16(static_cast<bf16_t*>(meta_out) + off, v);
        *reinterpret_cast<uint4*>(&tail_lds[r0][c * 8]) = v;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  // Physical layout: every wavefront of a refresh launch folds (its tiles'
  // table round trip has to pass anyway; the fold needs no branch).
  if constexpr (REFRESH && !LOGICAL) {
    float mx[8], mn[8];
    tail_keys.fold(len - tail * kPage, lane, mx, mn);
    publish_tail(mx, mn);
  }

  // 3. per tile: one accumulator per (sign, 32-coordinate block), lo then mid
  // then hi, summed in a fixed tree; max over the group's heads
  float* out = scores + (int64_t)unit * max_pages;
  auto score_tile = [&](int t, const uint4 (&bx_in)[ML], const uint4 (&bn_in)[ML], bool last) {
    if constexpr (REFRESH && LOGICAL) {
      // Logical layout: only the wavefront holding the last page reads its
      // keys and folds them, just before its last tile (folding earlier, with
      // the keys held in registers or staged in LDS, measured no faster).
      if (last && has_tail) {
        tail_keys.load(k_pool + ((int64_t)phys_tail * hkv + g) * kPage * D, lane);
        float mx[8], mn[8];
        tail_keys.fold(len - tail * kPage, lane, mx, mn);
        publish_tail(mx, mn);
      }
    }
    uint4 bx[KB], bn[KB];
#pragma unroll
    for (int i = 0; i < ML; ++i) {
      if constexpr (META8) {
        bx[2 * i] = fp8x8_to_bf16x8(bx_in[i].x, bx_in[i].y);
        bx[2 * i + 1] = fp8x8_to_bf16x8(bx_in[i].z, bx_in[i].w);
        bn[2 * i] = fp8x8_to_bf16x8(bn_in[i].x, bn_in[i].y);
        bn[2 * i + 1] = fp8x8_to_bf16x8(bn_in[i].z, bn_in[i].w);
      } else {
        bx[i] = bx_in[i];
        bn[i] = bn_in[i];
      }
    }
    if (REFRESH && last && has_tail && col == col_tail) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        bx[kb] = *reinterpret_cast<const uint4*>(&tail_lds[0][coord(kgrp, kb)]);
        bn[kb] = *reinterpret_cast<const uint4*>(&tail_lds[1][coord(kgrp, kb)]);
      }
    }
    f32x4_t acc[2 * KB];
#pragma unroll
    for (int i = 0; i < 2 * KB; ++i) acc[i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 2; k >= 0; --k) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        acc[kb] = mfma_bf16_16x16x32(a[0][k][kb], bx[kb], acc[kb]);
        acc[KB + kb] = mfma_bf16_16x16x32(a[1][k][kb], bn[kb], acc[KB + kb]);
      }
    }
    const f32x4_t u = tree_sum<2 * KB>(acc);  // u[i] = bound of head 4*kgrp+i on page col
    float best = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) best = (4 * kgrp + i < G) ? fmax_(best, u[i]) : best;
    best = fmax_(best, __shfl_xor(best, 16));  // heads 0-3 with 4-7
    const int64_t p = tile_page(t) + col;
    if (kgrp == 0 && p < np) out[p] = best;
  };
  // Steady state: every iteration scores NF tiles and requests the next NF,
  // so the number of loads in flight is the same on every path.
  // The main loop never scores the run's last tile (the one that can hold
  // the request's last page). A scheduling barrier follows each request:
  // left free, the scheduler moved the next tile's waits above it (register
  // pressure), which left one tile in flight instead of NF.
  int t = 0;
  if constexpr (NF == 2) {
    auto& xa = xs[0];
    auto& na = ns[0];
    auto& xb = xs[1];
    auto& nb = ns[1];
    for (; t + 3 < n_tiles; t += 2) {
      score_tile(t, xa, na, false);
      load(t + 2, xa, na);
      __builtin_amdgcn_sched_barrier(0);
      score_tile(t + 1, xb, nb, false);
      load(t + 3, xb, nb);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (t + 2 < n_tiles) {  // three tiles left
      score_tile(t, xa, na, false);
      load(t + 2, xa, na);
      __builtin_amdgcn_sched_barrier(0);
      score_tile(t + 1, xb, nb, false);
      score_tile(t + 2, xa, na, true);
    } else {
      if (t < n_tiles) score_tile(t, xa, na, t + 1 == n_tiles);
      if (t + 1 < n_tiles) score_tile(t + 1, xb, nb, true);
    }
  } else {
    for (; t + 2 * NF - 1 < n_tiles; t += NF) {
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        score_tile(t + f, xs[f], ns[f], false);
        load(t + f + NF, xs[f], ns[f]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // fewer than 2 NF tiles left, the first NF of them in flight
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      if (t + f < n_tiles) {
        score_tile(t + f, xs[f], ns[f], t + f + 1 == n_tiles);
        if (t + f + NF < n_tiles) load(t + f + NF, xs[f], ns[f]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int f = 0; f < NF; ++f)
      if (t + NF + f < n_tiles) score_tile(t + NF + f, xs[f], ns[f], t + NF + f + 1 == n_tiles);
  }
}

hipError_t launch_score_pages(const Shape& s, const float* q, const void* meta,
                              const int32_t* page_table, const int32_t* seq_lens, float* scores,
                              const void* k_pool, void* meta_out, hipStream_t st) {
  const dim3 block(kScoreWaves * kWave);
  if (s.kv_bf16) {
    // Tiles per wavefront: about two wavefronts per SIMD (1024 SIMDs), each
    // streaming the tiles that leaves (runs of 4 to 8 16-page tiles measured
    // best at 32 x 4096 pages, 2 and 16 worse). With the metadata in logical
    // order a wavefront's prologue is one round trip shorter, and twice the
    // wavefronts with half the tiles each measured faster (32 x 4096 pages:
    // score 26.4 -> 25.0 us); in the physical layout, and with 8-bit codes
    // in either, that lost (learned sink +2 us, 8-bit metadata +4 to +6 us).
    const int tiles_per_unit = (s.max_pages + 15) / 16;
    const int64_t tiles = (int64_t)tiles_per_unit * s.batch * s.hkv;
    const int64_t waves_target = (s.meta_logical && !s.meta8) ? 4096 : 2048;
    // In the logical layout runs are also capped at 8 tiles: with requests of
    // very different lengths (tiles count max_pages, not the lengths) the
    // longest requests' wavefronts would otherwise stream 16 tiles each
    // (ragged batch of 4k to 128k tokens: refresh+score 116.7-119.3 -> 114.5 us;
    // a cap of 4 lost, 128 us).
    const int cap = (s.meta_logical && !s.meta8) ? 8 : kMaxTiles;
    const int tpw = (int)std::min<int64_t>(cap, std::max<int64_t>(1, tiles / waves_target));
    const int per_block = kMfmaWaves * tpw * 16;
    const int chunks = (s.max_pages + per_block - 1) / per_block;
    const int64_t blocks = (int64_t)chunks * s.batch * s.hkv;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks);
    const int last_phys = (int)std::min<int64_t>(s.num_phys_pages - 1, 0x7fffffff);
    const bf16_t* kp = static_cast<const bf16_t*>(k_pool);
#define PS_SCORE_MFMA(DD, RR, M8, LG)                                                      \
  hipLaunchKernelGGL((score_pages_mfma_kernel<DD, kG, RR, M8, LG, M8 ? kMeta8InFlight : 2>),  \
                     grid, block, 0, st, q, meta,                                            \
                     page_table, seq_lens, s.hkv, s.max_pages, last_phys, chunks, tpw,       \
                     scores, kp, meta_out)
#define PS_SCORE_MFMA_L(DD, RR, M8)                       \
  do {                                                    \
    if (s.meta_logical) PS_SCORE_MFMA(DD, RR, M8, true);  \
    else PS_SCORE_MFMA(DD, RR, M8, false);                \
  } while (0)
#define PS_SCORE_MFMA_M(DD, RR)                  \
  do {                                           \
    if (s.meta8) PS_SCORE_MFMA_L(DD, RR, true);  \
    else PS_SCORE_MFMA_L(DD, RR, false);         \
  } while (0)
    PS_WITH_GROUP(s.group, {
      if (s.head_dim == 64) {
        if (kp) PS_SCORE_MFMA_M(64, true);
        else PS_SCORE_MFMA_M(64, false);
      } else {
        if (kp) PS_SCORE_MFMA_M(128, true);
        else PS_SCORE_MFMA_M(128, false);
      }
    });
#undef PS_SCORE_MFMA_M
#undef PS_SCORE_MFMA_L
#undef PS_SCORE_MFMA
    return hipGetLastError();
  }
  // fp32 K: the vector-ALU kernel (fp32 or 8-bit metadata)
  const float* kp = static_cast<const float*>(k_pool);
#define PS_SCORE_F32_LAUNCH_L(DD, RR, M8, LG)                                               \
  hipLaunchKernelGGL((score_pages_kernel<float, DD, kG, RR, M8, LG>), grid, block, 0, st, q, \
                     meta, page_table, seq_lens, s.hkv, s.max_pages, chunks, scores, kp,   \
                     meta_out)
#define PS_SCORE_F32_LAUNCH(DD, RR, M8)                                    \
  do {                                                                     \
    if (s.meta_logical) PS_SCORE_F32_LAUNCH_L(DD, RR, M8, true);           \
    else PS_SCORE_F32_LAUNCH_L(DD, RR, M8, false);                         \
  } while (0)
#define PS_SCORE_F32(DD)                                                                    \
  do {                                                                                      \
    const int per_block = ScoreCfg<float, DD>::kPagesPerBlock;                              \
    const int chunks = (s.max_pages + per_block - 1) / per_block;                           \
    const int64_t blocks = (int64_t)chunks * s.batch * s.hkv;                               \
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;                           \
    const dim3 grid((unsigned)blocks);                                                      \
    PS_WITH_GROUP(s.group, {                                                                \
      if (kp) {                                                                             \
        if (s.meta8) PS_SCORE_F32_LAUNCH(DD, true, true);                                   \
        else PS_SCORE_F32_LAUNCH(DD, true, false);                                          \
      } else {                                                                              \
        if (s.meta8) PS_SCORE_F32_LAUNCH(DD, false, true);                                  \
        else PS_SCORE_F32_LAUNCH(DD, false, false);                                         \
      }                                                                                     \
    });                                                                                     \
  } while (0)
  if (s.head_dim == 64)
    PS_SCORE_F32(64);
  else
    PS_SCORE_F32(128);
#undef PS_SCORE_F32
#undef PS_SCORE_F32_LAUNCH
#undef PS_SCORE_F32_LAUNCH_L
  return hipGetLastError();
}

}  // namespace ps
