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
// Work split: a workgroup of 4 wavefronts covers a chunk of consecutive
// logical pages of one (request, KV head). Within a wavefront, lane =
// (page slot, column vector): a page's kmax and kmin rows are read as
// coalesced 16-byte vectors, several pages per wave-load, and all loads of a
// wavefront's pages are issued before any arithmetic.
#include "ps_device.h"
#include "ps_launch.h"

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

template <typename T, int D, int G>
__global__ __launch_bounds__(kScoreWaves * kWave) void score_pages_kernel(
    const float* __restrict__ q, const T* __restrict__ meta,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens, int hkv,
    int max_pages, int chunks_per_unit, float* __restrict__ scores) {
  using C = ScoreCfg<T, D>;
  using L = typename C::L;
  constexpr int V = L::kVec;
  constexpr int LPR = L::kLanesPerRow;

  const int unit = blockIdx.x / chunks_per_unit;  // b * hkv + g
  const int chunk = blockIdx.x % chunks_per_unit;
  const int b = unit / hkv;
  const int g = unit % hkv;
  const int np = ceil_div(seq_lens[b], kPage);
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int p0 = chunk * C::kPagesPerBlock + wave * C::kPagesPerWave;
  if (p0 >= np) return;  // uniform per wavefront
  const int slot = lane / LPR;
  const int c = lane % LPR;

  // Issue every metadata load of this wavefront first.
  uint4 vmax[kScoreIters], vmin[kScoreIters];
#pragma unroll
  for (int it = 0; it < kScoreIters; ++it) {
    const int p = p0 + it * C::kPagesPerLoad + slot;
    if (p < np) {
      const int phys = page_table[(int64_t)b * max_pages + p];
      const T* src = meta + ((int64_t)phys * hkv + g) * 2 * D + c * V;
      vmax[it] = ld16(src);
      vmin[it] = ld16(src + D);
    } else {
      vmax[it] = make_uint4(0, 0, 0, 0);
      vmin[it] = make_uint4(0, 0, 0, 0);
    }
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

  float* out = scores + (int64_t)unit * max_pages;
#pragma unroll
  for (int it = 0; it < kScoreIters; ++it) {
    float kx[V], kn[V];
    unpack(vmax[it], kx);
    unpack(vmin[it], kn);
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
    const int p = p0 + it * C::kPagesPerLoad + slot;
    if (c == 0 && p < np) out[p] = best;
  }
}

hipError_t launch_score_pages(const Shape& s, const float* q, const void* meta,
                              const int32_t* page_table, const int32_t* seq_lens, float* scores,
                              hipStream_t st) {
  const dim3 block(kScoreWaves * kWave);
  PS_WITH_KV(s.kv_bf16, s.head_dim, {
    const int per_block = ScoreCfg<TElem, kD>::kPagesPerBlock;
    const int chunks = (s.max_pages + per_block - 1) / per_block;
    const int64_t blocks = (int64_t)chunks * s.batch * s.hkv;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks);
    PS_WITH_GROUP(s.group, {
      hipLaunchKernelGGL((score_pages_kernel<TElem, kD, kG>), grid, block, 0, st, q,
                         static_cast<const TElem*>(meta), page_table, seq_lens, s.hkv,
                         s.max_pages, chunks, scores);
    });
  });
  return hipGetLastError();
}

}  // namespace ps
