// Page metadata: elementwise max and min of the valid keys of each page.
// ("Don't read the haystack", section "Part two: the skipping".)
//
// One wavefront per (request, logical page, KV head) folds the page
// (PageFold), and two lane groups write the kmax and kmin rows: in the key
// dtype, or as 8-bit codes with kmax rounded up and kmin rounded down
// (fp8_e4m3_directed). The rows go to the physical page's slot
// [phys, g] or to the request's logical slot [b, g, p].
#include "ps_launch.h"
#include "ps_meta.h"

namespace ps {

constexpr int kMetaWaves = 4;

template <typename T, int D, bool META8>
__global__ __launch_bounds__(kMetaWaves * kWave) void build_page_meta_kernel(
    const T* __restrict__ k_pool, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ page_begin, int n_pages,
    int batch, int hkv, int max_pages, int items_per_req, int logical, void* __restrict__ meta) {
  using L = RowLayout<T, D>;
  constexpr int V = L::kVec;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int64_t flat = (int64_t)blockIdx.x * kMetaWaves + wave;
  if (flat >= (int64_t)items_per_req * batch) return;  // tail of the last block
  const int b = (int)(flat / items_per_req);
  const int item = (int)(flat % items_per_req);

  const int len = seq_lens[b];
  const int np = ceil_div(len, kPage);
  const int64_t begin = page_begin ? page_begin[b] : 0;
  const int64_t end = begin + n_pages < np ? begin + n_pages : np;
  const int64_t p = begin + item / hkv;
  const int g = item % hkv;
  if (p >= end) return;  // uniform per wavefront

  const int phys = page_table[(int64_t)b * max_pages + p];
  const int cnt = min(kPage, len - (int)p * kPage);
  const int r0 = lane / L::kLanesPerRow;
  const int c = lane % L::kLanesPerRow;
  PageFold<T, D> pf;
  pf.load(k_pool + ((int64_t)phys * hkv + g) * kPage * D, lane);
  float mx[V], mn[V];
  pf.fold(cnt, lane, mx, mn);
  if (r0 < 2) {
    const int64_t slot = logical ? ((int64_t)b * hkv + g) * max_pages + p
                                 : (int64_t)phys * hkv + g;
    const int64_t off = slot * 2 * D + r0 * D + c * V;
    if constexpr (META8 && V == 8) {
      *reinterpret_cast<uint2*>(static_cast<uint8_t*>(meta) + off) =
          r0 == 0 ? fp8_pack8(mx, true) : fp8_pack8(mn, false);
    } else if constexpr (META8) {
      *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(meta) + off) =
          r0 == 0 ? fp8_pack4(mx, true) : fp8_pack4(mn, false);
    } else {
      st16(static_cast<T*>(meta) + off, r0 == 0 ? pack(mx) : pack(mn));
    }
  }
}

hipError_t launch_build_page_meta(const Shape& s, const void* k_pool, const int32_t* page_table,
                                  const int32_t* seq_lens, const int32_t* page_begin,
                                  int n_pages, void* meta, hipStream_t st) {
  const int pages = n_pages < s.max_pages ? n_pages : s.max_pages;
  const int items_per_req = pages * s.hkv;
  const int64_t waves = (int64_t)items_per_req * s.batch;
  const int64_t blocks = (waves + kMetaWaves - 1) / kMetaWaves;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)blocks), block(kMetaWaves * kWave);
  if (s.meta8) {
    PS_WITH_KV(s.kv_bf16, s.head_dim, {
      hipLaunchKernelGGL((build_page_meta_kernel<TElem, kD, true>), grid, block, 0, st,
                         static_cast<const TElem*>(k_pool), page_table, seq_lens, page_begin,
                         pages, s.batch, s.hkv, s.max_pages, items_per_req, s.meta_logical,
                         meta);
    });
    return hipGetLastError();
  }
  PS_WITH_KV(s.kv_bf16, s.head_dim, {
    hipLaunchKernelGGL((build_page_meta_kernel<TElem, kD, false>), grid, block, 0, st,
                       static_cast<const TElem*>(k_pool), page_table, seq_lens, page_begin,
                       pages, s.batch, s.hkv, s.max_pages, items_per_req, s.meta_logical,
                         meta);
  });
  return hipGetLastError();
}

}  // namespace ps
