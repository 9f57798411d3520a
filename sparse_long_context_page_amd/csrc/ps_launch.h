// Host-side launchers of the pagesparse kernels. Arguments reaching these
// functions have already been validated by the C ABI layer (ps_api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ps {

struct Shape {
  int batch, hq, hkv, group, head_dim, max_pages;
  int64_t num_phys_pages;
  int kv_bf16;  // 1: bf16 pools, 0: fp32 pools
  int meta8;    // 1: 8-bit metadata bounds, 0: metadata in the pool dtype
  int meta_logical;  // 1: metadata [B, Hkv, max_pages, 2, D], 0: [P_phys, Hkv, 2, D]
};

hipError_t launch_build_page_meta(const Shape& s, const void* k_pool, const int32_t* page_table,
                                  const int32_t* seq_lens, const int32_t* page_begin,
                                  int n_pages, void* meta, hipStream_t st);

// k_pool and meta_out non-null: also rebuild each request's last page's
// metadata from k_pool into meta_out before scoring it.
hipError_t launch_score_pages(const Shape& s, const float* q, const void* meta,
                              const int32_t* page_table, const int32_t* seq_lens, float* scores,
                              const void* k_pool, void* meta_out, hipStream_t st);

// Largest max_pages the selection kernel holds in registers (1M tokens).
constexpr int kSelectMaxPages = 65536;
// Largest max_pages, and list slots per split, of the decode that makes its
// own selection (a workgroup of 256 threads holds the scores in registers,
// 32 per lane: 128k tokens).
constexpr int kSelectDecodeMaxPages = 8192;
constexpr int kMaxSplitPages = 512;

hipError_t launch_select_topk(const Shape& s, const float* scores, const int32_t* seq_lens,
                              int budget, int n_sink, int n_local, int32_t* sel,
                              int32_t* sel_count, hipStream_t st);

hipError_t launch_select_topdelta(const Shape& s, const float* q, const void* k_pool,
                                  const int32_t* page_table, const float* scores,
                                  const int32_t* seq_lens, int budget, int n_sink, int n_local,
                                  float scale, float delta, int32_t* sel, int32_t* sel_count,
                                  hipStream_t st);

hipError_t launch_select_decode(const Shape& s, const float* q, const void* k_pool,
                                const void* v_pool, const int32_t* page_table,
                                const int32_t* seq_lens, const float* scores, int budget,
                                int n_sink, int n_local, float scale, int n_splits, int32_t* sel,
                                int32_t* sel_count, float* part_acc, float* part_ml,
                                const float* sink, float* out, float* lse, int32_t* arrivals,
                                hipStream_t st);

// Fixed size of the library's own workspace array (ps_noalloc.hip), and the
// bytes a scratch-backed selecting decode of this shape needs in it.
constexpr int64_t kNoAllocScratchBytes = int64_t(8) << 20;
constexpr int64_t scratch_align(int64_t x) { return (x + 255) & ~int64_t(255); }
// Scratch layout: arrivals [B, Hkv] int32, then part_ml [B, Hq, S, 2] and
// part_acc [B, Hq, S, D] fp32, each at a 256-byte boundary. -1 when a size
// does not fit in 64 bits (the caller validated the geometry first).
inline int64_t noalloc_scratch_bytes(const Shape& s, int n_splits) {
  const int64_t units = (int64_t)s.batch * s.hkv;
  const int64_t rows = (int64_t)s.batch * s.hq * n_splits;
  if (units < 0 || rows < 0 || rows > (INT64_MAX / 4) / (s.head_dim + 2)) return -1;
  return scratch_align(units * 4) + scratch_align(rows * 2 * 4) +
         scratch_align(rows * s.head_dim * 4);
}

// launch_select_decode with the partials and arrival counters in that array
// (the merged output is always written).
hipError_t launch_select_decode_noalloc(const Shape& s, const float* q, const void* k_pool,
                                        const void* v_pool, const int32_t* page_table,
                                        const int32_t* seq_lens, const float* scores,
                                        int budget, int n_sink, int n_local, float scale,
                                        int n_splits, int32_t* sel, int32_t* sel_count,
                                        const float* sink, float* out, float* lse,
                                        hipStream_t st);

hipError_t launch_select_topdelta_decode(const Shape& s, const float* q, const void* k_pool,
                                         const void* v_pool, const int32_t* page_table,
                                         const int32_t* seq_lens, const float* scores,
                                         int budget, int n_sink, int n_local, float scale,
                                         float delta, int n_splits, int32_t* sel,
                                         int32_t* sel_count, float* part_acc, float* part_ml,
                                         const float* sink, float* out, float* lse,
                                         int32_t* arrivals, hipStream_t st);

hipError_t launch_decode(const Shape& s, bool sparse, const float* q, const void* k_pool,
                         const void* v_pool, const int32_t* page_table, const int32_t* seq_lens,
                         const int32_t* sel, const int32_t* sel_count, int budget, float scale,
                         int n_splits, float* part_acc, float* part_ml, hipStream_t st);

hipError_t launch_combine(const Shape& s, const float* part_acc, const float* part_ml,
                          int n_splits, const float* sink, float* out, float* lse,
                          hipStream_t st);

}  // namespace ps

// Instantiate BODY with a compile-time group size kG in [1, 8].
#define PS_WITH_GROUP(G, ...)                  \
  switch (G) {                                 \
    case 1: { constexpr int kG = 1; __VA_ARGS__; } break; \
    case 2: { constexpr int kG = 2; __VA_ARGS__; } break; \
    case 3: { constexpr int kG = 3; __VA_ARGS__; } break; \
    case 4: { constexpr int kG = 4; __VA_ARGS__; } break; \
    case 5: { constexpr int kG = 5; __VA_ARGS__; } break; \
    case 6: { constexpr int kG = 6; __VA_ARGS__; } break; \
    case 7: { constexpr int kG = 7; __VA_ARGS__; } break; \
    case 8: { constexpr int kG = 8; __VA_ARGS__; } break; \
    default: return hipErrorInvalidValue;      \
  }

// Instantiate BODY with element type TElem and head dimension kD.
#define PS_WITH_KV(BF16, D, ...)                                          \
  if (BF16) {                                                             \
    using TElem = ::ps::bf16_t;                                           \
    if ((D) == 64) { constexpr int kD = 64; __VA_ARGS__; }                \
    else { constexpr int kD = 128; __VA_ARGS__; }                         \
  } else {                                                                \
    using TElem = float;                                                  \
    if ((D) == 64) { constexpr int kD = 64; __VA_ARGS__; }                \
    else { constexpr int kD = 128; __VA_ARGS__; }                         \
  }
