// C ABI of the pagesparse library: host-side validation, overflow-checked
// sizing and dispatch to the kernel launchers. Every check here runs before
// any HIP call, so a rejected call enqueues nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <initializer_list>

#include "pagesparse.h"
#include "ps_device.h"
#include "ps_launch.h"

#define PS_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kMaxGroup = 8;
constexpr int kMaxSplits = 4096;

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

// Overflow-checked product of positive factors.
bool prod_ok(std::initializer_list<int64_t> xs, int64_t* out) {
  int64_t acc = 1;
  for (int64_t x : xs) {
    if (!mul_ok(acc, x, &acc)) return false;
  }
  *out = acc;
  return true;
}

int check_geom(const ps_geom* g, ps::Shape* s) {
  if (!g) return PS_ERR_NULL;
  if (g->meta_format != PS_META_KV && g->meta_format != PS_META_FP8_E4M3) return PS_ERR_SHAPE;
  if (g->meta_layout != PS_META_PHYSICAL && g->meta_layout != PS_META_LOGICAL)
    return PS_ERR_SHAPE;
  if (g->batch < 0 || g->num_q_heads < 1 || g->num_kv_heads < 1 || g->head_dim < 1 ||
      g->page_size < 1 || g->max_pages < 1 || g->num_phys_pages < 1)
    return PS_ERR_SHAPE;
  if (g->num_q_heads % g->num_kv_heads != 0) return PS_ERR_SHAPE;
  const int group = g->num_q_heads / g->num_kv_heads;
  if (group > kMaxGroup) return PS_ERR_UNSUPPORTED;
  if (g->head_dim != 64 && g->head_dim != 128) return PS_ERR_UNSUPPORTED;
  if (g->page_size != ps::kPage) return PS_ERR_UNSUPPORTED;
  if (g->kv_dtype != PS_F32 && g->kv_dtype != PS_BF16) return PS_ERR_UNSUPPORTED;
  const int64_t elem = g->kv_dtype == PS_BF16 ? 2 : 4;
  int64_t t;
  // token positions p * page_size and page counts stay inside int32
  if (!prod_ok({g->max_pages, g->page_size}, &t) || t > INT32_MAX) return PS_ERR_OVERFLOW;
  // pool bytes, metadata bytes, per-request page-table, score and query sizes
  if (!prod_ok({g->num_phys_pages, g->num_kv_heads, g->page_size, g->head_dim, elem}, &t))
    return PS_ERR_OVERFLOW;
  // logical-layout metadata [B, Hkv, max_pages, 2, D]
  if (g->meta_layout == PS_META_LOGICAL &&
      !prod_ok({g->batch, g->num_kv_heads, g->max_pages, 2, g->head_dim, elem}, &t))
    return PS_ERR_OVERFLOW;
  if (!prod_ok({g->batch, g->max_pages}, &t)) return PS_ERR_OVERFLOW;
  if (!prod_ok({g->batch, g->num_kv_heads, g->max_pages, 4}, &t)) return PS_ERR_OVERFLOW;
  if (!prod_ok({g->max_pages, g->num_kv_heads}, &t) || t > INT32_MAX) return PS_ERR_OVERFLOW;
  if (!prod_ok({g->batch, g->num_q_heads, g->head_dim, 4}, &t)) return PS_ERR_OVERFLOW;
  if (g->num_phys_pages > INT32_MAX) return PS_ERR_OVERFLOW;  // page ids are int32
  s->batch = g->batch;
  s->hq = g->num_q_heads;
  s->hkv = g->num_kv_heads;
  s->group = group;
  s->head_dim = g->head_dim;
  s->max_pages = g->max_pages;
  s->num_phys_pages = g->num_phys_pages;
  s->kv_bf16 = g->kv_dtype == PS_BF16;
  s->meta8 = g->meta_format == PS_META_FP8_E4M3;
  s->meta_logical = g->meta_layout == PS_META_LOGICAL;
  return PS_OK;
}

int check_partials(const ps::Shape& s, int n_splits) {
  int64_t t;
  if (!prod_ok({s.batch, s.hq, n_splits, s.head_dim, 4}, &t)) return PS_ERR_OVERFLOW;
  if (!prod_ok({s.batch, s.hkv, n_splits}, &t) || t > INT32_MAX) return PS_ERR_OVERFLOW;
  return PS_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? PS_OK : PS_ERR_HIP; }

}  // namespace

PS_API int ps_build_page_meta(const ps_geom* geom, const void* k_pool, const int32_t* page_table,
                              const int32_t* seq_lens, const int32_t* page_begin, int32_t n_pages,
                              void* meta, void* stream) {
  ps::Shape s;
  int rc = check_geom(geom, &s);
  if (rc) return rc;
  if (!k_pool || !page_table || !seq_lens || !meta) return PS_ERR_NULL;
  if (n_pages < 1) return PS_ERR_SHAPE;
  if (s.batch == 0) return PS_OK;
  return hip_status(ps::launch_build_page_meta(s, k_pool, page_table, seq_lens, page_begin,
                                               n_pages, meta, (hipStream_t)stream));
}

PS_API int ps_score_pages(const ps_geom* geom, const float* q, const void* meta,
                          const int32_t* page_table, const int32_t* seq_lens, float* scores,
                          void* stream) {
  ps::Shape s;
  int rc = check_geom(geom, &s);
  if (rc) return rc;
  if (!q || !meta || !page_table || !seq_lens || !scores) return PS_ERR_NULL;
  if (s.batch == 0) return PS_OK;
  return hip_status(
      ps::launch_score_pages(s, q, meta, page_table, seq_lens, scores, nullptr, nullptr,
                             (hipStream_t)stream));
}

PS_API int ps_refresh_score_pages(const ps_geom* geom, const float* q, const void* k_pool,
                                  void* meta, const int32_t* page_table,
                                  const int32_t* seq_lens, float* scores, void* stream) {
  ps::Shape s;
  int rc = check_geom(geom, &s);
  if (rc) return rc;
  if (!q || !k_pool || !meta || !page_table || !seq_lens || !scores) return PS_ERR_NULL;
  if (s.batch == 0) return PS_OK;
  return hip_status(ps::launch_score_pages(s, q, meta, page_table, seq_lens, scores, k_pool, meta,
                                           (hipStream_t)stream));
}

PS_API int ps_select_topk(const ps_geom* geom, const float* scores, const int32_t* seq_lens,
                          int32_t budget_pages, int32_t n_sink_pages, int32_t n_local_pages,
                          int32_t* sel, int32_t* sel_count, void* stream) {
  ps::Shape s;
  int rc = check_geom(geom, &s);
  if (rc) return rc;
  if (!scores || !seq_lens || !sel || !sel_count) return PS_ERR_NULL;
  if (budget_pages < 1 || n_sink_pages < 0 || n_local_pages < 0) return PS_ERR_BUDGET;
  if ((int64_t)n_sink_pages + n_local_pages > budget_pages) return PS_ERR_BUDGET;
  if (s.max_pages > ps::kSelectMaxPages) return PS_ERR_UNSUPPORTED;
  int64_t t;
  if (!prod_ok({s.batch, s.hkv, budget_pages, 4}, &t)) return PS_ERR_OVERFLOW;
  if (s.batch == 0) return PS_OK;
  return hip_status(ps::launch_select_topk(s, scores, seq_lens, budget_pages, n_sink_pages,
                                           n_local_pages, sel, sel_count, (hipStream_t)stream));
}

PS_API int ps_select_topdelta(const ps_geom* geom, const float* q, const void* k_pool,
                              const int32_t* page_table, const int32_t* seq_lens,
                              const float* scores, int32_t budget_pages, int32_t n_sink_pages,
                              int32_t n_local_pages, float scale, float delta, int32_t* sel,
                              int32_t* sel_count, void* stream) {
  ps::Shape s;
  int rc = check_geom(geom, &s);
  if (rc) return rc;
  if (!q || !k_pool || !page_table || !seq_lens || !scores || !sel || !sel_count)
    return PS_ERR_NULL;
  if (budget_pages < 1 || n_sink_pages < 0 || n_local_pages < 0) return PS_ERR_BUDGET;
  if ((int64_t)n_sink_pages + n_local_pages > budget_pages) return PS_ERR_BUDGET;
  if (!(delta >= 0.0f) || !(scale > 0.0f) || !(scale < INFINITY)) return PS_ERR_BUDGET;
  if (s.max_pages > ps::kSelectMaxPages) return PS_ERR_UNSUPPORTED;
  int64_t t;
  if (!prod_ok({s.batch, s.hkv, budget_pages, 4}, &t)) return PS_ERR_OVERFLOW;
  if (s.batch == 0) return PS_OK;
  return hip_status(ps::launch_select_topdelta(s, q, k_pool, page_table, scores, seq_lens,
                                               budget_pages, n_sink_pages, n_local_pages, scale,
                                               delta, sel, sel_count, (hipStream_t)stream));
}

PS_API int ps_sparse_decode(const ps_geom* geom, const float* q, const void* k_pool,
                            const void* v_pool, const int32_t* page_table,
                            const int32_t* seq_lens, const int32_t* sel,
                            const int32_t* sel_count, int32_t budget_pages, float scale,
                            int32_t n_splits, float* part_acc, float* part_ml, void* stream) {
  ps::Shape s;
  int rc = check_geom(geom, &s);
  if (rc) return rc;
  if (!q || !k_pool || !v_pool || !page_table || !seq_lens || !sel || !sel_count || !part_acc ||
      !part_ml)
    return PS_ERR_NULL;
  if (budget_pages < 1) return PS_ERR_BUDGET;
  if (n_splits < 1 || n_splits > budget_pages || n_splits > kMaxSplits) return PS_ERR_BUDGET;
  int64_t t;
  if (!prod_ok({s.batch, s.hkv, budget_pages, 4}, &t)) return PS_ERR_OVERFLOW;
  rc = check_partials(s, n_splits);
  if (rc) return rc;
  if (s.batch == 0) return PS_OK;
  return hip_status(ps::launch_decode(s, true, q, k_pool, v_pool, page_table, seq_lens, sel,
                                      sel_count, budget_pages, scale, n_splits, part_acc,
                                      part_ml, (hipStream_t)stream));
}

// Host checks shared by the two selecting decodes.
static int check_select_decode(const ps_geom* geom, ps::Shape* s, const float* q,
                               const void* k_pool, const void* v_pool,
                               const int32_t* page_table, const int32_t* seq_lens,
                               const float* scores, int32_t budget_pages, int32_t n_sink_pages,
                               int32_t n_local_pages, int32_t n_splits, const int32_t* sel,
                               const int32_t* sel_count, const float* part_acc,
                               const float* part_ml, const float* sink, const float* out,
                               const float* lse, const int32_t* arrivals) {
  int rc = check_geom(geom, s);
  if (rc) return rc;
  if (!q || !k_pool || !v_pool || !page_table || !seq_lens || !scores) return PS_ERR_NULL;
  if ((sel == nullptr) != (sel_count == nullptr)) return PS_ERR_NULL;
  if ((!out || n_splits > 1) && (!part_acc || !part_ml)) return PS_ERR_NULL;
  if (budget_pages < 1 || n_sink_pages < 0 || n_local_pages < 0) return PS_ERR_BUDGET;
  if ((int64_t)n_sink_pages + n_local_pages > budget_pages) return PS_ERR_BUDGET;
  if (n_splits < 1 || n_splits > budget_pages || n_splits > kMaxSplits) return PS_ERR_BUDGET;
  if (out ? (n_splits != 1 && !arrivals) : (sink || lse || arrivals)) return PS_ERR_BUDGET;
  if (s->max_pages > ps::kSelectDecodeMaxPages ||
      (budget_pages + n_splits - 1) / n_splits > ps::kMaxSplitPages)
    return PS_ERR_UNSUPPORTED;
  int64_t t;
  if (!prod_ok({s->batch, s->hkv, budget_pages, 4}, &t)) return PS_ERR_OVERFLOW;
  return check_partials(*s, n_splits);
}

PS_API int ps_select_sparse_decode(const ps_geom* geom, const float* q, const void* k_pool,
                                   const void* v_pool, const int32_t* page_table,
                                   const int32_t* seq_lens, const float* scores,
                                   int32_t budget_pages, int32_t n_sink_pages,
                                   int32_t n_local_pages, float scale, int32_t n_splits,
                                   int32_t* sel, int32_t* sel_count, float* part_acc,
                                   float* part_ml, const float* sink, float* out, float* lse,
                                   int32_t* arrivals, void* stream) {
  ps::Shape s;
  const int rc = check_select_decode(geom, &s, q, k_pool, v_pool, page_table, seq_lens, scores,
                                     budget_pages, n_sink_pages, n_local_pages, n_splits, sel,
                                     sel_count, part_acc, part_ml, sink, out, lse, arrivals);
  if (rc) return rc;
  if (s.batch == 0) return PS_OK;
  return hip_status(ps::launch_select_decode(s, q, k_pool, v_pool, page_table, seq_lens, scores,
                                             budget_pages, n_sink_pages, n_local_pages, scale,
                                             n_splits, sel, sel_count, part_acc, part_ml, sink,
                                             out, lse, arrivals, (hipStream_t)stream));
}

PS_API int ps_select_sparse_decode_noalloc(const ps_geom* geom, const float* q,
                                           const void* k_pool, const void* v_pool,
                                           const int32_t* page_table, const int32_t* seq_lens,
                                           const float* scores, int32_t budget_pages,
                                           int32_t n_sink_pages, int32_t n_local_pages,
                                           float scale, int32_t n_splits, int32_t* sel,
                                           int32_t* sel_count, const float* sink, float* out,
                                           float* lse, void* stream) {
  ps::Shape s;
  // the workspace stands in for the caller's partials and counters in the
  // checks they share with ps_select_sparse_decode
  const float* ws = reinterpret_cast<const float*>(out);
  int rc = check_select_decode(geom, &s, q, k_pool, v_pool, page_table, seq_lens, scores,
                               budget_pages, n_sink_pages, n_local_pages, n_splits, sel,
                               sel_count, ws, ws, sink, out, lse,
                               reinterpret_cast<const int32_t*>(out));
  if (rc) return rc;
  if (!out) return PS_ERR_NULL;
  const int64_t need = ps::noalloc_scratch_bytes(s, n_splits);
  if (need < 0 || need > ps::kNoAllocScratchBytes) return PS_ERR_WORKSPACE;
  if (s.batch == 0) return PS_OK;
  return hip_status(ps::launch_select_decode_noalloc(
      s, q, k_pool, v_pool, page_table, seq_lens, scores, budget_pages, n_sink_pages,
      n_local_pages, scale, n_splits, sel, sel_count, sink, out, lse, (hipStream_t)stream));
}

PS_API int ps_select_topdelta_sparse_decode(const ps_geom* geom, const float* q,
                                            const void* k_pool, const void* v_pool,
                                            const int32_t* page_table, const int32_t* seq_lens,
                                            const float* scores, int32_t budget_pages,
                                            int32_t n_sink_pages, int32_t n_local_pages,
                                            float scale, float delta, int32_t n_splits,
                                            int32_t* sel, int32_t* sel_count, float* part_acc,
                                            float* part_ml, const float* sink, float* out,
                                            float* lse, int32_t* arrivals, void* stream) {
  ps::Shape s;
  const int rc = check_select_decode(geom, &s, q, k_pool, v_pool, page_table, seq_lens, scores,
                                     budget_pages, n_sink_pages, n_local_pages, n_splits, sel,
                                     sel_count, part_acc, part_ml, sink, out, lse, arrivals);
  if (rc) return rc;
  if (!(delta >= 0.0f) || !(scale > 0.0f) || !(scale < INFINITY)) return PS_ERR_BUDGET;
  if (s.batch == 0) return PS_OK;
  return hip_status(ps::launch_select_topdelta_decode(
      s, q, k_pool, v_pool, page_table, seq_lens, scores, budget_pages, n_sink_pages,
      n_local_pages, scale, delta, n_splits, sel, sel_count, part_acc, part_ml, sink, out, lse,
      arrivals, (hipStream_t)stream));
}

PS_API int ps_full_decode(const ps_geom* geom, const float* q, const void* k_pool,
                          const void* v_pool, const int32_t* page_table, const int32_t* seq_lens,
                          float scale, int32_t n_splits, float* part_acc, float* part_ml,
                          void* stream) {
  ps::Shape s;
  int rc = check_geom(geom, &s);
  if (rc) return rc;
  if (!q || !k_pool || !v_pool || !page_table || !seq_lens || !part_acc || !part_ml)
    return PS_ERR_NULL;
  if (n_splits < 1 || n_splits > s.max_pages || n_splits > kMaxSplits) return PS_ERR_BUDGET;
  rc = check_partials(s, n_splits);
  if (rc) return rc;
  if (s.batch == 0) return PS_OK;
  return hip_status(ps::launch_decode(s, false, q, k_pool, v_pool, page_table, seq_lens, nullptr,
                                      nullptr, 0, scale, n_splits, part_acc, part_ml,
                                      (hipStream_t)stream));
}

PS_API int ps_combine(const ps_geom* geom, const float* part_acc, const float* part_ml,
                      int32_t n_splits, const float* sink, float* out, float* lse, void* stream) {
  ps::Shape s;
  int rc = check_geom(geom, &s);
  if (rc) return rc;
  if (!part_acc || !part_ml || !out) return PS_ERR_NULL;
  if (n_splits < 1 || n_splits > kMaxSplits) return PS_ERR_BUDGET;
  rc = check_partials(s, n_splits);
  if (rc) return rc;
  if (s.batch == 0) return PS_OK;
  return hip_status(ps::launch_combine(s, part_acc, part_ml, n_splits, sink, out, lse,
                                       (hipStream_t)stream));
}

PS_API const char* ps_strerror(int status) {
  switch (status) {
    case PS_OK: return "PS_OK: enqueued";
    case PS_ERR_NULL: return "PS_ERR_NULL: a required pointer is NULL";
    case PS_ERR_SHAPE: return "PS_ERR_SHAPE: inconsistent or out-of-range dimension";
    case PS_ERR_UNSUPPORTED: return "PS_ERR_UNSUPPORTED: shape or dtype not implemented";
    case PS_ERR_OVERFLOW: return "PS_ERR_OVERFLOW: a size computation overflows";
    case PS_ERR_BUDGET: return "PS_ERR_BUDGET: budget, forced-page or split arguments invalid";
    case PS_ERR_HIP: return "PS_ERR_HIP: the HIP runtime reported a launch error";
    case PS_ERR_WORKSPACE:
      return "PS_ERR_WORKSPACE: the call needs more than the library's fixed workspace";
    default: return "unknown ps_status";
  }
}

PS_API int ps_abi_version(void) { return (2 << 16) | 0; }  // 2.0: ps_geom.meta_layout
