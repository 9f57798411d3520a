/*
 * pagesparse.h -- C ABI of page-selected sparse decode attention for AMD
 * Instinct MI355X (gfx950).
 *
 * One decode step for a batch of requests whose keys and values live in a
 * paged cache:
 *   1. ps_build_page_meta  per-page elementwise key max/min   (metadata)
 *   2. ps_score_pages      per-page upper bound of q.k         (page score)
 *   3. ps_select_topk      forced pages + top-k per KV head    (selection)
 *      ps_select_topdelta  the same, kept pages also above a threshold
 *   4. ps_sparse_decode    split-KV softmax partials over the kept pages
 *      ps_full_decode      the same over every page            (dense twin)
 *   5. ps_combine          log-sum-exp merge of the partials + optional sink
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer except `geom` is a DEVICE pointer owned by the caller, to a
 *   contiguous row-major array laid out as documented. The library allocates
 *   nothing, never synchronises and enqueues work only on `stream` (a
 *   hipStream_t; NULL means the null stream). The calls are therefore safe
 *   to capture into a HIP graph. No call keeps state between calls except
 *   ps_select_sparse_decode_noalloc, whose workspace is one fixed device
 *   array of the library per GPU (see there).
 * - The return value is a ps_status. PS_OK means the work was enqueued.
 *   Arguments are validated on the host BEFORE any HIP call; a failed
 *   validation returns its code and enqueues nothing. Device-resident values
 *   (seq_lens, page_table, sel) cannot be checked without a synchronisation,
 *   so their preconditions are documented per call and are the caller's
 *   responsibility. PS_ERR_HIP reports a launch failure.
 * - Sizes are computed with overflow-checked 64-bit arithmetic; a product that
 *   would overflow returns PS_ERR_OVERFLOW (never a saturated size).
 *   ("perf(core): fused sparse-attention decode via page indirection - #1005",
 *   commit "gate fused sparse decode on sparsity": checked, not saturating,
 *   multiplication.)
 * - Query head h belongs to KV head h / (num_q_heads / num_kv_heads).
 * - A request b holds seq_lens[b] >= 1 tokens on n_b = ceil(seq_lens[b] /
 *   page_size) logical pages; logical page p holds tokens
 *   [p*page_size, min((p+1)*page_size, seq_lens[b])). Only those tokens are
 *   read as data; the unused slots of a partial last page are never used.
 */
#ifndef PAGESPARSE_H
#define PAGESPARSE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PS_OK = 0,
  PS_ERR_NULL = -1,        /* a required pointer is NULL                          */
  PS_ERR_SHAPE = -2,       /* an inconsistent or out-of-range dimension          */
  PS_ERR_UNSUPPORTED = -3, /* a valid shape the library does not implement       */
  PS_ERR_OVERFLOW = -4,    /* a size computation overflows 64 bits / int32 index */
  PS_ERR_BUDGET = -5,      /* budget, forced-page or split arguments inconsistent */
  PS_ERR_HIP = -6,         /* the HIP runtime reported an error at launch        */
  PS_ERR_WORKSPACE = -7    /* needs more than the library's fixed workspace       */
} ps_status;

typedef enum {
  PS_F32 = 0,  /* IEEE binary32                                          */
  PS_BF16 = 1  /* bfloat16 (the high 16 bits of a binary32), RNE-rounded */
} ps_dtype;

/* Element type of the metadata pool.
 *   PS_META_KV        kmax and kmin in kv_dtype (exact).
 *   PS_META_FP8_E4M3  8-bit bounds (bf16 or fp32 pools): kmax rounded up and
 *                     kmin rounded down to OCP E4M3 (no infinities; bias 7;
 *                     largest finite 448), so for every query the bound can
 *                     only grow and stays an upper bound of q.k. The page
 *                     score then reads half the metadata bytes. A zero bound
 *                     is code 0x00. Requires |K| <= 448: a larger magnitude
 *                     saturates to 448 and its bound is no longer admissible.
 *   ("Faster Than Flash: Exploiting Attention Sparsity for Efficient
 *   Long-Context Decoding", section "Methodology", item 1: the scan that
 *   decides which blocks to read runs on a low-bit copy of the cache.) */
typedef enum {
  PS_META_KV = 0,
  PS_META_FP8_E4M3 = 1
} ps_meta_format;

/* Where a page's metadata lives.
 *   PS_META_PHYSICAL  with the physical page: meta [num_phys_pages, Hkv, 2, D],
 *                     the entry of (b, p) at page_table[b, p] (pages shared
 *                     by several requests share their metadata).
 *   PS_META_LOGICAL   per request, in logical page order: meta
 *                     [B, Hkv, max_pages, 2, D], the entry of (b, g, p) at
 *                     [b, g, p]. The page score then reads the metadata
 *                     without going through the page table (one dependent
 *                     memory round trip fewer before its first page);
 *                     entries at p >= n_b are neither written nor used. A
 *                     page shared by several requests has one entry per
 *                     request. */
typedef enum {
  PS_META_PHYSICAL = 0,
  PS_META_LOGICAL = 1
} ps_meta_layout;

/* Geometry shared by every call of one decode step.
 *   batch           B  >= 0 (0: validate, enqueue nothing, return PS_OK)
 *   num_q_heads     Hq >= 1, a multiple of num_kv_heads, with
 *                   Hq / Hkv (the group size G) in [1, 8]
 *   num_kv_heads    Hkv >= 1
 *   head_dim        D, 64 or 128
 *   page_size       tokens per page, 16
 *   max_pages       row stride of page_table; >= n_b for every request
 *   num_phys_pages  rows of the K, V and metadata pools (>= 1)
 *   kv_dtype        element type of K and V
 *   meta_format     element type of the metadata (ps_meta_format); entry
 *                   points that do not read metadata ignore it. A value
 *                   outside ps_meta_format is PS_ERR_SHAPE in every entry
 *                   point
 *   meta_layout     where the metadata of a page lives (ps_meta_layout);
 *                   a value outside it is PS_ERR_SHAPE in every entry point */
typedef struct {
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t max_pages;
  int64_t num_phys_pages;
  int32_t kv_dtype;    /* ps_dtype */
  int32_t meta_format; /* ps_meta_format */
  int32_t meta_layout; /* ps_meta_layout */
} ps_geom;

/* Array layouts (all contiguous, row-major):
 *   k_pool, v_pool [num_phys_pages, Hkv, page_size, D]    kv_dtype
 *   meta           [num_phys_pages, Hkv, 2, D] (PS_META_PHYSICAL) or
 *                  [B, Hkv, max_pages, 2, D] (PS_META_LOGICAL)
 *                                                          kv_dtype (PS_META_KV) or uint8 codes
 *                                                          (PS_META_FP8_E4M3); [..,0,:] = kmax,
 *                                                          [..,1,:] = kmin
 *   page_table     [B, max_pages]  int32, logical page -> physical page; entries
 *                  at p >= n_b are ignored
 *   seq_lens       [B]             int32
 *   q              [B, Hq, D]      float32
 *   scores         [B, Hkv, max_pages]       float32
 *   sel            [B, Hkv, budget_pages]    int32
 *   sel_count      [B, Hkv]                  int32
 *   part_acc       [B, Hq, n_splits, D]      float32
 *   part_ml        [B, Hq, n_splits, 2]      float32  ([..,0] = m, [..,1] = l)
 *   out            [B, Hq, D]      float32
 *   lse            [B, Hq]         float32
 *   sink           [Hq]            float32
 */

/* 1. Page metadata. ("Don't read the haystack", section "Part two: the
 * skipping": each page keeps the elementwise min and max of its keys.)
 * For every request b, KV head g and logical page p in
 * [begin_b, min(begin_b + n_pages, n_b)) with begin_b = page_begin[b] (or 0
 * when page_begin is NULL), with M = meta[page_table[b,p], g] (physical
 * layout) or meta[b, g, p] (logical layout):
 *   M[0, d] = max over the page's valid tokens t of K[t, d]
 *   M[1, d] = min over the same tokens.
 * The result is exact (a selection among stored values); with
 * PS_META_FP8_E4M3 it is kmax rounded up and kmin rounded down to E4M3. Passing
 * page_begin[b] = n_b - 1 and n_pages = 1 refreshes only the tail page, the
 * incremental update of a decode step. Other metadata rows are untouched.
 * n_pages >= 1 (use max_pages for a full build).
 * Device preconditions: 1 <= seq_lens[b] <= max_pages*page_size;
 * 0 <= page_table[b,p] < num_phys_pages for p < n_b; 0 <= page_begin[b];
 * no physical page is mapped by two (b, p) within the rebuilt ranges
 * (physical layout). */
int ps_build_page_meta(const ps_geom* geom, const void* k_pool, const int32_t* page_table,
                       const int32_t* seq_lens, const int32_t* page_begin, int32_t n_pages,
                       void* meta, void* stream);

/* 2. Page score. ("Don't read the haystack", section "Part two: the
 * skipping": the bound sum_d max(q_d*kmin_d, q_d*kmax_d) is at least q.k for
 * every key of the page.) For every b, KV head g and logical page p < n_b:
 *   scores[b,g,p] = max over the group's query heads h of
 *                   sum_d max(q[b,h,d]*kmin_d, q[b,h,d]*kmax_d)
 * with (kmax, kmin) the page's metadata (meta[page_table[b,p], g], or
 * meta[b, g, p] in the logical layout). Unscaled; the max over the
 * group makes one page list per KV head admissible for all its heads.
 * Computed in fp32 as sum_d (max(q,0)*kmax_d + min(q,0)*kmin_d) with exact
 * products and a fixed summation order (bf16 metadata: on the matrix cores,
 * q split exactly into three bf16 terms; fp32 metadata: fma; 8-bit metadata:
 * widened exactly to the pool's dtype, then as that metadata), so results are bitwise
 * reproducible; entries at p >= n_b are not written.
 * Device preconditions: as ps_build_page_meta, with meta built for every
 * page read. */
int ps_score_pages(const ps_geom* geom, const float* q, const void* meta,
                   const int32_t* page_table, const int32_t* seq_lens, float* scores,
                   void* stream);

/* 1+2. The last page's metadata refreshed inside the page score: one launch
 * does the work of ps_build_page_meta with page_begin[b] = n_b - 1 and
 * n_pages = 1, followed by ps_score_pages, with bitwise the same metadata and
 * scores. ("Don't read the haystack", section "Part two: the skipping": the
 * page summaries are maintained incrementally as tokens append; a decode step
 * appends to each request's last page only.) meta is read for every page and
 * written for page n_b - 1 of every request.
 * Host checks: those of ps_score_pages.
 * Device preconditions: as ps_build_page_meta and ps_score_pages; in the
 * physical layout, no two requests share their last physical page. */
int ps_refresh_score_pages(const ps_geom* geom, const float* q, const void* k_pool, void* meta,
                           const int32_t* page_table, const int32_t* seq_lens, float* scores,
                           void* stream);

/* 3. Selection. ("Don't read the haystack", section "Part two: the
 * skipping": keep the top pages by bound plus the sink page and the last
 * local pages; "perf(core): fused sparse-attention decode via page
 * indirection - #1005", section "The reduction...": the kept count is known
 * on the host, so nothing is read back.) For every (b, g), with n = n_b:
 *   if budget_pages >= n: every page 0..n-1 is kept;
 *   else the first n_sink_pages and the last n_local_pages pages are kept and
 *   the remaining budget_pages - n_sink_pages - n_local_pages slots go to the
 *   other pages by decreasing scores[b,g,p], ties to the lower p.
 * sel[b,g,:] lists the kept logical pages in ascending order followed by -1
 * padding; sel_count[b,g] = min(budget_pages, n).
 * Host checks: budget_pages >= 1, n_sink_pages >= 0, n_local_pages >= 0,
 * n_sink_pages + n_local_pages <= budget_pages (else PS_ERR_BUDGET);
 * max_pages <= 65536 (else PS_ERR_UNSUPPORTED).
 * Device precondition: scores are finite (no NaN). */
int ps_select_topk(const ps_geom* geom, const float* scores, const int32_t* seq_lens,
                   int32_t budget_pages, int32_t n_sink_pages, int32_t n_local_pages,
                   int32_t* sel, int32_t* sel_count, void* stream);

/* 3'. Top-delta selection. ("Faster Than Flash: Exploiting Attention
 * Sparsity for Efficient Long-Context Decoding", section "Methodology", item
 * 2, eq. (1)-(3): a block is kept when its logit is at least the maximum
 * minus delta, the maximum replaced by a pseudo-max over the sink and local
 * tokens; "Pseudo-Max Robustness as Fail-Safe": the pseudo-max is never
 * larger, so the kept set only grows.) For every (b, g) with n = n_b:
 *   if budget_pages >= n: every page 0..n-1 is kept (as ps_select_topk);
 *   else, with F the first n_sink_pages and last n_local_pages pages,
 *     m_h = max over the valid tokens t of the pages of F of
 *           scale * q[b,h,:] . K[t, g, :]   for each query head h of g,
 *     tau = min_h m_h - delta  (-infinity when F is empty),
 *   the pages of F and, of the other pages with scale * scores[b,g,p] >= tau,
 *   the best by decreasing score (ties to the lower p), at most
 *   budget_pages - |F| of them, are kept.
 * The logits and the comparison are evaluated in fp64 (exact products).
 * sel and sel_count as ps_select_topk; sel_count[b,g] <= min(budget_pages, n)
 * (fewer pages when few pass the threshold).
 * Host checks: those of ps_select_topk; delta >= 0 (+infinity gives
 * ps_select_topk's selection) and 0 < scale < infinity (else PS_ERR_BUDGET).
 * Device preconditions: those of ps_select_topk and ps_score_pages. */
int ps_select_topdelta(const ps_geom* geom, const float* q, const void* k_pool,
                       const int32_t* page_table, const int32_t* seq_lens, const float* scores,
                       int32_t budget_pages, int32_t n_sink_pages, int32_t n_local_pages,
                       float scale, float delta, int32_t* sel, int32_t* sel_count, void* stream);


/* 4a. Sparse split-KV decode. ("Don't read the haystack", sections "Part one:
 * hitting the wall on purpose" and "Part two: the skipping": the sparse twin
 * of a split-KV flash-decode walks a page list; each split writes its running
 * max, normaliser and unnormalised accumulator in fp32.)
 * Split s of (b, query head h, KV head g) covers the list slots
 * [s*c, min((s+1)*c, sel_count[b,g])) with c = ceil(budget_pages / n_splits),
 * i.e. the pages sel[b,g,slot]. Over the valid tokens t of those pages, with
 * x_t = scale * (q[b,h] . K_t):
 *   part_ml[b,h,s,0] = m = max_t x_t
 *   part_ml[b,h,s,1] = l = sum_t exp(x_t - m)
 *   part_acc[b,h,s,:] =    sum_t exp(x_t - m) V_t
 * An empty split writes (m, l, acc) = (-inf, 0, 0).
 * Host checks: 1 <= n_splits <= budget_pages.
 * Device preconditions: sel_count[b,g] <= budget_pages; each sel entry in
 * [0, sel_count) is a logical page < n_b (any order). */
int ps_sparse_decode(const ps_geom* geom, const float* q, const void* k_pool, const void* v_pool,
                     const int32_t* page_table, const int32_t* seq_lens, const int32_t* sel,
                     const int32_t* sel_count, int32_t budget_pages, float scale,
                     int32_t n_splits, float* part_acc, float* part_ml, void* stream);

/* 3+4a. Selection fused into the sparse decode: one launch does the work of
 * ps_select_topk followed by ps_sparse_decode, with bitwise the same page
 * list and partials. ("Training-free sparse attention for long-context LLM
 * decode", section "Reusable code": a fused single-launch variant of the
 * sparse decode; "Don't read the haystack", section "Part one: hitting the
 * wall on purpose": a decode step of small kernels is bound by launches.)
 * Every split's workgroup selects the (b, g) page list from scores itself
 * and attends the list slots of its split, so no page list is read back.
 * sel and sel_count, when not NULL, receive what ps_select_topk writes.
 * The partials are written as by ps_sparse_decode. With out != NULL the
 * merge happens in the same launch: out and lse (when not NULL) receive what
 * ps_combine writes for these partials with the given sink (NULL = none),
 * bitwise. With one split the single partial is merged directly (part_acc
 * and part_ml are then not used and may be NULL). With more splits,
 * arrivals [B, Hkv] int32 counts the splits of each (b, g) that have
 * written their partials, and the last one to finish merges them ("Attention:
 * Undivided & Uncompressed", section "Traffic": the split-KV merge; here it
 * saves the merge launch). arrivals is device memory owned by the caller:
 * all zero when the launch starts, all zero again when it ends (allocate it
 * zeroed once and reuse it; launches that overlap in time must not share
 * it). Without out, sink, lse and arrivals must be NULL.
 * Host checks: those of ps_select_topk and ps_sparse_decode (same codes);
 * sel and sel_count both NULL or both set, and the partials set unless out
 * is set with one split (else PS_ERR_NULL); out != NULL with n_splits != 1
 * and no arrivals, or sink, lse or arrivals set without out (PS_ERR_BUDGET);
 * max_pages <= 8192 and ceil(budget_pages / n_splits) <= 512 (else
 * PS_ERR_UNSUPPORTED).
 * Device preconditions: scores are finite (no NaN); arrivals as above. */
int ps_select_sparse_decode(const ps_geom* geom, const float* q, const void* k_pool,
                            const void* v_pool, const int32_t* page_table,
                            const int32_t* seq_lens, const float* scores, int32_t budget_pages,
                            int32_t n_sink_pages, int32_t n_local_pages, float scale,
                            int32_t n_splits, int32_t* sel, int32_t* sel_count, float* part_acc,
                            float* part_ml, const float* sink, float* out, float* lse,
                            int32_t* arrivals, void* stream);

/* 3+4a+5 without allocation: ps_select_sparse_decode with out, with the
 * split partials and the arrival counters in a fixed-size device array of
 * the library instead of caller buffers. For callers that cannot allocate
 * or pass workspace: code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc. The caller passes inputs and outputs only;
 * nothing is allocated (no hipMalloc, hipFree or allocating library call).
 * Results are bitwise those of ps_select_sparse_decode with out (sel,
 * sel_count when not NULL, out, lse when not NULL).
 * Workspace: one array of 8 MiB per GPU, held from the library's first use
 * on that GPU until the process ends; its device address is looked up once
 * per device. A call needs 256-byte-aligned room for B*Hkv int32 counters
 * plus B*Hq*n_splits*(D+2) floats of partials (none of the partials with one
 * split); a call needing more returns PS_ERR_WORKSPACE and enqueues nothing.
 * Each call first clears the counters (a small kernel on `stream`, so a
 * captured graph replays it), then launches the decode. Every call on one
 * GPU uses the same array: calls that overlap in time on one GPU (other
 * streams, other threads) race and must be serialised by the caller.
 * Arguments as ps_select_sparse_decode; out is required.
 * Host checks: those of ps_select_sparse_decode with out set (same codes;
 * out NULL is PS_ERR_NULL), then PS_ERR_WORKSPACE as above.
 * Device preconditions: those of ps_select_sparse_decode. */
int ps_select_sparse_decode_noalloc(const ps_geom* geom, const float* q, const void* k_pool,
                                    const void* v_pool, const int32_t* page_table,
                                    const int32_t* seq_lens, const float* scores,
                                    int32_t budget_pages, int32_t n_sink_pages,
                                    int32_t n_local_pages, float scale, int32_t n_splits,
                                    int32_t* sel, int32_t* sel_count, const float* sink,
                                    float* out, float* lse, void* stream);

/* 3'+4a. Top-delta selection fused into the sparse decode: one launch does
 * the work of ps_select_topdelta followed by ps_sparse_decode, with bitwise
 * the same page list and partials (and, with out, the merge of ps_combine as
 * in ps_select_sparse_decode, with arrivals as there). ("Faster Than Flash: Exploiting Attention
 * Sparsity for Efficient Long-Context Decoding", section "Methodology", item
 * 2; "Training-free sparse attention for long-context LLM decode", section
 * "Reusable code": a fused single-launch variant of the sparse decode.)
 * Every split's workgroup computes the (b, g) threshold from the forced
 * pages' keys and selects the page list itself.
 * Arguments as ps_select_sparse_decode, with delta as in ps_select_topdelta.
 * Host checks: those of ps_select_sparse_decode (same codes), then delta >= 0
 * and 0 < scale < infinity (else PS_ERR_BUDGET).
 * Device preconditions: those of ps_select_topdelta and ps_sparse_decode. */
int ps_select_topdelta_sparse_decode(const ps_geom* geom, const float* q, const void* k_pool,
                                     const void* v_pool, const int32_t* page_table,
                                     const int32_t* seq_lens, const float* scores,
                                     int32_t budget_pages, int32_t n_sink_pages,
                                     int32_t n_local_pages, float scale, float delta,
                                     int32_t n_splits, int32_t* sel, int32_t* sel_count,
                                     float* part_acc, float* part_ml, const float* sink,
                                     float* out, float* lse, int32_t* arrivals, void* stream);

/* 4b. Dense split-KV decode: ps_sparse_decode over every page. Split s of a
 * request covers logical pages [s*c_b, min((s+1)*c_b, n_b)) with
 * c_b = ceil(n_b / n_splits). ("Don't read the haystack", section "Part one:
 * hitting the wall on purpose".)
 * Host checks: 1 <= n_splits <= max_pages. */
int ps_full_decode(const ps_geom* geom, const float* q, const void* k_pool, const void* v_pool,
                   const int32_t* page_table, const int32_t* seq_lens, float scale,
                   int32_t n_splits, float* part_acc, float* part_ml, void* stream);

/* 5. Merge of split partials with an optional sink. ("Attention: Undivided &
 * Uncompressed", section "Traffic": partial softmaxes merge by rescaling with
 * exp of the difference of their maxima; "Training-free sparse attention for
 * long-context LLM decode", section "Strongest signals", item 1: a learned
 * per-head sink is a virtual key with zero value that enters only the
 * denominator.) For every (b, h), with sigma = sink[h] (or -inf when sink is
 * NULL):
 *   M   = max(max_s m_s, sigma)
 *   L   = sum_s exp(m_s - M) l_s + exp(sigma - M)
 *   out = sum_s exp(m_s - M) acc_s / L
 *   lse = M + ln L                       (written only when lse != NULL)
 * If every split is empty and there is no sink, out = 0 and lse = -inf.
 * Host checks: n_splits >= 1. */
int ps_combine(const ps_geom* geom, const float* part_acc, const float* part_ml, int32_t n_splits,
               const float* sink, float* out, float* lse, void* stream);

/* Human-readable name of a ps_status (static storage; never NULL). */
const char* ps_strerror(int status);

/* ABI version of this library: (major << 16) | minor. This header is 2.0
 * (ps_geom gained meta_layout: a caller built against 1.x passes a shorter
 * struct, so the major version changed). */
int ps_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGESPARSE_H */
