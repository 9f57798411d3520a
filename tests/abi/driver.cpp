// Exercises the C ABI layer's host code (validation, overflow-checked sizing,
// dispatch) through every entry point, with the kernel launchers replaced by
// counting stubs. Built and run under the address and undefined-behaviour
// sanitizers by tests/test_abi_sanitizers.py; exits non-zero on the first
// unexpected status.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "pagesparse.h"

extern int g_launches;

static int failures = 0;

static void expect(const char* what, int got, int want) {
  if (got != want) {
    fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
    ++failures;
  }
}

static ps_geom geom(int32_t batch = 2, int32_t hq = 12, int32_t hkv = 2, int32_t d = 128,
                    int32_t max_pages = 64, int64_t phys = 128, int32_t dtype = PS_BF16,
                    int32_t meta = PS_META_KV) {
  ps_geom g;
  memset(&g, 0, sizeof g);
  g.batch = batch;
  g.num_q_heads = hq;
  g.num_kv_heads = hkv;
  g.head_dim = d;
  g.page_size = 16;
  g.max_pages = max_pages;
  g.num_phys_pages = phys;
  g.kv_dtype = dtype;
  g.meta_format = meta;
  return g;
}

int main() {
  // never dereferenced: the launchers are stubs
  alignas(16) static char buf[64];
  void* X = buf;
  float* F = reinterpret_cast<float*>(buf);
  int32_t* I = reinterpret_cast<int32_t*>(buf);
  const ps_geom g = geom();

  // geometry checks, through the score entry point
  expect("null geom", ps_score_pages(nullptr, F, X, I, I, F, nullptr), PS_ERR_NULL);
  struct {
    ps_geom g;
    int want;
  } bad[] = {
      {geom(-1), PS_ERR_SHAPE},
      {geom(2, 0), PS_ERR_SHAPE},
      {geom(2, 13), PS_ERR_SHAPE},
      {geom(2, 32, 2), PS_ERR_UNSUPPORTED},
      {geom(2, 12, 2, 96), PS_ERR_UNSUPPORTED},
      {geom(2, 12, 2, 128, 0), PS_ERR_SHAPE},
      {geom(2, 12, 2, 128, 64, 0), PS_ERR_SHAPE},
      {geom(2, 12, 2, 128, 64, int64_t(1) << 60), PS_ERR_OVERFLOW},
      {geom(2, 12, 2, 128, 64, int64_t(1) << 31), PS_ERR_OVERFLOW},
      {geom(2, 12, 2, 128, 1 << 28), PS_ERR_OVERFLOW},
      {geom(0x7fffffff, 64, 8, 128, 1 << 27), PS_ERR_OVERFLOW},
      {geom(2, 12, 2, 128, 64, 128, 7), PS_ERR_UNSUPPORTED},
      {geom(2, 12, 2, 128, 64, 128, PS_BF16, 2), PS_ERR_SHAPE},
  };
  for (auto& c : bad) expect("bad geometry", ps_score_pages(&c.g, F, X, I, I, F, nullptr), c.want);
  ps_geom ps16 = g;
  ps16.page_size = 32;
  expect("page size", ps_score_pages(&ps16, F, X, I, I, F, nullptr), PS_ERR_UNSUPPORTED);
  ps_geom layout = g;
  layout.meta_layout = 2;
  expect("meta layout", ps_score_pages(&layout, F, X, I, I, F, nullptr), PS_ERR_SHAPE);
  layout.meta_layout = -1;
  expect("meta layout", ps_score_pages(&layout, F, X, I, I, F, nullptr), PS_ERR_SHAPE);
  // logical metadata B * Hkv * max_pages * 2 * D * 4 bytes beyond int64; the
  // physical layout of the same geometry passes the size checks
  ps_geom huge = geom(0x7fffffff, 8, 8, 128, (1 << 26) - 1, 128, PS_F32);
  huge.meta_layout = PS_META_LOGICAL;
  expect("logical overflow", ps_score_pages(&huge, F, X, I, I, F, nullptr), PS_ERR_OVERFLOW);

  // every entry point: a missing pointer, then a valid call (one launch)
  int before = g_launches;
  expect("meta null", ps_build_page_meta(&g, nullptr, I, I, nullptr, 4, X, nullptr), PS_ERR_NULL);
  expect("meta n_pages", ps_build_page_meta(&g, X, I, I, nullptr, 0, X, nullptr), PS_ERR_SHAPE);
  expect("meta", ps_build_page_meta(&g, X, I, I, nullptr, 64, X, nullptr), PS_OK);
  expect("score null", ps_score_pages(&g, nullptr, X, I, I, F, nullptr), PS_ERR_NULL);
  expect("score", ps_score_pages(&g, F, X, I, I, F, nullptr), PS_OK);
  expect("refresh null", ps_refresh_score_pages(&g, F, nullptr, X, I, I, F, nullptr), PS_ERR_NULL);
  expect("refresh", ps_refresh_score_pages(&g, F, X, X, I, I, F, nullptr), PS_OK);
  expect("select budget", ps_select_topk(&g, F, I, 0, 0, 0, I, I, nullptr), PS_ERR_BUDGET);
  expect("select forced", ps_select_topk(&g, F, I, 4, 3, 2, I, I, nullptr), PS_ERR_BUDGET);
  expect("select", ps_select_topk(&g, F, I, 8, 1, 2, I, I, nullptr), PS_OK);
  ps_geom wide = geom(2, 12, 2, 128, 65537, 200000);
  expect("select rows", ps_select_topk(&wide, F, I, 8, 1, 2, I, I, nullptr), PS_ERR_UNSUPPORTED);
  expect("topdelta delta",
         ps_select_topdelta(&g, F, X, I, I, F, 8, 1, 1, 0.1f, -1.0f, I, I, nullptr),
         PS_ERR_BUDGET);
  expect("topdelta", ps_select_topdelta(&g, F, X, I, I, F, 8, 1, 1, 0.1f, 2.0f, I, I, nullptr),
         PS_OK);
  expect("sparse splits",
         ps_sparse_decode(&g, F, X, X, I, I, I, I, 8, 0.1f, 9, F, F, nullptr), PS_ERR_BUDGET);
  expect("sparse", ps_sparse_decode(&g, F, X, X, I, I, I, I, 8, 0.1f, 4, F, F, nullptr), PS_OK);
  expect("fused arrivals",
         ps_select_sparse_decode(&g, F, X, X, I, I, F, 8, 1, 1, 0.1f, 2, I, I, F, F, nullptr, F,
                                 nullptr, nullptr, nullptr),
         PS_ERR_BUDGET);
  expect("fused", ps_select_sparse_decode(&g, F, X, X, I, I, F, 8, 1, 1, 0.1f, 2, I, I, F, F,
                                          nullptr, F, F, I, nullptr),
         PS_OK);
  expect("noalloc null", ps_select_sparse_decode_noalloc(&g, F, X, X, I, I, F, 8, 1, 1, 0.1f, 2,
                                                         I, I, nullptr, nullptr, nullptr, nullptr),
         PS_ERR_NULL);
  expect("noalloc", ps_select_sparse_decode_noalloc(&g, F, X, X, I, I, F, 8, 1, 1, 0.1f, 2, I, I,
                                                    F, F, F, nullptr),
         PS_OK);
  ps_geom big = geom(64, 64, 8, 128, 64, 128);
  expect("noalloc workspace",
         ps_select_sparse_decode_noalloc(&big, F, X, X, I, I, F, 64, 0, 0, 0.1f, 8, I, I, nullptr,
                                         F, nullptr, nullptr),
         PS_ERR_WORKSPACE);
  expect("topdelta fused",
         ps_select_topdelta_sparse_decode(&g, F, X, X, I, I, F, 8, 1, 1, 0.1f, 3.0f, 1, I, I,
                                          nullptr, nullptr, nullptr, F, F, nullptr, nullptr),
         PS_OK);
  expect("full splits", ps_full_decode(&g, F, X, X, I, I, 0.1f, 65, F, F, nullptr), PS_ERR_BUDGET);
  expect("full", ps_full_decode(&g, F, X, X, I, I, 0.1f, 8, F, F, nullptr), PS_OK);
  expect("combine null", ps_combine(&g, F, F, 4, nullptr, nullptr, nullptr, nullptr), PS_ERR_NULL);
  expect("combine", ps_combine(&g, F, F, 4, nullptr, F, nullptr, nullptr), PS_OK);
  // the metadata entry points with the logical layout
  ps_geom logical = g;
  logical.meta_layout = PS_META_LOGICAL;
  expect("meta logical", ps_build_page_meta(&logical, X, I, I, nullptr, 64, X, nullptr), PS_OK);
  expect("score logical", ps_score_pages(&logical, F, X, I, I, F, nullptr), PS_OK);
  expect("refresh logical", ps_refresh_score_pages(&logical, F, X, X, I, I, F, nullptr), PS_OK);
  const int launched = g_launches - before;
  if (launched != 14) {
    fprintf(stderr, "%d launches, expected 14\n", launched);
    ++failures;
  }

  // an empty batch validates and launches nothing
  before = g_launches;
  ps_geom empty = geom(0);
  expect("empty score", ps_score_pages(&empty, F, X, I, I, F, nullptr), PS_OK);
  expect("empty fused", ps_select_sparse_decode(&empty, F, X, X, I, I, F, 8, 1, 1, 0.1f, 2, I, I,
                                                F, F, nullptr, F, F, I, nullptr),
         PS_OK);
  if (g_launches != before) {
    fprintf(stderr, "an empty batch launched\n");
    ++failures;
  }

  // status strings and the version
  for (int c = -8; c <= 1; ++c) {
    const char* m = ps_strerror(c);
    if (!m || !m[0]) {
      fprintf(stderr, "empty message for %d\n", c);
      ++failures;
    }
  }
  if ((ps_abi_version() >> 16) != 2) ++failures;
  if (failures) return 1;
  printf("abi driver: all checks passed\n");
  return 0;
}
