// Launch of the decode that selects its own pages by top-k (kernels in
// ps_decode.h).
#include "ps_decode.h"

namespace ps {

hipError_t launch_select_decode(const Shape& s, const float* q, const void* k_pool,
                                const void* v_pool, const int32_t* page_table,
                                const int32_t* seq_lens, const float* scores, int budget,
                                int n_sink, int n_local, float scale, int n_splits, int32_t* sel,
                                int32_t* sel_count, float* part_acc, float* part_ml,
                                const float* sink, float* out, float* lse, int32_t* arrivals,
                                hipStream_t st) {
  const SelectArgs sa{scores, n_sink, n_local, sel, sel_count, sink, out, lse, scale, 0.0f,
                      arrivals};
  return launch_selecting_decode<kSelect>(s, q, k_pool, v_pool, page_table, seq_lens, budget,
                                          scale, n_splits, part_acc, part_ml, sa, st);
}

}  // namespace ps
