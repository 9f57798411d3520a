// Launches of the split-KV decode over a page list or over every page
// (kernels in ps_decode.h).
#include "ps_decode.h"

namespace ps {

hipError_t launch_decode(const Shape& s, bool sparse, const float* q, const void* k_pool,
                         const void* v_pool, const int32_t* page_table, const int32_t* seq_lens,
                         const int32_t* sel, const int32_t* sel_count, int budget, float scale,
                         int n_splits, float* part_acc, float* part_ml, hipStream_t st) {
  const int64_t blocks = (int64_t)s.batch * s.hkv * n_splits;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks), block(kDecWaves * kWave);
  const float qscale = scale * 1.44269504088896340736f;  // log2(e)
  const SelectArgs none{nullptr, 0, 0, nullptr, nullptr, nullptr, nullptr, nullptr, 0.0f, 0.0f};
  if (s.kv_bf16) {
    const int waves = decode_waves(blocks);
    const dim3 wblock(waves * kWave);
#define PS_DECODE_MFMA(DD, MM, WW)                                                             \
  hipLaunchKernelGGL((decode_mfma_kernel<DD, kG, MM, 1, WW, 2>), grid, wblock, 0, st, q,       \
                     static_cast<const bf16_t*>(k_pool), static_cast<const bf16_t*>(v_pool),   \
                     page_table, seq_lens, sel, sel_count, sparse ? budget : 0, s.hkv,          \
                     s.max_pages, n_splits, qscale, part_acc, part_ml, none)
#define PS_DECODE_MFMA_W(DD, MM)                      \
  do {                                                \
    if (waves == 8) PS_DECODE_MFMA(DD, MM, 8);        \
    else PS_DECODE_MFMA(DD, MM, 4);                   \
  } while (0)
    PS_WITH_GROUP(s.group, {
      if (s.head_dim == 64) {
        if (sparse) PS_DECODE_MFMA_W(64, kList);
        else PS_DECODE_MFMA_W(64, kDense);
      } else {
        if (sparse) PS_DECODE_MFMA_W(128, kList);
        else PS_DECODE_MFMA_W(128, kDense);
      }
    });
#undef PS_DECODE_MFMA_W
#undef PS_DECODE_MFMA
    return hipGetLastError();
  }
  // fp32 K/V: the vector-ALU decode
  const float* kp = static_cast<const float*>(k_pool);
  const float* vp = static_cast<const float*>(v_pool);
#define PS_DECODE_F32(DD)                                                                     \
  do {                                                                                        \
  PS_WITH_GROUP(s.group, {                                                                    \
    if (sparse)                                                                               \
      hipLaunchKernelGGL((decode_kernel<float, DD, kG, kList, 1>), grid, block, 0, st, q, kp, \
                         vp, page_table, seq_lens, sel, sel_count, budget, s.hkv,             \
                         s.max_pages, n_splits, qscale, part_acc, part_ml, none);             \
    else                                                                                      \
      hipLaunchKernelGGL((decode_kernel<float, DD, kG, kDense, 1>), grid, block, 0, st, q,    \
                         kp, vp, page_table, seq_lens, nullptr, nullptr, 0, s.hkv,            \
                         s.max_pages, n_splits, qscale, part_acc, part_ml, none);             \
  });                                                                                         \
  } while (0)
  if (s.head_dim == 64)
    PS_DECODE_F32(64);
  else
    PS_DECODE_F32(128);
#undef PS_DECODE_F32
  return hipGetLastError();
}

}  // namespace ps
