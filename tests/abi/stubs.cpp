// Stand-ins for the kernel launchers of the library (no device code): each
// counts its call and returns success, so the C ABI layer's host code can be
// built and run alone, under the address and undefined-behaviour sanitizers.
#include "ps_launch.h"

int g_launches = 0;

namespace ps {

hipError_t launch_build_page_meta(const Shape&, const void*, const int32_t*, const int32_t*,
                                  const int32_t*, int, void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_score_pages(const Shape&, const float*, const void*, const int32_t*,
                              const int32_t*, float*, const void*, void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_select_topk(const Shape&, const float*, const int32_t*, int, int, int,
                              int32_t*, int32_t*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_select_topdelta(const Shape&, const float*, const void*, const int32_t*,
                                  const float*, const int32_t*, int, int, int, float, float,
                                  int32_t*, int32_t*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_select_decode(const Shape&, const float*, const void*, const void*,
                                const int32_t*, const int32_t*, const float*, int, int, int,
                                float, int, int32_t*, int32_t*, float*, float*, const float*,
                                float*, float*, int32_t*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_select_decode_noalloc(const Shape&, const float*, const void*, const void*,
                                        const int32_t*, const int32_t*, const float*, int, int,
                                        int, float, int, int32_t*, int32_t*, const float*,
                                        float*, float*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_select_topdelta_decode(const Shape&, const float*, const void*, const void*,
                                         const int32_t*, const int32_t*, const float*, int, int,
                                         int, float, float, int, int32_t*, int32_t*, float*,
                                         float*, const float*, float*, float*, int32_t*,
                                         hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_decode(const Shape&, bool, const float*, const void*, const void*,
                         const int32_t*, const int32_t*, const int32_t*, const int32_t*, int,
                         float, int, float*, float*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_combine(const Shape&, const float*, const float*, int, const float*, float*,
                          float*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}

}  // namespace ps
