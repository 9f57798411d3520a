// The selecting decode that merges its own splits, with its workspace in a
// fixed-size device array of the library instead of caller buffers: for
// callers that cannot allocate (code under HIP graph capture, serving loops
// or harnesses that forbid hipMalloc). Same kernels as
// ps_select_sparse_decode; only where the split partials and the arrival
// counters live differs.
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy, at its own address, until the process ends. In host
// code the variable's name is only a host-side stand-in, so the device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is handed to kernels. Every call on one GPU
// shares the array: calls that overlap in time on one GPU race.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "ps_launch.h"

namespace ps {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device.
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// Clears the arrival counters (a kernel, not a memset node, so a captured
// graph replays it correctly).
__global__ void zero_counters(int32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

hipError_t launch_select_decode_noalloc(const Shape& s, const float* q, const void* k_pool,
                                        const void* v_pool, const int32_t* page_table,
                                        const int32_t* seq_lens, const float* scores,
                                        int budget, int n_sink, int n_local, float scale,
                                        int n_splits, int32_t* sel, int32_t* sel_count,
                                        const float* sink, float* out, float* lse,
                                        hipStream_t st) {
  const int64_t bytes = noalloc_scratch_bytes(s, n_splits);
  if (bytes < 0 || bytes > kNoAllocScratchBytes) return hipErrorInvalidValue;
  void* base = nullptr;
  hipError_t e = scratch_address(&base);
  if (e != hipSuccess) return e;
  uint8_t* p = static_cast<uint8_t*>(base);
  const int64_t units = (int64_t)s.batch * s.hkv;
  const int64_t rows = (int64_t)s.batch * s.hq * n_splits;
  int32_t* arrivals = reinterpret_cast<int32_t*>(p);
  float* part_ml = reinterpret_cast<float*>(p + scratch_align(units * 4));
  float* part_acc =
      reinterpret_cast<float*>(p + scratch_align(units * 4) + scratch_align(rows * 2 * 4));
  if (n_splits > 1) {
    const int n = (int)units;  // units * 4 <= kNoAllocScratchBytes
    hipLaunchKernelGGL(zero_counters, dim3((n + 255) / 256), dim3(256), 0, st, arrivals, n);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_select_decode(s, q, k_pool, v_pool, page_table, seq_lens, scores, budget,
                              n_sink, n_local, scale, n_splits, sel, sel_count,
                              n_splits > 1 ? part_acc : nullptr,
                              n_splits > 1 ? part_ml : nullptr, sink, out, lse,
                              n_splits > 1 ? arrivals : nullptr, st);
}

}  // namespace ps
