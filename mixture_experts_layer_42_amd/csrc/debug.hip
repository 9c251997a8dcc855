// Debug-mode input checks (MOE_DEBUG=1 in the environment): every floating-point input of an
// entry point is scanned on the device for NaN and infinity before any work is enqueued. The
// result goes to a flag in device memory that the host reads back after a stream
// synchronisation, so a non-finite input becomes MOE_ERR_INVALID_ARG with nothing else
// enqueued. Off by default: the hot path checks nothing.
#include <cstdlib>
#include <cstring>

#include "common.h"
#include "kernels.h"

namespace moe {

__device__ int g_nonfinite;   // set to 1 by any check kernel that meets a non-finite value

__global__ void clear_nonfinite_kernel() { g_nonfinite = 0; }

// n elements of `elt` bytes (2: bf16, 4: float32); with n_rows_dev the count is
// n_rows_dev[0] * row_elems (rows produced on the device, e.g. the kept rows)
__global__ __launch_bounds__(256) void finite_check_kernel(const void *__restrict__ p, size_t n,
                                                           int elt,
                                                           const int32_t *__restrict__ n_rows_dev,
                                                           int row_elems) {
  if (n_rows_dev) n = (size_t)n_rows_dev[0] * row_elems;
  int bad = 0;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x) {
    if (elt == 2) {
      const uint32_t u = ((const uint16_t *)p)[i];
      bad |= (u & 0x7F80u) == 0x7F80u;
    } else {
      const uint32_t u = ((const uint32_t *)p)[i];
      bad |= (u & 0x7F800000u) == 0x7F800000u;
    }
  }
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(&g_nonfinite, 1);
}

bool debug_checks_enabled() {
  const char *e = std::getenv("MOE_DEBUG");
  return e && e[0] && std::strcmp(e, "0") != 0;
}

hipError_t debug_any_nonfinite(const DebugSpan *spans, int n_spans, hipStream_t st, bool *found) {
  *found = false;
  hipLaunchKernelGGL(clear_nonfinite_kernel, dim3(1), dim3(1), 0, st);
  for (int i = 0; i < n_spans; ++i) {
    const DebugSpan &s = spans[i];
    if (!s.p) continue;
    hipLaunchKernelGGL(finite_check_kernel, dim3(1024), dim3(256), 0, st, s.p, s.n, s.elt,
                       s.n_rows_dev, s.row_elems);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int h = 0;
  e = hipMemcpyFromSymbolAsync(&h, HIP_SYMBOL(g_nonfinite), sizeof(int), 0,
                               hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(st);
  if (e != hipSuccess) return e;
  *found = h != 0;
  return hipSuccess;
}

}  // namespace moe
