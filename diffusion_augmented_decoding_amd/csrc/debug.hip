// Data-contract checks for debugging (off unless UNO_DEBUG is set in the
// environment or uno_debug_checks(1) is called): token ids and uniforms of a
// call are checked on the device before its kernels run, and the call waits
// for the result, so a violation is reported as UNO_ERR_INVALID_ARGUMENT by
// the call itself.  With the checks off nothing here runs.
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "internal.h"

namespace uno {

namespace {

__device__ unsigned int g_debug_bad;   // violations seen by the last check

__global__ void debug_clear_kernel(unsigned int* bad) { *bad = 0u; }

// ids[r * stride + c] for r < rows, c in [c0, cols): count those outside [lo, hi)
__global__ __launch_bounds__(256) void debug_ids_kernel(const int32_t* ids, int64_t rows, int64_t cols,
                                                       int64_t stride, int64_t c0, int32_t lo, int32_t hi,
                                                       unsigned int* bad) {
  const int64_t n = rows * (cols - c0);
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
    const int64_t r = i / (cols - c0), c = c0 + i % (cols - c0);
    const int32_t v = ids[r * stride + c];
    if (v < lo || v >= hi) atomicAdd(bad, 1u);
  }
}

// uniforms outside [0, 1) (NaN included)
__global__ __launch_bounds__(256) void debug_unit_kernel(const float* u, int64_t n, unsigned int* bad) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
    const float v = u[i];
    if (!(v >= 0.f && v < 1.f)) atomicAdd(bad, 1u);
  }
}

std::atomic<int> g_mode{-1};   // -1: not yet read from the environment

unsigned int* bad_counter() {
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_debug_bad)) != hipSuccess) return nullptr;
  return static_cast<unsigned int*>(p);
}

uno_status finish(hipStream_t stream, unsigned int* bad, const char* what) {
  unsigned int host = 0;
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = hipMemcpyAsync(&host, bad, sizeof(host), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return check_hip(e, "debug check");
  if (host) return fail(UNO_ERR_INVALID_ARGUMENT, "%s: %u value(s) outside the data contract", what, host);
  return UNO_OK;
}

unsigned blocks_for(int64_t n) { return unsigned(std::min<int64_t>((n + 255) / 256, 1024)); }

}  // namespace

bool debug_checks() {
  int m = g_mode.load(std::memory_order_acquire);
  if (m < 0) {
    const char* env = getenv("UNO_DEBUG");
    m = (env && env[0] && strcmp(env, "0") != 0) ? 1 : 0;
    int expected = -1;
    g_mode.compare_exchange_strong(expected, m);
    m = g_mode.load(std::memory_order_acquire);
  }
  return m == 1;
}

uno_status debug_check_ids(hipStream_t stream, const int32_t* ids, int64_t rows, int64_t cols, int64_t stride,
                           int64_t first_col, int32_t lo, int32_t hi, const char* what) {
  if (!ids || rows <= 0 || cols <= first_col) return UNO_OK;
  unsigned int* bad = bad_counter();
  if (!bad) return fail(UNO_ERR_HIP, "debug check: no device counter");
  hipLaunchKernelGGL(debug_clear_kernel, dim3(1), dim3(1), 0, stream, bad);
  hipLaunchKernelGGL(debug_ids_kernel, dim3(blocks_for(rows * (cols - first_col))), dim3(256), 0, stream, ids, rows,
                     cols, stride, first_col, lo, hi, bad);
  return finish(stream, bad, what);
}

uno_status debug_check_unit(hipStream_t stream, const float* u, int64_t n, const char* what) {
  if (!u || n <= 0) return UNO_OK;
  unsigned int* bad = bad_counter();
  if (!bad) return fail(UNO_ERR_HIP, "debug check: no device counter");
  hipLaunchKernelGGL(debug_clear_kernel, dim3(1), dim3(1), 0, stream, bad);
  hipLaunchKernelGGL(debug_unit_kernel, dim3(blocks_for(n)), dim3(256), 0, stream, u, n, bad);
  return finish(stream, bad, what);
}

}  // namespace uno

extern "C" {

void uno_debug_checks(int32_t on) { uno::g_mode.store(on ? 1 : 0, std::memory_order_release); }

int32_t uno_debug_checks_enabled(void) { return uno::debug_checks() ? 1 : 0; }

}  // extern "C"
