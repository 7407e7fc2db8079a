// Opt-in checks of the device-data preconditions the entry points document
// (CGS_VALIDATE=1 in the environment, or cgs_set_validate(1)): index lists
// ascending, unique and in range; values finite and inside the fixed-point
// ranges of the token scores and contribution scores.  A checked call runs a
// small kernel on its stream, waits for it and returns CGS_ERR_DATA before
// any of its own kernels are launched.  The mode synchronises the stream and
// allocates one flag per device on first use, so it is a debugging aid: it
// must not be enabled while a stream is being captured.
#include <math.h>
#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "common.hpp"
#include "validate.hpp"

namespace cgs {
namespace {

constexpr int kMaxDevices = 64;
int* g_flag[kMaxDevices] = {};
std::mutex g_flag_mu;
std::atomic<int> g_validate{-1};  // -1: not read from the environment yet

// Sets *bad when idx[0..n) is not strictly ascending or leaves [0, limit).
__global__ __launch_bounds__(256) void check_index_kernel(const int32_t* __restrict__ idx, int n, int limit,
                                                          int* __restrict__ bad) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    const int32_t v = idx[i];
    if (v < 0 || v >= limit || (i > 0 && idx[i - 1] >= v)) atomicOr(bad, 1);
  }
}

// Sets *bad when an element of a[0..n) is not finite or |a| > bound.
template <typename T>
__global__ __launch_bounds__(256) void check_abs_kernel(const T* __restrict__ a, size_t n, float bound,
                                                        int* __restrict__ bad) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const float v = Elem<T>::to_f32(a[i]);
    if (!(fabsf(v) <= bound)) atomicOr(bad, 1);
  }
}

__global__ void zero_flag_kernel(int* flag) { *flag = 0; }

// Sets *bad when an element of a[0..n) is not finite (or, with nonneg, negative).
__global__ void check_finite_f64_kernel(const double* __restrict__ a, int n, int nonneg, int* __restrict__ bad) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    if (!isfinite(a[i]) || (nonneg && a[i] < 0.0)) atomicOr(bad, 1);
}

// The calling thread's device flag (allocated once per device).
int* device_flag() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_flag_mu);
  if (!g_flag[dev] && hipMalloc(reinterpret_cast<void**>(&g_flag[dev]), sizeof(int)) != hipSuccess) {
    g_flag[dev] = nullptr;
    return nullptr;
  }
  return g_flag[dev];
}

template <typename Launch>
int run_check(hipStream_t s, Launch launch) {
  // A check reads its verdict back to the host, which a stream under graph
  // capture cannot do: refuse before enqueuing anything, so that the caller's
  // capture stays valid.
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess) return CGS_ERR_LAUNCH;
  if (cs != hipStreamCaptureStatusNone) return CGS_ERR_UNSUPPORTED;
  int* flag = device_flag();
  if (!flag) return CGS_ERR_LAUNCH;
  hipLaunchKernelGGL(zero_flag_kernel, dim3(1), dim3(1), 0, s, flag);
  launch(flag);
  if (!launch_ok()) return CGS_ERR_LAUNCH;
  int h = 0;
  if (hipMemcpyAsync(&h, flag, sizeof(int), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return CGS_ERR_LAUNCH;
  return h ? CGS_ERR_DATA : CGS_OK;
}

int grid_for(size_t n) { return static_cast<int>(std::min<size_t>((n + 255) / 256, 1024)); }

}  // namespace

bool validate_on() {
  int v = g_validate.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* e = getenv("CGS_VALIDATE");
    int expect = -1;
    // the first reader publishes the environment's setting unless a call of
    // cgs_set_validate got there first
    g_validate.compare_exchange_strong(expect, (e && e[0] && e[0] != '0') ? 1 : 0);
    v = g_validate.load(std::memory_order_relaxed);
  }
  return v == 1;
}

int validate_index(const int32_t* idx, int n, int limit, hipStream_t s) {
  if (!validate_on() || n <= 0 || !idx) return CGS_OK;
  return run_check(s, [&](int* flag) {
    hipLaunchKernelGGL(check_index_kernel, dim3(grid_for(n)), dim3(256), 0, s, idx, n, limit, flag);
  });
}

int validate_abs(const void* a, size_t n, int dtype, float bound, hipStream_t s) {
  if (!validate_on() || n == 0 || !a) return CGS_OK;
  return run_check(s, [&](int* flag) {
    if (dtype == CGS_BF16)
      hipLaunchKernelGGL((check_abs_kernel<uint16_t>), dim3(grid_for(n)), dim3(256), 0, s,
                         static_cast<const uint16_t*>(a), n, bound, flag);
    else
      hipLaunchKernelGGL((check_abs_kernel<float>), dim3(grid_for(n)), dim3(256), 0, s,
                         static_cast<const float*>(a), n, bound, flag);
  });
}

int validate_finite_f64(const double* a, int n, hipStream_t s, bool nonneg) {
  if (!validate_on() || n <= 0 || !a) return CGS_OK;
  return run_check(s, [&](int* flag) {
    hipLaunchKernelGGL(check_finite_f64_kernel, dim3(grid_for(n)), dim3(256), 0, s, a, n, nonneg ? 1 : 0, flag);
  });
}

}  // namespace cgs

extern "C" int cgs_set_validate(int on) {
  cgs::validate_on();  // settle the environment default first
  return cgs::g_validate.exchange(on ? 1 : 0) == 1 ? 1 : 0;
}
