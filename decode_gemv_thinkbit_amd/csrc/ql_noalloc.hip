// Grouped GEMV for callers that cannot allocate device memory: the task
// scheduler and split-K state live in a static device array of the library
// instead of a caller buffer.  Same kernels and results as
// qlinear_gemv_grouped.
#include <mutex>

#include "ql_internal.hpp"

namespace {

constexpr int kMaxDevices = 64;

// The state array.  Its name is only a host-side stand-in for the device
// symbol: host code uses the per-device address obtained below, never the name.
static __device__ __align__(256) uint32_t scratch[QL_NOALLOC_STATE_WORDS];

std::mutex g_mu;
uint32_t* g_ptr[kMaxDevices] = {};  // device address of `scratch` on each device (null until set up)

__global__ void __launch_bounds__(256) clear_words_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

// Address of the current device's copy of `scratch`.  The first call on a
// device looks it up and clears the array with a fill kernel on `stream`
// (a fill kernel, not a memset, so that the clear is also correct inside a
// captured graph).  Every completed grouped launch leaves its counters at zero
// again, so later calls need no clear.
ql_status state_on_device(hipStream_t stream, uint32_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return ql::set_error(QL_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return ql::set_error(QL_EUNSUPPORTED, "device %d is beyond the %d devices this entry point supports", dev,
                         kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return ql::set_error(QL_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    hipLaunchKernelGGL(clear_words_kernel, dim3(256), dim3(256), 0, stream, static_cast<uint32_t*>(p),
                       (int64_t)QL_NOALLOC_STATE_WORDS);
    e = hipGetLastError();
    if (e != hipSuccess) return ql::set_error(QL_EHIP, "state clear launch: %s", hipGetErrorString(e));
    g_ptr[dev] = static_cast<uint32_t*>(p);
  }
  *out = g_ptr[dev];
  return QL_OK;
}

}  // namespace

extern "C" {

ql_status qlinear_gemv_grouped_noalloc(const ql_gemv_desc* descs, int32_t count, int64_t total_tasks, int32_t M,
                                       int64_t state_words, hipStream_t stream) {
  if (M < 1 || M > 16) return ql::set_error(QL_EINVAL, "grouped gemv needs 1 <= M <= 16 (M=%d)", M);
  if (count <= 0 || total_tasks <= 0 || total_tasks >= ((int64_t)1 << 31))
    return ql::set_error(QL_EINVAL, "bad count (%d) or task total (%lld)", count, (long long)total_tasks);
  if (!descs || ((uintptr_t)descs & 15u))
    return ql::set_error(QL_EINVAL, "descs must be a non-null, 16-byte aligned device pointer");
  if (state_words < QL_SCHED_WORDS || state_words > (int64_t)QL_NOALLOC_STATE_WORDS)
    return ql::set_error(QL_EINVAL,
                         "state_words %lld outside [%d, %d]: the launch needs more state than the static array "
                         "holds (use qlinear_gemv_grouped with a caller buffer, or fewer split parts)",
                         (long long)state_words, QL_SCHED_WORDS, QL_NOALLOC_STATE_WORDS);
  uint32_t* state = nullptr;
  const ql_status st = state_on_device(stream, &state);
  if (st != QL_OK) return st;
  const hipError_t e = ql::launch_gemv_grouped(descs, count, total_tasks, M, state, stream);
  if (e != hipSuccess) return ql::set_error(QL_EHIP, "grouped gemv launch: %s", hipGetErrorString(e));
  return QL_OK;
}

}  // extern "C"
