// Scratch memory of the allocation-free entry point (msa_indexer_topk_noalloc):
// the per-sequence arrival counters of the fused scan + selection live in a
// file-scope device array instead of a caller workspace.
//
// Each GPU holds its own copy of `scratch` at its own address, kept until the
// process ends.  In host code the array's name is not a device address, so it
// is never passed to a kernel: its address on the current device is looked up
// once per device with hipGetSymbolAddress and cached, and only that pointer
// reaches the kernels.  Every call on a device shares the array; calls that
// overlap on one device race on it.
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace msa {

// One arrival counter per sequence (uint32), for at most kStaticMaxBatch sequences.
static __device__ __align__(256) uint32_t scratch[kStaticMaxBatch];

__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

hipError_t static_scratch(uint32_t** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static uint32_t* ptr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    ptr[dev] = static_cast<uint32_t*>(p);
  }
  *out = ptr[dev];
  return hipSuccess;
}

// Clears n counters with a kernel (not a memset node, so the call can be captured
// into a HIP graph).
hipError_t launch_zero_u32(uint32_t* p, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace msa
