// Measurement probes of the benchmark: a streaming read of a device buffer and
// the dense f16 MFMA issue rate.  Not part of the MSA path (built into
// libmsa_probe.so, not libmsa.so); they give the ceilings the path's kernels
// are measured against on the GPU at hand.
#include <hip/hip_runtime.h>

#include "probe.h"

namespace msa_probe {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kProbeMagic = 0x9E3779B9u;

// One workgroup per contiguous 32 KiB slice: 8 independent 16-byte loads per
// thread, all issued before the first is used (indices past the end clamp to
// the last element, so no load is guarded by a branch).
constexpr int kProbeLoads = 8;
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ src, size_t n,
                                                          uint32_t* __restrict__ sink) {
  const size_t base = (size_t)blockIdx.x * 256 * kProbeLoads + threadIdx.x;
  uint4 v[kProbeLoads];
#pragma unroll
  for (int k = 0; k < kProbeLoads; ++k) v[k] = src[min(base + (size_t)k * 256, n - 1)];
  uint32_t x = 0;
#pragma unroll
  for (int k = 0; k < kProbeLoads; ++k) x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  if (x == kProbeMagic) sink[blockIdx.x % MSA_PROBE_SINK_WORDS] = x;
}

// Sixteen independent accumulation chains per wave keep the MFMA pipe fed.
__global__ __launch_bounds__(256) void mfma_peak_kernel(float* __restrict__ out, int iters) {
  const _Float16 v = (_Float16)(1.0f / 1024.0f) * (_Float16)(threadIdx.x & 7);
  const h8 a = h8{v, v, v, v, v, v, v, v};
  const h8 b = h8{v, -v, v, -v, v, -v, v, -v};
  f4 acc[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) acc[k] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace msa_probe

extern "C" msa_status msa_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (buf == nullptr || sink == nullptr || bytes == 0 || bytes % 16 != 0 ||
      reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return MSA_ERR_INVALID_ARG;
  const size_t n = bytes / 16;
  const size_t per_wg = (size_t)256 * msa_probe::kProbeLoads;
  if ((n + per_wg - 1) / per_wg > 0x7FFFFFFFu) return MSA_ERR_INVALID_ARG;
  const unsigned grid = (unsigned)((n + per_wg - 1) / per_wg);
  hipLaunchKernelGGL(msa_probe::stream_read_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const uint4*>(buf), n,
                     sink);
  return hipGetLastError() == hipSuccess ? MSA_OK : MSA_ERR_HIP;
}

extern "C" msa_status msa_probe_mfma_f16(float* out, int32_t workgroups, int32_t iters, hipStream_t stream) {
  if (out == nullptr || workgroups < 1 || iters < 1) return MSA_ERR_INVALID_ARG;
  hipLaunchKernelGGL(msa_probe::mfma_peak_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream, out, (int)iters);
  return hipGetLastError() == hipSuccess ? MSA_OK : MSA_ERR_HIP;
}
