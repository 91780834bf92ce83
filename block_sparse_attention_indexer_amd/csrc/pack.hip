// FP8 / NVFP4 pack and unpack kernels.
//
// Source: "vLLM 為 MiniMax-M3.1-Flash 提供 Day-0 支援" -- K, V and the index
// key are quantised to NVFP4 as they are written into their caches (section
// "QKV GEMM + norm + RoPE + KV insert fusion"); NVFP4 is an E2M1 code per
// element with one E4M3 scale per 16 elements and an fp32 tensor scale
// ("What is new in the MiniMax-M3.1 architecture": 4.5 bits per element).
// The quantiser itself is not described there; the one here rounds to
// nearest-even with every step in fp32 in a fixed order (see msa.h).
#include "common.hpp"
#include "launch.hpp"

namespace msa {

__global__ void pack_fp8_kernel(const float* __restrict__ x, int64_t n, float scale,
                                uint8_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    out[i] = (uint8_t)e4m3_encode2(x[i] / scale, 0.0f);
  }
}

__global__ void unpack_fp8_kernel(const uint8_t* __restrict__ x, int64_t n, float scale,
                                  float* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    out[i] = scale * e4m3_to_f(x[i]);
  }
}

// One thread per group of 16 consecutive elements.
__global__ void pack_nvfp4_kernel(const float* __restrict__ x, int64_t groups, float tensor_scale,
                                  uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gi < groups; gi += stride) {
    const float4* src = reinterpret_cast<const float4*>(x + gi * 16);
    float v[16];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 f = src[k];
      v[4 * k + 0] = f.x; v[4 * k + 1] = f.y; v[4 * k + 2] = f.z; v[4 * k + 3] = f.w;
    }
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) amax = fmaxf(amax, __builtin_fabsf(v[k]));
    const float six_s = 6.0f * tensor_scale;
    const float t = amax / six_s;
    const uint32_t sb = e4m3_encode2(t, 0.0f) & 0xFFu;
    const float denom = e4m3_value(sb) * tensor_scale;
    uint32_t w[2] = {0u, 0u};
    if (denom > 0.0f) {
#pragma unroll
      for (int j = 0; j < 8; ++j)   // elements 2j, 2j+1: byte j of the group's 8
        w[j >> 2] |= e2m1_encode2(v[2 * j] / denom, v[2 * j + 1] / denom) << (8 * (j & 3));
    }
    reinterpret_cast<uint2*>(codes)[gi] = make_uint2(w[0], w[1]);
    scales[gi] = (uint8_t)sb;
  }
}

// One thread per group of 16: scale * value, value per the dequant mode.
template <bool FP8MODE>
__global__ void unpack_nvfp4_kernel(const uint8_t* __restrict__ codes,
                                    const uint8_t* __restrict__ scales, int64_t groups,
                                    float tensor_scale, float* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gi < groups; gi += stride) {
    const uint2 w = reinterpret_cast<const uint2*>(codes)[gi];
    const uint32_t sb = scales[gi];
    const float s = e4m3_value(sb);
    float4* dst = reinterpret_cast<float4*>(out + gi * 16);
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      float r[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int k = 4 * k4 + u;
        const uint32_t c = ((k < 8 ? w.x : w.y) >> (4 * (k & 7))) & 0xFu;
        float val = e2m1_magnitude(c) * s;              // exact in fp32
        if (FP8MODE) val = e4m3_value(e4m3_encode(val)); // re-round to E4M3
        if (c & 8u) val = -val;
        r[u] = tensor_scale * val;
      }
      dst[k4] = make_float4(r[0], r[1], r[2], r[3]);
    }
  }
}

static inline unsigned grid_for(int64_t n, int threads) {
  int64_t g = (n + threads - 1) / threads;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (unsigned)g;
}

hipError_t launch_pack_fp8(const float* x, int64_t n, float scale, uint8_t* out, hipStream_t s) {
  hipLaunchKernelGGL(pack_fp8_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, x, n, scale, out);
  return hipGetLastError();
}
hipError_t launch_unpack_fp8(const uint8_t* x, int64_t n, float scale, float* out, hipStream_t s) {
  hipLaunchKernelGGL(unpack_fp8_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, x, n, scale, out);
  return hipGetLastError();
}
hipError_t launch_pack_nvfp4(const float* x, int64_t groups, float ts, uint8_t* codes,
                             uint8_t* scales, hipStream_t s) {
  hipLaunchKernelGGL(pack_nvfp4_kernel, dim3(grid_for(groups, 256)), dim3(256), 0, s, x, groups,
                     ts, codes, scales);
  return hipGetLastError();
}
hipError_t launch_unpack_nvfp4(const uint8_t* codes, const uint8_t* scales, int64_t groups,
                               float ts, bool fp8mode, float* out, hipStream_t s) {
  if (fp8mode)
    hipLaunchKernelGGL(unpack_nvfp4_kernel<true>, dim3(grid_for(groups, 256)), dim3(256), 0, s,
                       codes, scales, groups, ts, out);
  else
    hipLaunchKernelGGL(unpack_nvfp4_kernel<false>, dim3(grid_for(groups, 256)), dim3(256), 0, s,
                       codes, scales, groups, ts, out);
  return hipGetLastError();
}

}  // namespace msa
