// One MSA decode layer step (T = 1) in one launch: index scan and block
// max-pool, top-16 selection and sparse attention, with the same results as
// the three separate calls.
//
// Source: "vLLM 為 MiniMax-M3.1-Flash 提供 Day-0 支援", section "MSA primer"
// (the four steps) and the AMD section, which mentions a single ("mono")
// kernel for low-latency decode.
//
// The three calls leave the GPU half idle twice per step: the selection can
// only start once every block of the batch has been scored, and the
// attention only once every row is selected, although each of them needs
// just one sequence's scores.  Here a grid of persistent workgroups (two
// per CU) first takes the scan's chunks (a sequence's 64-block chunk per
// item, in sequence order) from a work counter.  The workgroup that
// finishes the last chunk of a sequence selects that sequence's blocks (one
// wave per group) and marks its four rows ready.  Once the chunks run out,
// the workgroups take the rows in order and attend each one as soon as it is
// ready (4 waves per row).  A workgroup only ever waits for chunks that
// running workgroups have already taken, so the step completes whether or
// not the whole grid is resident; the wait is bounded all the same (a row
// whose flag never comes is written as NaN).  Scores and selections pass
// between workgroups through device-coherent stores and loads, ordered by
// completed-store waits before each counter or flag update.
//
// Workspace (uint32): [0] next chunk, [1] next row, [2] workgroups done,
// [3] unused, [4, 4+B) per-sequence arrival counts, [4+B, 4+5B) per-row
// ready flags.  All zero before the call; every word is reset to zero by its
// last user, so the workspace is left zeroed.
#include "attn_row.hpp"
#include "launch.hpp"
#include "scan1.hpp"

namespace msa {

template <int KT>
__global__ __launch_bounds__(kDecWaves * 64, 2) void decode_step_kernel(Scan1Args sa, AttnArgs aa,
                                                                        int32_t* __restrict__ sel,
                                                                        uint32_t* __restrict__ ws, int B,
                                                                        int nchunks, uint32_t spin_limit) {
  __shared__ int item_sh, ok_sh;
  uint32_t* next_chunk = ws;
  uint32_t* next_row = ws + 1;
  uint32_t* done = ws + 2;
  uint32_t* arrival = ws + 4;
  uint32_t* ready = ws + 4 + B;
  const int nscan = B * nchunks, rows = B * kGroups;

  // 1. scan chunks; the workgroup that completes a sequence selects its blocks
  for (;;) {
    if (threadIdx.x == 0)
      item_sh = (int)__hip_atomic_fetch_add(next_chunk, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int item = item_sh;
    __syncthreads();
    if (item >= nscan) break;
    const int b = item / nchunks;
    scan1_chunk<KT, false, true>(sa, b, item - b * nchunks);
    if (scan1_select_if_last(sa, b, nchunks, sel, arrival)) {
      __builtin_amdgcn_s_waitcnt(0);   // the selection is stored before its rows are marked
      __syncthreads();
      if (threadIdx.x < kGroups)
        __hip_atomic_store(&ready[b * kGroups + threadIdx.x], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }

  // 2. attention rows, each as soon as its sequence is selected
  for (;;) {
    if (threadIdx.x == 0)
      item_sh = (int)__hip_atomic_fetch_add(next_row, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int r = item_sh;
    __syncthreads();
    if (r >= rows) break;
    if (threadIdx.x == 0) {
      uint32_t n = 0;
      while (__hip_atomic_load(&ready[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) == 0u && ++n < spin_limit)
        __builtin_amdgcn_s_sleep(2);
      ok_sh = n < spin_limit ? 1 : 0;
      __hip_atomic_store(&ready[r], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    __syncthreads();
    if (ok_sh) {
      attend_row<KT, false, kDecWaves, true>(aa, r);
    } else {
      float* o = aa.out + (size_t)r * kHeadsPerGroup * kHeadDim;   // T = 1: row r is heads 16g.. of sequence b
      for (int e = threadIdx.x; e < kHeadsPerGroup * kHeadDim; e += kDecWaves * 64) o[e] = __builtin_nanf("");
      if (aa.lse != nullptr && threadIdx.x < kHeadsPerGroup) aa.lse[(size_t)r * kHeadsPerGroup + threadIdx.x] = __builtin_nanf("");
    }
    __syncthreads();
  }

  // 3. the last workgroup out resets the work counters
  if (threadIdx.x == 0 &&
      __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1) {
    __hip_atomic_store(next_chunk, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(next_row, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

bool decode_step_fits(const ProblemArgs& p, const CacheArgs& idx_k, const CacheArgs& k, const CacheArgs& v,
                      bool fp8mode) {
  if (p.T != 1 || idx_k.dtype == 0 || k.dtype == 0 || k.dtype != v.dtype || idx_k.dtype != k.dtype) return false;
  return !(k.dtype == 2 && fp8mode);   // the FP8-rounded NVFP4 reading takes the three calls
}

size_t decode_step_workspace_words(int B) { return 4 + 5 * (size_t)B; }

hipError_t launch_decode_step(const ProblemArgs& p, const void* idx_q, float idx_q_scale, const CacheArgs& idx_k,
                              const void* q, float q_scale, const CacheArgs& k, const CacheArgs& v,
                              float softmax_scale, float* block_scores, int32_t* sel, float* out, float* lse,
                              uint32_t* ws, hipStream_t s) {
  const int nchunks = (p.max_blocks + kScan1Blocks - 1) / kScan1Blocks;
  const Scan1Args sa{static_cast<const uint8_t*>(idx_q), idx_k.data, idx_k.scales, idx_k.num_pages, p.seq_lens,
                     p.block_table, p.max_blocks, idx_q_scale * idx_k.tensor_scale, block_scores, nullptr};
  const float c_log2 = softmax_scale * q_scale * k.tensor_scale * 1.4426950408889634f;
  const AttnArgs aa{static_cast<const uint8_t*>(q), c_log2, k.data, k.scales, k.num_pages, v.data, v.scales,
                    v.num_pages, v.tensor_scale, sel, p.seq_lens, p.block_table, p.max_blocks, 1, out, lse};
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int nscan = p.B * nchunks;
  const unsigned grid = (unsigned)min(2 * max(cus, 1), nscan);
  const uint32_t spin_limit = 1u << 18;   // well under a second of polling; a step takes ~0.2 ms
  if (k.dtype == 1)
    hipLaunchKernelGGL(decode_step_kernel<1>, dim3(grid), dim3(kDecWaves * 64), 0, s, sa, aa, sel, ws, p.B,
                       nchunks, spin_limit);
  else
    hipLaunchKernelGGL(decode_step_kernel<2>, dim3(grid), dim3(kDecWaves * 64), 0, s, sa, aa, sel, ws, p.B,
                       nchunks, spin_limit);
  return hipGetLastError();
}

}  // namespace msa
