// Step 3 of MSA: the top-16 blocks of every (sequence, query token, group)
// row, the query's own (most recent) block always kept.
//
// Source: "vLLM 為 MiniMax-M3.1-Flash 提供 Day-0 支援", section "MSA primer":
// attention runs over the top 16 blocks and the most recent block is always
// kept, capping a query at 2,048 keys.  Rows with 16 or fewer visible blocks
// select them all.  Otherwise the own block is joined by the 15 best older
// blocks under the strict order (score descending, block index ascending).
//
// One wavefront per row.  Each candidate is a 64-bit key (order-preserving
// score bits, then the complement of the block index), so all keys are
// distinct and the order above is plain integer order.  Fifteen rounds each
// take the wave-wide maximum among keys below the previous round's winner --
// no per-element state, the row is read from L1/L2.  The 16 winners are then
// ranked with a 16-way compare and written ascending.
#include "common.hpp"
#include "launch.hpp"

namespace msa {

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t o = __shfl_xor(v, off);
    v = o > v ? o : v;
  }
  return v;
}

__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ block_scores,
                                                   int32_t* __restrict__ sel,
                                                   const int32_t* __restrict__ seq_lens, int B,
                                                   int T, int max_blocks) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t rows = (int64_t)B * T * kGroups;
  if (row >= rows) return;
  const int b = (int)(row / ((int64_t)T * kGroups));
  const int t = (int)((row / kGroups) % T);
  const int L = seq_lens[b];
  int own = (L - T + t) / kBlock;
  own = max(0, min(own, max_blocks - 1));
  int32_t* out = sel + row * kTopK;
  if (own + 1 <= kTopK) {
    if (lane < kTopK) out[lane] = lane <= own ? lane : -1;
    return;
  }
  const float* S = block_scores + row * max_blocks;
  uint64_t prev = ~0ull;
  int32_t mine = -1;
  for (int r = 0; r < kTopK - 1; ++r) {
    uint64_t best = 0;
    for (int i = lane; i < own; i += 64) {
      const uint64_t key = ((uint64_t)order_key(S[i]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
      if (key < prev && key > best) best = key;
    }
    best = wave_max_u64(best);
    prev = best;
    if (lane == r) mine = (int32_t)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFu));
  }
  if (lane == kTopK - 1) mine = own;
  int rank = 0;
#pragma unroll
  for (int s = 0; s < kTopK; ++s) {
    const int32_t other = __shfl(mine, s);
    rank += (other < mine) ? 1 : 0;
  }
  if (lane < kTopK) out[rank] = mine;
}

hipError_t launch_topk(const ProblemArgs& p, const float* block_scores, int32_t* sel,
                       hipStream_t s) {
  const int64_t rows = (int64_t)p.B * p.T * kGroups;
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, block_scores,
                     sel, p.seq_lens, p.B, p.T, p.max_blocks);
  return hipGetLastError();
}

}  // namespace msa
