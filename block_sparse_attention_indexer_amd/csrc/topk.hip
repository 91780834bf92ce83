// Step 3 of MSA: the top-16 blocks of every (sequence, query token, group)
// row, the query's own (most recent) block always kept.
//
// Source: "vLLM 為 MiniMax-M3.1-Flash 提供 Day-0 支援", section "MSA primer":
// per group 16 blocks are kept, the newest block always among them, which
// bounds a query at 2,048 keys.  Rows with 16 or fewer visible blocks
// select them all.  Otherwise the own block is joined by the 15 best older
// blocks under the strict order (score descending, block index ascending).
//
// Each older block becomes a 64-bit key: order-preserving score bits above
// the complemented block index, so the keys are distinct and the order above
// is plain integer order.  The row is read once into registers.  Rows of up
// to 2,048 blocks take one wave each (topk_wave_kernel; a bound from the
// lanes' largest keys, no workgroup barrier); longer rows one 1,024-thread
// workgroup each (topk_row_kernel), running the selecting attention's
// bound-then-rank selection (a per-wave bound from ballots over 16-bit key
// prefixes, then an exact rank of the few keys above it; a radix cut when
// many keys tie at the bound).  The 15 winners plus the own block are
// written ascending.
#include "common.hpp"
#include "launch.hpp"
#include "select.hpp"
#include "topk_wave.hpp"

namespace msa {

constexpr int kTopkThreads = 1024;   // threads per row in the workgroup form (E keys each)

template <int E, int NT = kTopkThreads>   // keys per thread: rows of up to NT*E older blocks
__global__ __launch_bounds__(NT) void topk_row_kernel(
    const float* __restrict__ block_scores, int32_t* __restrict__ sel,
    const int32_t* __restrict__ seq_lens, int T, int max_blocks) {
  __shared__ int32_t sel_sh[kTopK];
  const int64_t row = blockIdx.x;
  const int b = (int)(row / ((int64_t)T * kGroups));
  const int t = (int)((row / kGroups) % T);
  const int own = max(0, min((seq_lens[b] - T + t) / kBlock, max_blocks - 1));
  // the bound-then-rank selection (the radix cut when many keys tie at the bound)
  select_row<NT, E>(block_scores + row * max_blocks, own, sel_sh);
  __syncthreads();
  if (threadIdx.x < kTopK) sel[row * kTopK + threadIdx.x] = sel_sh[threadIdx.x];
}

// Rows of up to 64*E blocks: one wave per row, the row held in registers and
// its selection done with wave operations only (no workgroup barrier).
constexpr int kTopkWaveRows = 4;   // rows (waves) per workgroup

// Grid: (token, sequence); wave w of the workgroup takes group w.
template <int E>
__global__ __launch_bounds__(64 * kTopkWaveRows) void topk_wave_kernel(
    const float* __restrict__ block_scores, int32_t* __restrict__ sel,
    const int32_t* __restrict__ seq_lens, int T, int max_blocks) {
  static_assert(kTopkWaveRows == kGroups, "one wave per group of a (sequence, token)");
  __shared__ WaveTopkLds sh[kTopkWaveRows];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int t = blockIdx.x, b = blockIdx.y;
  const int64_t row = ((int64_t)b * T + t) * kGroups + w;
  const int own = max(0, min((seq_lens[b] - T + t) / kBlock, max_blocks - 1));
  wave_topk_row_regs<E, false>(block_scores + row * max_blocks, own, sel + row * kTopK, sh[w], lane);
}

hipError_t launch_topk(const ProblemArgs& p, const float* block_scores, int32_t* sel,
                       hipStream_t s) {
  const int64_t rows = (int64_t)p.B * p.T * kGroups;
  const dim3 grid((unsigned)rows), block(kTopkThreads);
  const dim3 wgrid((unsigned)p.T, (unsigned)p.B), wblock(64 * kTopkWaveRows);   // B <= 65535
  // Rows of up to 2,048 blocks: a wave per row, at any row count (c3_128k's
  // 256 rows take as long as in the workgroup form, 2,048 rows of 1,023 blocks
  // 6.9 against 23 us).  Longer rows: a 1,024-thread workgroup per row.
  if (p.max_blocks <= 64 * 16)
    hipLaunchKernelGGL(topk_wave_kernel<16>, wgrid, wblock, 0, s, block_scores, sel, p.seq_lens, p.T,
                       p.max_blocks);
  else if (p.max_blocks <= 64 * 32)
    hipLaunchKernelGGL(topk_wave_kernel<32>, wgrid, wblock, 0, s, block_scores, sel, p.seq_lens, p.T,
                       p.max_blocks);
  else if (p.max_blocks <= kTopkThreads)
    hipLaunchKernelGGL(topk_row_kernel<1>, grid, block, 0, s, block_scores, sel, p.seq_lens, p.T,
                       p.max_blocks);
  else if (p.max_blocks <= 2 * kTopkThreads)
    hipLaunchKernelGGL(topk_row_kernel<2>, grid, block, 0, s, block_scores, sel, p.seq_lens, p.T,
                       p.max_blocks);
  else
    hipLaunchKernelGGL(topk_row_kernel<8>, grid, block, 0, s, block_scores, sel, p.seq_lens,
                       p.T, p.max_blocks);
  return hipGetLastError();
}

}  // namespace msa
