// Context-parallel (DCP) selection: each shard's local top-16 and the owner's
// exact merge.
//
// Source: "vLLM 為 MiniMax-M3.1-Flash 提供 Day-0 支援", sections "NVFP4
// indexer DCP" (NVIDIA and AMD): every GPU scores all four groups over its
// share of the pages and sends its local top-16 per group to the GPU that
// owns the group; the owner merges them into the final top-16 and the
// selection stays exact.  Shard s of P holds logical blocks s, s+P, s+2P, ...
// A shard's candidates for a (sequence, token, group) row are its blocks
// older than the row's own block (the owner forces the own block); it sends
// its 16 best under (score descending, block ascending), best first.  The
// owner keeps the own block and the 15 best of all candidates -- which are
// the 15 best older blocks overall, since each of those is among its own
// shard's 16 best -- and reports them ascending, as msa_block_topk does.
//
// Both kernels rank (score, block) pairs by select.hpp's 64-bit keys and
// narrow them with its radix cut, then rank the winners.
#include "common.hpp"
#include "launch.hpp"
#include "scan1.hpp"
#include "select.hpp"

namespace msa {

// One workgroup per row: the shard's 16 best blocks older than the own block.
constexpr int kShardThreads = 256;

template <int E>
__global__ __launch_bounds__(kShardThreads) void shard_topk_kernel(
    const float* __restrict__ block_scores, const int32_t* __restrict__ seq_lens, int T, int max_blocks,
    int shard, int num_shards, float* __restrict__ cand_scores, int32_t* __restrict__ cand_blocks) {
  __shared__ uint64_t won[kTopK];
  __shared__ uint32_t n_won;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int b = (int)(row / ((int64_t)T * kGroups));
  const int t = (int)((row / kGroups) % T);
  const int own = max(0, min((seq_lens[b] - T + t) / kBlock, max_blocks - 1));
  const float* S = block_scores + row * max_blocks;
  const int nc = shard_count(own, shard, num_shards);   // candidates: shard blocks < own
  uint64_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = tid + e * kShardThreads;
    const int blk = shard + num_shards * j;
    key[e] = j < nc ? select_key(S[blk], blk) : 0ull;
  }
  const uint32_t need = (uint32_t)min(nc, kTopK);
  uint64_t prefix = 0, mask = 0;   // nc <= 16: every candidate wins
  if (nc > kTopK) radix_cut<kShardThreads, E>(key, need, prefix, mask);
  if (tid == 0) n_won = 0;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (key[e] != 0ull && (key[e] & mask) >= prefix) {
      const uint32_t slot = atomicAdd(&n_won, 1u);
      if (slot < (uint32_t)kTopK) won[slot] = key[e];
    }
  }
  __syncthreads();
  if (tid < 64) {
    const bool mine_ok = tid < (int)need;
    const uint64_t mine = mine_ok ? won[tid] : 0ull;
    int rank = 0;   // winners with a larger key come first
    for (int l = 0; l < (int)need; ++l) rank += won[l] > mine ? 1 : 0;
    float* cs = cand_scores + row * kTopK;
    int32_t* cb = cand_blocks + row * kTopK;
    if (mine_ok) {
      const int blk = select_key_block(mine);
      cs[rank] = S[blk];
      cb[rank] = blk;
    } else if (tid < kTopK) {
      cs[tid] = __builtin_nanf("");
      cb[tid] = -1;
    }
  }
}

// One wave (workgroup of 64) per row: the own block plus the 15 best of the
// num_shards * 16 candidates (E = 2 per lane: up to 8 shards).
constexpr int kMergeMaxShards = 8;

__global__ __launch_bounds__(64) void topk_merge_kernel(
    const float* __restrict__ cand_scores, const int32_t* __restrict__ cand_blocks,
    const int32_t* __restrict__ seq_lens, int T, int max_blocks, int num_shards, int64_t rows,
    int32_t* __restrict__ sel) {
  __shared__ int32_t won[kTopK];
  __shared__ uint32_t n_won;
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int b = (int)(row / ((int64_t)T * kGroups));
  const int t = (int)((row / kGroups) % T);
  const int own = max(0, min((seq_lens[b] - T + t) / kBlock, max_blocks - 1));
  int32_t* out = sel + row * kTopK;
  if (own + 1 <= kTopK) {
    if (lane < kTopK) out[lane] = lane <= own ? lane : -1;
    return;
  }
  constexpr int E = kMergeMaxShards * kTopK / 64;
  uint64_t key[E];
  uint32_t nvalid = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int c = lane + 64 * e;            // candidate c: shard c / 16, slot c % 16
    const int sh = c / kTopK;
    key[e] = 0ull;
    if (sh < num_shards) {
      const size_t at = ((size_t)sh * rows + row) * kTopK + (c % kTopK);
      const int blk = cand_blocks[at];
      // only older blocks are candidates; anything else is ignored (the own block is added below)
      if (blk >= 0 && blk < own) key[e] = select_key(cand_scores[at], blk);
    }
    nvalid += (uint32_t)__popcll(__ballot(key[e] != 0ull));
  }
  const uint32_t need = min(nvalid, (uint32_t)(kTopK - 1));
  uint64_t prefix = 0, mask = 0;
  if (nvalid > need) radix_cut<64, E>(key, need, prefix, mask);
  if (lane == 0) n_won = 0;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (key[e] != 0ull && (key[e] & mask) >= prefix) {
      const uint32_t slot = atomicAdd(&n_won, 1u);
      if (slot < need) won[slot] = select_key_block(key[e]);
    }
  }
  __syncthreads();
  // the need winners and the own block, ranked ascending by block id; the rest -1
  const int32_t mine = lane < (int)need ? won[lane] : lane == (int)need ? own : 0x7FFFFFFF;
  int rank = 0;
#pragma unroll
  for (int k = 0; k < kTopK; ++k) rank += (__builtin_amdgcn_readlane(mine, k) < mine) ? 1 : 0;
  if (lane <= (int)need) out[rank] = mine;
  else if (lane < kTopK) out[lane] = -1;
}

hipError_t launch_shard_topk(const ProblemArgs& p, int shard, int num_shards, const float* block_scores,
                             float* cand_scores, int32_t* cand_blocks, hipStream_t s) {
  const int64_t rows = (int64_t)p.B * p.T * kGroups;
  const int nloc = shard_count(p.max_blocks, shard, num_shards);
  if (nloc <= 4 * kShardThreads)
    hipLaunchKernelGGL(shard_topk_kernel<4>, dim3((unsigned)rows), dim3(kShardThreads), 0, s, block_scores,
                       p.seq_lens, p.T, p.max_blocks, shard, num_shards, cand_scores, cand_blocks);
  else
    hipLaunchKernelGGL(shard_topk_kernel<32>, dim3((unsigned)rows), dim3(kShardThreads), 0, s, block_scores,
                       p.seq_lens, p.T, p.max_blocks, shard, num_shards, cand_scores, cand_blocks);
  return hipGetLastError();
}

hipError_t launch_topk_merge(const ProblemArgs& p, int num_shards, const float* cand_scores,
                             const int32_t* cand_blocks, int32_t* sel, hipStream_t s) {
  if (num_shards < 1 || num_shards > kMergeMaxShards) return hipErrorInvalidValue;
  const int64_t rows = (int64_t)p.B * p.T * kGroups;
  hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)rows), dim3(64), 0, s, cand_scores, cand_blocks,
                     p.seq_lens, p.T, p.max_blocks, num_shards, rows, sel);
  return hipGetLastError();
}

}  // namespace msa
