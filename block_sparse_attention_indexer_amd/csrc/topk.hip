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
// is plain integer order.  The row is read once into registers; a
// most-significant-digit radix select over 8-bit digits (LDS histogram, the
// digit found by one wave) narrows a key prefix until exactly 15 keys lie at
// or above it -- usually after two or three digits.  The 15 winners plus the
// own block are then ranked and written ascending.  Rows of up to 2,048
// blocks take one wave each (topk_wave_kernel; no workgroup barrier), longer
// rows one workgroup of 256 threads (topk_radix_kernel).
#include "common.hpp"
#include "launch.hpp"
#include "topk_wave.hpp"

namespace msa {

constexpr int kTopkThreads = 256;

template <int E, int NT = kTopkThreads>   // keys per thread: rows of up to NT*E older blocks
__global__ __launch_bounds__(NT) void topk_radix_kernel(
    const float* __restrict__ block_scores, int32_t* __restrict__ sel,
    const int32_t* __restrict__ seq_lens, int T, int max_blocks) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t pick_digit, pick_above, pick_count, n_won;
  __shared__ int32_t won[kTopK];

  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t row = blockIdx.x;
  const int b = (int)(row / ((int64_t)T * kGroups));
  const int t = (int)((row / kGroups) % T);
  const int L = seq_lens[b];
  int own = (L - T + t) / kBlock;
  own = max(0, min(own, max_blocks - 1));
  int32_t* out = sel + row * kTopK;
  if (own + 1 <= kTopK) {
    if (tid < kTopK) out[tid] = tid <= own ? tid : -1;
    return;
  }
  const float* S = block_scores + row * max_blocks;
  const int n = own;   // candidates: blocks 0 .. own-1

  // The row's loads are all issued before the first is used: ne (uniform) is
  // the number of slots that reach a candidate, and indices past the row are
  // clamped to its last candidate (their keys are dropped below).
  const int ne = min(E, (n + NT - 1) / NT);
  float v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    v[e] = 0.0f;
    if (e < ne) v[e] = S[min(tid + e * NT, n - 1)];
  }
  uint64_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = tid + e * NT;
    key[e] = (e < ne && i < n) ? ((uint64_t)order_key(v[e]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i) : 0ull;
  }
  // Index 0xFFFFFFFF is never a block, so a real key is never 0: 0 marks "no key".
  uint64_t prefix = 0, mask = 0;
  uint32_t need = kTopK - 1;
  if (tid == 0) n_won = 0;
#pragma unroll 1
  for (int shift = 56; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (key[e] != 0ull && (key[e] & mask) == prefix)
        atomicAdd(&hist[(uint32_t)(key[e] >> shift) & 255u], 1u);
    __syncthreads();
    if (tid < 64) {
      // lane l holds bins 4l..4l+3; find digit d with above(d) < need <= above(d) + hist[d]
      uint32_t h[4], s = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) { h[u] = hist[4 * lane + u]; s += h[u]; }
      // suffix sum over lanes above this one
      uint32_t incl = s;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_down(incl, off);
        if (lane + off < 64) incl += o;
      }
      uint32_t above = incl - s;          // keys in bins of higher lanes
#pragma unroll
      for (int u = 3; u >= 0; --u) {
        if (above < need && need <= above + h[u]) {
          pick_digit = 4 * lane + u;
          pick_above = above;
          pick_count = h[u];
        }
        above += h[u];
      }
    }
    __syncthreads();
    const uint32_t d = pick_digit, a = pick_above, c = pick_count;
    prefix |= (uint64_t)d << shift;
    mask |= 255ull << shift;
    need -= a;
    // pick_* is next written after two more barriers, so no barrier is needed here
    if (c == need) break;
  }
  // exactly 15 keys satisfy (key & mask) >= prefix
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (key[e] != 0ull && (key[e] & mask) >= prefix) {
      const uint32_t slot = atomicAdd(&n_won, 1u);
      if (slot < (uint32_t)(kTopK - 1)) won[slot] = tid + e * NT;
    }
  }
  __syncthreads();
  if (tid < 64) {
    const int32_t mine = lane < kTopK - 1 ? won[lane] : (lane == kTopK - 1 ? own : 0x7FFFFFFF);
    int rank = 0;
#pragma unroll
    for (int s = 0; s < kTopK; ++s) rank += (__shfl(mine, s) < mine) ? 1 : 0;
    if (lane < kTopK) out[rank] = mine;
  }
}

// Rows of up to 64*E blocks: one wave per row, the row held in registers and
// the digit search done with wave operations only (no workgroup barrier).
constexpr int kTopkWaveRows = 4;   // rows (waves) per workgroup
constexpr int kTopkManyRows = 4096;

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
  // Many rows: a wave per row keeps every CU busy.  Few rows (decode): a
  // workgroup per row shortens each row's critical path.
  const bool many = rows >= kTopkManyRows;
  if (many && p.max_blocks <= 64 * 16)
    hipLaunchKernelGGL(topk_wave_kernel<16>, wgrid, wblock, 0, s, block_scores, sel, p.seq_lens, p.T,
                       p.max_blocks);
  else if (many && p.max_blocks <= 64 * 32)
    hipLaunchKernelGGL(topk_wave_kernel<32>, wgrid, wblock, 0, s, block_scores, sel, p.seq_lens, p.T,
                       p.max_blocks);
  else if (p.max_blocks <= 8 * kTopkThreads)
    hipLaunchKernelGGL(topk_radix_kernel<8>, grid, block, 0, s, block_scores, sel, p.seq_lens, p.T,
                       p.max_blocks);
  else
    hipLaunchKernelGGL(topk_radix_kernel<32>, grid, block, 0, s, block_scores, sel, p.seq_lens,
                       p.T, p.max_blocks);
  return hipGetLastError();
}

}  // namespace msa
