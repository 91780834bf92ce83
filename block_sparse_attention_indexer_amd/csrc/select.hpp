// Workgroup-level selection helpers shared by the DCP kernels and the
// attention kernel that selects its own row's blocks.
//
// Source: "vLLM 為 MiniMax-M3.1-Flash 提供 Day-0 支援", section "MSA primer":
// 16 blocks per group, chosen by score, the newest one always included.  A (score,
// block) pair becomes one 64-bit key: order-preserving score bits (NaN
// lowest, -0 == +0) over the complemented block id, so keys are distinct and
// (score descending, block ascending) is plain integer order.
#pragma once
#include "common.hpp"

namespace msa {

constexpr int kMaxBlocksSelect = 8192;   // the largest max_blocks a problem may have

__device__ __forceinline__ uint64_t select_key(float score, int block) {
  return ((uint64_t)order_key(score) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)block);
}
__device__ __forceinline__ int select_key_block(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }

// The workgroup's keys (E per thread of NT, 0 = none, others distinct) hold at
// least `need` >= 1 keys.  Returns prefix/mask such that exactly `need` keys
// satisfy (key & mask) >= prefix.  Every thread of the workgroup calls it.
template <int NT, int E>
__device__ void radix_cut(const uint64_t (&key)[E], uint32_t need, uint64_t& prefix, uint64_t& mask) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t pick[3];
  const int tid = threadIdx.x, lane = tid & 63;
  prefix = 0;
  mask = 0;
#pragma unroll 1
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += NT) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (key[e] != 0ull && (key[e] & mask) == prefix) atomicAdd(&hist[(uint32_t)(key[e] >> shift) & 255u], 1u);
    __syncthreads();
    if (tid < 64) {
      // lane l holds bins 4l..4l+3; find digit d with above(d) < need <= above(d) + hist[d]
      uint32_t h[4], sum = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) { h[u] = hist[4 * lane + u]; sum += h[u]; }
      uint32_t incl = sum;             // suffix sum over lanes >= this one
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_down(incl, off);
        if (lane + off < 64) incl += o;
      }
      uint32_t above = incl - sum;
#pragma unroll
      for (int u = 3; u >= 0; --u) {
        if (above < need && need <= above + h[u]) {
          pick[0] = 4 * lane + u;
          pick[1] = above;
          pick[2] = h[u];
        }
        above += h[u];
      }
    }
    __syncthreads();
    const uint32_t d = pick[0], a = pick[1], c = pick[2];
    prefix |= (uint64_t)d << shift;
    mask |= 255ull << shift;
    need -= a;
    // pick is written again only after two more barriers
    if (c == need) break;   // uniform across the workgroup
  }
}


// The top-16 of one (sequence, token, group) row, selected by the whole
// workgroup (NT threads; every thread calls it; own is the same for all):
// with own+1 <= 16 visible blocks all of them, else the own block and the 15
// best older blocks (keys as above).  Leaves sel_sh[0..15] (LDS) ascending,
// padded with -1; the caller synchronises before reading it.  S: the row's
// block scores; E*NT >= own.
template <int NT, int E>
__device__ void select_row(const float* S, int own, int32_t* sel_sh) {
  __shared__ int32_t won[kTopK - 1];
  __shared__ uint32_t n_won;
  const int tid = threadIdx.x;
  if (own + 1 <= kTopK) {
    if (tid < kTopK) sel_sh[tid] = tid <= own ? tid : -1;
    return;
  }
  // all of the row's loads in flight before the first use (ne is uniform;
  // indices past the candidates are clamped and their keys dropped)
  const int ne = min(E, (own + NT - 1) / NT);
  float v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    v[e] = 0.0f;
    if (e < ne) v[e] = S[min(tid + e * NT, own - 1)];
  }
  uint64_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = tid + e * NT;
    key[e] = (e < ne && i < own) ? select_key(v[e], i) : 0ull;
  }
  uint64_t prefix, mask;
  radix_cut<NT, E>(key, kTopK - 1, prefix, mask);   // own >= 16 older blocks
  if (tid == 0) n_won = 0;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (key[e] != 0ull && (key[e] & mask) >= prefix) {
      const uint32_t slot = atomicAdd(&n_won, 1u);
      if (slot < (uint32_t)(kTopK - 1)) won[slot] = select_key_block(key[e]);
    }
  }
  __syncthreads();
  if (tid < 64) {
    const int32_t mine = tid < kTopK - 1 ? won[tid] : (tid == kTopK - 1 ? own : 0x7FFFFFFF);
    int rank = 0;
#pragma unroll
    for (int k = 0; k < kTopK; ++k) rank += (__shfl(mine, k) < mine) ? 1 : 0;
    if (tid < kTopK) sel_sh[rank] = mine;
  }
}

}  // namespace msa
