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
//
// First a bound, then an exact rank.  Each wave finds, with 16 ballots over
// the top 16 bits of its keys, the largest prefix x_w such that at least C of
// its keys are >= x_w << 48; with tau the R-th largest x_w over the waves
// (C * R >= 15; C = max(2, ceil(15 / the number of waves full of candidates))),
// at least 15 keys are >= tau << 48, so tau is at most the row's 15th-best key
// and every winner is >= it.  The keys >= tau (a few dozen
// on block-max score rows: a 16-bit prefix resolves a score to 2^-7 relative)
// go to an LDS list, and one wave ranks them exactly (keys are distinct).  Two
// barriers instead of three per radix digit.  When more than 64 keys pass --
// scores that agree in their top 16 bits, as when a row's spread is small
// beside a common offset -- 16 more ballots set the low 16 bits of each
// wave's bound (the same argument over the keys' upper 32 bits); when still
// more than 64 pass (many equal scores), the radix cut over all keys decides.
// Optionally a row of the block table is copied into LDS while the selection
// runs (its loads go out with the score loads; up to TE * NT entries), so the
// caller reads the selected blocks' pages from LDS after its next barrier.
struct TablePrefetch {
  const int32_t* row = nullptr;   // nullptr: no copy
  int n = 0;
  int32_t* lds = nullptr;
};

template <int NT, int E, int TE = 0>
__device__ void select_row(const float* S, int own, int32_t* sel_sh, TablePrefetch tp = {}) {
  __shared__ int32_t won[kTopK - 1];
  __shared__ uint32_t n_won;
  __shared__ uint32_t tau_sh[NT / 64];
  __shared__ uint64_t cand[64];
  const int tid = threadIdx.x, lane = tid & 63;
  int32_t tv[TE > 0 ? TE : 1];
  auto table_loads = [&]() {
    if constexpr (TE > 0) {
      if (tp.row != nullptr) {
#pragma unroll
        for (int u = 0; u < TE; ++u) tv[u] = tid + u * NT < tp.n ? tp.row[tid + u * NT] : 0;
      }
    }
  };
  auto table_stores = [&]() {
    if constexpr (TE > 0) {
      if (tp.row != nullptr) {
#pragma unroll
        for (int u = 0; u < TE; ++u)
          if (tid + u * NT < tp.n) tp.lds[tid + u * NT] = tv[u];
      }
    }
  };
  if (own + 1 <= kTopK) {
    if (tid < kTopK) sel_sh[tid] = tid <= own ? tid : -1;
    table_loads();
    table_stores();
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
  table_loads();
  uint64_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = tid + e * NT;
    key[e] = (e < ne && i < own) ? select_key(v[e], i) : 0ull;
  }

  // the wave's bound x (wave-uniform): at least C of its keys have a prefix >= x.
  // C and R follow the number of waves whose 64 keys are all candidates (nwa):
  // R <= nwa of them reach the R-th largest bound, with C * R >= 15.
  constexpr int NW = NT / 64;
  static_assert(NW >= 1 && (NW & (NW - 1)) == 0 && NW <= 64, "a power-of-two number of waves");
  const int nwa = max(1, min(NW, min(own, NT) / 64));
  const int C = max(2, (kTopK - 1 + nwa - 1) / nwa);
  const int R = (kTopK - 1 + C - 1) / C;
  // pass 0 sets the top 16 bits of each wave's bound x (over the keys' upper
  // 32 bits); when more than 64 keys reach the resulting tau, pass 1 sets the
  // low 16 bits (x is then the wave's C-th largest score key itself)
  uint32_t x = 0, M = 0;
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    const uint32_t top = pass == 0 ? 0x80000000u : 0x8000u;
#pragma unroll 1
    for (int i = 0; i < 16; ++i) {
      const uint32_t c = x | (top >> i);   // c >= 1, so only real keys count
      uint32_t cnt = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) cnt += ballot_count((uint32_t)(key[e] >> 32) >= c);
      if (cnt >= (uint32_t)C) x = c;
    }
    if (pass == 1) __syncthreads();   // the first pass's tau_sh and n_won have been read
    if (lane == 0) tau_sh[tid >> 6] = x;
    if (tid == 0) n_won = 0;
    __syncthreads();
    // tau: the R-th largest wave bound, found in every wave (lane i < NW holds
    // bound i; ranks break ties by wave index, so exactly one lane has rank R-1)
    const uint32_t bnd = tau_sh[lane & (NW - 1)];
    int rk = 0;
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      const uint32_t o = (uint32_t)__builtin_amdgcn_readlane(bnd, j);
      rk += (o > bnd || (o == bnd && j < lane)) ? 1 : 0;
    }
    const uint64_t at_r = __ballot(lane < NW && rk == R - 1);
    const uint32_t tau = (uint32_t)__builtin_amdgcn_readlane(bnd, __builtin_ctzll(at_r));
    const uint64_t tau64 = (uint64_t)tau << 32;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (key[e] != 0ull && key[e] >= tau64) {
        const uint32_t slot = atomicAdd(&n_won, 1u);
        if (slot < 64u) cand[slot] = key[e];
      }
    }
    __syncthreads();
    M = n_won;   // >= 15; the same for every thread
    if (M <= 64u) break;
  }
  if (M <= 64u) {
    if (tid < 64) {
      // lane l holds candidate l (lanes past M hold 0, below every key); each
      // lane counts the candidates above its own, read lane by lane
      const uint64_t mine = (uint32_t)tid < M ? cand[tid] : 0ull;
      const uint32_t mhi = (uint32_t)(mine >> 32), mlo = (uint32_t)mine;
      int rank = 0;
#pragma unroll
      for (int jj = 0; jj < 64; ++jj) {
        // readlane yields a signed int: widen each half through uint32_t
        const uint64_t o = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(mhi, jj) << 32) |
                           (uint64_t)(uint32_t)__builtin_amdgcn_readlane(mlo, jj);
        rank += o > mine ? 1 : 0;
      }
      if ((uint32_t)tid < M && rank < kTopK - 1) won[rank] = select_key_block(mine);
      // the wave's own LDS writes are seen by its later reads
      const int32_t id = tid < kTopK - 1 ? won[tid] : (tid == kTopK - 1 ? own : 0x7FFFFFFF);
      int r2 = 0;
#pragma unroll
      for (int k = 0; k < kTopK; ++k) r2 += (__builtin_amdgcn_readlane(id, k) < id) ? 1 : 0;
      if (tid < kTopK) sel_sh[r2] = id;
    }
    table_stores();
    return;
  }

  // many keys at the bound (ties): the radix cut over every key
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
    for (int k = 0; k < kTopK; ++k) rank += (__builtin_amdgcn_readlane(mine, k) < mine) ? 1 : 0;
    if (tid < kTopK) sel_sh[rank] = mine;
  }
  table_stores();
}

}  // namespace msa
