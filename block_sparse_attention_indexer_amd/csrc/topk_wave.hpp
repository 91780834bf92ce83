// Top-16 selection for one row by a single wavefront (step 3 of MSA).
//
// Source: "vLLM 為 MiniMax-M3.1-Flash 提供 Day-0 支援", section "MSA primer":
// per group 16 blocks are kept, the newest block always among them.  With own+1 <= 16 visible blocks all are selected; otherwise the own
// block joins the 15 best older blocks under (score descending, block index
// ascending).  NaN ranks below every number.
//
// Each older block i is a 64-bit key: order-preserving score bits above the
// complemented index, so keys are distinct and the order above is integer
// order.  A most-significant-digit radix select over 8-bit digits narrows a
// key prefix until exactly 15 keys lie at or above it; each pass streams the
// row from memory (written just before by other workgroups), counts
// digits in a 256-bin histogram in LDS, and lets one wave scan find the digit.
// Only one wave takes part, so no workgroup barrier is needed.  The form that
// holds the row in registers first tries a threshold pass: the 15th largest of
// the 64 lane maxima bounds the 15th best key from below, and when at most 64
// keys reach it they are ranked directly, with no histogram atomics (on rows
// whose best keys crowd into a few lanes the radix select runs instead).
#pragma once
#include "common.hpp"

namespace msa {

struct WaveTopkLds {
  uint32_t hist[256];
  int32_t won[kTopK];
  uint32_t n_won;
  uint64_t cand[64];   // threshold candidates (wave_topk_row_regs)
};

__device__ __forceinline__ uint64_t readlane_u64(uint64_t x, int j) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)x, j);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(x >> 32), j);
  return ((uint64_t)hi << 32) | lo;
}

// The 15 winners in sh.won (any order) plus the own block, written ascending to
// out[0..15] by one wave.
template <bool COHERENT>
__device__ __forceinline__ void wave_rank_and_store(const WaveTopkLds& sh, int own, int32_t* out, int lane) {
  const int32_t mine = lane < kTopK - 1 ? sh.won[lane] : (lane == kTopK - 1 ? own : 0x7FFFFFFF);
  int rank = 0;
#pragma unroll
  for (int k = 0; k < kTopK; ++k) rank += (__shfl(mine, k) < mine) ? 1 : 0;
  if (lane < kTopK) {
    if (COHERENT) __hip_atomic_store(out + rank, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else out[rank] = mine;
  }
}

__device__ __forceinline__ uint64_t topk_key(float s, int i) {
  return ((uint64_t)order_key(s) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
}

// Scores written by other workgroups of the same kernel are read with
// device-coherent loads (they bypass the per-XCD caches that may hold stale
// lines); no cache-wide fence is needed.
__device__ __forceinline__ float coherent_load(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Writes out[0..15] (ascending block ids, -1 padded) for one row of scores S;
// the scores were written, and the selection is read, by other workgroups of
// the running kernel (device-coherent loads and stores).
__device__ inline void wave_topk_row(const float* S, int own, int32_t* out, WaveTopkLds& sh, int lane) {
  if (own + 1 <= kTopK) {
    if (lane < kTopK) __hip_atomic_store(out + lane, lane <= own ? lane : -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  const int n = own;               // candidates: blocks 0 .. own-1
  uint64_t prefix = 0, mask = 0;
  uint32_t need = kTopK - 1;
#pragma unroll 1
  for (int shift = 56; shift >= 0; shift -= 8) {
#pragma unroll
    for (int u = 0; u < 4; ++u) sh.hist[4 * lane + u] = 0;
    lds_wait();
    for (int i = lane; i < n; i += 64) {
      const uint64_t key = topk_key(coherent_load(S + i), i);
      if ((key & mask) == prefix) atomicAdd(&sh.hist[(uint32_t)(key >> shift) & 255u], 1u);
    }
    lds_wait();
    // lane l holds bins 4l..4l+3; find digit d with above(d) < need <= above(d) + hist[d]
    uint32_t h[4], s = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) { h[u] = sh.hist[4 * lane + u]; s += h[u]; }
    uint32_t incl = s;             // suffix sum over lanes >= this one
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_down(incl, off);
      if (lane + off < 64) incl += o;
    }
    uint32_t above = incl - s;     // keys in bins of higher lanes
    uint32_t d = 0, a = 0, c = 0;
    bool found = false;
#pragma unroll
    for (int u = 3; u >= 0; --u) {
      if (!found && above < need && need <= above + h[u]) {
        found = true;
        d = 4 * lane + u;
        a = above;
        c = h[u];
      }
      above += h[u];
    }
    const int src = __ffsll((unsigned long long)__ballot(found)) - 1;
    d = __shfl(d, src);
    a = __shfl(a, src);
    c = __shfl(c, src);
    prefix |= (uint64_t)d << shift;
    mask |= 255ull << shift;
    need -= a;
    if (c == need) break;          // wave-uniform
  }
  // exactly 15 keys satisfy (key & mask) >= prefix
  if (lane == 0) sh.n_won = 0;
  lds_wait();
  for (int i = lane; i < n; i += 64) {
    const uint64_t key = topk_key(coherent_load(S + i), i);
    if ((key & mask) >= prefix) {
      const uint32_t slot = atomicAdd(&sh.n_won, 1u);
      if (slot < (uint32_t)(kTopK - 1)) sh.won[slot] = i;
    }
  }
  lds_wait();
  wave_rank_and_store<true>(sh, own, out, lane);
}

// The same selection with the row held in registers: each lane loads its
// E scores once (lane + 64e), all loads in flight together, and the radix
// passes run on registers.  For rows of up to 64*E older blocks.  COHERENT:
// the scores were written, and the selection is read, by other workgroups of
// the running kernel (device-coherent loads and stores).
template <int E, bool COHERENT = true>
__device__ inline void wave_topk_row_regs(const float* S, int own, int32_t* out, WaveTopkLds& sh, int lane) {
  if (own + 1 <= kTopK) {
    if (lane < kTopK) {
      if (COHERENT) __hip_atomic_store(out + lane, lane <= own ? lane : -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else out[lane] = lane <= own ? lane : -1;
    }
    return;
  }
  const int n = own;
  // ne (uniform): the slots that reach a candidate; their loads are all issued
  // before the first is used, indices past the row clamped to its last candidate
  const int ne = min(E, (n + 63) / 64);
  float v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    v[e] = 0.0f;
    if (e < ne) {
      const float* p = S + min(lane + 64 * e, n - 1);
      v[e] = COHERENT ? coherent_load(p) : *p;
    }
  }
  uint32_t k32[E];
#pragma unroll
  for (int e = 0; e < E; ++e) k32[e] = (e < ne && lane + 64 * e < n) ? order_key(v[e]) : 0u;
  auto key_of = [&](int e) -> uint64_t {
    return ((uint64_t)k32[e] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(lane + 64 * e));
  };

  // Threshold pass.  tau, the 15th largest of the 64 lane maxima, is at most the
  // row's 15th best key (at least 15 lanes hold a key >= tau), so the 15 winners
  // are among the keys >= tau.  With n >= 16 candidates lanes 0..15 all hold one,
  // so exactly one lane has 14 larger lane maxima.  When at most 64 keys reach
  // tau (the usual case) they are ranked directly; otherwise the radix select
  // below runs.  No LDS atomics either way on this path.
  {
    uint64_t lmax = 0;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (lane + 64 * e < n) lmax = key_of(e) > lmax ? key_of(e) : lmax;
    int greater = 0;
#pragma unroll 1
    for (int j = 0; j < 64; ++j) greater += readlane_u64(lmax, j) > lmax ? 1 : 0;
    const uint64_t at15 = __ballot(lmax != 0ull && greater == kTopK - 2);
    const uint64_t tau = readlane_u64(lmax, __builtin_ctzll(at15));
    uint32_t ncand = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) ncand += (uint32_t)__popcll(__ballot(lane + 64 * e < n && key_of(e) >= tau));
    if (ncand <= 64) {
      uint32_t base = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool c = lane + 64 * e < n && key_of(e) >= tau;
        const uint64_t bm = __ballot(c);
        if (c) sh.cand[base + (uint32_t)__popcll(bm & ((1ull << lane) - 1ull))] = key_of(e);
        base += (uint32_t)__popcll(bm);
      }
      lds_wait();
      const uint64_t mine = (uint32_t)lane < ncand ? sh.cand[lane] : 0ull;
      int r = 0;
#pragma unroll 1
      for (uint32_t j = 0; j < ncand; ++j) r += sh.cand[j] > mine ? 1 : 0;
      if ((uint32_t)lane < ncand && r < kTopK - 1) sh.won[r] = (int32_t)(0xFFFFFFFFu - (uint32_t)mine);
      lds_wait();
      wave_rank_and_store<COHERENT>(sh, own, out, lane);
      return;
    }
  }

  uint64_t prefix = 0, mask = 0;
  uint32_t need = kTopK - 1;
#pragma unroll 1
  for (int shift = 56; shift >= 0; shift -= 8) {
#pragma unroll
    for (int u = 0; u < 4; ++u) sh.hist[4 * lane + u] = 0;
    lds_wait();
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint64_t key = key_of(e);
      if (lane + 64 * e < n && (key & mask) == prefix) atomicAdd(&sh.hist[(uint32_t)(key >> shift) & 255u], 1u);
    }
    lds_wait();
    uint32_t h[4], s = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) { h[u] = sh.hist[4 * lane + u]; s += h[u]; }
    uint32_t incl = s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_down(incl, off);
      if (lane + off < 64) incl += o;
    }
    uint32_t above = incl - s;
    uint32_t d = 0, a = 0, c = 0;
    bool found = false;
#pragma unroll
    for (int u = 3; u >= 0; --u) {
      if (!found && above < need && need <= above + h[u]) {
        found = true;
        d = 4 * lane + u;
        a = above;
        c = h[u];
      }
      above += h[u];
    }
    const int src = __ffsll((unsigned long long)__ballot(found)) - 1;
    d = __shfl(d, src);
    a = __shfl(a, src);
    c = __shfl(c, src);
    prefix |= (uint64_t)d << shift;
    mask |= 255ull << shift;
    need -= a;
    if (c == need) break;
  }
  if (lane == 0) sh.n_won = 0;
  lds_wait();
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (lane + 64 * e < n && (key_of(e) & mask) >= prefix) {
      const uint32_t slot = atomicAdd(&sh.n_won, 1u);
      if (slot < (uint32_t)(kTopK - 1)) sh.won[slot] = lane + 64 * e;
    }
  }
  lds_wait();
  wave_rank_and_store<COHERENT>(sh, own, out, lane);
}

}  // namespace msa
