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
// holds the row in registers first bounds the 15th best key from below with
// the lanes' largest keys, and when at most 64 keys reach the bound they are
// ranked directly, with no histogram atomics (on rows whose best keys crowd
// into a few lanes the radix select runs instead).
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
  for (int k = 0; k < kTopK; ++k) rank += (__builtin_amdgcn_readlane(mine, k) < mine) ? 1 : 0;
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


// A 32-bit key of a score for the selection by one wave, in the score order
// of the selection: -0 and +0 equal, NaN 0 (below every number), other
// distinct scores distinct.  Non-negative scores keep their bits with the top
// bit set; negative ones take the two's-complement negation of their bits.
__device__ __forceinline__ uint32_t wave_score_key(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t s = (uint32_t)((int32_t)u >> 31);
  const uint32_t k = (u ^ (s | 0x80000000u)) - s;
  return x != x ? 0u : k;
}

// The same selection with the row held in registers: each lane loads its
// scores once (blocks lane + 64e, all loads in flight together) and the
// selection runs on registers.  For rows of up to 64*E older blocks.
// COHERENT: the scores were written, and the selection is read, by other
// workgroups of the running kernel (device-coherent loads and stores).
//
// First a bound, then an exact rank.  With 16 ballots the wave finds the
// largest 16-bit prefix x such that at least 15 lanes hold a key whose top 16
// bits reach x (each lane compares its largest key).  Those lanes hold at
// least 15 keys >= x << 16, so every winner is >= it.  The keys that reach
// the bound (the 15 winners and a few more on ordinary rows) go to an LDS
// list as (key, complemented block) pairs and are ranked exactly.  When more
// than 64 reach it (scores that agree in their top 16 bits, as when a row's
// spread is small beside its magnitude), 16 more ballots set the bound's low
// bits; when that still leaves more than 64 (many equal or crowded scores),
// or fewer than 15 lanes hold a number at all, a most-significant-digit radix
// select over all keys decides instead.
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
  // ne (uniform): the slots that hold a candidate; later slots are skipped
  const int ne = min(E, (n + 63) / 64);
  float v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    v[e] = 0.0f;
    if (lane + 64 * e < n) v[e] = COHERENT ? coherent_load(S + lane + 64 * e) : S[lane + 64 * e];
  }
  uint32_t k32[E];
  uint32_t lmax = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    k32[e] = 0;
    if (e < ne) {
      k32[e] = lane + 64 * e < n ? wave_score_key(v[e]) : 0u;
      lmax = max(lmax, k32[e]);
    }
  }
  auto key_of = [&](int e) -> uint64_t {
    return ((uint64_t)k32[e] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(lane + 64 * e));
  };

  // pass 0 sets the top 16 bits of x; when more than 64 keys reach that bound,
  // pass 1 sets the low 16 (x is then the 15th largest lane maximum itself)
  uint32_t x = 0;
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    const uint32_t top = pass == 0 ? 0x80000000u : 0x8000u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t c = x | (top >> i);
      if (ballot_count(lmax >= c) >= (uint32_t)(kTopK - 1)) x = c;
    }
    if (x == 0) break;   // fewer than 15 lanes hold a number
    // the keys >= x (x > 0 leaves out the empty slots), listed in slot order
    uint32_t M = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (e < ne) {
        const bool c = k32[e] >= x;
        const uint64_t bm = __ballot(c);
        if (bm != 0ull) {
          // position M + (the lanes below this one that hold a key >= x); past 64
          // entries the list is not used, so positions wrap instead of being tested
          const uint32_t pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bm, M));
          if (c) sh.cand[pos & 63u] = key_of(e);
          M += ballot_count(c);
        }
      }
    }
    if (M <= 64u) {
      // zero entries (below every key) up to a multiple of four, read four at a time
      if ((uint32_t)lane >= M && (uint32_t)lane < ((M + 3u) & ~3u)) sh.cand[lane] = 0ull;
      lds_wait();
      const uint64_t mine = (uint32_t)lane < M ? sh.cand[lane] : 0ull;
      int r = 0;
#pragma unroll 1
      for (uint32_t j = 0; j < M; j += 4) {
        const uint64_t a0 = sh.cand[j], a1 = sh.cand[j + 1], a2 = sh.cand[j + 2], a3 = sh.cand[j + 3];
        r += (a0 > mine ? 1 : 0) + (a1 > mine ? 1 : 0) + (a2 > mine ? 1 : 0) + (a3 > mine ? 1 : 0);
      }
      if ((uint32_t)lane < M && r < kTopK - 1) sh.won[r] = (int32_t)(0xFFFFFFFFu - (uint32_t)mine);
      lds_wait();
      wave_rank_and_store<COHERENT>(sh, own, out, lane);
      return;
    }
    // the list's writes are complete before the next pass writes it again
    lds_wait();
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
