// One-token decode scan (steps 1+2 of MSA for T = 1) as device code shared
// by the scan kernel and the scan with top-16 (msa_indexer_topk).
//
// Source: "vLLM 為 MiniMax-M3.1-Flash 提供 Day-0 支援", section "MSA primer":
// one index query per GQA group is dotted with every key of a single shared
// index-key head, and the scores are max-pooled into one score per block.
#pragma once
#include "common.hpp"
#include "launch.hpp"
#include "topk_wave.hpp"

namespace msa {

constexpr int kDecWaves = 4;   // waves per workgroup of the decode scans

// Single-token decode (T = 1): a streaming scan on the 4x4x4 f16 MFMA.
//
// With one query token there are only 4 query rows (the groups), so a 16-row
// MFMA tile would leave 12 rows empty.  The 4x4x4 form computes 16
// independent 4x4 blocks: block b = lane/4; lane (b, i) supplies row i of A
// (group i of the index query), lane (b, j) supplies column j of B (key
// 4b+j), and lane (b, j) receives all 4 rows of its column.  So every lane
// owns one key of a 64-key set and gets that key's 4 group scores.
// NVFP4 keys are contracted one 16-dim scale group at a time (4 MFMAs on the
// unscaled E2M1 values; products and sums exact), then each group's partial
// dot is multiplied by its E4M3 scale in one fp32 FMA -- one FMA per 16
// elements instead of a multiply per element.  FP8 keys chain all 32 MFMAs.
// A lane reads its own key's row (4 x 16 B of NVFP4 codes + 8 B of scales,
// or 8 x 16 B of FP8); the loads of a set together cover every cache line
// of the set's 64 rows.
template <int KT> struct KeySet;
template <> struct KeySet<2> { uint4 c[4]; uint2 s; };   // NVFP4: 64 B codes + 8 scale bytes
template <> struct KeySet<1> { uint4 c[8]; };            // FP8: 128 B

template <int KT>
__device__ __forceinline__ void load_key_set(KeySet<KT>& u, const uint8_t* __restrict__ kdata,
                                             const uint8_t* __restrict__ kscales, size_t row) {
  if constexpr (KT == 2) {
    const uint4* src = reinterpret_cast<const uint4*>(kdata + row * kNvfp4RowBytes);
#pragma unroll
    for (int q = 0; q < 4; ++q) u.c[q] = src[q];
    u.s = *reinterpret_cast<const uint2*>(kscales + row * kNvfp4ScaleBytes);
  } else {
    const uint4* src = reinterpret_cast<const uint4*>(kdata + row * kHeadDim);
#pragma unroll
    for (int q = 0; q < 8; ++q) u.c[q] = src[q];
  }
}

__device__ __forceinline__ uint32_t dword_of(const uint4& v, int k) {
  return k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
}
__device__ __forceinline__ h4 cat4(h2 a, h2 b) { return h4{a[0], a[1], b[0], b[1]}; }
// E4M3 byte k (0..3, a constant after unrolling) of w, as float.
__device__ __forceinline__ float e4m3_byte_to_f(uint32_t w, int k) {
  switch (k) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8(w, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8(w, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8(w, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8(w, 3);
  }
}

constexpr int kDec1Chains = 2;   // independent MFMA accumulation chains (divides 8)

// The 4 group scores of this lane's key (before the tensor scales).
// A[c] gives dims 4c .. 4c+3 of this lane's group (lane % 4) -- for the
// FP8-rounded NVFP4 reading (FP8MODE) dims 8i + {0,2,4,6} (c = 2i) and
// 8i + {1,3,5,7} (c = 2i+1), the order the table decode produces.
// FP8MODE: each element is the E4M3 re-rounding of e2m1 x scale, read from
// the 2 KB table in LDS (`lut`, two words per scale byte), so the scale
// cannot be applied after the dot: all 32 MFMAs take decoded values.
template <int KT, bool FP8MODE, typename ASrc>
__device__ __forceinline__ f4 score_key_set(const KeySet<KT>& u, const ASrc& A, const uint32_t* lut) {
  f4 tot = {0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (KT == 2 && FP8MODE) {
    f4 part[2] = {f4{0.0f, 0.0f, 0.0f, 0.0f}, f4{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int sg = 0; sg < 8; ++sg) {              // scale group sg: dims 16sg .. 16sg+15
      const uint32_t sb = ((sg < 4 ? u.s.x : u.s.y) >> (8 * (sg & 3))) & 0xFFu;
      const uint2 lh = reinterpret_cast<const uint2*>(lut)[sb];   // one 8-byte LDS read
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const h8 v = fp4x8_lut_to_h8(dword_of(u.c[sg >> 1], 2 * (sg & 1) + h), lh.x, lh.y);
        const int c = 4 * sg + 2 * h;
        part[h] = __builtin_amdgcn_mfma_f32_4x4x4f16(A[c], h4{v[0], v[1], v[2], v[3]}, part[h], 0, 0, 0);
        part[h] = __builtin_amdgcn_mfma_f32_4x4x4f16(A[c + 1], h4{v[4], v[5], v[6], v[7]}, part[h], 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) tot[i] = part[0][i] + part[1][i];
  } else if constexpr (KT == 2) {
    // kDec1Chains scale groups at a time, their MFMA chains interleaved
#pragma unroll
    for (int s0 = 0; s0 < 8; s0 += kDec1Chains) {
      f4 part[kDec1Chains];
#pragma unroll
      for (int g = 0; g < kDec1Chains; ++g) part[g] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int h = 0; h < 2; ++h) {               // dword 2s+h: dims 16s+8h .. +7, low nibble first
#pragma unroll
        for (int e = 0; e < 2; ++e) {
#pragma unroll
          for (int g = 0; g < kDec1Chains; ++g) {
            const int s = s0 + g;
            const uint32_t w = dword_of(u.c[s >> 1], 2 * (s & 1) + h);
            const h4 bv = e == 0 ? cat4(fp4x2_to_h2<0>(w), fp4x2_to_h2<1>(w)) : cat4(fp4x2_to_h2<2>(w), fp4x2_to_h2<3>(w));
            part[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(A[4 * s + 2 * h + e], bv, part[g], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int g = 0; g < kDec1Chains; ++g) {
        const int s = s0 + g;
        const float sc = e4m3_byte_to_f(s < 4 ? u.s.x : u.s.y, s & 3);
#pragma unroll
        for (int i = 0; i < 4; ++i) tot[i] = fmaf(sc, part[g][i], tot[i]);
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < 32; ++c) {                // dword c = dims 4c .. 4c+3
      const uint32_t w = dword_of(u.c[c >> 2], c & 3);
      tot = __builtin_amdgcn_mfma_f32_4x4x4f16(A[c], cat4(fp8x2_to_h2<false>(w), fp8x2_to_h2<true>(w)), tot, 0, 0, 0);
    }
  }
  return tot;
}

// The index-query operand of a lane: 32 x h4 in registers.  (Reading it from
// an LDS copy per MFMA instead frees 64 VGPRs but measured slower.)
struct AInRegs {
  h4 v[32];
  __device__ __forceinline__ h4 operator[](int c) const { return v[c]; }
};

constexpr int kDec1PagesPerWave = 16;

// Each wave keeps a ring of kDec1Ring key sets in registers, kDec1Ring - 1 of
// them in flight while one is contracted; at ~170 VGPRs that is two
// workgroups per CU, so about 24 sets (110 KB) are in flight per CU.
constexpr int kDec1Ring = 4;

// FUSE: the last workgroup of a sequence to finish (a per-sequence arrival
// counter in `counters`, zero before the call and reset to zero by that
// workgroup) also selects the sequence's top-16 blocks, one wave per group.
// Nothing waits on another workgroup: the last arrival does the work.
// Everything one workgroup of the one-token scan needs.
struct Scan1Args {
  const uint8_t* idx_q;
  const uint8_t* kdata;
  const uint8_t* kscales;
  int64_t num_pages;
  const int32_t* seq_lens;
  const int32_t* table;
  int max_blocks;
  float sigma;
  float* block_scores;
  float* token_scores;
  // Context-parallel shard: the scan covers logical blocks blk_off + blk_step*j
  // (j = 0, 1, ...) only, writing their scores at those positions; 0 and 1 for
  // the whole context.
  int blk_off = 0;
  int blk_step = 1;
  // Shared-prefix decode: device [B], nullable -- the first skip[b] logical
  // blocks of sequence b are scored by another kernel and left untouched here.
  const int32_t* skip = nullptr;
};
// Blocks of the shard among the first n logical blocks.
__host__ __device__ __forceinline__ int shard_count(int n, int off, int step) {
  return n > off ? (n - off + step - 1) / step : 0;
}
constexpr int kScan1Blocks = kDecWaves * kDec1PagesPerWave;   // blocks per workgroup chunk

// Blocks [w0, wend) (local shard indices, wend - w0 <= PPW) of sequence b,
// scored by one wave: blocks at or past the sequence's end get -inf, the others
// their pooled score (NaN for an unreadable page).  pooled: this wave's
// [PPW][4] LDS slice.  b, w0 and wend are wave-uniform.
// COHERENT: the pooled scores are stored device-coherently, for another
// workgroup of the same kernel to read.
template <int KT, bool TOKSC, bool COHERENT, int PPW, bool FP8MODE>
__device__ __forceinline__ void scan1_blocks(const Scan1Args& a, int b, int w0, int wend, const uint32_t* lut,
                                             float (*pooled)[kGroups]) {
  static_assert(PPW >= 1 && PPW <= 64, "page ids are held one per lane");
  const int lane = threadIdx.x & 63;
  const float NEG_INF = -__builtin_inff();
  const float QNAN = __builtin_nanf("");
  const int L = a.seq_lens[b];
  const int nb = min((L + kBlock - 1) / kBlock, a.max_blocks);
  // local index j of the shard is logical block gblk(j)
  auto gblk = [&](int j) { return a.blk_off + a.blk_step * j; };
  const int nb_loc = shard_count(nb, a.blk_off, a.blk_step);
  const int nreal = max(0, min(wend, nb_loc) - w0);

  int pid = 0;
  if (lane < nreal) pid = a.table[(size_t)b * a.max_blocks + gblk(w0 + lane)];
  const int pid_bad = (pid < 0 || (int64_t)pid >= a.num_pages) ? 1 : 0;
  const int pid_safe = pid_bad ? 0 : pid;

  // A operand: this lane's group g = lane % 4, all 128 dims as f16
  AInRegs A;
  {
    const uint4* src = reinterpret_cast<const uint4*>(a.idx_q + ((size_t)b * kGroups + (lane & 3)) * kHeadDim);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint4 v = src[q];
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
      if constexpr (FP8MODE) {   // dims 16q+8h + {0,2,4,6} then + {1,3,5,7}
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const h8 d = fp8x8_to_h8(wv[2 * h], wv[2 * h + 1]);
          A.v[4 * q + 2 * h] = h4{d[0], d[2], d[4], d[6]};
          A.v[4 * q + 2 * h + 1] = h4{d[1], d[3], d[5], d[7]};
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) A.v[4 * q + k] = cat4(fp8x2_to_h2<false>(wv[k]), fp8x2_to_h2<true>(wv[k]));
      }
    }
  }
  const size_t tstride = (size_t)a.max_blocks * kBlock;
  float* tsc = TOKSC ? a.token_scores + (size_t)b * kGroups * tstride : nullptr;

  // blocks of this range past the sequence: -inf
  for (int e = lane; e < kGroups * (wend - w0 - nreal); e += 64) {
    const int n = wend - w0 - nreal;
    a.block_scores[((size_t)b * kGroups + e / n) * a.max_blocks + gblk(w0 + nreal + e % n)] = NEG_INF;
  }
  if (TOKSC) {
    for (int i = w0 + nreal; i < wend; ++i)
#pragma unroll
      for (int g = 0; g < kGroups; ++g)
        for (int kk = lane; kk < kBlock; kk += 64) tsc[g * tstride + (size_t)gblk(i) * kBlock + kk] = NEG_INF;
  }

  const int nsets = 2 * nreal;               // two 64-key sets per page
  f4 bmax = {NEG_INF, NEG_INF, NEG_INF, NEG_INF};
  // score set u (64 keys of block u/2) and fold it into the block maxima
  auto consume = [&](int u, const KeySet<KT>& cur) {
    const int blk = u >> 1, half = u & 1;
    f4 sc = score_key_set<KT, FP8MODE>(cur, A, lut);
    const int key = gblk(w0 + blk) * kBlock + half * 64 + lane;
    if (gblk(w0 + blk) == nb - 1) {              // only the last block can hold keys past L - 1
      if (key >= L) sc = f4{NEG_INF, NEG_INF, NEG_INF, NEG_INF};
    }
    bmax[0] = fmaxf(bmax[0], sc[0]);
    bmax[1] = fmaxf(bmax[1], sc[1]);
    bmax[2] = fmaxf(bmax[2], sc[2]);
    bmax[3] = fmaxf(bmax[3], sc[3]);
    if constexpr (TOKSC) {
#pragma unroll
      for (int g = 0; g < kGroups; ++g) tsc[g * tstride + key] = key < L ? sc[g] * a.sigma : NEG_INF;
    }
    if (half == 1) {
      const bool bad = __builtin_amdgcn_readlane(pid_bad, blk) != 0;
      const float m = wave_max4(bmax);
      if ((lane & 15) == 0) pooled[blk][2 * (lane >> 5) + ((lane >> 4) & 1)] = bad ? QNAN : m * a.sigma;
      if (TOKSC && bad) {
#pragma unroll
        for (int g = 0; g < kGroups; ++g)
          for (int kk = lane; kk < kBlock; kk += 64) tsc[g * tstride + (size_t)gblk(w0 + blk) * kBlock + kk] = QNAN;
      }
      bmax = f4{NEG_INF, NEG_INF, NEG_INF, NEG_INF};
    }
  };
  {
    // a ring of kDec1Ring key sets in registers, kDec1Ring - 1 loads ahead; loads
    // past the wave's last set re-read that set (cache hits), so that every
    // load is unconditional and each wait covers exactly one set
    constexpr int R = kDec1Ring;
    KeySet<KT> buf[R];
    auto load_set = [&](KeySet<KT>& dst, int u) {
      const int uc = min(u, nsets - 1);
      load_key_set<KT>(dst, a.kdata, a.kscales,
                       (size_t)__builtin_amdgcn_readlane(pid_safe, uc >> 1) * kBlock + (uc & 1) * 64 + lane);
    };
#pragma unroll
    for (int r = 0; r < R - 1; ++r) load_set(buf[r], r);
    for (int u0 = 0; u0 < nsets; u0 += R) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        load_set(buf[(r + R - 1) % R], u0 + r + R - 1);
        if (u0 + r < nsets) consume(u0 + r, buf[r]);
      }
    }
  }
  lds_wait();
  for (int e = lane; e < kGroups * nreal; e += 64) {
    const int g = e / nreal, i = e % nreal;
    float* dst = a.block_scores + ((size_t)b * kGroups + g) * a.max_blocks + gblk(w0 + i);
    if (COHERENT)   // device-coherent store: read back by another workgroup in this kernel
      __hip_atomic_store(dst, pooled[i][g], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      *dst = pooled[i][g];
  }
  lds_wait();   // the slice is reused by the wave's next range
}

// One workgroup's chunk of the scan: shard blocks [4*PPW*chunk, +4*PPW) of
// sequence b, PPW per wave (blocks past the sequence get -inf).  Smaller PPW
// gives more, shorter chunks: used when the grid would not fill the chip.
template <int KT, bool TOKSC, bool COHERENT, int PPW = kDec1PagesPerWave, bool FP8MODE = false>
__device__ __forceinline__ void scan1_chunk(const Scan1Args& a, int b, int chunk, const uint32_t* lut = nullptr) {
  __shared__ float pooled[kDecWaves][PPW][kGroups];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nloc = shard_count(a.max_blocks, a.blk_off, a.blk_step);
  const int wbase = (chunk * kDecWaves + wave) * PPW;
  const int wend = min(wbase + PPW, nloc);
  // local blocks below skip[b] belong to the shared-prefix kernel
  const int w0 = a.skip == nullptr ? wbase : max(wbase, shard_count(a.skip[b], a.blk_off, a.blk_step));
  if (w0 < wend) scan1_blocks<KT, TOKSC, COHERENT, PPW, FP8MODE>(a, b, w0, wend, lut, pooled[wave]);
}

// The whole one-token scan spread evenly: the blocks of all sequences, taken
// in (sequence, block) order, are cut into one contiguous share per wave of
// the grid (sizes differ by at most one), and each share into ranges that end
// at sequence boundaries or after 64 blocks.  With ragged contexts every CU
// then reads the same number of pages, where per-sequence chunks leave some
// CUs a chunk more than others.  The blocks past each sequence (up to
// max_blocks) are spread the same way and get -inf.  SKIP: the blocks of a
// sequence of prefix group q start at groups.blocks[q] (those below belong to
// another kernel), and its -inf run at the larger of that and its block count.  pre, padpre: LDS, B + 1 ints
// each, filled here with the exclusive prefix sums of the sequences' scanned
// and -inf block counts (padpre only with SKIP; without it the -inf counts
// follow from pre).
constexpr int kFlatMaxSeqs = 1024;   // sequences the prefix sums in LDS cover
template <int KT, bool FP8MODE, bool SKIP>
__device__ __forceinline__ void scan1_flat(const Scan1Args& a, int B, const uint32_t* lut, int* pre, int* padpre,
                                           const PrefixGroups& groups) {
  __shared__ float pooled[kDecWaves][64][kGroups];
  __shared__ int wsum[kDecWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // exclusive prefix sums of v over the threads of the workgroup: returns
  // (sum over the threads before this one, sum over all of them)
  auto block_scan = [&](int v, int& total) {
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int w2 = 0; w2 < kDecWaves; ++w2) {
      before += w2 < wave ? wsum[w2] : 0;
      total += wsum[w2];
    }
    __syncthreads();   // wsum is rewritten by the next scan
    return before + x - v;
  };
  int carry = 0, pcarry = 0;
  for (int base = 0; base < B; base += kDecWaves * 64) {
    const int i = base + tid;
    int v = 0, pv = 0;
    if (i < B) {
      const int nbi = min((a.seq_lens[i] + kBlock - 1) / kBlock, a.max_blocks);
      int sk = 0;   // the shared blocks of i's prefix group (a uniform loop over the groups)
      if constexpr (SKIP) {
        for (int q = 0; q < groups.n; ++q)
          if (i >= groups.start[q] && i < groups.start[q + 1]) sk = groups.blocks[q];
      }
      v = max(0, nbi - sk);
      pv = a.max_blocks - max(nbi, sk);
    }
    int total;
    const int ex = block_scan(v, total);
    if (i < B) pre[i] = carry + ex;
    carry += total;
    if constexpr (SKIP) {
      const int pex = block_scan(pv, total);
      if (i < B) padpre[i] = pcarry + pex;
      pcarry += total;
    }
  }
  if (tid == 0) {
    pre[B] = carry;
    if constexpr (SKIP) padpre[B] = pcarry;
  }
  __syncthreads();
  // padpre[b]: -inf blocks of the sequences before b (b * max_blocks - pre[b] without SKIP)
  auto pad_before = [&](int bb) -> int64_t {
    if constexpr (SKIP) return padpre[bb];
    else return (int64_t)bb * a.max_blocks - pre[bb];
  };
  const int64_t N = carry;                                   // blocks to scan, all sequences
  const int64_t W = (int64_t)gridDim.x * kDecWaves;
  const int64_t gw = (int64_t)blockIdx.x * kDecWaves + wave;
  int s = (int)(N * gw / W);
  const int s1 = (int)(N * (gw + 1) / W);
  // the sequence holding flat block s: the last b with pre[b] <= s
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= s) lo = mid; else hi = mid;
  }
  int b = lo;
  while (s < s1) {
    while (pre[b + 1] <= s) ++b;                             // sequences with no block
    // first block of b's range: its skip count, which is max_blocks less its
    // -inf and scanned block counts
    const int j = s - pre[b] +
                  (SKIP ? a.max_blocks - (padpre[b + 1] - padpre[b]) - (pre[b + 1] - pre[b]) : 0);
    const int n = min(min(s1, pre[b + 1]) - s, 64);
    scan1_blocks<KT, false, false, 64, FP8MODE>(a, b, j, j + n, lut, pooled[wave]);
    s += n;
  }
  // -inf past each sequence: pad entry p of sequence b is block
  // max_blocks - (its -inf count) + (p - pad_before(b))
  const int64_t P = pad_before(B);
  const int64_t p0 = P * gw / W, p1 = P * (gw + 1) / W;
  const float NEG_INF = -__builtin_inff();
  for (int64_t pp = p0 + lane; pp < p1; pp += 64) {
    int l2 = 0, h2 = B;   // the last b with pad_before(b) <= pp
    while (h2 - l2 > 1) {
      const int mid = (l2 + h2) >> 1;
      if (pad_before(mid) <= pp) l2 = mid; else h2 = mid;
    }
    const int64_t pb = pad_before(l2);
    const int blk = a.max_blocks - (int)(pad_before(l2 + 1) - pb) + (int)(pp - pb);
#pragma unroll
    for (int g = 0; g < kGroups; ++g) a.block_scores[((size_t)l2 * kGroups + g) * a.max_blocks + blk] = NEG_INF;
  }
}

// After scan1_chunk: counts this workgroup's chunk of sequence b in
// arrival[b] (zero before the sequence's first chunk; reset to zero by the
// last); the workgroup that completes the sequence (nchunks chunks) selects
// its top-16 blocks for the four groups, one wave per group, and returns
// true.  The scores and -inf fills are complete (not merely issued) before
// the count, and the count is taken at system scope, so the last arrival
// reads every workgroup's scores with device-coherent loads.  No cache-wide
// fence: on a GPU with one L2 per XCD that would write back and invalidate
// the whole L2.  The selection is stored device-coherently.
__device__ __forceinline__ bool scan1_select_if_last(const Scan1Args& a, int b, int nchunks, int32_t* sel,
                                                     uint32_t* arrival) {
  __shared__ int last_sh;
  __shared__ WaveTopkLds tk[kDecWaves];
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    last_sh = __hip_atomic_fetch_add(&arrival[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) ==
                      (uint32_t)nchunks - 1 ? 1 : 0;
  __syncthreads();
  if (!last_sh) return false;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (threadIdx.x == 0) __hip_atomic_store(&arrival[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  const int L = a.seq_lens[b];
  const int own = max(0, min((L - 1) / kBlock, a.max_blocks - 1));
  const size_t r = (size_t)b * kGroups + wave;   // one group per wave
  if (own <= 64 * 16)
    wave_topk_row_regs<16>(a.block_scores + r * a.max_blocks, own, sel + r * kTopK, tk[wave], lane);
  else
    wave_topk_row(a.block_scores + r * a.max_blocks, own, sel + r * kTopK, tk[wave], lane);
  return true;
}

}  // namespace msa
