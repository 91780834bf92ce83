// Steps 1+2 of MSA for decode and speculative decode (T <= 4 query tokens):
// index scores over the paged index-key cache, max-pooled per 128-token block
// in the same pass.  (Many query tokens: indexer_prefill.hip.)
//
// Source: "vLLM 為 MiniMax-M3.1-Flash 提供 Day-0 支援", section "MSA primer":
// one index query per GQA group is dotted with every key of a single shared
// index-key head, and the scores are max-pooled into one score per block.
// Decode is bound by reading the index keys of the whole context (128 B per
// token in FP8, 72 B in NVFP4), so these kernels are coalesced streaming
// scans: every page is read once, dequantised in registers, contracted on f16
// MFMAs against all query rows at once, and reduced to one max per (row,
// block) before anything is written.  Per-key scores are written only when
// the caller asks for them (a separate template instance).
#include "common.hpp"
#include "launch.hpp"
#include "topk_wave.hpp"

namespace msa {

// ---------------------------------------------------------------------------
// Decode and speculative decode (T <= 4): a streaming scan.
//
// Grid (page range, sequence); each of the 4 waves of a workgroup owns
// kDecPagesPerWave consecutive logical blocks.  A wave reads its page ids
// once (one lane per block), then walks its pages in units of TPU key tiles
// (16 keys each).  With PIPE the next unit's loads are issued before the
// current unit is contracted, so memory and math overlap inside the wave;
// those loads are unconditional (past the last unit a wave re-reads its last
// unit, which hits in cache) so that every wait covers exactly one unit.
// The MFMA rows are 4 tokens x 4 groups.  sigma > 0 is applied to the pooled
// maximum only: fl(sigma*x) is monotone in x, so this equals the maximum of
// the scaled scores.
#ifndef MSA_DEC_PAGES_PER_WAVE
#define MSA_DEC_PAGES_PER_WAVE 8
#endif
#ifndef MSA_DEC_TPU
#define MSA_DEC_TPU 4
#endif
#ifndef MSA_DEC_PIPE
#define MSA_DEC_PIPE 1
#endif
constexpr int kDecWaves = 4;
constexpr int kDecPagesPerWave = MSA_DEC_PAGES_PER_WAVE;

template <int KT, int TPU> struct IdxUnit;
template <int TPU> struct IdxUnit<2, TPU> { uint4 c[TPU]; uint32_t s[TPU]; };   // NVFP4 codes + 2 scale bytes
template <int TPU> struct IdxUnit<1, TPU> { uint4 c[TPU][2]; };                 // FP8

template <int KT, int TPU>
__device__ __forceinline__ void load_idx_unit(IdxUnit<KT, TPU>& u, const uint8_t* __restrict__ kdata,
                                              const uint8_t* __restrict__ kscales, size_t row0, int Q) {
#pragma unroll
  for (int kt = 0; kt < TPU; ++kt) {
    const size_t row = row0 + kt * 16;
    if constexpr (KT == 2) {
      u.c[kt] = *reinterpret_cast<const uint4*>(kdata + row * kNvfp4RowBytes + 16 * Q);
      u.s[kt] = *reinterpret_cast<const uint16_t*>(kscales + row * kNvfp4ScaleBytes + 2 * Q);
    } else {
      const uint4* src = reinterpret_cast<const uint4*>(kdata + row * kHeadDim + 32 * Q);
      u.c[kt][0] = src[0];
      u.c[kt][1] = src[1];
    }
  }
}

// One 16-key tile -> the four 32-dim B fragments (k-chunk c = dims 32Q+8c .. +7).
template <int KT, bool FP8MODE, int TPU>
__device__ __forceinline__ void decode_idx_tile(const IdxUnit<KT, TPU>& u, int kt, const uint32_t* lut,
                                                h8 (&Bc)[4]) {
  if constexpr (KT == 2) {
    const uint32_t w[4] = {u.c[kt].x, u.c[kt].y, u.c[kt].z, u.c[kt].w};
    if constexpr (FP8MODE) {
      const uint32_t s0 = u.s[kt] & 0xFFu, s1 = (u.s[kt] >> 8) & 0xFFu;
      const uint32_t l0 = lut[2 * s0], h0 = lut[2 * s0 + 1];
      const uint32_t l1 = lut[2 * s1], h1 = lut[2 * s1 + 1];
      Bc[0] = fp4x8_lut_to_h8(w[0], l0, h0);
      Bc[1] = fp4x8_lut_to_h8(w[1], l0, h0);
      Bc[2] = fp4x8_lut_to_h8(w[2], l1, h1);
      Bc[3] = fp4x8_lut_to_h8(w[3], l1, h1);
    } else {
      const h2 sc = fp8x2_to_h2<false>(u.s[kt]);
      const h8 s0 = h8{sc[0], sc[0], sc[0], sc[0], sc[0], sc[0], sc[0], sc[0]};
      const h8 s1 = h8{sc[1], sc[1], sc[1], sc[1], sc[1], sc[1], sc[1], sc[1]};
      Bc[0] = fp4x8_to_h8(w[0]) * s0;
      Bc[1] = fp4x8_to_h8(w[1]) * s0;
      Bc[2] = fp4x8_to_h8(w[2]) * s1;
      Bc[3] = fp4x8_to_h8(w[3]) * s1;
    }
  } else {
    Bc[0] = fp8x8_to_h8(u.c[kt][0].x, u.c[kt][0].y);
    Bc[1] = fp8x8_to_h8(u.c[kt][0].z, u.c[kt][0].w);
    Bc[2] = fp8x8_to_h8(u.c[kt][1].x, u.c[kt][1].y);
    Bc[3] = fp8x8_to_h8(u.c[kt][1].z, u.c[kt][1].w);
  }
}

// Contract one unit: per tile four 16x16x32 MFMAs and the masked running max.
// Lane (Q, j) gets token Q, groups 0..3 of key `key0 + 16*kt` (key0 includes j).
template <int KT, bool FP8MODE, bool TOKSC, int TPU>
__device__ __forceinline__ void contract_idx_unit(const IdxUnit<KT, TPU>& u, const h8 (&A)[4],
                                                  const uint32_t* lut, int key0, int p_tok, bool tok_ok,
                                                  float sigma, float (&bmax)[4], float* tsc_row,
                                                  size_t tsc_stride) {
  const float NEG_INF = -__builtin_inff();
#pragma unroll
  for (int kt = 0; kt < TPU; ++kt) {
    h8 Bc[4];
    decode_idx_tile<KT, FP8MODE, TPU>(u, kt, lut, Bc);
    f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < 4; ++c) acc = mfma_16x16x32(A[c], Bc[c], acc);
    const int key = key0 + 16 * kt;
    const bool vis = tok_ok && key <= p_tok;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      bmax[r] = fmaxf(bmax[r], vis ? acc[r] : NEG_INF);
      if constexpr (TOKSC) {
        if (tok_ok) tsc_row[r * tsc_stride + key] = vis ? acc[r] * sigma : NEG_INF;
      }
    }
  }
}

template <int KT, bool FP8MODE, bool TOKSC, int TPU, bool PIPE>
__global__ __launch_bounds__(kDecWaves * 64) void indexer_decode_kernel(
    const uint8_t* __restrict__ idx_q, const uint8_t* __restrict__ kdata,
    const uint8_t* __restrict__ kscales, int64_t num_pages, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ table, int max_blocks, int T, float sigma,
    float* __restrict__ block_scores, float* __restrict__ token_scores) {
  constexpr int UPP = 8 / TPU;             // units per page
  static_assert(kDecPagesPerWave >= 1 && kDecPagesPerWave <= 64, "page ids are held one per lane");
  __shared__ uint32_t lut[FP8MODE ? 512 : 2];
  // pooled scores of each wave's blocks, [block][token*4 + group], written out at the end
  __shared__ float pooled[kDecWaves][kDecPagesPerWave][16];
  if (FP8MODE) {
    build_fp8_lut(lut);
    __syncthreads();
  }
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int Q = lane >> 4, j = lane & 15;
  const float NEG_INF = -__builtin_inff();
  const float QNAN = __builtin_nanf("");
  const int L = seq_lens[b];
  const int nb = min((L + kBlock - 1) / kBlock, max_blocks);
  const int w0 = (blockIdx.x * kDecWaves + wave) * kDecPagesPerWave;   // first block of this wave
  if (w0 >= max_blocks) return;
  const int wend = min(w0 + kDecPagesPerWave, max_blocks);
  const int nreal = max(0, min(wend, nb) - w0);                        // blocks with keys

  // page ids of this wave's blocks: lane i holds block w0 + i; bad ids read page 0
  int pid = 0;
  if (lane < nreal) pid = table[(size_t)b * max_blocks + w0 + lane];
  const int pid_bad = (pid < 0 || (int64_t)pid >= num_pages) ? 1 : 0;
  const int pid_safe = pid_bad ? 0 : pid;

  // A operand: row j = token j/4, group j%4; k-chunk c = dims 32Q+8c .. +7
  h8 A[4];
  {
    const int t = j >> 2, g = j & 3;
    if (t < T) {
      const uint4* src =
          reinterpret_cast<const uint4*>(idx_q + (((size_t)b * T + t) * kGroups + g) * kHeadDim + 32 * Q);
      const uint4 u0 = src[0], u1 = src[1];
      const uint32_t wq[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const h8 a = fp8x8_to_h8(wq[2 * c], wq[2 * c + 1]);
        A[c] = (KT == 2 && FP8MODE) ? h8{a[0], a[2], a[4], a[6], a[1], a[3], a[5], a[7]} : a;
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) A[c] = h8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  const bool tok_ok = Q < T;
  const int p_tok = L - T + Q;
  const size_t tstride = (size_t)max_blocks * kBlock;
  float* tsc_row = TOKSC ? token_scores + (((size_t)b * T + (tok_ok ? Q : 0)) * kGroups) * tstride : nullptr;

  // blocks of this wave past the sequence: -inf
  if (TOKSC && tok_ok) {
    for (int i = w0 + nreal; i < wend; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        for (int kk = j; kk < kBlock; kk += 16) tsc_row[r * tstride + (size_t)i * kBlock + kk] = NEG_INF;
  }
  for (int e = lane; e < 16 * (wend - w0 - nreal); e += 64) {
    const int n = wend - w0 - nreal;
    const int rowi = e / n, i = w0 + nreal + e % n;
    if ((rowi >> 2) < T) block_scores[(((size_t)b * T + (rowi >> 2)) * kGroups + (rowi & 3)) * max_blocks + i] = NEG_INF;
  }

  const int nunits = nreal * UPP;
  float bmax[4] = {NEG_INF, NEG_INF, NEG_INF, NEG_INF};
  IdxUnit<KT, TPU> buf0, buf1;
  if (PIPE && nunits > 0)
    load_idx_unit<KT, TPU>(buf0, kdata, kscales, (size_t)__builtin_amdgcn_readlane(pid_safe, 0) * kBlock + j, Q);
  for (int uu = 0; uu < nunits; ++uu) {
    const int blk = uu / UPP, part = uu % UPP;
    if (PIPE) {
      const int un = min(uu + 1, nunits - 1);
      const size_t row_n = (size_t)__builtin_amdgcn_readlane(pid_safe, un / UPP) * kBlock + (un % UPP) * (16 * TPU) + j;
      load_idx_unit<KT, TPU>(buf1, kdata, kscales, row_n, Q);
    } else {
      const size_t row0 = (size_t)__builtin_amdgcn_readlane(pid_safe, blk) * kBlock + part * (16 * TPU) + j;
      load_idx_unit<KT, TPU>(buf0, kdata, kscales, row0, Q);
    }
    contract_idx_unit<KT, FP8MODE, TOKSC, TPU>(buf0, A, lut, (w0 + blk) * kBlock + part * (16 * TPU) + j,
                                               p_tok, tok_ok, sigma, bmax, tsc_row, tstride);
    if (PIPE) buf0 = buf1;
    if (part == UPP - 1) {
      const bool bad = __builtin_amdgcn_readlane(pid_bad, blk) != 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float m = max16(bmax[r]);
        if (j == 0) pooled[wave][blk][4 * Q + r] = bad ? QNAN : m * sigma;
        bmax[r] = NEG_INF;
      }
      if (TOKSC && bad && tok_ok) {
        const int i = w0 + blk;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          for (int kk = j; kk < kBlock; kk += 16) tsc_row[r * tstride + (size_t)i * kBlock + kk] = QNAN;
      }
    }
  }
  lds_wait();
  // write the pooled scores: entry e -> row (token, group) e / nreal, block w0 + e % nreal
  for (int e = lane; e < 16 * nreal; e += 64) {
    const int rowi = e / nreal, i = e % nreal;
    const int tt = rowi >> 2, g = rowi & 3;
    if (tt < T) block_scores[(((size_t)b * T + tt) * kGroups + g) * max_blocks + w0 + i] = pooled[wave][i][rowi];
  }
}

// ---------------------------------------------------------------------------
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

#ifndef MSA_DEC1_CHAINS
#define MSA_DEC1_CHAINS 2
#endif
constexpr int kDec1Chains = MSA_DEC1_CHAINS;   // independent MFMA accumulation chains (divides 8)

// The 4 group scores of this lane's key (before the tensor scales).
// A[c] gives dims 4c .. 4c+3 of this lane's group (lane % 4).
template <int KT, typename ASrc>
__device__ __forceinline__ f4 score_key_set(const KeySet<KT>& u, const ASrc& A) {
  f4 tot = {0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (KT == 2) {
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

#ifndef MSA_DEC1_PAGES_PER_WAVE
#define MSA_DEC1_PAGES_PER_WAVE 16
#endif
constexpr int kDec1PagesPerWave = MSA_DEC1_PAGES_PER_WAVE;

// Each wave keeps a ring of kDec1Ring key sets in registers, kDec1Ring - 1 of
// them in flight while one is contracted; at ~170 VGPRs that is two
// workgroups per CU, so about 24 sets (110 KB) are in flight per CU.
#ifndef MSA_DEC1_RING
#define MSA_DEC1_RING 4
#endif
constexpr int kDec1Ring = MSA_DEC1_RING;

// FUSE: the last workgroup of a sequence to finish (a per-sequence arrival
// counter in `counters`, zero before the call and reset to zero by that
// workgroup) also selects the sequence's top-16 blocks, one wave per group.
// Nothing waits on another workgroup: the last arrival does the work.
template <int KT, bool TOKSC, bool FUSE>
__global__ __launch_bounds__(kDecWaves * 64, 2) void indexer_decode1_kernel(
    const uint8_t* __restrict__ idx_q, const uint8_t* __restrict__ kdata,
    const uint8_t* __restrict__ kscales, int64_t num_pages, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ table, int max_blocks, float sigma, float* __restrict__ block_scores,
    float* __restrict__ token_scores, int32_t* __restrict__ sel, uint32_t* __restrict__ counters) {
  static_assert(kDec1PagesPerWave >= 1 && kDec1PagesPerWave <= 64, "page ids are held one per lane");
  __shared__ float pooled[kDecWaves][kDec1PagesPerWave][kGroups];
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const float NEG_INF = -__builtin_inff();
  const float QNAN = __builtin_nanf("");
  const int L = seq_lens[b];
  const int nb = min((L + kBlock - 1) / kBlock, max_blocks);
  const int w0 = (blockIdx.x * kDecWaves + wave) * kDec1PagesPerWave;
  if (w0 < max_blocks) {
  const int wend = min(w0 + kDec1PagesPerWave, max_blocks);
  const int nreal = max(0, min(wend, nb) - w0);

  int pid = 0;
  if (lane < nreal) pid = table[(size_t)b * max_blocks + w0 + lane];
  const int pid_bad = (pid < 0 || (int64_t)pid >= num_pages) ? 1 : 0;
  const int pid_safe = pid_bad ? 0 : pid;

  // A operand: this lane's group g = lane % 4, all 128 dims as f16
  AInRegs A;
  {
    const uint4* src = reinterpret_cast<const uint4*>(idx_q + ((size_t)b * kGroups + (lane & 3)) * kHeadDim);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint4 v = src[q];
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) A.v[4 * q + k] = cat4(fp8x2_to_h2<false>(wv[k]), fp8x2_to_h2<true>(wv[k]));
    }
  }
  const size_t tstride = (size_t)max_blocks * kBlock;
  float* tsc = TOKSC ? token_scores + (size_t)b * kGroups * tstride : nullptr;

  // blocks of this wave past the sequence: -inf
  for (int e = lane; e < kGroups * (wend - w0 - nreal); e += 64) {
    const int n = wend - w0 - nreal;
    block_scores[((size_t)b * kGroups + e / n) * max_blocks + w0 + nreal + e % n] = NEG_INF;
  }
  if (TOKSC) {
    for (int i = w0 + nreal; i < wend; ++i)
#pragma unroll
      for (int g = 0; g < kGroups; ++g)
        for (int kk = lane; kk < kBlock; kk += 64) tsc[g * tstride + (size_t)i * kBlock + kk] = NEG_INF;
  }

  const int nsets = 2 * nreal;               // two 64-key sets per page
  f4 bmax = {NEG_INF, NEG_INF, NEG_INF, NEG_INF};
  // score set u (64 keys of block u/2) and fold it into the block maxima
  auto consume = [&](int u, const KeySet<KT>& cur) {
    const int blk = u >> 1, half = u & 1;
    f4 sc = score_key_set<KT>(cur, A);
    const int key = (w0 + blk) * kBlock + half * 64 + lane;
    if (w0 + blk == nb - 1) {                    // only the last block can hold keys past L - 1
      if (key >= L) sc = f4{NEG_INF, NEG_INF, NEG_INF, NEG_INF};
    }
    bmax[0] = fmaxf(bmax[0], sc[0]);
    bmax[1] = fmaxf(bmax[1], sc[1]);
    bmax[2] = fmaxf(bmax[2], sc[2]);
    bmax[3] = fmaxf(bmax[3], sc[3]);
    if constexpr (TOKSC) {
#pragma unroll
      for (int g = 0; g < kGroups; ++g) tsc[g * tstride + key] = key < L ? sc[g] * sigma : NEG_INF;
    }
    if (half == 1) {
      const bool bad = __builtin_amdgcn_readlane(pid_bad, blk) != 0;
      const float m = wave_max4(bmax, lane);
      if ((lane & 15) == 0) pooled[wave][blk][2 * (lane >> 5) + ((lane >> 4) & 1)] = bad ? QNAN : m * sigma;
      if (TOKSC && bad) {
#pragma unroll
        for (int g = 0; g < kGroups; ++g)
          for (int kk = lane; kk < kBlock; kk += 64) tsc[g * tstride + (size_t)(w0 + blk) * kBlock + kk] = QNAN;
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
      load_key_set<KT>(dst, kdata, kscales,
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
    float* dst = block_scores + ((size_t)b * kGroups + g) * max_blocks + w0 + i;
    if (FUSE)   // device-coherent store: read back by another workgroup in this kernel
      __hip_atomic_store(dst, pooled[wave][i][g], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      *dst = pooled[wave][i][g];
  }
  }   // w0 < max_blocks

  if constexpr (FUSE) {
    // The scores and -inf fills above are complete (not merely issued) before the
    // count, and the count is taken at system scope, so the last arrival reads every
    // workgroup's scores with device-coherent loads.  No cache-wide fence: on a GPU
    // with one L2 per XCD that would write back and invalidate the whole L2.
    __shared__ int last_sh;
    __shared__ WaveTopkLds tk[kDecWaves];
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
      last_sh = __hip_atomic_fetch_add(&counters[b], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) ==
                        gridDim.x - 1 ? 1 : 0;
    __syncthreads();
    if (last_sh) {
      if (threadIdx.x == 0) __hip_atomic_store(&counters[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      const int own = max(0, min((L - 1) / kBlock, max_blocks - 1));
      const size_t r = (size_t)b * kGroups + wave;   // one group per wave
      if (own <= 64 * 16)
        wave_topk_row_regs<16>(block_scores + r * max_blocks, own, sel + r * kTopK, tk[wave], lane);
      else
        wave_topk_row(block_scores + r * max_blocks, own, sel + r * kTopK, tk[wave], lane);
    }
  }
}

// fp32 index keys and queries: one workgroup per (block, sequence), one
// thread per key, fp32 FMAs in dimension order.
__global__ __launch_bounds__(128) void indexer_f32_kernel(
    const float* __restrict__ idx_q, const float* __restrict__ kdata, int64_t num_pages,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ table, int max_blocks, int T,
    float sigma, float* __restrict__ block_scores, float* __restrict__ token_scores) {
  __shared__ float red[2];
  const int b = blockIdx.y, i = blockIdx.x, r = threadIdx.x;
  const int lane = r & 63, wave = r >> 6;
  const int L = seq_lens[b];
  const int nb = min((L + kBlock - 1) / kBlock, max_blocks);
  const float NEG_INF = -__builtin_inff();
  bool bad = false;
  const float* krow = nullptr;
  if (i < nb) {
    const int pg = table[(size_t)b * max_blocks + i];
    if (pg < 0 || (int64_t)pg >= num_pages) bad = true;
    else krow = kdata + ((size_t)pg * kBlock + r) * kHeadDim;
  }
  const int key = i * kBlock + r;
  for (int t = 0; t < T; ++t) {
    const int p = L - T + t;
    for (int g = 0; g < kGroups; ++g) {
      float v = NEG_INF;
      if (krow != nullptr && key <= p) {
        const float* qrow = idx_q + (((size_t)b * T + t) * kGroups + g) * kHeadDim;
        float acc = 0.0f;
        for (int d = 0; d < kHeadDim; ++d) acc = fmaf(qrow[d], krow[d], acc);
        v = acc * sigma;
      }
      if (bad) v = __builtin_nanf("");
      if (token_scores != nullptr)
        token_scores[(((size_t)b * T + t) * kGroups + g) * ((size_t)max_blocks * kBlock) + key] = v;
      float m = v;
      for (int off = 1; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
      if (lane == 0) red[wave] = m;
      __syncthreads();
      if (r == 0) {
        block_scores[(((size_t)b * T + t) * kGroups + g) * max_blocks + i] =
            bad ? __builtin_nanf("") : fmaxf(red[0], red[1]);
      }
      __syncthreads();
    }
  }
}

bool indexer_can_fuse_topk(const ProblemArgs& p, const CacheArgs& k, bool fp8mode) {
  return p.T == 1 && k.dtype != 0 && !(k.dtype == 2 && fp8mode);
}

hipError_t launch_indexer(const ProblemArgs& p, const void* idx_q, int q_dtype, float q_scale,
                          const CacheArgs& k, bool fp8mode, float* block_scores,
                          float* token_scores, hipStream_t s, int32_t* sel, uint32_t* counters) {
  const float sigma = q_scale * k.tensor_scale;
  if (k.dtype == 0) {
    hipLaunchKernelGGL(indexer_f32_kernel, dim3(p.max_blocks, p.B), dim3(128), 0, s,
                       (const float*)idx_q, (const float*)k.data, k.num_pages, p.seq_lens,
                       p.block_table, p.max_blocks, p.T, sigma, block_scores, token_scores);
    return hipGetLastError();
  }
  const uint8_t* q8 = (const uint8_t*)idx_q;
  if (p.T == 1 && !(k.dtype == 2 && fp8mode)) {
    // one token: 4x4x4 MFMA scan (the FP8-rounded NVFP4 reading keeps the 16-row path,
    // since its re-rounded values cannot take the scale after the dot)
    const unsigned per_wg = kDecWaves * kDec1PagesPerWave;
    const dim3 grid((unsigned)((p.max_blocks + per_wg - 1) / per_wg), (unsigned)p.B);
    const bool ts = token_scores != nullptr;
#define MSA_DEC1_LAUNCH(KT, TS, FU)                                                                  \
  hipLaunchKernelGGL((indexer_decode1_kernel<KT, TS, FU>), grid, dim3(kDecWaves * 64), 0, s, q8, k.data, \
                     k.scales, k.num_pages, p.seq_lens, p.block_table, p.max_blocks, sigma,            \
                     block_scores, token_scores, sel, counters)
    const bool fu = sel != nullptr;
    if (k.dtype == 1) {
      if (ts) MSA_DEC1_LAUNCH(1, true, false); else if (fu) MSA_DEC1_LAUNCH(1, false, true); else MSA_DEC1_LAUNCH(1, false, false);
    } else {
      if (ts) MSA_DEC1_LAUNCH(2, true, false); else if (fu) MSA_DEC1_LAUNCH(2, false, true); else MSA_DEC1_LAUNCH(2, false, false);
    }
#undef MSA_DEC1_LAUNCH
  } else if (p.T <= 4) {
    const unsigned per_wg = kDecWaves * kDecPagesPerWave;
    const dim3 grid((unsigned)((p.max_blocks + per_wg - 1) / per_wg), (unsigned)p.B);
#define MSA_DEC_LAUNCH(KT, FM, TS)                                                              \
  hipLaunchKernelGGL((indexer_decode_kernel<KT, FM, TS, (KT == 2 ? MSA_DEC_TPU : MSA_DEC_TPU / 2), MSA_DEC_PIPE != 0>), grid, dim3(kDecWaves * 64), 0, s, q8,  \
                     k.data, k.scales, k.num_pages, p.seq_lens, p.block_table, p.max_blocks, p.T, \
                     sigma, block_scores, token_scores)
    const bool ts = token_scores != nullptr;
    if (k.dtype == 1) {
      if (ts) MSA_DEC_LAUNCH(1, false, true); else MSA_DEC_LAUNCH(1, false, false);
    } else if (fp8mode) {
      if (ts) MSA_DEC_LAUNCH(2, true, true); else MSA_DEC_LAUNCH(2, true, false);
    } else {
      if (ts) MSA_DEC_LAUNCH(2, false, true); else MSA_DEC_LAUNCH(2, false, false);
    }
#undef MSA_DEC_LAUNCH
  } else {
    return launch_indexer_prefill(p, idx_q, k, fp8mode, sigma, block_scores, token_scores, s);
  }
  return hipGetLastError();
}

}  // namespace msa
