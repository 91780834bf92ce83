// Steps 1+2 of MSA for many query tokens (chunked prefill): index scores
// max-pooled per 128-key block, as a dense GEMM with the pooling fused into
// its epilogue.
//
// Source: "vLLM 為 MiniMax-M3.1-Flash 提供 Day-0 支援", section "MSA primer"
// (each group's index query scores every key against the one index-key head
// all groups use; a block keeps its best key's score) and section "Performance
// optimizations" (separate indexer prefill and decode kernels).
//
// For one sequence the scores are Q K^T with Q = [T tokens x 4 groups, 128]
// and K = [L keys, 128]; only the per-(row, block) maxima are kept, so the
// T x L score matrix never exists.  A workgroup owns 64 tokens x 4 groups =
// 256 rows and a chunk of kPfChunk consecutive blocks.  Its 4 waves keep
// their 64 rows of Q as f16 MFMA operands in registers for the whole chunk.
// Per block the page is read once (raw bytes are prefetched into registers
// two blocks ahead of the block being multiplied), dequantised into an f16
// tile in LDS (double-buffered; rows padded to 288 B, the 16-byte-aligned
// stride that measured the fewest LDS bank-conflict cycles), and contracted
// on 16x16x32 f16 MFMAs (exact
// products, fp32 sums) as S^T = K Q^T: keys are the MFMA rows, so a lane
// holds 16 keys of one query row per 64-key half.  The epilogue takes the
// max over the block's keys in-lane, then across the four lane quarters
// (3 exchanges, leaving one query row per lane).  Causality is per key
// (key <= the token's position), applied only in the blocks at or past the
// tile's first own block.
#include "common.hpp"
#include "launch.hpp"

namespace msa {

constexpr int kPfTokens = 64;                  // query tokens per workgroup (x 4 groups = 256 rows)
constexpr int kPfXcds = 8;                     // XCDs the workgroups are spread over, round-robin
constexpr int kPfChunk = 16;         // blocks per workgroup
constexpr int kPfWriteWindow = 8;    // blocks whose scores a lane writes back to back
constexpr int kPfRowHalves = kHeadDim + 16;   // f16 per LDS key row (288 B)
constexpr int kPfTileHalves = kBlock * kPfRowHalves;

// 8 NVFP4 codes (one dword, one scale) -> 8 FP8-rounded values as f16, in element order.
__device__ __forceinline__ h8 fp4x8_lut_to_h8_ordered(uint32_t w, uint32_t lut_lo, uint32_t lut_hi) {
  const uint32_t me = w & 0x07070707u, mo = (w >> 4) & 0x07070707u;
  const uint32_t fe = __builtin_amdgcn_perm(lut_hi, lut_lo, me) ^ ((w << 4) & 0x80808080u);
  const uint32_t fo = __builtin_amdgcn_perm(lut_hi, lut_lo, mo) ^ (w & 0x80808080u);
  // interleave even (fe) and odd (fo) elements: bytes e0 e1 e2 e3 | e4 e5 e6 e7
  return fp8x8_to_h8(__builtin_amdgcn_perm(fo, fe, 0x05010400u), __builtin_amdgcn_perm(fo, fe, 0x07030602u));
}

// The raw bytes of half a key row (64 dims) that one thread dequantises.
template <int KT> struct PfRaw;
template <> struct PfRaw<2> { uint4 c[2]; uint32_t s; };   // NVFP4: 32 B codes + 4 scale bytes
template <> struct PfRaw<1> { uint4 c[4]; };               // FP8: 64 B

template <int KT>
__device__ __forceinline__ void pf_load(PfRaw<KT>& r, const uint8_t* __restrict__ kdata,
                                        const uint8_t* __restrict__ kscales, size_t row, int half) {
  if constexpr (KT == 2) {
    const uint4* src = reinterpret_cast<const uint4*>(kdata + row * kNvfp4RowBytes + 32 * half);
    r.c[0] = src[0];
    r.c[1] = src[1];
    r.s = *reinterpret_cast<const uint32_t*>(kscales + row * kNvfp4ScaleBytes + 4 * half);
  } else {
    const uint4* src = reinterpret_cast<const uint4*>(kdata + row * kHeadDim + 64 * half);
#pragma unroll
    for (int q = 0; q < 4; ++q) r.c[q] = src[q];
  }
}

// LDS offset (in f16) of the 16-byte chunk c (dims 8c .. 8c+7) of a tile row.
__device__ __forceinline__ int pf_chunk(int c) { return 8 * c; }

// Dequantise 64 dims (half `half`) of one key into its f16 tile row.
template <int KT, bool FP8MODE>
__device__ __forceinline__ void pf_store(const PfRaw<KT>& r, const uint32_t* lut, _Float16* row, int half) {
  h8 v[8];
  if constexpr (KT == 2) {
#pragma unroll
    for (int d = 0; d < 8; ++d) {                 // dword d: dims 8d .. 8d+7, scale byte d/2
      const uint4& c = r.c[d >> 2];
      const uint32_t w = (d & 3) == 0 ? c.x : (d & 3) == 1 ? c.y : (d & 3) == 2 ? c.z : c.w;
      const uint32_t sb = (r.s >> (8 * (d >> 1))) & 0xFFu;
      if constexpr (FP8MODE) {
        v[d] = fp4x8_lut_to_h8_ordered(w, lut[2 * sb], lut[2 * sb + 1]);
      } else {
        const _Float16 sh = e4m3_to_h(sb);
        v[d] = fp4x8_to_h8(w) * h8{sh, sh, sh, sh, sh, sh, sh, sh};
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = fp8x8_to_h8(r.c[q].x, r.c[q].y);
      v[2 * q + 1] = fp8x8_to_h8(r.c[q].z, r.c[q].w);
    }
  }
#pragma unroll
  for (int d = 0; d < 8; ++d) *reinterpret_cast<h8*>(row + pf_chunk(8 * half + d)) = v[d];
}

// SHARED (shared-prefix decode): the workgroup's rows are the query rows of
// prefix group blockIdx.z -- sequences [start, start + n), whose first
// `blocks` logical blocks are the same pages -- taken as n*T row tokens in
// batch order (row token t = token t % T of sequence start + t / T, which is
// row start*T + t of idx_q and block_scores, the same linear index as for one
// sequence).  Only those shared blocks are scored, each page read and
// dequantised once for all n sequences; each row keeps its own position.
template <int KT, bool FP8MODE, bool TOKSC, bool SHARED = false, int CHUNK = kPfChunk>
__global__ __launch_bounds__(256, 2) void indexer_prefill_kernel(
    const uint8_t* __restrict__ idx_q, const uint8_t* __restrict__ kdata,
    const uint8_t* __restrict__ kscales, int64_t num_pages, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ table, int max_blocks, int T, float sigma,
    float* __restrict__ block_scores, float* __restrict__ token_scores, PrefixGroups groups, int nitems = 0) {
  static_assert(!(SHARED && TOKSC), "per-key scores are not written for shared prefixes");
  __shared__ uint32_t lut[FP8MODE ? 512 : 2];
  __shared__ __attribute__((aligned(16))) _Float16 tile[2][kPfTileHalves];
  __shared__ int page_of[CHUNK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int Q = lane >> 4, n = lane & 15;
  // b: the sequence of row token 0 (whose block-table row gives the pages); Tn: row tokens
  // Work item (token tile tx, chunk cy, sequence or group bz).  Without SHARED the
  // grid is 1-D: workgroups go to the 8 XCDs round-robin (workgroup w on XCD
  // w % 8), and XCD x takes the x-th eighth of the items in (sequence, chunk,
  // token tile) order, so one key chunk's token tiles share one L2 instead of
  // every XCD reading every chunk.  SHARED keeps its 3-D grid.
  int tx, cy, bz;
  if constexpr (SHARED) {
    tx = blockIdx.x;
    cy = blockIdx.y;
    bz = blockIdx.z;
  } else {
    const int ntx = (T + kPfTokens - 1) / kPfTokens, ncy = (max_blocks + CHUNK - 1) / CHUNK;
    const int per = (int)(gridDim.x / kPfXcds);   // the grid is kPfXcds * per
    const int item = (int)(blockIdx.x % kPfXcds) * per + (int)(blockIdx.x / kPfXcds);
    if (item >= nitems) return;
    tx = item % ntx;
    cy = (item / ntx) % ncy;
    bz = item / (ntx * ncy);
  }
  const int b = SHARED ? groups.start[bz] : bz;
  const int Tn = SHARED ? (groups.start[bz + 1] - b) * T : T;
  const int blim = SHARED ? min(groups.blocks[bz], max_blocks) : max_blocks;
  const int t0 = tx * kPfTokens;
  const int c0 = cy * CHUNK;
  if (SHARED && (t0 >= Tn || c0 >= blim)) return;   // the grid covers the largest group
  const int L = seq_lens[b];
  // position of row token t (t < Tn)
  auto pos = [&](int t) { return SHARED ? seq_lens[b + t / T] - T + t % T : L - T + t; };
  const int t_last = min(Tn, t0 + kPfTokens) - 1;
  int own_first, own_last;   // smallest and largest own block of the tile's rows
  if constexpr (SHARED) {
    own_first = 0x7FFFFFFF;
    own_last = -1;
    for (int t = t0; t <= t_last; ++t) {
      const int o = pos(t) / kBlock;
      own_first = min(own_first, o);
      own_last = max(own_last, o);
    }
  } else {
    own_first = (L - T + t0) / kBlock;          // own block of the tile's first token
    own_last = (L - T + t_last) / kBlock;
  }
  const int nb = SHARED ? blim : min((L + kBlock - 1) / kBlock, max_blocks);
  const int c_end = min(c0 + CHUNK, blim);
  // blocks [c0, c_comp) of this chunk have visible keys; [c_comp, c_end) get -inf
  const int c_comp = max(c0, min(c_end, min(nb, own_last + 1)));
  const float NEG_INF = -__builtin_inff();
  // A block whose page id is unreadable is marked NaN through the bit pattern
  // (an integer select and store): this file is compiled without NaN
  // semantics (-fno-honor-nans: no MFMA result is NaN, and without the flag
  // every fmaxf of one is preceded by a canonicalising max), under which a
  // float select of a NaN constant could be folded away.
  constexpr uint32_t kQNanBits = 0x7FC00000u;
  auto mark = [&](float* dst, bool bad_blk, float v) {
    *reinterpret_cast<uint32_t*>(dst) = bad_blk ? kQNanBits : __builtin_bit_cast(uint32_t, v);
  };
  const size_t tstride = (size_t)max_blocks * kBlock;

  if (FP8MODE) build_fp8_lut(lut);
  if (tid < CHUNK) {
    int pg = -1;
    if (c0 + tid < c_comp) {
      pg = table[(size_t)b * max_blocks + c0 + tid];
      if (pg < 0 || (int64_t)pg >= num_pages) pg = -2;     // unreadable page
    }
    page_of[tid] = pg;
  }

  // rows of this wave: 4 row tiles rr; row m of tile rr = token 4*(4*wave+rr) + m/4, group m%4
  // A operand fragment [rr][ks]: lane (Q, m=n) holds dims 32ks + 8Q .. +7 of that row
  h8 A[4][4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int t = t0 + 4 * (4 * wave + rr) + (n >> 2);
    const int g = n & 3;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (t < Tn) {
        const uint2 u = *reinterpret_cast<const uint2*>(idx_q + (((size_t)b * T + t) * kGroups + g) * kHeadDim +
                                                        32 * ks + 8 * Q);
        A[rr][ks] = fp8x8_to_h8(u.x, u.y);
      } else {
        A[rr][ks] = h8{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
  }
  // the position of this lane's query row (row n of each row tile: token n/4)
  int p_of[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int t = t0 + 4 * (4 * wave + rr) + (n >> 2);
    p_of[rr] = t < Tn ? pos(t) : -1;   // rows past the last token see nothing
  }
  // LDS offsets of this lane's operand chunks (dims 32ks + 8Q .. +7)
  int kofs[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) kofs[ks] = pf_chunk(4 * ks + Q);
  __syncthreads();

  // blocks of the chunk with no visible key for any row: -inf
  for (int e = tid; e < kPfTokens * kGroups * (c_end - c_comp); e += 256) {
    const int nblk = c_end - c_comp;
    const int row = e / nblk, i = c_comp + e % nblk;
    const int t = t0 + (row >> 2);
    if (t < Tn) block_scores[(((size_t)b * T + t) * kGroups + (row & 3)) * max_blocks + i] = NEG_INF;
    if (TOKSC && t < T)
      for (int kk = 0; kk < kBlock; ++kk)
        token_scores[(((size_t)b * T + t) * kGroups + (row & 3)) * tstride + (size_t)i * kBlock + kk] = NEG_INF;
  }
  const int nblocks = c_comp - c0;
  if (nblocks <= 0) return;

  const int key_ld = tid >> 1, half_ld = tid & 1;   // the half key row this thread dequantises
  auto page_row = [&](int k) -> size_t {
    const int pg = page_of[k];
    return (size_t)(pg < 0 ? 0 : pg) * kBlock + key_ld;
  };
  // raw bytes run two blocks ahead of the block being multiplied
  PfRaw<KT> raw, raw2;
  pf_load<KT>(raw, kdata, kscales, page_row(0), half_ld);
  if (nblocks > 1) pf_load<KT>(raw2, kdata, kscales, page_row(1), half_ld);
  pf_store<KT, FP8MODE>(raw, lut, &tile[0][key_ld * kPfRowHalves], half_ld);
  raw = raw2;
  __syncthreads();

  // (with per-key scores, which write every key anyway, one block at a time)
  constexpr int WW = TOKSC ? 1 : kPfWriteWindow;
  uint32_t win[WW];   // this lane's row: scores of the current window's blocks
#pragma unroll
  for (int u = 0; u < WW; ++u) win[u] = 0u;
  for (int k = 0; k < nblocks; ++k) {
    const int i = c0 + k;
    const _Float16* B = tile[k & 1];
    if (k + 2 < nblocks) pf_load<KT>(raw2, kdata, kscales, page_row(k + 2), half_ld);

    // two halves of 64 keys; in the 16x16 output tile (kt, rr), lane (Q, n) holds keys
    // kh*64 + kt*16 + 4Q + r (r = 0..3) of query row n of row tile rr
    const bool bad = page_of[k] == -2;
    const bool all_visible = i < own_first;
    f4 m;   // per row tile rr: this lane's running max over its keys
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      f4 acc[4][4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) acc[rr][kt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        h8 Kf[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
          Kf[kt] = *reinterpret_cast<const h8*>(B + (kh * 64 + kt * 16 + n) * kPfRowHalves + kofs[ks]);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) acc[rr][kt] = mfma_16x16x32(Kf[kt], A[rr][ks], acc[rr][kt]);
      }
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        float v;
        if (all_visible) {
          float u[4];
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
            u[kt] = fmaxf(fmaxf(acc[rr][kt][0], acc[rr][kt][1]), fmaxf(acc[rr][kt][2], acc[rr][kt][3]));
          v = fmaxf(fmaxf(u[0], u[1]), fmaxf(u[2], u[3]));
        } else {
          v = NEG_INF;
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              v = fmaxf(v, (i * kBlock + kh * 64 + kt * 16 + 4 * Q + r <= p_of[rr]) ? acc[rr][kt][r] : NEG_INF);
        }
        m[rr] = kh == 0 ? v : fmaxf(m[rr], v);
      }
      if constexpr (TOKSC) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int t = t0 + 4 * (4 * wave + rr) + (n >> 2);
          if (t < T) {
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int key = i * kBlock + kh * 64 + kt * 16 + 4 * Q + r;
                mark(&token_scores[(((size_t)b * T + t) * kGroups + (n & 3)) * tstride + key], bad,
                     key <= p_of[rr] ? acc[rr][kt][r] * sigma : NEG_INF);
              }
          }
        }
      }
    }
    const float mx = quarter_max4(m);              // query row n of row tile Q
    {
      // this lane's row keeps the scores of kPfWriteWindow consecutive blocks and
      // writes them back to back: one score per block would touch each 128-byte
      // line of the row many times, and lines evicted partly written between
      // touches multiply the HBM writes
      const uint32_t bits = bad ? kQNanBits : __builtin_bit_cast(uint32_t, mx * sigma);
      const int slot = k % WW;
#pragma unroll
      for (int u = 0; u < WW; ++u) win[u] = slot == u ? bits : win[u];
      if (slot == WW - 1 || k == nblocks - 1) {
        const int t = t0 + 4 * (4 * wave + Q) + (n >> 2);
        if (t < Tn) {
          uint32_t* dst = reinterpret_cast<uint32_t*>(block_scores) +
                          (((size_t)b * T + t) * kGroups + (n & 3)) * max_blocks + (i - slot);
#pragma unroll
          for (int u = 0; u < WW; ++u)
            if (u <= slot) dst[u] = win[u];
        }
      }
    }

    if (k + 1 < nblocks) pf_store<KT, FP8MODE>(raw, lut, &tile[(k + 1) & 1][key_ld * kPfRowHalves], half_ld);
    raw = raw2;
    __syncthreads();
  }
}

hipError_t launch_indexer_prefill(const ProblemArgs& p, const void* idx_q, const CacheArgs& k,
                                  bool fp8mode, float sigma, float* block_scores, float* token_scores,
                                  hipStream_t s) {
  // 1-D grid over the XCDs (see the kernel): 8 * ceil(items / 8) workgroups,
  // those past the items return at once
  const int64_t items = (int64_t)((p.T + kPfTokens - 1) / kPfTokens) * ((p.max_blocks + kPfChunk - 1) / kPfChunk) * p.B;
  if (items > 0x7FFFFFFF - kPfXcds) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(kPfXcds * ((items + kPfXcds - 1) / kPfXcds)), 1, 1);
  const uint8_t* q8 = static_cast<const uint8_t*>(idx_q);
  const bool ts = token_scores != nullptr;
  const PrefixGroups none{};
#define MSA_PF_LAUNCH(KT, FM, TS)                                                                \
  hipLaunchKernelGGL((indexer_prefill_kernel<KT, FM, TS>), grid, dim3(256), 0, s, q8, k.data,     \
                     k.scales, k.num_pages, p.seq_lens, p.block_table, p.max_blocks, p.T, sigma,  \
                     block_scores, token_scores, none, (int)items)
  if (k.dtype == 1) {
    if (ts) MSA_PF_LAUNCH(1, false, true); else MSA_PF_LAUNCH(1, false, false);
  } else if (fp8mode) {
    if (ts) MSA_PF_LAUNCH(2, true, true); else MSA_PF_LAUNCH(2, true, false);
  } else {
    if (ts) MSA_PF_LAUNCH(2, false, true); else MSA_PF_LAUNCH(2, false, false);
  }
#undef MSA_PF_LAUNCH
  return hipGetLastError();
}

hipError_t launch_indexer_shared(const ProblemArgs& p, const void* idx_q, const CacheArgs& k, bool fp8mode,
                                 float sigma, const PrefixGroups& g, float* block_scores, hipStream_t s) {
  int max_rows = 0, max_blocks = 0;
  for (int i = 0; i < g.n; ++i) {
    max_rows = max(max_rows, (g.start[i + 1] - g.start[i]) * p.T);
    max_blocks = max(max_blocks, min(g.blocks[i], p.max_blocks));
  }
  if (g.n == 0 || max_rows == 0 || max_blocks == 0) return hipSuccess;
  const unsigned gx = (unsigned)((max_rows + kPfTokens - 1) / kPfTokens);
  // blocks per workgroup: the largest of 16, 8, 4, 2 that still gives every CU two workgroups
  const int want = 2 * current_cu_count();
  int chunk = 2;
  for (int c = 16; c > 2; c /= 2)
    if ((int64_t)gx * ((max_blocks + c - 1) / c) * g.n >= want) { chunk = c; break; }
  const dim3 grid(gx, (unsigned)((max_blocks + chunk - 1) / chunk), (unsigned)g.n);
  const uint8_t* q8 = static_cast<const uint8_t*>(idx_q);
#define MSA_SH_LAUNCH(KT, FM, C)                                                                      \
  hipLaunchKernelGGL((indexer_prefill_kernel<KT, FM, false, true, C>), grid, dim3(256), 0, s, q8, k.data, \
                     k.scales, k.num_pages, p.seq_lens, p.block_table, p.max_blocks, p.T, sigma,          \
                     block_scores, nullptr, g)
#define MSA_SH_CHUNK(KT, FM)                                                 \
  do {                                                                       \
    if (chunk == 16) MSA_SH_LAUNCH(KT, FM, 16);                              \
    else if (chunk == 8) MSA_SH_LAUNCH(KT, FM, 8);                           \
    else if (chunk == 4) MSA_SH_LAUNCH(KT, FM, 4);                           \
    else MSA_SH_LAUNCH(KT, FM, 2);                                           \
  } while (0)
  if (k.dtype == 1) MSA_SH_CHUNK(1, false);
  else if (fp8mode) MSA_SH_CHUNK(2, true);
  else MSA_SH_CHUNK(2, false);
#undef MSA_SH_CHUNK
#undef MSA_SH_LAUNCH
  return hipGetLastError();
}

}  // namespace msa
