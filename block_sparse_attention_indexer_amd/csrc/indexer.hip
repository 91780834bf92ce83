// Steps 1+2 of MSA for decode and speculative decode (T <= 8 query tokens):
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
#include "scan1.hpp"

namespace msa {

// ---------------------------------------------------------------------------
// Decode and speculative decode (T <= 8): a streaming scan.
//
// Grid (page range, sequence); each of the 4 waves of a workgroup owns PPW
// consecutive blocks (kDecPagesPerWave, or a half or a quarter of it when the
// grid would otherwise leave CUs idle).  A wave reads its page ids
// once (one lane per block), then walks its pages in units of TPU key tiles
// (16 keys each).  With PIPE the next unit's loads are issued before the
// current unit is contracted, so memory and math overlap inside the wave;
// those loads are unconditional (past the last unit a wave re-reads its last
// unit, which hits in cache) so that every wait covers exactly one unit.
// A key tile is the MFMAs' first operand and a row tile of 16 query rows
// (4 tokens x 4 groups) their second; NT = 2 row tiles (T = 5..8) contract
// each decoded key tile twice, so the dequantisation is shared by all T
// tokens and the scan stays bound by the page reads.  sigma > 0 is applied
// to the pooled maximum only: fl(sigma*x) is monotone in x, so this equals
// the maximum of the scaled scores.
constexpr int kDecPagesPerWave = 8;
constexpr int kDecTpu = 4;          // 16-key units per NVFP4 lane load (half for FP8)
constexpr bool kDecPipe = true;     // next unit loaded while the current one is contracted
constexpr int kDec1WgPerCu = 1;     // one-token scan: workgroups per CU the chunking aims for
constexpr int kDec1FlatWgPerCu = 2; // flat one-token scan: workgroups per CU for large batches (all resident)

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

// Contract one unit: per tile and row tile four 16x16x32 MFMAs with the keys
// as the first operand, so lane (Q, j) gets keys 4Q .. 4Q+3 of the tile
// (`kq` = this lane's first key of the unit) for query row j of row tile n,
// and folds them into its running maximum bmax[n].  MASK: keys past a row's
// token position count as -inf (only the units that reach the last T keys
// of the sequence need it; the caller picks the instance per unit).
template <int KT, bool FP8MODE, bool TOKSC, int TPU, int NT, bool MASK>
__device__ __forceinline__ void contract_idx_unit(const IdxUnit<KT, TPU>& u, const h8 (&A)[NT][4],
                                                  const uint32_t* lut, int kq, const int (&p_tok)[NT],
                                                  const bool (&tok_ok)[NT], float sigma, float (&bmax)[NT],
                                                  float* const (&tsc_row)[NT]) {
  const float NEG_INF = -__builtin_inff();
#pragma unroll
  for (int kt = 0; kt < TPU; ++kt) {
    h8 Bc[4];
    decode_idx_tile<KT, FP8MODE, TPU>(u, kt, lut, Bc);
    const int key = kq + 16 * kt;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < 4; ++c) acc = mfma_16x16x32(Bc[c], A[n][c], acc);
      bool vis[4] = {true, true, true, true};
      if constexpr (MASK) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          vis[r] = key + r <= p_tok[n];
          acc[r] = vis[r] ? acc[r] : NEG_INF;
        }
      }
      bmax[n] = vmax(vmax(vmax(vmax(bmax[n], acc[0]), acc[1]), acc[2]), acc[3]);
      if constexpr (TOKSC) {
        if (tok_ok[n]) {
#pragma unroll
          for (int r = 0; r < 4; ++r) tsc_row[n][key + r] = vis[r] ? acc[r] * sigma : NEG_INF;
        }
      }
    }
  }
}

template <int KT, bool FP8MODE, bool TOKSC, int TPU, bool PIPE, int PPW, int NT>
__global__ __launch_bounds__(kDecWaves * 64) void indexer_decode_kernel(
    const uint8_t* __restrict__ idx_q, const uint8_t* __restrict__ kdata,
    const uint8_t* __restrict__ kscales, int64_t num_pages, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ table, int max_blocks, int T, float sigma,
    float* __restrict__ block_scores, float* __restrict__ token_scores, int blk_off, int blk_step,
    const int32_t* __restrict__ skip) {
  constexpr int UPP = 8 / TPU;             // units per page
  static_assert(PPW >= 1 && PPW <= 64, "page ids are held one per lane");
  static_assert(NT == 1 || NT == 2, "one or two row tiles");
  __shared__ uint32_t lut[FP8MODE ? 512 : 2];
  // pooled scores of each wave's blocks, [block][token*4 + group], written out at the end
  __shared__ float pooled[kDecWaves][PPW][16 * NT];
  if (FP8MODE) {
    build_fp8_lut(lut);
    __syncthreads();
  }
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform, held in a scalar register
  const int Q = lane >> 4, j = lane & 15;
  const float NEG_INF = -__builtin_inff();
  const float QNAN = __builtin_nanf("");
  const int L = seq_lens[b];
  const int nb = min((L + kBlock - 1) / kBlock, max_blocks);
  // shard (context-parallel) view: local block j is logical block gblk(j); w0,
  // wend and nreal count local blocks (blk_off 0, blk_step 1: the whole context)
  auto gblk = [&](int jj) { return blk_off + blk_step * jj; };
  const int nloc = shard_count(max_blocks, blk_off, blk_step);
  const int wbase = (blockIdx.x * kDecWaves + wave) * PPW;
  const int wend = min(wbase + PPW, nloc);
  // first block of this wave (local blocks below skip[b] belong to the shared-prefix kernel)
  const int w0 = skip == nullptr ? wbase : max(wbase, shard_count(skip[b], blk_off, blk_step));
  if (w0 >= wend) return;
  const int nreal = max(0, min(wend, shard_count(nb, blk_off, blk_step)) - w0);   // blocks with keys

  // page ids of this wave's blocks: lane i holds block w0 + i; bad ids read page 0
  int pid = 0;
  if (lane < nreal) pid = table[(size_t)b * max_blocks + gblk(w0 + lane)];
  const int pid_bad = (pid < 0 || (int64_t)pid >= num_pages) ? 1 : 0;
  const int pid_safe = pid_bad ? 0 : pid;

  // query operand: row j of tile n = token 4n + j/4, group j%4; k-chunk c = dims 32Q+8c .. +7
  h8 A[NT][4];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int t = 4 * n + (j >> 2), g = j & 3;
    if (t < T) {
      const uint4* src =
          reinterpret_cast<const uint4*>(idx_q + (((size_t)b * T + t) * kGroups + g) * kHeadDim + 32 * Q);
      const uint4 u0 = src[0], u1 = src[1];
      const uint32_t wq[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const h8 a = fp8x8_to_h8(wq[2 * c], wq[2 * c + 1]);
        A[n][c] = (KT == 2 && FP8MODE) ? h8{a[0], a[2], a[4], a[6], a[1], a[3], a[5], a[7]} : a;
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) A[n][c] = h8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  // this lane's query row of each tile: its token's position and token-score row
  bool tok_ok[NT];
  int p_tok[NT];
  const size_t tstride = (size_t)max_blocks * kBlock;
  float* tsc_row[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int t = 4 * n + (j >> 2);
    tok_ok[n] = t < T;
    p_tok[n] = L - T + t;
    tsc_row[n] = TOKSC ? token_scores + (((size_t)b * T + (tok_ok[n] ? t : 0)) * kGroups + (j & 3)) * tstride
                       : nullptr;
  }
  // fill the token scores of block i with v: lane (Q, j) writes keys 4Q + 16m .. +3 of its rows
  auto fill_token_scores = [&](int i, float v) {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      if (!tok_ok[n]) continue;
      for (int kk = 4 * Q; kk < kBlock; kk += 16)
#pragma unroll
        for (int r = 0; r < 4; ++r) tsc_row[n][(size_t)i * kBlock + kk + r] = v;
    }
  };

  // blocks of this wave past the sequence: -inf
  if (TOKSC) {
    for (int i = w0 + nreal; i < wend; ++i) fill_token_scores(gblk(i), NEG_INF);
  }
  for (int e = lane; e < 16 * NT * (wend - w0 - nreal); e += 64) {
    const int n = wend - w0 - nreal;
    const int rowi = e / n, i = gblk(w0 + nreal + e % n);
    if ((rowi >> 2) < T) block_scores[(((size_t)b * T + (rowi >> 2)) * kGroups + (rowi & 3)) * max_blocks + i] = NEG_INF;
  }

  const int nunits = nreal * UPP;
  float bmax[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) bmax[n] = NEG_INF;
  // units alternate between two register buffers (UPP is even, so a unit's
  // buffer is fixed by its part); with PIPE the next unit's loads are in
  // flight while the current one is contracted
  static_assert(UPP % 2 == 0, "units of a page alternate between two buffers");
  IdxUnit<KT, TPU> buf[2];
  auto load_unit = [&](IdxUnit<KT, TPU>& dst, int un) {
    const size_t row = (size_t)__builtin_amdgcn_readlane(pid_safe, un / UPP) * kBlock + (un % UPP) * (16 * TPU) + j;
    load_idx_unit<KT, TPU>(dst, kdata, kscales, row, Q);
  };
  if (PIPE && nunits > 0) load_unit(buf[0], 0);
  // units wholly at or below the first token's position need no mask
  const int vis_end = L - T;
  for (int blk = 0; blk < nreal; ++blk) {
    const int kblk = gblk(w0 + blk) * kBlock;
#pragma unroll
    for (int part = 0; part < UPP; ++part) {
      const int uu = blk * UPP + part;
      IdxUnit<KT, TPU>& cur = buf[part & 1];
      if (PIPE) load_unit(buf[(part + 1) & 1], min(uu + 1, nunits - 1));
      else load_unit(cur, uu);
      const int ku = kblk + part * (16 * TPU);
      if (ku + 16 * TPU - 1 <= vis_end)
        contract_idx_unit<KT, FP8MODE, TOKSC, TPU, NT, false>(cur, A, lut, ku + 4 * Q, p_tok, tok_ok, sigma, bmax,
                                                              tsc_row);
      else
        contract_idx_unit<KT, FP8MODE, TOKSC, TPU, NT, true>(cur, A, lut, ku + 4 * Q, p_tok, tok_ok, sigma, bmax,
                                                             tsc_row);
    }
    // block maxima: lane 32h + 16q + j holds tile h's row j (NT = 2) or tile 0's row j (NT = 1)
    const bool bad = __builtin_amdgcn_readlane(pid_bad, blk) != 0;
    const float m = quarter_max2(bmax[0], bmax[NT - 1]);
    if ((Q & 1) == 0 && (NT == 2 || Q == 0)) pooled[wave][blk][16 * (Q >> 1) + j] = bad ? QNAN : m * sigma;
    if (TOKSC && bad) fill_token_scores(gblk(w0 + blk), QNAN);
#pragma unroll
    for (int n = 0; n < NT; ++n) bmax[n] = NEG_INF;
  }
  lds_wait();
  // write the pooled scores: entry e -> row (token, group) e / nreal, block w0 + e % nreal
  for (int e = lane; e < 16 * NT * nreal; e += 64) {
    const int rowi = e / nreal, i = e % nreal;
    const int tt = rowi >> 2, g = rowi & 3;
    if (tt < T) block_scores[(((size_t)b * T + tt) * kGroups + g) * max_blocks + gblk(w0 + i)] = pooled[wave][i][rowi];
  }
}

// ---------------------------------------------------------------------------
// Single-token decode (T = 1): the streaming scan of scan1.hpp, one chunk per
// workgroup.  FUSE: the last workgroup of a sequence to finish (a
// per-sequence arrival counter in `counters`, zero before the call and reset
// to zero by that workgroup) also selects the sequence's top-16 blocks.
// Nothing waits on another workgroup: the last arrival does the work.
template <int KT, bool TOKSC, bool FUSE, int PPW, bool FP8MODE = false>
__global__ __launch_bounds__(kDecWaves * 64, 2) void indexer_decode1_kernel(Scan1Args a, int32_t* __restrict__ sel,
                                                                            uint32_t* __restrict__ counters) {
  __shared__ __align__(8) uint32_t lut[FP8MODE ? 512 : 2];
  if constexpr (FP8MODE) {
    build_fp8_lut(lut);
    __syncthreads();
  }
  scan1_chunk<KT, TOKSC, FUSE, PPW, FP8MODE>(a, blockIdx.y, blockIdx.x, lut);
  if constexpr (FUSE) scan1_select_if_last(a, blockIdx.y, gridDim.x, sel, counters);
}

// The one-token scan spread evenly over a fixed grid (scan1_flat): for
// ragged contexts, with no selection or shard and no per-key scores.  SKIP:
// each sequence of a prefix group g starts after the group's shared blocks
// (the rest of the shared-prefix call).
template <int KT, bool FP8MODE, bool SKIP = false>
__global__ __launch_bounds__(kDecWaves * 64, 2) void indexer_decode1_flat_kernel(Scan1Args a, int B,
                                                                                 PrefixGroups g) {
  __shared__ __align__(8) uint32_t lut[FP8MODE ? 512 : 2];
  __shared__ int pre[kFlatMaxSeqs + 1];
  __shared__ int padpre[SKIP ? kFlatMaxSeqs + 1 : 1];
  if constexpr (FP8MODE) build_fp8_lut(lut);   // the prefix pass below synchronises
  scan1_flat<KT, FP8MODE, SKIP>(a, B, lut, pre, padpre, g);
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

// skip[b] = the shared block count of b's prefix group (0 outside every group).
__global__ void fill_skip_kernel(PrefixGroups g, int B, int32_t* __restrict__ skip) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int v = 0;
  for (int k = 0; k < g.n; ++k)
    if (b >= g.start[k] && b < g.start[k + 1]) v = g.blocks[k];
  skip[b] = v;
}

hipError_t launch_fill_skip(const PrefixGroups& g, int B, int32_t* skip, hipStream_t s) {
  hipLaunchKernelGGL(fill_skip_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, s, g, B, skip);
  return hipGetLastError();
}

// The one-token scan over a fixed grid, each wave a contiguous share of all
// sequences' blocks: two workgroups per CU (the scan's residency), or one when
// even B x max_blocks would give a wave fewer than 16 blocks -- long-lived
// waves win there (32 x 256 blocks: 35.0 us against 39.5 us).  groups
// non-null: the SKIP form, each group's shared blocks left out.
static void launch_flat(const Scan1Args& sa, int B, int kdtype, bool fp8mode, const PrefixGroups* groups,
                        hipStream_t s) {
  const int cus = current_cu_count();
  const int64_t bound = (int64_t)B * sa.max_blocks;
  const int per_cu = bound >= (int64_t)kDec1FlatWgPerCu * cus * kDecWaves * 16 ? kDec1FlatWgPerCu : 1;
  const dim3 grid((unsigned)(per_cu * cus)), block(kDecWaves * 64);
  const PrefixGroups g = groups != nullptr ? *groups : PrefixGroups{};
#define MSA_FLAT(KT, FM)                                                                      \
  do {                                                                                        \
    if (groups != nullptr)                                                                    \
      hipLaunchKernelGGL((indexer_decode1_flat_kernel<KT, FM, true>), grid, block, 0, s, sa, B, g); \
    else hipLaunchKernelGGL((indexer_decode1_flat_kernel<KT, FM>), grid, block, 0, s, sa, B, g);  \
  } while (0)
  if (kdtype == 1) MSA_FLAT(1, false);
  else if (fp8mode) MSA_FLAT(2, true);
  else MSA_FLAT(2, false);
#undef MSA_FLAT
}

hipError_t launch_indexer_skipping(const ProblemArgs& p, const void* idx_q, int q_dtype, float q_scale,
                                   const CacheArgs& k, bool fp8mode, float* block_scores, const PrefixGroups& g,
                                   int32_t* skip_ws, hipStream_t s) {
  if (k.dtype == 0) return hipErrorInvalidValue;
  if (p.T == 1 && p.B <= kFlatMaxSeqs) {
    const Scan1Args sa{(const uint8_t*)idx_q, k.data, k.scales, k.num_pages, p.seq_lens, p.block_table, p.max_blocks,
                       q_scale * k.tensor_scale, block_scores, nullptr};
    launch_flat(sa, p.B, k.dtype, fp8mode, &g, s);
    return hipGetLastError();
  }
  const hipError_t e = launch_fill_skip(g, p.B, skip_ws, s);
  if (e != hipSuccess) return e;
  return launch_indexer(p, idx_q, q_dtype, q_scale, k, fp8mode, block_scores, nullptr, s, nullptr, nullptr, 0, 1,
                        skip_ws);
}

bool indexer_can_fuse_topk(const ProblemArgs& p, const CacheArgs& k, bool fp8mode) {
  return p.T == 1 && k.dtype != 0 && !(k.dtype == 2 && fp8mode);
}

hipError_t launch_indexer(const ProblemArgs& p, const void* idx_q, int q_dtype, float q_scale,
                          const CacheArgs& k, bool fp8mode, float* block_scores,
                          float* token_scores, hipStream_t s, int32_t* sel, uint32_t* counters,
                          int shard, int num_shards, const int32_t* skip) {
  const float sigma = q_scale * k.tensor_scale;
  const int nloc = shard_count(p.max_blocks, shard, num_shards);   // blocks of the shard
  if ((num_shards != 1 || skip != nullptr) && (k.dtype == 0 || p.T > 8 || sel != nullptr)) return hipErrorInvalidValue;
  if (nloc == 0) return hipSuccess;   // a shard past the last block has nothing to score
  if (k.dtype == 0) {
    hipLaunchKernelGGL(indexer_f32_kernel, dim3(p.max_blocks, p.B), dim3(128), 0, s,
                       (const float*)idx_q, (const float*)k.data, k.num_pages, p.seq_lens,
                       p.block_table, p.max_blocks, p.T, sigma, block_scores, token_scores);
    return hipGetLastError();
  }
  const uint8_t* q8 = (const uint8_t*)idx_q;
  // Pages per wave: the largest of the kernel's three sizes whose grid still gives
  // every CU `per_cu` workgroups (a shard, or few long sequences, has few chunks).
  // The one-token scan asks for one workgroup per CU: long-lived waves beat a
  // second, shorter workgroup (32 sequences x 256 blocks: 8 pages per wave in
  // 31 us against 4 pages in 34.6 us); longer contexts are unchanged by it.
  auto pick_ppw = [&](int big, int per_cu) {
    const int want = per_cu * current_cu_count();
    for (int ppw = big; ppw > big / 4; ppw /= 2)
      if ((int64_t)p.B * ((nloc + kDecWaves * ppw - 1) / (kDecWaves * ppw)) >= want) return ppw;
    return big / 4;
  };
  const bool flat = p.T == 1 && sel == nullptr && token_scores == nullptr && num_shards == 1 && skip == nullptr &&
                    p.B <= kFlatMaxSeqs;
  if (flat) {
    const Scan1Args sa{q8, k.data, k.scales, k.num_pages, p.seq_lens, p.block_table, p.max_blocks, sigma,
                       block_scores, nullptr};
    launch_flat(sa, p.B, k.dtype, fp8mode, nullptr, s);
  } else if (p.T == 1 && !(fp8mode && k.dtype == 2 && sel != nullptr)) {
    // one token: 4x4x4 MFMA scan; the FP8-rounded NVFP4 reading decodes through the
    // LDS table instead of scaling partial dots (not fused with the selection)
    const int ppw = pick_ppw(kDec1PagesPerWave, kDec1WgPerCu);
    const bool f8 = fp8mode && k.dtype == 2;
    const dim3 grid((unsigned)((nloc + kDecWaves * ppw - 1) / (kDecWaves * ppw)), (unsigned)p.B);
    const bool ts = token_scores != nullptr;
    const bool fu = sel != nullptr;
    const Scan1Args sa{q8, k.data, k.scales, k.num_pages, p.seq_lens, p.block_table, p.max_blocks, sigma,
                       block_scores, token_scores, shard, num_shards, skip};
#define MSA_DEC1_LAUNCH(KT, TS, FU, PPW, FM)                                                        \
  hipLaunchKernelGGL((indexer_decode1_kernel<KT, TS, FU, PPW, FM>), grid, dim3(kDecWaves * 64), 0, s, sa, sel, \
                     counters)
#define MSA_DEC1_PPW(KT, TS, FU, FM)                                                                \
  do {                                                                                              \
    if (ppw == kDec1PagesPerWave) MSA_DEC1_LAUNCH(KT, TS, FU, kDec1PagesPerWave, FM);               \
    else if (ppw == kDec1PagesPerWave / 2) MSA_DEC1_LAUNCH(KT, TS, FU, kDec1PagesPerWave / 2, FM);  \
    else MSA_DEC1_LAUNCH(KT, TS, FU, kDec1PagesPerWave / 4, FM);                                    \
  } while (0)
    if (k.dtype == 1) {
      if (ts) MSA_DEC1_PPW(1, true, false, false); else if (fu) MSA_DEC1_PPW(1, false, true, false);
      else MSA_DEC1_PPW(1, false, false, false);
    } else if (f8) {
      if (ts) MSA_DEC1_PPW(2, true, false, true); else MSA_DEC1_PPW(2, false, false, true);
    } else {
      if (ts) MSA_DEC1_PPW(2, true, false, false); else if (fu) MSA_DEC1_PPW(2, false, true, false);
      else MSA_DEC1_PPW(2, false, false, false);
    }
#undef MSA_DEC1_PPW
#undef MSA_DEC1_LAUNCH
  } else if (p.T <= 8) {
    // speculative decode: one row tile of 4 tokens x 4 groups for T <= 4, two for T <= 8
    const int ppw = pick_ppw(kDecPagesPerWave, 2);
    const dim3 grid((unsigned)((nloc + kDecWaves * ppw - 1) / (kDecWaves * ppw)), (unsigned)p.B);
#define MSA_DEC_LAUNCH(KT, FM, TS, PPW, NT)                                                                  \
  hipLaunchKernelGGL((indexer_decode_kernel<KT, FM, TS, (KT == 2 ? kDecTpu : kDecTpu / 2),            \
                                            kDecPipe, PPW, NT>), grid, dim3(kDecWaves * 64), 0, s, q8, \
                     k.data, k.scales, k.num_pages, p.seq_lens, p.block_table, p.max_blocks, p.T,             \
                     sigma, block_scores, token_scores, shard, num_shards, skip)
#define MSA_DEC_PPW(KT, FM, TS, NT)                                                                   \
  do {                                                                                                \
    if (ppw == kDecPagesPerWave) MSA_DEC_LAUNCH(KT, FM, TS, kDecPagesPerWave, NT);                    \
    else if (ppw == kDecPagesPerWave / 2) MSA_DEC_LAUNCH(KT, FM, TS, kDecPagesPerWave / 2, NT);       \
    else MSA_DEC_LAUNCH(KT, FM, TS, kDecPagesPerWave / 4, NT);                                        \
  } while (0)
#define MSA_DEC_NT(KT, FM, TS)                      \
  do {                                              \
    if (p.T <= 4) MSA_DEC_PPW(KT, FM, TS, 1);       \
    else MSA_DEC_PPW(KT, FM, TS, 2);                \
  } while (0)
    const bool ts = token_scores != nullptr;
    if (k.dtype == 1) {
      if (ts) MSA_DEC_NT(1, false, true); else MSA_DEC_NT(1, false, false);
    } else if (fp8mode) {
      if (ts) MSA_DEC_NT(2, true, true); else MSA_DEC_NT(2, true, false);
    } else {
      if (ts) MSA_DEC_NT(2, false, true); else MSA_DEC_NT(2, false, false);
    }
#undef MSA_DEC_NT
#undef MSA_DEC_PPW
#undef MSA_DEC_LAUNCH
  } else {
    return launch_indexer_prefill(p, idx_q, k, fp8mode, sigma, block_scores, token_scores, s);
  }
  return hipGetLastError();
}

}  // namespace msa
