// Step 4 of MSA: exact attention over the selected blocks (kernels and
// launcher; the MFMA path's device code is in attn_row.hpp).
//
// Source: "vLLM 為 MiniMax-M3.1-Flash 提供 Day-0 支援", section "MSA primer"
// and its Figure 1 caption: attention is computed exactly, restricted to
// the keys of the kept blocks, and all query heads of a GQA group share their
// group's blocks -- so full K/V is read for 2,048 keys at most per query.
//
// One workgroup per (sequence, query token, group) with 16 waves; wave w
// takes the w-th selected block.  All of a block's K loads and the first V
// tiles are issued together right after the block-table lookup, so a wave
// waits on memory about twice (K, then the rest of V) rather than once per
// tile.  Per block (one KV head, 16 query heads):
//   S^T = K Q^T on 16x16x32 f16 MFMAs (A = 16 keys x 32 dims of K, straight
//         from the page: lane quarter Q loads dims [32Q, 32Q+32) of its key;
//         B = Q^T, the 16 heads of the group);
//   softmax over the block's <= 128 keys in fp32 (exp2 domain);
//   O^T += V^T P^T on 16x16x32 f16 MFMAs, two 16-key tiles per product.  The
//         lane layout of S^T is the B operand P^T of the next product, so P
//         never leaves registers; it enters as f16 (round to nearest, at most
//         2^-12 relative error per element; the softmax sum stays fp32).
//         Each 16-key V tile is dequantised into a wave-private LDS slice in
//         its natural [key][dim] f16 layout (16-byte writes, chunks
//         XOR-swizzled per key so that neither the writes nor the reads meet
//         bank conflicts) and read back with gfx950's transposing LDS read
//         (ds_read_b64_tr_b16), which hands each lane 4 consecutive keys of
//         one dim: the A operand of V^T.  Keys past the query's position are
//         zeroed before decoding (their scale byte, or their FP8 bytes).
// The 16 per-block partial states (max, sum, O) are merged in one pass over
// LDS, summed in wave order, so results are deterministic.
// FP8 and NVFP4 values are exact in f16, so Q K^T is exact up to its fp32
// accumulation; P V carries P's f16 rounding.
#include <math.h>

#include "attn_row.hpp"
#include "launch.hpp"

namespace msa {

// SELECT: each workgroup first selects its row's 16 blocks from the block
// scores (msa_topk_sparse_attn), so the selection needs no launch of its own.
constexpr int kDecodeWaves = 16;   // waves per row below kAttnManyRows rows
constexpr int kAttnManyWg = 3;     // resident workgroups per CU of the 4-wave form
template <int KT, bool FP8MODE, int WAVES, bool SELECT = false>
__global__ __launch_bounds__(WAVES * 64, WAVES == 16 ? 1 : WAVES == 8 ? 2 : kAttnManyWg) void attn_mfma_kernel(
    AttnArgs a) {
  attend_row<KT, FP8MODE, WAVES, SELECT>(a, blockIdx.x);
}

// Many rows (prefill): workgroups go to the 8 XCDs round-robin, so workgroup
// w runs on XCD w % 8.  Rows are renumbered (sequence, group)-major -- r' =
// (b*4 + g)*T + t -- and XCD x takes the contiguous run of r' starting at
// x * per: each XCD's L2 then serves consecutive tokens of as few (sequence,
// KV head) pairs as possible, which share their own block, planted blocks and
// many others (c5: one pair per XCD instead of two sequences' alternate
// tokens).  The grid is 8 * per; workgroups past the rows return at once.
constexpr int kXcds = 8;
template <int KT, bool FP8MODE>
__global__ __launch_bounds__(256, kAttnManyWg) void attn_many_kernel(AttnArgs a, int nrows, int per) {
  const int rr = (int)(blockIdx.x % kXcds) * per + (int)(blockIdx.x / kXcds);
  if (rr >= nrows) return;
  const int bg = rr / a.T, t = rr - bg * a.T;
  const int b = bg >> 2, g = bg & 3;
  attend_row<KT, FP8MODE, 4, false>(a, (b * a.T + t) * kGroups + g);
}

// Shared-prefix form: staged prefix blocks come from their operand images.
// Always the 16-wave form (decode row counts), whatever the number of rows.
template <int KT, bool FP8MODE, int WAVES>
__global__ __launch_bounds__(WAVES * 64, 1) void attn_prefix_kernel(AttnArgs a, PrefixAttnArgs pa) {
  attend_row<KT, FP8MODE, WAVES, false, true>(a, blockIdx.x, &pa);
}

// fp32 queries and caches: plain fp32 arithmetic on the vector ALUs.  One
// workgroup per (sequence, token, group); thread (head h = tid/16, part =
// tid%16) owns dims part*8 .. part*8+7 of head h's output.
__global__ __launch_bounds__(256) void attn_f32_kernel(
    const float* __restrict__ q, float c_nat, const float* __restrict__ kdata, int64_t kpages,
    const float* __restrict__ vdata, int64_t vpages, float v_scale, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ table, int max_blocks, int T,
    float* __restrict__ out, float* __restrict__ lse) {
  __shared__ float qs[16][kHeadDim];
  __shared__ float logit[16][kBlock];
  const int row = blockIdx.x;
  const int g = row & 3, bt = row >> 2, t = bt % T, b = bt / T;
  const int tid = threadIdx.x, h = tid >> 4, part = tid & 15;
  const int L = seq_lens[b];
  const int p = L - T + t;
  const float NEG_INF = -__builtin_inff();
  const float* qbase = q + (((size_t)b * T + t) * kHeads + g * kHeadsPerGroup) * kHeadDim;
  for (int e = tid; e < 16 * kHeadDim; e += 256) qs[e / kHeadDim][e % kHeadDim] = qbase[e];
  float m = NEG_INF, lsum = 0.0f, o[8];
  for (int d = 0; d < 8; ++d) o[d] = 0.0f;
  bool bad = false;
  for (int w = 0; w < kTopK; ++w) {
    const int blk = sel[(size_t)row * kTopK + w];
    if (blk < 0) continue;
    if (blk >= max_blocks) { bad = true; continue; }
    const int pg = table[(size_t)b * max_blocks + blk];
    if (pg < 0 || (int64_t)pg >= kpages || (int64_t)pg >= vpages) { bad = true; continue; }
    const int nkeys = min(kBlock, p + 1 - blk * kBlock);
    if (nkeys <= 0) continue;
    const size_t rowbase = ((size_t)pg * kGroups + g) * kBlock;
    __syncthreads();
    for (int kk = part; kk < kBlock; kk += 16) {
      float v = NEG_INF;
      if (kk < nkeys) {
        const float* krow = kdata + (rowbase + kk) * kHeadDim;
        float acc = 0.0f;
        for (int d = 0; d < kHeadDim; ++d) acc = fmaf(qs[h][d], krow[d], acc);
        v = acc * c_nat;
      }
      logit[h][kk] = v;
    }
    __syncthreads();
    float bm = NEG_INF;
    for (int kk = 0; kk < nkeys; ++kk) bm = fmaxf(bm, logit[h][kk]);
    const float mn = fmaxf(m, bm);
    const float corr = (m == NEG_INF) ? 0.0f : expf(m - mn);
    lsum *= corr;
    for (int d = 0; d < 8; ++d) o[d] *= corr;
    for (int kk = 0; kk < nkeys; ++kk) {
      const float pk = expf(logit[h][kk] - mn);
      lsum += pk;
      const float* vrow = vdata + (rowbase + kk) * kHeadDim + part * 8;
      for (int d = 0; d < 8; ++d) o[d] = fmaf(pk, vrow[d], o[d]);
    }
    m = mn;
  }
  const int head = g * kHeadsPerGroup + h;
  float* dst = out + (((size_t)b * T + t) * kHeads + head) * kHeadDim + part * 8;
  for (int d = 0; d < 8; ++d) dst[d] = bad ? __builtin_nanf("") : o[d] * (v_scale / lsum);
  if (lse != nullptr && part == 0)
    lse[((size_t)b * T + t) * kHeads + head] = bad ? __builtin_nanf("") : m + logf(lsum);
}

hipError_t launch_attention(const ProblemArgs& p, const void* q, int q_dtype, float q_scale,
                            const CacheArgs& k, const CacheArgs& v, bool fp8mode,
                            const int32_t* sel, float softmax_scale, float* out, float* lse,
                            hipStream_t s, const float* block_scores, int32_t* sel_out,
                            const PrefixAttnArgs* pa) {
  const unsigned rows = (unsigned)((int64_t)p.B * p.T * kGroups);
  const bool many = rows >= kAttnManyRows;
  // The selection inside the attention launch pays off for decode (few rows: it
  // saves a launch); with many rows (prefill, many speculative tokens) each
  // workgroup's selection latency adds up (2 x 4,096 prefill tokens on
  // 69,632-token contexts: 1.94 ms against 0.10 + 1.68 ms), and the fp32 kernel
  // takes a selection -- there the top-16 kernel runs first.
  bool select = block_scores != nullptr;
  if (select && (k.dtype == 0 || many)) {
    const hipError_t e = launch_topk(p, block_scores, sel_out, s);
    if (e != hipSuccess) return e;
    sel = sel_out;
    select = false;
  }
  if (k.dtype == 0) {
    const float c_nat = softmax_scale * q_scale * k.tensor_scale;
    hipLaunchKernelGGL(attn_f32_kernel, dim3(rows), dim3(256), 0, s, (const float*)q, c_nat,
                       (const float*)k.data, k.num_pages, (const float*)v.data, v.num_pages,
                       v.tensor_scale, sel, p.seq_lens, p.block_table, p.max_blocks, p.T, out, lse);
    return hipGetLastError();
  }
  const float c_log2 = softmax_scale * q_scale * k.tensor_scale * 1.4426950408889634f;
  const uint8_t* q8 = (const uint8_t*)q;
  // Few rows (decode): 16 waves per row, one selected block each, so every
  // block of the step is in flight at once, but one row per CU at a time.
  // Many rows (>= 1,024: prefill, or 8 speculative tokens on 64 sequences): 4
  // waves per row with 4 blocks each and a 4-way merge -- a small LDS
  // footprint and three resident rows per CU (2,048 rows: 165 us against
  // 215 us).  The choice depends only on the row count.
  const int per = (int)((rows + kXcds - 1) / kXcds);   // rows per XCD in the many-rows form
  const AttnArgs aa{q8, c_log2, k.data, k.scales, k.num_pages, v.data, v.scales, v.num_pages, v.tensor_scale,
                    sel, p.seq_lens, p.block_table, p.max_blocks, p.T, out, lse, block_scores, sel_out};
#define MSA_ATTN_LAUNCH(KT, FM)                                                                        \
  if (pa != nullptr)                                                                                   \
    hipLaunchKernelGGL((attn_prefix_kernel<KT, FM, kDecodeWaves>), dim3(rows), dim3(kDecodeWaves * 64), 0, s, \
                       aa, *pa);                                                                       \
  else if (many)                                                                                       \
    hipLaunchKernelGGL((attn_many_kernel<KT, FM>), dim3(kXcds * per), dim3(256), 0, s, aa, (int)rows, per); \
  else if (select)                                                                                     \
    hipLaunchKernelGGL((attn_mfma_kernel<KT, FM, kDecodeWaves, true>), dim3(rows), dim3(kDecodeWaves * 64), 0, \
                       s, aa);                                                                         \
  else                                                                                                 \
    hipLaunchKernelGGL((attn_mfma_kernel<KT, FM, kDecodeWaves, false>), dim3(rows), dim3(kDecodeWaves * 64), 0, \
                       s, aa)
  if (k.dtype == 1) { MSA_ATTN_LAUNCH(1, false); }
  else if (fp8mode) { MSA_ATTN_LAUNCH(2, true); }
  else { MSA_ATTN_LAUNCH(2, false); }
#undef MSA_ATTN_LAUNCH
  return hipGetLastError();
}

}  // namespace msa
