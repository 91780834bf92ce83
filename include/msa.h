/*
 * msa.h -- C ABI of libmsa, the MI355X (gfx950) hot path of MiniMax Sparse
 * Attention (MSA).
 *
 * The method (source: "vLLM 為 MiniMax-M3.1-Flash 提供 Day-0 支援", English
 * post, section "MSA primer" and its Figure 1 caption): keys are grouped in
 * blocks of 128 tokens.  A small indexer gives every key a score per GQA
 * group (the group's 128-dim index query dotted with the key's entry in one
 * index-key head common to all groups) and reduces each block to the maximum
 * of its keys' scores.  Per group 16 blocks are kept -- always including the
 * newest -- and exact attention runs over those keys only (2,048 at most),
 * shared by the group's query heads.  K/V and index keys are held as FP8 or
 * NVFP4, queries as FP8 (sections "What is new in the MiniMax-M3.1
 * architecture" and "NVIDIA Blackwell optimized MSA kernels").
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Shapes are fixed by the model: groups G = 4 (= KV heads), 16 query
 *    heads per group (64 query heads), head_dim 128, block 128 tokens,
 *    top-k 16.  Other values return MSA_ERR_UNSUPPORTED.
 *  - Sequence b has length L_b = seq_lens[b], counting its T new query
 *    tokens; query token t sits at position p = L_b - T + t, sees keys 0..p,
 *    and its own ("most recent") block is p / 128.
 *  - A paged cache holds pages of 128 tokens.  Page `pg`, head `h`, token `r`
 *    of a cache with `heads` heads is row ((pg*heads + h)*128 + r):
 *       MSA_F32      : 128 floats per row
 *       MSA_FP8_E4M3 : 128 bytes per row (OCP E4M3)
 *       MSA_NVFP4    : 64 bytes of E2M1 codes per row in `data` (two per
 *                      byte, even dim in the low nibble) and 8 E4M3 scale
 *                      bytes per row in `scales` (one per 16 dims)
 *    Logical block i of sequence b lives in page block_table[b*max_blocks+i].
 *    The index-key cache has heads = 1; the K and V caches have heads = 4.
 *  - Every decoded value is tensor_scale * element (NVFP4: tensor_scale *
 *    e4m3(scale byte) * e2m1(code), or that product re-rounded to E4M3 under
 *    MSA_DQ_FP8).
 *  - Ownership: every array is caller-owned device memory (except where a
 *    host pointer is stated).  The library allocates nothing on these
 *    paths and keeps no state besides immutable code; calls are re-entrant.
 *  - Asynchrony: every compute call enqueues its kernels on `stream` and
 *    returns at once; outputs are valid once the stream reaches that point.
 *  - Errors: argument errors that can be seen from the host (null pointers,
 *    unsupported shapes or dtype pairs, non-positive scales, a workspace
 *    that is too small) return their status before any HIP call and leave
 *    the outputs untouched.  A failed launch returns MSA_ERR_HIP.  Device
 *    arrays are not validated from the host: seq_lens must satisfy
 *    T <= L_b <= max_blocks*128; a page id outside [0, num_pages) is never
 *    dereferenced -- that block's scores and any attention output touching
 *    it become NaN.
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_ABI_VERSION 2

typedef enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARG = 1,   /* null pointer, bad size, non-positive scale   */
  MSA_ERR_UNSUPPORTED = 2,   /* shape or dtype combination not implemented   */
  MSA_ERR_WORKSPACE = 3,     /* workspace null or smaller than required      */
  MSA_ERR_HIP = 4            /* a HIP launch or query failed                 */
} msa_status;

typedef enum { MSA_F32 = 0, MSA_FP8_E4M3 = 1, MSA_NVFP4 = 2 } msa_dtype;

/* How NVFP4 elements are decoded before a dot product (ignored for F32/FP8).
 *  MSA_DQ_FP8:   e2m1 * e4m3 scale re-rounded to E4M3 (nearest-even,
 *    saturating at 448) -- what the kernels that dequantise NVFP4 to FP8 for
 *    an FP8 matrix product compute ("NVIDIA Blackwell optimized MSA kernels";
 *    the CDNA4 kernel's table of pre-rounded products, "NVFP4 MSA kernel").
 *  MSA_DQ_EXACT: the product e2m1 * e4m3 scale itself, as a 16-bit
 *    dequantisation keeps it ("NVIDIA Rubin optimized MSA", where the scores
 *    are exact).
 * Every call takes the reading explicitly; neither is implied. */
typedef enum { MSA_DQ_FP8 = 0, MSA_DQ_EXACT = 1 } msa_dequant;

typedef struct {
  msa_dtype dtype;
  const void* data;          /* F32 floats, FP8 bytes, or NVFP4 codes        */
  const uint8_t* scales;     /* NVFP4 only: 8 E4M3 bytes per row; else NULL  */
  float tensor_scale;        /* > 0, finite                                  */
  int32_t heads;             /* 1 for the index-key cache, 4 for K and V     */
  int32_t head_dim;          /* 128                                          */
  int64_t num_pages;         /* pages in the pool                            */
} msa_cache;

typedef struct {
  int32_t batch;             /* B >= 1                                       */
  int32_t tokens;            /* T >= 1 query tokens per sequence             */
  int32_t groups;            /* 4                                            */
  int32_t heads_per_group;   /* 16                                           */
  int32_t head_dim;          /* 128                                          */
  int32_t block_size;        /* 128                                          */
  int32_t topk;              /* 16                                           */
  const int32_t* seq_lens;   /* device [B]                                   */
  const int32_t* block_table;/* device [B][max_blocks]                       */
  int32_t max_blocks;        /* >= 1; <= 8192                                */
} msa_problem;

/* Steps 1+2: index scores max-pooled per block ("MSA primer": each GQA group
 * has one index query, dotted with the single index-key head that all groups
 * share, for every key of the context; a block's score is the largest of its
 * keys' scores).
 *   idx_q        device [B][T][4][128]: F32 floats or FP8 bytes (q_dtype),
 *                each decoded value times q_scale.
 *   idx_k        the index-key cache (heads = 1): F32 with F32 queries;
 *                FP8 or NVFP4 with FP8 queries.
 *   block_scores device out [B][T][4][max_blocks] fp32:
 *                max over block i's keys j <= p of (q . k); -inf for blocks
 *                wholly after p and for i >= ceil(L_b/128).
 *   token_scores device out, nullable, [B][T][4][max_blocks*128] fp32:
 *                the per-key scores (-inf past p), for inspection only.
 * Any T >= 1: T <= 8 runs the decode scans, larger T the prefill kernel. */
msa_status msa_indexer_scores(const msa_problem* prob, const void* idx_q, msa_dtype q_dtype,
                              float q_scale, const msa_cache* idx_k, msa_dequant dequant,
                              float* block_scores, float* token_scores, hipStream_t stream);

/* Step 3: top-16 blocks per (sequence, token, group) ("MSA primer": 16
 * blocks are kept per group, one of them always the newest).  With own+1 <=
 * 16 visible blocks all of them are selected; otherwise the own block plus
 * the 15 best older blocks by (score descending, block index ascending).
 * NaN ranks below every number.
 *   block_scores device [B][T][4][max_blocks] (as written above).
 *   sel          device out [B][T][4][16] int32 logical block ids,
 *                ascending, padded with -1.
 *   workspace    device scratch of at least msa_workspace_size(prob,
 *                MSA_CALL_TOPK) bytes; that size is 0, so NULL and 0 are
 *                accepted. */
msa_status msa_block_topk(const msa_problem* prob, const float* block_scores, int32_t* sel,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Step 4: exact attention over the selected blocks ("MSA primer" and Figure
 * 1: exact attention, restricted to the keys of the kept blocks; every query
 * head of a group uses its group's selection).  Head h uses group h / 16.
 *   q            device [B][T][64][128]: F32 floats or FP8 bytes, times q_scale.
 *   k, v         caches with heads = 4 (F32 with F32 q; FP8 or NVFP4 with FP8 q).
 *   sel          device [B][T][4][16] as written by msa_block_topk.
 *   softmax_scale  logits are softmax_scale * (q . k) (1/sqrt(128) for MSA).
 *                softmax_scale * q_scale * k->tensor_scale * log2(e) must be a
 *                positive finite float, else MSA_ERR_INVALID_ARG.
 *   out          device out [B][T][64][128] fp32.
 *   lse          device out, nullable, [B][T][64] fp32: natural-log
 *                log-sum-exp of the scaled logits.
 *   workspace    device scratch of at least msa_workspace_size(prob,
 *                MSA_CALL_ATTN) bytes (may be NULL when that size is 0).
 * msa_sparse_attn_decode requires T <= 8; msa_sparse_attn_prefill takes any
 * T >= 1 (same results). */
msa_status msa_sparse_attn_decode(const msa_problem* prob, const void* q, msa_dtype q_dtype,
                                  float q_scale, const msa_cache* k, const msa_cache* v,
                                  msa_dequant dequant, const int32_t* sel, float softmax_scale,
                                  float* out, float* lse, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);
msa_status msa_sparse_attn_prefill(const msa_problem* prob, const void* q, msa_dtype q_dtype,
                                   float q_scale, const msa_cache* k, const msa_cache* v,
                                   msa_dequant dequant, const int32_t* sel, float softmax_scale,
                                   float* out, float* lse, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/* Indexer decode context parallelism (DCP), on one GPU (sections "NVFP4
 * indexer DCP", NVIDIA and AMD parts: each of P GPUs scores all four groups
 * over its share of the pages; each sends its local top-16 per group to the
 * group's owner, which merges them into the final top-16 -- an exact
 * selection; on AMD the scores themselves, bit-identical to a single-GPU
 * run, are written into the owner's buffer).  Shard s of num_shards holds
 * the logical blocks i with i % num_shards == s.  1 <= num_shards <=
 * MSA_MAX_SHARDS and 0 <= shard < num_shards, else MSA_ERR_INVALID_ARG.
 *
 * msa_indexer_scores_shard: msa_indexer_scores restricted to the shard's
 *   blocks: their entries of block_scores [B][T][4][max_blocks] are written
 *   (the same bits as one msa_indexer_scores call writes there, -inf past the
 *   sequence); every other entry is left untouched, so running every shard
 *   once fills block_scores exactly as msa_indexer_scores does.  FP8 or NVFP4
 *   index keys and tokens <= 8 (decode and speculative decode), else
 *   MSA_ERR_UNSUPPORTED; no per-key scores.
 * msa_shard_topk: the shard's local top-16 per (sequence, token, group) row
 *   of block_scores: among the shard's blocks older than the row's own block
 *   (p / 128), the 16 best by (score descending, block ascending), best
 *   first, as cand_scores [B][T][4][16] fp32 (the score bits as read) and
 *   cand_blocks [B][T][4][16] int32; a shard with fewer candidates pads with
 *   NaN / -1.  NaN ranks below every number.  Reads only the shard's entries.
 * msa_topk_merge: the owner's merge.  cand_scores / cand_blocks are
 *   [num_shards][B][T][4][16], shard s's lists from msa_shard_topk at offset
 *   s*B*T*4*16.  Writes sel [B][T][4][16] equal to msa_block_topk on the full
 *   block_scores: with own+1 <= 16 visible blocks 0..own, else the own block
 *   and the 15 best candidates, ascending, -1 padded.  Candidates that are
 *   not older than the row's own block are ignored; the lists must come from
 *   distinct shards of one partition. */
#define MSA_MAX_SHARDS 8
msa_status msa_indexer_scores_shard(const msa_problem* prob, int32_t shard, int32_t num_shards,
                                    const void* idx_q, msa_dtype q_dtype, float q_scale,
                                    const msa_cache* idx_k, msa_dequant dequant, float* block_scores,
                                    hipStream_t stream);
msa_status msa_shard_topk(const msa_problem* prob, int32_t shard, int32_t num_shards,
                          const float* block_scores, float* cand_scores, int32_t* cand_blocks,
                          hipStream_t stream);
msa_status msa_topk_merge(const msa_problem* prob, int32_t num_shards, const float* cand_scores,
                          const int32_t* cand_blocks, int32_t* sel, hipStream_t stream);

/* Shared-prefix decode for the index scan (section "NVFP4 MSA kernel": a
 * prefix page common to as many as 64 requests is decoded a single time for
 * all of them).  Sequences [group_start[k], group_start[k+1]) of the batch form
 * prefix group k; their block-table rows hold the same page ids in their
 * first prefix_blocks[k] logical blocks (the caller's promise: the pages are
 * read through the group's first row).  Writes the same block_scores as
 * msa_indexer_scores: the shared blocks are scored once for the whole group,
 * as one GEMM over all of its query rows (every shared page read and
 * dequantised once), each row keeping its own causal position; the other
 * blocks of every sequence by the decode scan.  Shared-block scores equal
 * msa_indexer_scores' within fp32 summation order (a different MFMA shape);
 * the -inf pattern is identical.
 *   num_groups     0 .. MSA_MAX_PREFIX_GROUPS;
 *   group_start    HOST [num_groups+1], strictly increasing, within
 *                  [0, batch]; each group holds 1 .. MSA_MAX_PREFIX_SEQS
 *                  sequences; sequences outside every group are scanned alone;
 *   prefix_blocks  HOST [num_groups], each in [0, max_blocks];
 *   workspace      device, at least msa_workspace_size(prob,
 *                  MSA_CALL_INDEXER_PREFIX) bytes (4 per sequence), scratch:
 *                  overwritten by every call, so calls that share it must not
 *                  overlap.
 * FP8 or NVFP4 index keys and tokens <= 8, else MSA_ERR_UNSUPPORTED; other
 * arguments as for msa_indexer_scores (no per-key scores). */
#define MSA_MAX_PREFIX_GROUPS 64
#define MSA_MAX_PREFIX_SEQS 64
msa_status msa_indexer_scores_prefix(const msa_problem* prob, int32_t num_groups, const int32_t* group_start,
                                     const int32_t* prefix_blocks, const void* idx_q, msa_dtype q_dtype,
                                     float q_scale, const msa_cache* idx_k, msa_dequant dequant,
                                     float* block_scores, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/* Shared-prefix decode attention (section "NVFP4 MSA kernel": a prefix page
 * common to as many as 64 requests is decoded a single time for all of them).
 * The same out and lse as msa_sparse_attn_decode with the same arguments, bit
 * for bit.  Prefix groups as for msa_indexer_scores_prefix: sequences
 * [group_start[k], group_start[k+1]) hold the same page ids in their first
 * prefix_blocks[k] logical blocks.  Every block below prefix_blocks[k] that two
 * or more rows of group k selected as an older block (not their own block)
 * is dequantised once per KV head into the workspace, as the operands the
 * attention's matrix products take; those rows read it from there instead of
 * decoding the page again.  Other blocks are decoded as usual.
 *   num_groups, group_start, prefix_blocks  HOST arrays, as for
 *                msa_indexer_scores_prefix (0..64 groups of 1..64 sequences);
 *   workspace    device, 256-byte aligned, at least
 *                msa_sparse_attn_prefix_workspace_size(prob, num_groups,
 *                group_start, prefix_blocks) bytes (64 KiB per block slot,
 *                min(prefix_blocks[k], 16 * rows of group k) slots per group
 *                and KV head, plus a slot map); scratch, overwritten by every
 *                call, so calls sharing it must not overlap.
 * FP8 or NVFP4 K/V and tokens <= 8, else MSA_ERR_UNSUPPORTED; other arguments
 * and errors as for msa_sparse_attn_decode. */
msa_status msa_sparse_attn_decode_prefix(const msa_problem* prob, int32_t num_groups, const int32_t* group_start,
                                         const int32_t* prefix_blocks, const void* q, msa_dtype q_dtype,
                                         float q_scale, const msa_cache* k, const msa_cache* v, msa_dequant dequant,
                                         const int32_t* sel, float softmax_scale, float* out, float* lse,
                                         void* workspace, size_t workspace_bytes, hipStream_t stream);
/* Workspace bytes msa_sparse_attn_decode_prefix needs for these prefix groups
 * (reads only host memory and host-visible fields of prob); 0 for invalid
 * arguments. */
size_t msa_sparse_attn_prefix_workspace_size(const msa_problem* prob, int32_t num_groups,
                                             const int32_t* group_start, const int32_t* prefix_blocks);

/* Steps 3+4 in one launch ("MSA primer": keep the top 16 blocks with the most
 * recent one forced, then attend exactly over them): what msa_block_topk
 * followed by msa_sparse_attn_decode / _prefill computes, with sel written
 * as msa_block_topk writes it (bit for bit) and out / lse as the attention
 * call writes them given that selection (bit for bit).  With fewer than
 * 1,024 (sequence, token, group) rows (decode) each attention workgroup first
 * selects its own row's blocks from block_scores, so the selection needs no
 * launch of its own; with more rows (speculative decode of many tokens,
 * prefill), and for fp32 caches, the top-16 kernel runs first (there it is
 * the faster way).  Any T >= 1.
 *   block_scores  device [B][T][4][max_blocks], as msa_indexer_scores writes;
 *   sel           device out [B][T][4][16];
 * other arguments as for msa_sparse_attn_decode (no workspace). */
msa_status msa_topk_sparse_attn(const msa_problem* prob, const float* block_scores, int32_t* sel, const void* q,
                                msa_dtype q_dtype, float q_scale, const msa_cache* k, const msa_cache* v,
                                msa_dequant dequant, float softmax_scale, float* out, float* lse,
                                hipStream_t stream);

/* Steps 1-3 in one call ("MSA primer": score, max-pool per block, keep the top
 * 16 blocks with the most recent one forced): the same block_scores and sel as
 * msa_indexer_scores followed by msa_block_topk, bit for bit.  For one query
 * token with FP8 or NVFP4-exact keys a single kernel does both -- the last
 * workgroup to finish a sequence selects that sequence's blocks -- which
 * removes the separate selection pass from the decode step; otherwise the two
 * kernels run back to back.
 *   workspace  device, at least msa_workspace_size(prob, MSA_CALL_INDEXER_TOPK)
 *              bytes (4 per sequence), zero-filled before its first use; every
 *              call leaves it zero-filled again.  Calls that share a workspace
 *              must not overlap (they are ordered on one stream).
 * Other arguments as for msa_indexer_scores and msa_block_topk. */
msa_status msa_indexer_topk(const msa_problem* prob, const void* idx_q, msa_dtype q_dtype,
                            float q_scale, const msa_cache* idx_k, msa_dequant dequant,
                            float* block_scores, int32_t* sel, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* msa_indexer_topk for callers that cannot allocate device memory -- code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc: the
 * same block_scores and sel, bit for bit, with no workspace argument.  The
 * per-sequence arrival counters live in a file-scope device array inside the
 * library (one per GPU, MSA_NOALLOC_MAX_BATCH counters = 16 KiB, held until the
 * process ends); each call clears the counters it uses with a small kernel on
 * `stream` before scanning.  No allocation is made.  Calls on one GPU share
 * that array, so calls that overlap on one GPU (different streams without
 * ordering) race; calls ordered on one stream do not.
 *   batch > MSA_NOALLOC_MAX_BATCH returns MSA_ERR_UNSUPPORTED (before any HIP
 *   call); a failed lookup of the array's address returns MSA_ERR_HIP.
 * Other arguments and errors as for msa_indexer_topk. */
#define MSA_NOALLOC_MAX_BATCH 4096
msa_status msa_indexer_topk_noalloc(const msa_problem* prob, const void* idx_q, msa_dtype q_dtype,
                                    float q_scale, const msa_cache* idx_k, msa_dequant dequant,
                                    float* block_scores, int32_t* sel, hipStream_t stream);

/* Steps 1-4 of one decode layer step in one call ("MSA primer": score,
 * max-pool, select the top 16 blocks with the most recent one forced,
 * attend): msa_indexer_scores, then msa_topk_sparse_attn -- two launches,
 * leaving block_scores, sel, out and lse as msa_indexer_scores +
 * msa_block_topk + msa_sparse_attn_decode do, bit for bit.
 *   idx_q, idx_q_dtype, idx_q_scale, idx_k  as for msa_indexer_scores;
 *   q, q_dtype, q_scale, k, v, softmax_scale, out, lse  as for
 *                msa_sparse_attn_decode (k, v: same dtype; tokens <= 8);
 *   block_scores, sel  outputs as for the two selection calls;
 *   workspace, workspace_bytes  unused (msa_workspace_size reports 0); may
 *                be NULL and 0.
 * Errors as for the three calls. */
msa_status msa_decode_step(const msa_problem* prob, const void* idx_q, msa_dtype idx_q_dtype,
                           float idx_q_scale, const msa_cache* idx_k, const void* q, msa_dtype q_dtype,
                           float q_scale, const msa_cache* k, const msa_cache* v, msa_dequant dequant,
                           float softmax_scale, float* block_scores, int32_t* sel, float* out,
                           float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Quantise-and-insert (section "QKV GEMM + norm + RoPE + KV insert fusion": K,
 * V and the index key are quantised to NVFP4 as they are written into their
 * caches; this is that insert step without the GEMM, norm and RoPE).
 *   x      device fp32 [batch, tokens, cache->heads, 128], contiguous and
 *          16-byte aligned (MSA_ERR_INVALID_ARG otherwise): the rows
 *          of the `tokens` new tokens of each sequence; token t of sequence b
 *          sits at position seq_lens[b] - tokens + t (seq_lens include them).
 *   cache  FP8, NVFP4 or fp32, heads 1 (index keys) or 4 (K or V).  Its data
 *          (and NVFP4 scales) are WRITTEN: the row of position p goes to row
 *          p % 128 of page block_table[b][p / 128], every head of it; nothing
 *          else is touched.  Quantisation as msa_pack_fp8 / msa_pack_nvfp4 with
 *          the cache's tensor_scale, so inserted rows are bit-identical to the
 *          same rows packed in one piece; fp32 rows are copied.
 * A row whose page id lies outside [0, num_pages) is not written (page ids
 * are device data: not checked on the host).  Rows of different calls may
 * share pages; rows of one call must not share a slot. */
msa_status msa_cache_insert(const msa_problem* prob, const float* x, const msa_cache* cache, hipStream_t stream);

/* Several quantise-and-inserts of the same new tokens in one launch (the K,
 * V and index-key rows a decode step appends): the same writes as n calls
 * of msa_cache_insert(prob, x[i], &caches[i]), bit for bit.
 *   n       1 .. MSA_MAX_INSERTS;
 *   x       HOST array of n device pointers, each as msa_cache_insert's x for
 *           caches[i] (fp32 [batch, tokens, caches[i].heads, 128], 16-byte
 *           aligned);
 *   caches  HOST array of n caches (FP8, NVFP4 or fp32; heads 1 or 4), whose
 *           data (and scales) are WRITTEN as msa_cache_insert writes them.
 * The caches must not overlap one another. */
#define MSA_MAX_INSERTS 4
msa_status msa_cache_insert_many(const msa_problem* prob, int32_t n, const float* const* x, const msa_cache* caches,
                                 hipStream_t stream);

typedef enum {
  MSA_CALL_INDEXER = 0,
  MSA_CALL_TOPK = 1,
  MSA_CALL_ATTN = 2,
  MSA_CALL_INDEXER_TOPK = 3,
  MSA_CALL_DECODE_STEP = 4,
  MSA_CALL_INDEXER_PREFIX = 5
} msa_call;

/* Bytes of device workspace a call needs for this problem (0 = none).
 * Reads only host-visible fields of prob. */
size_t msa_workspace_size(const msa_problem* prob, msa_call which);

/* Pack / unpack helpers (section "QKV GEMM + norm + RoPE + KV insert fusion":
 * K, V and the index key are quantised to NVFP4 when inserted).
 * FP8:   out[i] = E4M3_RNE_SAT(x[i] / scale), the division in fp32.
 * NVFP4: rows of row_len (a multiple of 16) floats; per 16 elements
 *        scale byte s = E4M3_RNE_SAT(amax / (6*tensor_scale)) and
 *        code = E2M1_RNE(x / (e4m3(s)*tensor_scale)) clamped to +-6, every
 *        step in fp32 in that order; s = 0 gives zero codes.  codes has
 *        rows*row_len/2 bytes, scales rows*row_len/16 bytes.
 * Unpack writes fp32: scale * value (NVFP4 value per `dequant`).
 * Inputs must be finite. */
msa_status msa_pack_fp8(const float* x, int64_t n, float scale, uint8_t* out, hipStream_t stream);
msa_status msa_unpack_fp8(const uint8_t* x, int64_t n, float scale, float* out, hipStream_t stream);
msa_status msa_pack_nvfp4(const float* x, int64_t rows, int32_t row_len, float tensor_scale,
                          uint8_t* codes, uint8_t* scales, hipStream_t stream);
msa_status msa_unpack_nvfp4(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                            int32_t row_len, float tensor_scale, msa_dequant dequant, float* out,
                            hipStream_t stream);

/* Static string for a status code; never NULL. */
const char* msa_status_string(msa_status s);
/* MSA_ABI_VERSION of the built library. */
int msa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MSA_H_ */
