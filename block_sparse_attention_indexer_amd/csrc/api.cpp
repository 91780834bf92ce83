// The C ABI of libmsa (declared in include/msa.h): host-side argument
// validation, then one or more kernel launches on the caller's stream.
// Validation makes no HIP call, so a rejected call has no side effect.
#include <math.h>
#include <stdint.h>


#include "../../include/msa.h"
#include "launch.hpp"

namespace {

using msa::CacheArgs;
using msa::ProblemArgs;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool good_scale(float s) { return isfinite(s) && s > 0.0f; }

msa_status check_problem(const msa_problem* p) {
  if (p == nullptr) return MSA_ERR_INVALID_ARG;
  if (p->groups != 4 || p->heads_per_group != 16 || p->head_dim != 128 || p->block_size != 128 ||
      p->topk != 16)
    return MSA_ERR_UNSUPPORTED;
  if (p->batch < 1 || p->tokens < 1 || p->max_blocks < 1) return MSA_ERR_INVALID_ARG;
  if (p->batch > 65535 || p->max_blocks > 8192 || p->tokens > 262144) return MSA_ERR_UNSUPPORTED;
  if ((int64_t)p->batch * p->tokens * 4 > 0x7FFFFFFF) return MSA_ERR_UNSUPPORTED;
  if (p->seq_lens == nullptr || p->block_table == nullptr) return MSA_ERR_INVALID_ARG;
  if (!aligned(p->seq_lens, 4) || !aligned(p->block_table, 4)) return MSA_ERR_INVALID_ARG;
  return MSA_OK;
}

msa_status check_cache(const msa_cache* c, int heads) {
  if (c == nullptr || c->data == nullptr) return MSA_ERR_INVALID_ARG;
  if (c->dtype != MSA_F32 && c->dtype != MSA_FP8_E4M3 && c->dtype != MSA_NVFP4) return MSA_ERR_UNSUPPORTED;
  if (c->head_dim != 128) return MSA_ERR_UNSUPPORTED;
  if (c->heads != heads) return MSA_ERR_INVALID_ARG;
  if (c->num_pages < 1 || c->num_pages > 0x7FFFFFFF) return MSA_ERR_INVALID_ARG;
  if (!good_scale(c->tensor_scale)) return MSA_ERR_INVALID_ARG;
  if (!aligned(c->data, 16)) return MSA_ERR_INVALID_ARG;
  if (c->dtype == MSA_NVFP4 && (c->scales == nullptr || !aligned(c->scales, 8))) return MSA_ERR_INVALID_ARG;
  return MSA_OK;
}

// Allowed pairs: F32 query with F32 cache; FP8 query with FP8 or NVFP4 cache.
msa_status check_pair(msa_dtype q_dtype, msa_dtype c_dtype) {
  if (q_dtype == MSA_F32 && c_dtype == MSA_F32) return MSA_OK;
  if (q_dtype == MSA_FP8_E4M3 && (c_dtype == MSA_FP8_E4M3 || c_dtype == MSA_NVFP4)) return MSA_OK;
  return MSA_ERR_UNSUPPORTED;
}

CacheArgs to_args(const msa_cache* c) {
  return CacheArgs{static_cast<const uint8_t*>(c->data), c->scales, c->num_pages, c->tensor_scale,
                   (int)c->dtype};
}
ProblemArgs to_args(const msa_problem* p) {
  return ProblemArgs{p->batch, p->tokens, p->max_blocks, p->seq_lens, p->block_table};
}
msa_status hip_status(hipError_t e) { return e == hipSuccess ? MSA_OK : MSA_ERR_HIP; }


// Prefix groups from the host arrays of a shared-prefix call: 0..64 groups of
// 1..64 consecutive sequences, group_start strictly increasing within [0, batch],
// prefix_blocks within [0, max_blocks].
msa_status read_prefix_groups(const msa_problem* prob, int32_t num_groups, const int32_t* group_start,
                              const int32_t* prefix_blocks, msa::PrefixGroups& g) {
  if (num_groups < 0 || num_groups > MSA_MAX_PREFIX_GROUPS) return MSA_ERR_INVALID_ARG;
  if (num_groups > 0 && (group_start == nullptr || prefix_blocks == nullptr)) return MSA_ERR_INVALID_ARG;
  g.n = num_groups;
  for (int k = 0; num_groups > 0 && k <= num_groups; ++k) {
    g.start[k] = group_start[k];
    if (g.start[k] < 0 || g.start[k] > prob->batch) return MSA_ERR_INVALID_ARG;
    if (k > 0) {
      const int n = g.start[k] - g.start[k - 1];
      if (n < 1 || n > MSA_MAX_PREFIX_SEQS) return MSA_ERR_INVALID_ARG;
    }
  }
  for (int k = 0; k < num_groups; ++k) {
    g.blocks[k] = prefix_blocks[k];
    if (g.blocks[k] < 0 || g.blocks[k] > prob->max_blocks) return MSA_ERR_INVALID_ARG;
  }
  return MSA_OK;
}

msa_status attention(const msa_problem* prob, const void* q, msa_dtype q_dtype, float q_scale,
                     const msa_cache* k, const msa_cache* v, msa_dequant dequant,
                     const int32_t* sel, float softmax_scale, float* out, float* lse,
                     void* workspace, size_t workspace_bytes, hipStream_t stream, int max_t,
                     const float* block_scores = nullptr) {
  msa_status st = check_problem(prob);
  if (st != MSA_OK) return st;
  if (prob->tokens > max_t) return MSA_ERR_UNSUPPORTED;
  if ((st = check_cache(k, 4)) != MSA_OK) return st;
  if ((st = check_cache(v, 4)) != MSA_OK) return st;
  if (k->dtype != v->dtype) return MSA_ERR_UNSUPPORTED;
  if ((st = check_pair(q_dtype, k->dtype)) != MSA_OK) return st;
  if (dequant != MSA_DQ_EXACT && dequant != MSA_DQ_FP8) return MSA_ERR_INVALID_ARG;
  if (q == nullptr || sel == nullptr || out == nullptr) return MSA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(sel, 4) || !aligned(out, 16) || (lse && !aligned(lse, 4)))
    return MSA_ERR_INVALID_ARG;
  if (block_scores != nullptr && !aligned(block_scores, 4)) return MSA_ERR_INVALID_ARG;
  if (!good_scale(q_scale) || !good_scale(softmax_scale)) return MSA_ERR_INVALID_ARG;
  // the combined logit scale (in the exp2 domain) must itself be a positive finite float
  if (!good_scale(softmax_scale * q_scale * k->tensor_scale * 1.4426950408889634f)) return MSA_ERR_INVALID_ARG;
  if (msa_workspace_size(prob, MSA_CALL_ATTN) > workspace_bytes) return MSA_ERR_WORKSPACE;
  (void)workspace;
  return hip_status(msa::launch_attention(to_args(prob), q, (int)q_dtype, q_scale, to_args(k),
                                          to_args(v), dequant == MSA_DQ_FP8, sel, softmax_scale,
                                          out, lse, stream, block_scores,
                                          block_scores != nullptr ? const_cast<int32_t*>(sel) : nullptr));
}

}  // namespace

extern "C" {

msa_status msa_indexer_scores(const msa_problem* prob, const void* idx_q, msa_dtype q_dtype,
                              float q_scale, const msa_cache* idx_k, msa_dequant dequant,
                              float* block_scores, float* token_scores, hipStream_t stream) {
  msa_status st = check_problem(prob);
  if (st != MSA_OK) return st;
  if ((st = check_cache(idx_k, 1)) != MSA_OK) return st;
  if ((st = check_pair(q_dtype, idx_k->dtype)) != MSA_OK) return st;
  if (dequant != MSA_DQ_EXACT && dequant != MSA_DQ_FP8) return MSA_ERR_INVALID_ARG;
  if (idx_q == nullptr || block_scores == nullptr) return MSA_ERR_INVALID_ARG;
  if (!aligned(idx_q, 16) || !aligned(block_scores, 4) || (token_scores && !aligned(token_scores, 4)))
    return MSA_ERR_INVALID_ARG;
  if (!good_scale(q_scale)) return MSA_ERR_INVALID_ARG;
  return hip_status(msa::launch_indexer(to_args(prob), idx_q, (int)q_dtype, q_scale,
                                        to_args(idx_k), dequant == MSA_DQ_FP8, block_scores,
                                        token_scores, stream));
}

msa_status msa_indexer_topk(const msa_problem* prob, const void* idx_q, msa_dtype q_dtype,
                            float q_scale, const msa_cache* idx_k, msa_dequant dequant,
                            float* block_scores, int32_t* sel, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  msa_status st = check_problem(prob);
  if (st != MSA_OK) return st;
  if ((st = check_cache(idx_k, 1)) != MSA_OK) return st;
  if ((st = check_pair(q_dtype, idx_k->dtype)) != MSA_OK) return st;
  if (dequant != MSA_DQ_EXACT && dequant != MSA_DQ_FP8) return MSA_ERR_INVALID_ARG;
  if (idx_q == nullptr || block_scores == nullptr || sel == nullptr) return MSA_ERR_INVALID_ARG;
  if (!aligned(idx_q, 16) || !aligned(block_scores, 4) || !aligned(sel, 4)) return MSA_ERR_INVALID_ARG;
  if (!good_scale(q_scale)) return MSA_ERR_INVALID_ARG;
  if (workspace == nullptr || !aligned(workspace, 4) ||
      workspace_bytes < msa_workspace_size(prob, MSA_CALL_INDEXER_TOPK))
    return MSA_ERR_WORKSPACE;
  const ProblemArgs pa = to_args(prob);
  const CacheArgs ka = to_args(idx_k);
  const bool fp8 = dequant == MSA_DQ_FP8;
  if (msa::indexer_can_fuse_topk(pa, ka, fp8))
    return hip_status(msa::launch_indexer(pa, idx_q, (int)q_dtype, q_scale, ka, fp8, block_scores, nullptr,
                                          stream, sel, static_cast<uint32_t*>(workspace)));
  hipError_t e = msa::launch_indexer(pa, idx_q, (int)q_dtype, q_scale, ka, fp8, block_scores, nullptr, stream);
  if (e != hipSuccess) return MSA_ERR_HIP;
  return hip_status(msa::launch_topk(pa, block_scores, sel, stream));
}

msa_status msa_indexer_topk_noalloc(const msa_problem* prob, const void* idx_q, msa_dtype q_dtype,
                                    float q_scale, const msa_cache* idx_k, msa_dequant dequant,
                                    float* block_scores, int32_t* sel, hipStream_t stream) {
  msa_status st = check_problem(prob);
  if (st != MSA_OK) return st;
  if (prob->batch > MSA_NOALLOC_MAX_BATCH) return MSA_ERR_UNSUPPORTED;
  if ((st = check_cache(idx_k, 1)) != MSA_OK) return st;
  if ((st = check_pair(q_dtype, idx_k->dtype)) != MSA_OK) return st;
  if (dequant != MSA_DQ_EXACT && dequant != MSA_DQ_FP8) return MSA_ERR_INVALID_ARG;
  if (idx_q == nullptr || block_scores == nullptr || sel == nullptr) return MSA_ERR_INVALID_ARG;
  if (!aligned(idx_q, 16) || !aligned(block_scores, 4) || !aligned(sel, 4)) return MSA_ERR_INVALID_ARG;
  if (!good_scale(q_scale)) return MSA_ERR_INVALID_ARG;
  static_assert(MSA_NOALLOC_MAX_BATCH <= msa::kStaticMaxBatch, "the static scratch holds every counter");
  const ProblemArgs pa = to_args(prob);
  const CacheArgs ka = to_args(idx_k);
  const bool fp8 = dequant == MSA_DQ_FP8;
  if (!msa::indexer_can_fuse_topk(pa, ka, fp8)) {
    // the two kernels, which need no scratch
    hipError_t e = msa::launch_indexer(pa, idx_q, (int)q_dtype, q_scale, ka, fp8, block_scores, nullptr, stream);
    if (e != hipSuccess) return MSA_ERR_HIP;
    return hip_status(msa::launch_topk(pa, block_scores, sel, stream));
  }
  uint32_t* counters = nullptr;
  if (msa::static_scratch(&counters) != hipSuccess) return MSA_ERR_HIP;
  // the counters of the previous call were left at zero; cleared again all the same
  hipError_t e = msa::launch_zero_u32(counters, prob->batch, stream);
  if (e != hipSuccess) return MSA_ERR_HIP;
  return hip_status(msa::launch_indexer(pa, idx_q, (int)q_dtype, q_scale, ka, fp8, block_scores, nullptr, stream,
                                        sel, counters));
}

msa_status msa_block_topk(const msa_problem* prob, const float* block_scores, int32_t* sel,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  msa_status st = check_problem(prob);
  if (st != MSA_OK) return st;
  if (block_scores == nullptr || sel == nullptr) return MSA_ERR_INVALID_ARG;
  if (!aligned(block_scores, 4) || !aligned(sel, 4)) return MSA_ERR_INVALID_ARG;
  if (msa_workspace_size(prob, MSA_CALL_TOPK) > workspace_bytes) return MSA_ERR_WORKSPACE;
  (void)workspace;   // the selection needs no scratch (its size is 0)
  return hip_status(msa::launch_topk(to_args(prob), block_scores, sel, stream));
}

msa_status msa_topk_sparse_attn(const msa_problem* prob, const float* block_scores, int32_t* sel, const void* q,
                                msa_dtype q_dtype, float q_scale, const msa_cache* k, const msa_cache* v,
                                msa_dequant dequant, float softmax_scale, float* out, float* lse,
                                hipStream_t stream) {
  if (block_scores == nullptr) return MSA_ERR_INVALID_ARG;
  return attention(prob, q, q_dtype, q_scale, k, v, dequant, sel, softmax_scale, out, lse, nullptr, 0, stream,
                   1 << 30, block_scores);
}

msa_status msa_indexer_scores_shard(const msa_problem* prob, int32_t shard, int32_t num_shards,
                                    const void* idx_q, msa_dtype q_dtype, float q_scale,
                                    const msa_cache* idx_k, msa_dequant dequant, float* block_scores,
                                    hipStream_t stream) {
  msa_status st = check_problem(prob);
  if (st != MSA_OK) return st;
  if (num_shards < 1 || num_shards > MSA_MAX_SHARDS || shard < 0 || shard >= num_shards) return MSA_ERR_INVALID_ARG;
  if ((st = check_cache(idx_k, 1)) != MSA_OK) return st;
  if ((st = check_pair(q_dtype, idx_k->dtype)) != MSA_OK) return st;
  if (idx_k->dtype == MSA_F32 || prob->tokens > 8) return MSA_ERR_UNSUPPORTED;
  if (dequant != MSA_DQ_EXACT && dequant != MSA_DQ_FP8) return MSA_ERR_INVALID_ARG;
  if (idx_q == nullptr || block_scores == nullptr) return MSA_ERR_INVALID_ARG;
  if (!aligned(idx_q, 16) || !aligned(block_scores, 4)) return MSA_ERR_INVALID_ARG;
  if (!good_scale(q_scale)) return MSA_ERR_INVALID_ARG;
  return hip_status(msa::launch_indexer(to_args(prob), idx_q, (int)q_dtype, q_scale, to_args(idx_k),
                                        dequant == MSA_DQ_FP8, block_scores, nullptr, stream, nullptr,
                                        nullptr, shard, num_shards));
}

msa_status msa_indexer_scores_prefix(const msa_problem* prob, int32_t num_groups, const int32_t* group_start,
                                     const int32_t* prefix_blocks, const void* idx_q, msa_dtype q_dtype,
                                     float q_scale, const msa_cache* idx_k, msa_dequant dequant,
                                     float* block_scores, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  msa_status st = check_problem(prob);
  if (st != MSA_OK) return st;
  if ((st = check_cache(idx_k, 1)) != MSA_OK) return st;
  if ((st = check_pair(q_dtype, idx_k->dtype)) != MSA_OK) return st;
  if (idx_k->dtype == MSA_F32 || prob->tokens > 8) return MSA_ERR_UNSUPPORTED;
  if (dequant != MSA_DQ_EXACT && dequant != MSA_DQ_FP8) return MSA_ERR_INVALID_ARG;
  if (idx_q == nullptr || block_scores == nullptr) return MSA_ERR_INVALID_ARG;
  if (!aligned(idx_q, 16) || !aligned(block_scores, 4)) return MSA_ERR_INVALID_ARG;
  if (!good_scale(q_scale)) return MSA_ERR_INVALID_ARG;
  msa::PrefixGroups g{};
  if ((st = read_prefix_groups(prob, num_groups, group_start, prefix_blocks, g)) != MSA_OK) return st;
  if (workspace == nullptr || !aligned(workspace, 4) ||
      workspace_bytes < msa_workspace_size(prob, MSA_CALL_INDEXER_PREFIX))
    return MSA_ERR_WORKSPACE;
  const msa::ProblemArgs pa = to_args(prob);
  const msa::CacheArgs ka = to_args(idx_k);
  const bool fp8 = dequant == MSA_DQ_FP8;
  int32_t* skip = static_cast<int32_t*>(workspace);
  hipError_t e =
      msa::launch_indexer_shared(pa, idx_q, ka, fp8, q_scale * idx_k->tensor_scale, g, block_scores, stream);
  if (e == hipSuccess)
    e = msa::launch_indexer_skipping(pa, idx_q, (int)q_dtype, q_scale, ka, fp8, block_scores, g, skip, stream);
  return hip_status(e);
}

msa_status msa_shard_topk(const msa_problem* prob, int32_t shard, int32_t num_shards, const float* block_scores,
                          float* cand_scores, int32_t* cand_blocks, hipStream_t stream) {
  msa_status st = check_problem(prob);
  if (st != MSA_OK) return st;
  if (num_shards < 1 || num_shards > MSA_MAX_SHARDS || shard < 0 || shard >= num_shards) return MSA_ERR_INVALID_ARG;
  if (block_scores == nullptr || cand_scores == nullptr || cand_blocks == nullptr) return MSA_ERR_INVALID_ARG;
  if (!aligned(block_scores, 4) || !aligned(cand_scores, 4) || !aligned(cand_blocks, 4)) return MSA_ERR_INVALID_ARG;
  return hip_status(msa::launch_shard_topk(to_args(prob), shard, num_shards, block_scores, cand_scores,
                                           cand_blocks, stream));
}

msa_status msa_topk_merge(const msa_problem* prob, int32_t num_shards, const float* cand_scores,
                          const int32_t* cand_blocks, int32_t* sel, hipStream_t stream) {
  msa_status st = check_problem(prob);
  if (st != MSA_OK) return st;
  if (num_shards < 1 || num_shards > MSA_MAX_SHARDS) return MSA_ERR_INVALID_ARG;
  if (cand_scores == nullptr || cand_blocks == nullptr || sel == nullptr) return MSA_ERR_INVALID_ARG;
  if (!aligned(cand_scores, 4) || !aligned(cand_blocks, 4) || !aligned(sel, 4)) return MSA_ERR_INVALID_ARG;
  return hip_status(msa::launch_topk_merge(to_args(prob), num_shards, cand_scores, cand_blocks, sel, stream));
}

msa_status msa_sparse_attn_decode(const msa_problem* prob, const void* q, msa_dtype q_dtype,
                                  float q_scale, const msa_cache* k, const msa_cache* v,
                                  msa_dequant dequant, const int32_t* sel, float softmax_scale,
                                  float* out, float* lse, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  return attention(prob, q, q_dtype, q_scale, k, v, dequant, sel, softmax_scale, out, lse,
                   workspace, workspace_bytes, stream, 8);
}

msa_status msa_sparse_attn_prefill(const msa_problem* prob, const void* q, msa_dtype q_dtype,
                                   float q_scale, const msa_cache* k, const msa_cache* v,
                                   msa_dequant dequant, const int32_t* sel, float softmax_scale,
                                   float* out, float* lse, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  return attention(prob, q, q_dtype, q_scale, k, v, dequant, sel, softmax_scale, out, lse,
                   workspace, workspace_bytes, stream, 262144);
}

msa_status msa_sparse_attn_decode_prefix(const msa_problem* prob, int32_t num_groups, const int32_t* group_start,
                                         const int32_t* prefix_blocks, const void* q, msa_dtype q_dtype,
                                         float q_scale, const msa_cache* k, const msa_cache* v, msa_dequant dequant,
                                         const int32_t* sel, float softmax_scale, float* out, float* lse,
                                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  msa_status st = check_problem(prob);
  if (st != MSA_OK) return st;
  if (prob->tokens > 8) return MSA_ERR_UNSUPPORTED;
  if ((st = check_cache(k, 4)) != MSA_OK) return st;
  if ((st = check_cache(v, 4)) != MSA_OK) return st;
  if (k->dtype != v->dtype || k->dtype == MSA_F32) return MSA_ERR_UNSUPPORTED;
  if ((st = check_pair(q_dtype, k->dtype)) != MSA_OK) return st;
  if (dequant != MSA_DQ_EXACT && dequant != MSA_DQ_FP8) return MSA_ERR_INVALID_ARG;
  if (q == nullptr || sel == nullptr || out == nullptr) return MSA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(sel, 4) || !aligned(out, 16) || (lse && !aligned(lse, 4)))
    return MSA_ERR_INVALID_ARG;
  if (!good_scale(q_scale) || !good_scale(softmax_scale)) return MSA_ERR_INVALID_ARG;
  if (!good_scale(softmax_scale * q_scale * k->tensor_scale * 1.4426950408889634f)) return MSA_ERR_INVALID_ARG;
  msa::PrefixGroups g{};
  if ((st = read_prefix_groups(prob, num_groups, group_start, prefix_blocks, g)) != MSA_OK) return st;
  const size_t need = msa::prefix_workspace_layout(g, prob->tokens).bytes;
  if (workspace == nullptr || !aligned(workspace, 256) || workspace_bytes < need) return MSA_ERR_WORKSPACE;
  return hip_status(msa::launch_attention_prefix(to_args(prob), q, q_scale, to_args(k), to_args(v),
                                                 dequant == MSA_DQ_FP8, sel, softmax_scale, out, lse, g, workspace,
                                                 stream));
}

size_t msa_sparse_attn_prefix_workspace_size(const msa_problem* prob, int32_t num_groups,
                                             const int32_t* group_start, const int32_t* prefix_blocks) {
  msa::PrefixGroups g{};
  if (check_problem(prob) != MSA_OK || read_prefix_groups(prob, num_groups, group_start, prefix_blocks, g) != MSA_OK)
    return 0;
  return msa::prefix_workspace_layout(g, prob->tokens).bytes;
}

msa_status msa_decode_step(const msa_problem* prob, const void* idx_q, msa_dtype idx_q_dtype,
                           float idx_q_scale, const msa_cache* idx_k, const void* q, msa_dtype q_dtype,
                           float q_scale, const msa_cache* k, const msa_cache* v, msa_dequant dequant,
                           float softmax_scale, float* block_scores, int32_t* sel, float* out,
                           float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  msa_status st = check_problem(prob);
  if (st != MSA_OK) return st;
  if (prob->tokens > 8) return MSA_ERR_UNSUPPORTED;
  if ((st = check_cache(idx_k, 1)) != MSA_OK) return st;
  if ((st = check_pair(idx_q_dtype, idx_k->dtype)) != MSA_OK) return st;
  if ((st = check_cache(k, 4)) != MSA_OK) return st;
  if ((st = check_cache(v, 4)) != MSA_OK) return st;
  if (k->dtype != v->dtype) return MSA_ERR_UNSUPPORTED;
  if ((st = check_pair(q_dtype, k->dtype)) != MSA_OK) return st;
  if (dequant != MSA_DQ_EXACT && dequant != MSA_DQ_FP8) return MSA_ERR_INVALID_ARG;
  if (idx_q == nullptr || q == nullptr || block_scores == nullptr || sel == nullptr || out == nullptr)
    return MSA_ERR_INVALID_ARG;
  if (!aligned(idx_q, 16) || !aligned(q, 16) || !aligned(block_scores, 4) || !aligned(sel, 4) ||
      !aligned(out, 16) || (lse && !aligned(lse, 4)))
    return MSA_ERR_INVALID_ARG;
  if (!good_scale(idx_q_scale) || !good_scale(q_scale) || !good_scale(softmax_scale)) return MSA_ERR_INVALID_ARG;
  (void)workspace;
  (void)workspace_bytes;   // no workspace is needed (msa_workspace_size reports 0)
  const ProblemArgs pa = to_args(prob);
  const CacheArgs ia = to_args(idx_k), ka = to_args(k), va = to_args(v);
  const bool fp8 = dequant == MSA_DQ_FP8;
  // the scan, then one launch that selects each row's blocks and attends
  hipError_t e = msa::launch_indexer(pa, idx_q, (int)idx_q_dtype, idx_q_scale, ia, fp8, block_scores, nullptr, stream);
  if (e == hipSuccess)
    e = msa::launch_attention(pa, q, (int)q_dtype, q_scale, ka, va, fp8, sel, softmax_scale, out, lse, stream,
                              block_scores, sel);
  return hip_status(e);
}

msa_status msa_cache_insert(const msa_problem* prob, const float* x, const msa_cache* cache, hipStream_t stream) {
  msa_status st = check_problem(prob);
  if (st != MSA_OK) return st;
  if (cache == nullptr) return MSA_ERR_INVALID_ARG;
  if (cache->heads != 1 && cache->heads != 4) return MSA_ERR_INVALID_ARG;
  if ((st = check_cache(cache, cache->heads)) != MSA_OK) return st;
  if (x == nullptr || !aligned(x, 16)) return MSA_ERR_INVALID_ARG;
  return hip_status(msa::launch_insert(to_args(prob), x, to_args(cache), cache->heads, stream));
}

msa_status msa_cache_insert_many(const msa_problem* prob, int32_t n, const float* const* x, const msa_cache* caches,
                                 hipStream_t stream) {
  msa_status st = check_problem(prob);
  if (st != MSA_OK) return st;
  if (n < 1 || n > MSA_MAX_INSERTS || x == nullptr || caches == nullptr) return MSA_ERR_INVALID_ARG;
  msa::CacheArgs c[MSA_MAX_INSERTS];
  int heads[MSA_MAX_INSERTS];
  for (int k = 0; k < n; ++k) {
    if (caches[k].heads != 1 && caches[k].heads != 4) return MSA_ERR_INVALID_ARG;
    if ((st = check_cache(&caches[k], caches[k].heads)) != MSA_OK) return st;
    if (x[k] == nullptr || !aligned(x[k], 16)) return MSA_ERR_INVALID_ARG;
    c[k] = to_args(&caches[k]);
    heads[k] = caches[k].heads;
  }
  return hip_status(msa::launch_insert_many(to_args(prob), n, x, c, heads, stream));
}

size_t msa_workspace_size(const msa_problem* prob, msa_call which) {
  if (prob == nullptr || prob->batch <= 0) return 0;
  if (which == MSA_CALL_INDEXER_TOPK)
    return (size_t)prob->batch * sizeof(uint32_t);   // one arrival counter per sequence
  if (which == MSA_CALL_INDEXER_PREFIX)
    return (size_t)prob->batch * sizeof(int32_t);     // shared block count per sequence
  return 0;
}

msa_status msa_pack_fp8(const float* x, int64_t n, float scale, uint8_t* out, hipStream_t stream) {
  if (x == nullptr || out == nullptr || n < 0) return MSA_ERR_INVALID_ARG;
  if (!good_scale(scale) || !aligned(x, 4)) return MSA_ERR_INVALID_ARG;
  if (n == 0) return MSA_OK;
  return hip_status(msa::launch_pack_fp8(x, n, scale, out, stream));
}

msa_status msa_unpack_fp8(const uint8_t* x, int64_t n, float scale, float* out, hipStream_t stream) {
  if (x == nullptr || out == nullptr || n < 0) return MSA_ERR_INVALID_ARG;
  if (!good_scale(scale) || !aligned(out, 4)) return MSA_ERR_INVALID_ARG;
  if (n == 0) return MSA_OK;
  return hip_status(msa::launch_unpack_fp8(x, n, scale, out, stream));
}

msa_status msa_pack_nvfp4(const float* x, int64_t rows, int32_t row_len, float tensor_scale,
                          uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  if (x == nullptr || codes == nullptr || scales == nullptr || rows < 0 || row_len <= 0)
    return MSA_ERR_INVALID_ARG;
  if (row_len % 16 != 0 || !good_scale(tensor_scale)) return MSA_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(codes, 8)) return MSA_ERR_INVALID_ARG;
  if (rows == 0) return MSA_OK;
  return hip_status(msa::launch_pack_nvfp4(x, rows * (row_len / 16), tensor_scale, codes, scales, stream));
}

msa_status msa_unpack_nvfp4(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                            int32_t row_len, float tensor_scale, msa_dequant dequant, float* out,
                            hipStream_t stream) {
  if (codes == nullptr || scales == nullptr || out == nullptr || rows < 0 || row_len <= 0)
    return MSA_ERR_INVALID_ARG;
  if (row_len % 16 != 0 || !good_scale(tensor_scale)) return MSA_ERR_INVALID_ARG;
  if (dequant != MSA_DQ_EXACT && dequant != MSA_DQ_FP8) return MSA_ERR_INVALID_ARG;
  if (!aligned(codes, 8) || !aligned(out, 16)) return MSA_ERR_INVALID_ARG;
  if (rows == 0) return MSA_OK;
  return hip_status(msa::launch_unpack_nvfp4(codes, scales, rows * (row_len / 16), tensor_scale,
                                             dequant == MSA_DQ_FP8, out, stream));
}

const char* msa_status_string(msa_status s) {
  switch (s) {
    case MSA_OK: return "ok";
    case MSA_ERR_INVALID_ARG: return "invalid argument";
    case MSA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MSA_ERR_WORKSPACE: return "workspace missing or too small";
    case MSA_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int msa_abi_version(void) { return MSA_ABI_VERSION; }

}  // extern "C"
