// Host-side launchers of the MSA kernels (internal to libmsa; the public
// surface is include/msa.h).  Each returns hipGetLastError() after enqueueing.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msa {

// Arguments common to the paged-cache kernels, already validated on the host.
struct CacheArgs {
  const uint8_t* data;     // F32 floats / FP8 bytes / NVFP4 codes
  const uint8_t* scales;   // NVFP4 scale bytes or nullptr
  int64_t num_pages;
  float tensor_scale;
  int dtype;               // 0 F32, 1 FP8, 2 NVFP4 (msa_dtype)
};

struct ProblemArgs {
  int B, T, max_blocks;
  const int32_t* seq_lens;
  const int32_t* block_table;
};

// Shared-prefix groups of one call: sequences [start[k], start[k+1]) share
// their first blocks[k] logical blocks (the same page ids).  Passed by value.
constexpr int kMaxPrefixGroups = 64;
struct PrefixGroups {
  int n;
  int start[kMaxPrefixGroups + 1];
  int blocks[kMaxPrefixGroups];
};

// Compute units of the current device, queried once per device (256 on MI355X;
// 256 is also the answer if the query fails).
inline int current_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) return 256;
    cached[dev] = c;
  }
  return cached[dev];
}

hipError_t launch_pack_fp8(const float* x, int64_t n, float scale, uint8_t* out, hipStream_t s);
hipError_t launch_unpack_fp8(const uint8_t* x, int64_t n, float scale, float* out, hipStream_t s);
hipError_t launch_pack_nvfp4(const float* x, int64_t groups, float tensor_scale, uint8_t* codes,
                             uint8_t* scales, hipStream_t s);
hipError_t launch_unpack_nvfp4(const uint8_t* codes, const uint8_t* scales, int64_t groups,
                               float tensor_scale, bool fp8mode, float* out, hipStream_t s);

// With sel and counters non-null (only where indexer_can_fuse_topk), the scan also
// writes the top-16 selection; counters: one zeroed uint32 per sequence, left zeroed.
// num_shards > 1: only the logical blocks i with i % num_shards == shard are scored
// (FP8 / NVFP4 keys, T <= 8, no fused selection).  skip (device [B], nullable): the
// first skip[b] blocks of sequence b are left to another kernel (same restrictions).
hipError_t launch_indexer(const ProblemArgs& p, const void* idx_q, int q_dtype, float q_scale,
                          const CacheArgs& k, bool fp8mode, float* block_scores,
                          float* token_scores, hipStream_t s, int32_t* sel = nullptr,
                          uint32_t* counters = nullptr, int shard = 0, int num_shards = 1,
                          const int32_t* skip = nullptr);

// Context-parallel selection: the local top-16 of one shard's blocks per row
// (cand_* [rows][16], best first, padded with NaN / -1), and the owner's merge of
// num_shards such lists (cand_* [num_shards][rows][16]) into sel.
hipError_t launch_shard_topk(const ProblemArgs& p, int shard, int num_shards, const float* block_scores,
                             float* cand_scores, int32_t* cand_blocks, hipStream_t s);
hipError_t launch_topk_merge(const ProblemArgs& p, int num_shards, const float* cand_scores,
                             const int32_t* cand_blocks, int32_t* sel, hipStream_t s);
bool indexer_can_fuse_topk(const ProblemArgs& p, const CacheArgs& k, bool fp8mode);

hipError_t launch_indexer_prefill(const ProblemArgs& p, const void* idx_q, const CacheArgs& k,
                                  bool fp8mode, float sigma, float* block_scores, float* token_scores,
                                  hipStream_t s);

// Shared-prefix decode: the shared blocks of every prefix group scored once for all
// of the group's query rows (T <= 8); skip: device [B] int32 filled with the shared
// block count of each sequence (0 outside the groups), for the per-sequence scans.
hipError_t launch_indexer_shared(const ProblemArgs& p, const void* idx_q, const CacheArgs& k, bool fp8mode,
                                 float sigma, const PrefixGroups& g, float* block_scores, hipStream_t s);
hipError_t launch_fill_skip(const PrefixGroups& g, int B, int32_t* skip, hipStream_t s);
// The decode scan of every block that no prefix group shares (the rest of the
// shared-prefix call): the evenly spread one-token scan reads the groups itself;
// the other scans take per-sequence skip counts, written into skip_ws (device
// [B] int32) first.
hipError_t launch_indexer_skipping(const ProblemArgs& p, const void* idx_q, int q_dtype, float q_scale,
                                   const CacheArgs& k, bool fp8mode, float* block_scores, const PrefixGroups& g,
                                   int32_t* skip_ws, hipStream_t s);

hipError_t launch_topk(const ProblemArgs& p, const float* block_scores, int32_t* sel,
                       hipStream_t s);

// The allocation-free entry point's scratch: arrival counters for at most
// kStaticMaxBatch sequences in a file-scope device array.  static_scratch gives
// its address on the current device (looked up once per device); launch_zero_u32
// clears n counters with a kernel.
constexpr int kStaticMaxBatch = 4096;
hipError_t static_scratch(uint32_t** out);
hipError_t launch_zero_u32(uint32_t* p, int n, hipStream_t s);

// With block_scores non-null the selection is made inside the attention launch
// (each workgroup selects its own row; written to sel_out) and sel is not read.
// With pa non-null (FP8 / NVFP4 caches, no block_scores) staged shared-prefix
// blocks are read from their images (launch_attention_prefix).
struct PrefixAttnArgs;
hipError_t launch_attention(const ProblemArgs& p, const void* q, int q_dtype, float q_scale,
                            const CacheArgs& k, const CacheArgs& v, bool fp8mode,
                            const int32_t* sel, float softmax_scale, float* out, float* lse,
                            hipStream_t s, const float* block_scores = nullptr, int32_t* sel_out = nullptr,
                            const PrefixAttnArgs* pa = nullptr);

// Shared-prefix decode attention: byte offsets of its workspace parts for a call
// with prefix groups gr and T query tokens (staged slot images, slot map, slot
// block ids, slot counts), and the attention through the staged blocks.
struct PrefixWorkspace {
  int slots;
  size_t staged, slot_of, slot_blk, count, bytes;
};
PrefixWorkspace prefix_workspace_layout(const PrefixGroups& gr, int T);
hipError_t launch_attention_prefix(const ProblemArgs& p, const void* q, float q_scale, const CacheArgs& k,
                                   const CacheArgs& v, bool fp8mode, const int32_t* sel, float softmax_scale,
                                   float* out, float* lse, const PrefixGroups& gr, void* workspace, hipStream_t s);

// Quantise the fp32 rows x [B, T, heads, 128] of the T new tokens and write them
// into their slots of cache c (heads = c's heads per page).
hipError_t launch_insert(const ProblemArgs& p, const float* x, const CacheArgs& c, int heads, hipStream_t s);
// Up to kMaxInserts inserts of the same new tokens (K, V, index keys) in one launch.
constexpr int kMaxInserts = 4;
struct InsertSet {
  struct One {
    const float* x;
    uint8_t* data;
    uint8_t* scales;
    int64_t num_pages;
    int hshift;
    float tensor_scale;
    int dtype;
    uint32_t rows;
  };
  int n;
  One one[kMaxInserts];
  uint32_t wg_begin[kMaxInserts + 1];
};
hipError_t launch_insert_many(const ProblemArgs& p, int n, const float* const* x, const CacheArgs* c,
                              const int* heads, hipStream_t s);

}  // namespace msa
