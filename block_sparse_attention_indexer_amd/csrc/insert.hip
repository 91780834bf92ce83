// Quantise-and-insert: new tokens' K, V or index-key rows (fp32) written into
// their slots of a paged cache as FP8 or NVFP4.
//
// Source: "vLLM 為 MiniMax-M3.1-Flash 提供 Day-0 支援", section "QKV GEMM +
// norm + RoPE + KV insert fusion": K, V and the index key are quantised to
// NVFP4 and written straight into their caches.  This is that insert step on
// its own (the GEMM, norm and RoPE need model weights).  The quantiser is the
// one of msa_pack_fp8 / msa_pack_nvfp4 (every step in fp32, in a fixed
// order), so a cache filled by inserts equals one packed in one piece.
//
// A lane takes one 16-dim group of one (sequence, new token, head) row: a
// wave covers 8 rows, 64 contiguous bytes of input per lane.  The group's
// absolute maximum, its E4M3 scale and its codes stay in the lane (no
// exchanges); the divisions by the shared denominator are most of the work.
// Each lane looks up its own row's slot (sequence length, then table entry:
// the 8 lanes of a row read the same words).  Per row the stores are 64
// contiguous code bytes (NVFP4; 128 for FP8, 512 for fp32) and 8 scale bytes.
#include "common.hpp"
#include "launch.hpp"

namespace msa {

constexpr int kInsertWaves = 4;
constexpr int kInsertRowsPerWave = 64 / kNvfp4ScaleBytes;   // 8: a lane per 16-dim group
constexpr int kInsertRowsPerWG = kInsertWaves * kInsertRowsPerWave;

// Workgroup `wg` of one insert: rows wg*32 .. wg*32+31 of x.
template <int DT>   // 0 F32, 1 FP8, 2 NVFP4
__device__ __forceinline__ void insert_rows(
    const float* __restrict__ x, uint8_t* __restrict__ data, uint8_t* __restrict__ scales, int64_t num_pages,
    int hshift, float tensor_scale, const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ table,
    int max_blocks, int T, uint32_t rows, uint32_t wg) {
  // rows = B*T*heads < 2^31 and heads = 1 << hshift, so 32-bit index arithmetic suffices
  const int heads = 1 << hshift;
  const int g = threadIdx.x & 7;   // group: dims 16g .. 16g+15
  const uint32_t row = wg * kInsertRowsPerWG + (threadIdx.x >> 3);   // (b*T + t)*heads + h
  if (row >= rows) return;
  const float4* src = reinterpret_cast<const float4*>(x + (size_t)row * kHeadDim + 16 * g);
  float4 f[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) f[k] = src[k];
  const uint32_t bt = row >> hshift;
  const uint32_t b = bt / (uint32_t)T;
  const int pos = seq_lens[b] - T + (int)(bt - b * (uint32_t)T);
  if (pos < 0 || pos / kBlock >= max_blocks) return;
  const int pg = table[(size_t)b * max_blocks + pos / kBlock];
  if (pg < 0 || (int64_t)pg >= num_pages) return;   // not a page of this pool: nothing is written
  const size_t slot = ((size_t)pg * heads + (row & (uint32_t)(heads - 1))) * kBlock + (pos & (kBlock - 1));
  if constexpr (DT == 0) {
    float4* dst = reinterpret_cast<float4*>(data + slot * kHeadDim * 4 + 64 * g);
#pragma unroll
    for (int k = 0; k < 4; ++k) dst[k] = f[k];
  } else if constexpr (DT == 1) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = e4m3_encode2(f[k].x / tensor_scale, f[k].y / tensor_scale) |
             (e4m3_encode2(f[k].z / tensor_scale, f[k].w / tensor_scale) << 16);
    *reinterpret_cast<uint4*>(data + slot * kHeadDim + 16 * g) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      amax = fmaxf(fmaxf(amax, fmaxf(__builtin_fabsf(f[k].x), __builtin_fabsf(f[k].y))),
                   fmaxf(__builtin_fabsf(f[k].z), __builtin_fabsf(f[k].w)));
    const uint32_t sb = e4m3_encode2(amax / (6.0f * tensor_scale), 0.0f) & 0xFFu;
    const float denom = e4m3_value(sb) * tensor_scale;
    uint32_t w[2] = {0u, 0u};
    if (denom > 0.0f) {
#pragma unroll
      for (int k = 0; k < 4; ++k)   // elements 4k .. 4k+3: bytes 2k, 2k+1 of the group's 8
        w[k >> 1] |= (e2m1_encode2(f[k].x / denom, f[k].y / denom) |
                      (e2m1_encode2(f[k].z / denom, f[k].w / denom) << 8)) << (16 * (k & 1));
    }
    *reinterpret_cast<uint2*>(data + slot * kNvfp4RowBytes + 8 * g) = make_uint2(w[0], w[1]);
    scales[slot * kNvfp4ScaleBytes + g] = (uint8_t)sb;
  }
}

template <int DT>
__global__ __launch_bounds__(64 * kInsertWaves) void insert_rows_kernel(
    const float* __restrict__ x, uint8_t* __restrict__ data, uint8_t* __restrict__ scales, int64_t num_pages,
    int hshift, float tensor_scale, const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ table,
    int max_blocks, int T, uint32_t rows) {
  insert_rows<DT>(x, data, scales, num_pages, hshift, tensor_scale, seq_lens, table, max_blocks, T, rows,
                  blockIdx.x);
}

// Several inserts in one launch: workgroups [wg_begin[k], wg_begin[k+1]) do insert k.
__global__ __launch_bounds__(64 * kInsertWaves) void insert_many_kernel(InsertSet set,
                                                                        const int32_t* __restrict__ seq_lens,
                                                                        const int32_t* __restrict__ table,
                                                                        int max_blocks, int T) {
  int k = 0;
  while (k + 1 < set.n && blockIdx.x >= set.wg_begin[k + 1]) ++k;
  const InsertSet::One& e = set.one[k];
  const uint32_t wg = blockIdx.x - set.wg_begin[k];
  if (e.dtype == 0)
    insert_rows<0>(e.x, e.data, e.scales, e.num_pages, e.hshift, e.tensor_scale, seq_lens, table, max_blocks, T,
                   e.rows, wg);
  else if (e.dtype == 1)
    insert_rows<1>(e.x, e.data, e.scales, e.num_pages, e.hshift, e.tensor_scale, seq_lens, table, max_blocks, T,
                   e.rows, wg);
  else
    insert_rows<2>(e.x, e.data, e.scales, e.num_pages, e.hshift, e.tensor_scale, seq_lens, table, max_blocks, T,
                   e.rows, wg);
}

hipError_t launch_insert(const ProblemArgs& p, const float* x, const CacheArgs& c, int heads, hipStream_t s) {
  const uint32_t rows = (uint32_t)((int64_t)p.B * p.T * heads);   // < 2^31: B*T*4 is bounded by the caller
  const int hshift = heads == 4 ? 2 : 0;
  const dim3 grid((rows + kInsertRowsPerWG - 1) / kInsertRowsPerWG), block(64 * kInsertWaves);
  uint8_t* data = const_cast<uint8_t*>(c.data);
  uint8_t* sc = const_cast<uint8_t*>(c.scales);
#define MSA_INSERT_LAUNCH(DT)                                                                               \
  hipLaunchKernelGGL(insert_rows_kernel<DT>, grid, block, 0, s, x, data, sc, c.num_pages, hshift, c.tensor_scale, \
                     p.seq_lens, p.block_table, p.max_blocks, p.T, rows)
  if (c.dtype == 0) MSA_INSERT_LAUNCH(0);
  else if (c.dtype == 1) MSA_INSERT_LAUNCH(1);
  else MSA_INSERT_LAUNCH(2);
#undef MSA_INSERT_LAUNCH
  return hipGetLastError();
}

hipError_t launch_insert_many(const ProblemArgs& p, int n, const float* const* x, const CacheArgs* c,
                              const int* heads, hipStream_t s) {
  InsertSet set{};
  set.n = n;
  uint32_t wgs = 0;
  for (int k = 0; k < n; ++k) {
    const uint32_t rows = (uint32_t)((int64_t)p.B * p.T * heads[k]);
    set.one[k] = InsertSet::One{x[k], const_cast<uint8_t*>(c[k].data), const_cast<uint8_t*>(c[k].scales),
                                c[k].num_pages, heads[k] == 4 ? 2 : 0, c[k].tensor_scale, c[k].dtype, rows};
    set.wg_begin[k] = wgs;
    wgs += (rows + kInsertRowsPerWG - 1) / kInsertRowsPerWG;
  }
  set.wg_begin[n] = wgs;
  hipLaunchKernelGGL(insert_many_kernel, dim3(wgs), dim3(64 * kInsertWaves), 0, s, set, p.seq_lens, p.block_table,
                     p.max_blocks, p.T);
  return hipGetLastError();
}

}  // namespace msa
