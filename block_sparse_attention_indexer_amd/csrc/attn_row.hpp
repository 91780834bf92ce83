// Step 4 of MSA: exact attention over the selected blocks -- the device
// code of one row, used by the attention kernels (with or without the row's
// own top-16 selection in front).
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
#pragma once
#include "common.hpp"
#include "select.hpp"

namespace msa {

constexpr int kAttnManyRows = 1024;   // rows from which the 4-wave form is used

// One 16-key V tile in LDS: f16 [16 keys][128 dims], 256 B per key.  The
// 16-byte chunk c of key k sits at chunk c ^ vt_swizzle(k): with it the
// 16-byte writes (8 keys per phase) and the transposing 8-byte reads (4 keys
// x 4 chunks per phase) each touch every bank once.
constexpr int kVtBytes = 16 * kHeadDim * 2;
constexpr int kVtSlotBytes = 2 * kVtBytes;   // per wave: the two tiles of one PV product
__device__ __forceinline__ int vt_swizzle(int k) { return (2 * k + (k >> 2) + 4 * (k >> 3)) & 15; }
__device__ __forceinline__ int vt_offset(int k, int chunk) { return k * 256 + 16 * (chunk ^ vt_swizzle(k)); }

// gfx950 transposing LDS read: in each group of 16 lanes, lane i receives for
// e = 0..3 the 16-bit element (i mod 4) of the 8-byte chunk addressed by lane
// 4e + i/4 of its group (fixed by an in-bounds probe).  With lane l pointing
// at key l/4, dims 4(l mod 4) .. +3 of a 16-dim tile, lane l gets dim l mod 16
// of keys 4(l/16) .. +3.
__device__ __forceinline__ h4 lds_read_tr16(const uint8_t* p) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)p);
  return __builtin_bit_cast(h4, v);
}
__device__ __forceinline__ h8 reorder_like_lut_a(h8 a) {
  return h8{a[0], a[2], a[4], a[6], a[1], a[3], a[5], a[7]};
}

// One 16-key tile of K or V as loaded from a page, before decoding.
//   K tile, lane (quarter Q, key j): dims [32Q, 32Q+32) of key j.
//   V tile, lane (key pair kp, 16-dim group dg): dims [16dg, 16dg+16) of keys 2kp, 2kp+1.
template <int KT> struct KRaw;
template <> struct KRaw<1> { uint4 c0, c1; };
template <> struct KRaw<2> { uint4 c; uint32_t s; };
template <int KT> struct VRaw;
template <> struct VRaw<1> { uint4 c[2]; };
template <> struct VRaw<2> { uint2 c[2]; uint32_t s[2]; };

// Loads go through buffer resources built once per block for its (page, KV
// head) slice -- a scalar base and the slice's byte size, uniform across the
// wave -- with offsets fixed per lane (computed once per row) and the tile's
// offset as a scalar, so a load costs no vector address arithmetic.  Reads past
// the slice's size return zero instead of touching memory.
struct KvRsrc {
  __amdgpu_buffer_rsrc_t codes, scales;
};
template <int KT>
__device__ __forceinline__ KvRsrc kv_rsrc(const uint8_t* codes, const uint8_t* scales, size_t rowbase) {
  constexpr int kRowBytes = KT == 2 ? kNvfp4RowBytes : kHeadDim;
  KvRsrc r;
  r.codes = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(codes + rowbase * kRowBytes), (short)0,
                                              kBlock * kRowBytes, kBufferFlags);
  r.scales = KT == 2 ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(scales + rowbase * kNvfp4ScaleBytes),
                                                         (short)0, kBlock * kNvfp4ScaleBytes, kBufferFlags)
                     : r.codes;
  return r;
}
// Per-lane byte offsets within a block's slice.
//   K tile kt, lane (quarter Q, key j): row kt*16 + j, dims [32Q, 32Q+32).
//   V tile kt, lane (key pair kp, 16-dim group dg): rows kt*16 + 2kp + u, dims [16dg, 16dg+16).
struct KvLaneOffsets {
  uint32_t k, ks, v[2], vs[2];
};
template <int KT>
__device__ __forceinline__ KvLaneOffsets kv_lane_offsets(int j, int Q, int kp, int dg) {
  constexpr int kRowBytes = KT == 2 ? kNvfp4RowBytes : kHeadDim;
  KvLaneOffsets o;
  o.k = j * kRowBytes + (KT == 2 ? 16 : 32) * Q;
  o.ks = j * kNvfp4ScaleBytes + 2 * Q;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    o.v[u] = (2 * kp + u) * kRowBytes + (KT == 2 ? 8 : 16) * dg;
    o.vs[u] = (2 * kp + u) * kNvfp4ScaleBytes + dg;
  }
  return o;
}

template <int KT>
__device__ __forceinline__ KRaw<KT> load_k_tile(const KvRsrc& rs, const KvLaneOffsets& o, int kt) {
  constexpr int kRowBytes = KT == 2 ? kNvfp4RowBytes : kHeadDim;
  KRaw<KT> t;
  if constexpr (KT == 2) {
    t.c = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs.codes, o.k, kt * 16 * kRowBytes, 0));
    t.s = __builtin_amdgcn_raw_buffer_load_b16(rs.scales, o.ks, kt * 16 * kNvfp4ScaleBytes, 0);
  } else {
    t.c0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs.codes, o.k, kt * 16 * kRowBytes, 0));
    t.c1 = __builtin_bit_cast(uint4,
                              __builtin_amdgcn_raw_buffer_load_b128(rs.codes, o.k + 16, kt * 16 * kRowBytes, 0));
  }
  return t;
}

template <int KT>
__device__ __forceinline__ VRaw<KT> load_v_tile(const KvRsrc& rs, const KvLaneOffsets& o, int kt) {
  constexpr int kRowBytes = KT == 2 ? kNvfp4RowBytes : kHeadDim;
  VRaw<KT> t;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if constexpr (KT == 2) {
      t.c[u] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs.codes, o.v[u],
                                                                              kt * 16 * kRowBytes, 0));
      t.s[u] = __builtin_amdgcn_raw_buffer_load_b8(rs.scales, o.vs[u], kt * 16 * kNvfp4ScaleBytes, 0);
    } else {
      t.c[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs.codes, o.v[u],
                                                                               kt * 16 * kRowBytes, 0));
    }
  }
  return t;
}

// K tile -> the four 16x32 A fragments of S^T = K Q^T (k-chunk c = dims 32Q+8c .. +7).
template <int KT, bool FP8MODE>
__device__ __forceinline__ void decode_k_tile(const KRaw<KT>& r, const uint32_t* lut, h8 (&Ak)[4]) {
  if constexpr (KT == 2) {
    const uint32_t wv[4] = {r.c.x, r.c.y, r.c.z, r.c.w};
    if constexpr (FP8MODE) {
      const uint32_t s0 = r.s & 0xFFu, s1 = (r.s >> 8) & 0xFFu;
      Ak[0] = fp4x8_lut_to_h8(wv[0], lut[2 * s0], lut[2 * s0 + 1]);
      Ak[1] = fp4x8_lut_to_h8(wv[1], lut[2 * s0], lut[2 * s0 + 1]);
      Ak[2] = fp4x8_lut_to_h8(wv[2], lut[2 * s1], lut[2 * s1 + 1]);
      Ak[3] = fp4x8_lut_to_h8(wv[3], lut[2 * s1], lut[2 * s1 + 1]);
    } else {
      const h2 sc = fp8x2_to_h2<false>(r.s);
      const h8 s0 = h8{sc[0], sc[0], sc[0], sc[0], sc[0], sc[0], sc[0], sc[0]};
      const h8 s1 = h8{sc[1], sc[1], sc[1], sc[1], sc[1], sc[1], sc[1], sc[1]};
      Ak[0] = fp4x8_to_h8(wv[0]) * s0;
      Ak[1] = fp4x8_to_h8(wv[1]) * s0;
      Ak[2] = fp4x8_to_h8(wv[2]) * s1;
      Ak[3] = fp4x8_to_h8(wv[3]) * s1;
    }
  } else {
    Ak[0] = fp8x8_to_h8(r.c0.x, r.c0.y);
    Ak[1] = fp8x8_to_h8(r.c0.z, r.c0.w);
    Ak[2] = fp8x8_to_h8(r.c1.x, r.c1.y);
    Ak[3] = fp8x8_to_h8(r.c1.z, r.c1.w);
  }
}

// V tile -> this lane's 2 keys x 16 dims as f16, written in [key][dim]
// layout into the wave's LDS slice (woff[u][hh]: byte offsets of key 2kp+u,
// dims 16dg+8hh .. +7).  Keys that are not kept are zeroed before decoding:
// an NVFP4 key through its scale bytes (E2M1 codes are always finite), an
// FP8 key through its bytes, so unwritten rows of a partly filled page never
// reach the product (0 * NaN would).
template <int KT, bool FP8MODE, bool MASK>
__device__ __forceinline__ void stage_v_tile(VRaw<KT> r, const uint32_t* lut, uint8_t* vt,
                                             const int (&woff)[2][2], bool keep0, bool keep1) {
  if constexpr (!MASK) {
  } else if constexpr (KT == 2) {
    r.s[0] = keep0 ? r.s[0] : 0u;
    r.s[1] = keep1 ? r.s[1] : 0u;
  } else {
    // masked per dword: a select of whole uint4 values went through scratch memory
    const uint32_t m0 = keep0 ? 0xFFFFFFFFu : 0u, m1 = keep1 ? 0xFFFFFFFFu : 0u;
    r.c[0].x &= m0; r.c[0].y &= m0; r.c[0].z &= m0; r.c[0].w &= m0;
    r.c[1].x &= m1; r.c[1].y &= m1; r.c[1].z &= m1; r.c[1].w &= m1;
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    h8 v[2];
    if constexpr (KT == 2) {
      const uint32_t sb = r.s[u];
      if constexpr (FP8MODE) {
        v[0] = fp4x8_lut_to_h8(r.c[u].x, lut[2 * sb], lut[2 * sb + 1]);
        v[1] = fp4x8_lut_to_h8(r.c[u].y, lut[2 * sb], lut[2 * sb + 1]);
      } else {
        const _Float16 sh = e4m3_to_h(sb);
        const h8 ss = h8{sh, sh, sh, sh, sh, sh, sh, sh};
        v[0] = fp4x8_to_h8(r.c[u].x) * ss;
        v[1] = fp4x8_to_h8(r.c[u].y) * ss;
      }
    } else {
      v[0] = fp8x8_to_h8(r.c[u].x, r.c[u].y);
      v[1] = fp8x8_to_h8(r.c[u].z, r.c[u].w);
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) *reinterpret_cast<h8*>(vt + woff[u][hh]) = v[hh];
  }
}

// V tiles in flight ahead of the one being multiplied.
template <int KT> constexpr int kVAhead = KT == 2 ? 4 : 2;
constexpr int kKRing = 8;   // K tiles of a block in flight (divides 8)
constexpr int kMergeStride = kHeadDim + 4;   // fp32 row of one head in the merge buffer (padded)
constexpr float kRescaleSlack = 8.0f;        // log2 headroom of the softmax weights before O is rescaled

// Shared-prefix staging (msa_sparse_attn_decode_prefix).  A staged block is
// one (page, KV head) slice dequantised once into the operand images the
// attention's MFMAs take, 64 KiB per slot:
//   K image: [tile kt 0..7][k-chunk c 0..3][lane 0..63] h8 -- lane's Ak[c] of tile kt;
//   V image: [tile pair 0..3][dim tile dt 0..7][lane 0..63] h8 -- lane's V^T operand.
// Lane mappings are those of attend_row, so a staged block gives the same
// operands, and the same results, as decoding the page in the attention.
constexpr int kStageKBytes = 8 * 4 * 64 * 16;
constexpr int kStageBytes = 2 * kStageKBytes;
constexpr int kMaxPrefixGroupsDev = 64;
struct PrefixAttnArgs {
  const uint8_t* staged;      // slot images
  const int32_t* slot_of;     // per group k: [4 heads][blocks[k]] slot ids, -1 = not staged
  int n;                      // prefix groups
  int start[kMaxPrefixGroupsDev + 1];   // sequences [start[k], start[k+1]) form group k
  int blocks[kMaxPrefixGroupsDev];      // shared leading blocks of group k
  int slot_of_base[kMaxPrefixGroupsDev];   // offset of group k's slot_of entries
};

// KT: 1 = FP8 K/V, 2 = NVFP4 K/V (queries FP8).  WAVES waves per workgroup;
// wave w takes selected blocks w, w + WAVES, ... and keeps a running (max,
// sum, O) over them (online softmax); the WAVES states merge at the end.
// Everything the attention of one row needs.
struct AttnArgs {
  const uint8_t* q;
  float c_log2;
  const uint8_t* kdata;
  const uint8_t* kscales;
  int64_t kpages;
  const uint8_t* vdata;
  const uint8_t* vscales;
  int64_t vpages;
  float v_scale;
  const int32_t* sel;
  const int32_t* seq_lens;
  const int32_t* table;
  int max_blocks;
  int T;
  float* out;
  float* lse;
  // SELECT: the row's block scores are read from here and its selection is
  // written to sel_out (sel is not read)
  const float* block_scores = nullptr;
  int32_t* sel_out = nullptr;
};

// Attention of one row (b*T + t)*4 + g by a workgroup of WAVES waves (all
// of which call it): KT 1 = FP8 K/V, 2 = NVFP4 K/V (queries FP8).  Wave w
// takes selected blocks w, w + WAVES, ... and keeps a running (max, sum, O)
// over them (online softmax); the WAVES states merge at the end.
// SELECT: the workgroup first selects the row's blocks itself from
// args.block_scores (select_row, the same rule and keys as msa_block_topk)
// and writes them to args.sel_out.
// PREFIX (with pa): blocks older than the row's own block that lie in its
// sequence's shared prefix and were staged are read from their images instead
// of being decoded from the pages.
template <int KT, bool FP8MODE, int WAVES, bool SELECT = false, bool PREFIX = false>
__device__ __forceinline__ void attend_row(const AttnArgs& args, int row, const PrefixAttnArgs* pa = nullptr) {
  const uint8_t* __restrict__ q = args.q;
  const float c_log2 = args.c_log2;
  const uint8_t* __restrict__ kdata = args.kdata;
  const uint8_t* __restrict__ kscales = args.kscales;
  const int64_t kpages = args.kpages;
  const uint8_t* __restrict__ vdata = args.vdata;
  const uint8_t* __restrict__ vscales = args.vscales;
  const int64_t vpages = args.vpages;
  const float v_scale = args.v_scale;
  const int32_t* __restrict__ sel = args.sel;
  const int32_t* __restrict__ seq_lens = args.seq_lens;
  const int32_t* __restrict__ table = args.table;
  const int max_blocks = args.max_blocks;
  const int T = args.T;
  float* __restrict__ out = args.out;
  float* __restrict__ lse = args.lse;
  static_assert(kTopK % WAVES == 0, "blocks split evenly over the waves");
  constexpr int kSmemDwords = WAVES * 16 * kMergeStride > WAVES * kVtSlotBytes / 4 ? WAVES * 16 * kMergeStride
                                                                                    : WAVES * kVtSlotBytes / 4;
  __shared__ uint32_t lut[FP8MODE ? 512 : 2];
  // V tile staging (WAVES x kVtSlotBytes), later reused as the merge buffer
  // [WAVES][16 heads][kMergeStride] fp32.
  __shared__ __attribute__((aligned(16))) uint32_t smem[kSmemDwords];
  __shared__ float m_sh[WAVES][16], l_sh[WAVES][16];
  __shared__ int nan_sh;

  const int g = row & 3;
  const int bt = row >> 2;
  const int t = bt % T, b = bt / T;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int Q = lane >> 4, j = lane & 15;
  const float NEG_INF = -__builtin_inff();

  // independent loads first: length, the query, this wave's blocks
  const int L = seq_lens[b];
  const uint4* qsrc =
      reinterpret_cast<const uint4*>(q + (((size_t)b * T + t) * kHeads + g * kHeadsPerGroup + j) * kHeadDim + 32 * Q);
  const uint4 qu0 = qsrc[0], qu1 = qsrc[1];
  int blks[kTopK / WAVES];
  // SELECT with 16 waves: the sequence's block-table row (up to 2,048 blocks)
  // is copied into LDS while the selection runs, so a wave's page id is an LDS
  // read instead of a memory round trip after the selection
  constexpr int kTblPerThread = (SELECT && WAVES == 16) ? 2 : 0;
  __shared__ int32_t tbl_sh[kTblPerThread > 0 ? kTblPerThread * WAVES * 64 : 1];
  const bool tbl_lds = kTblPerThread > 0 && max_blocks <= kTblPerThread * WAVES * 64;
  if constexpr (SELECT) {
    __shared__ int32_t sel_sh[kTopK];
    const int own = max(0, min((L - T + t) / kBlock, max_blocks - 1));
    // keys per thread sized to the row (uniform): a row of at most WAVES*64 older
    // blocks needs one slot per thread, not the 8,192-block maximum
    constexpr int NT = WAVES * 64, EMAX = kMaxBlocksSelect / NT;
    const float* srow = args.block_scores + (size_t)row * max_blocks;
    const int ne = (own + NT - 1) / NT;
    TablePrefetch tp;
    if (tbl_lds) tp = TablePrefetch{table + (size_t)b * max_blocks, max_blocks, tbl_sh};
    if (ne <= 1) select_row<NT, 1, kTblPerThread>(srow, own, sel_sh, tp);
    else if (ne <= 2 && EMAX >= 2) select_row<NT, (EMAX >= 2 ? 2 : EMAX), kTblPerThread>(srow, own, sel_sh, tp);
    else select_row<NT, EMAX, kTblPerThread>(srow, own, sel_sh, tp);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kTopK / WAVES; ++u) blks[u] = sel_sh[w + u * WAVES];
    if (threadIdx.x < kTopK) args.sel_out[(size_t)row * kTopK + threadIdx.x] = sel_sh[threadIdx.x];
  } else {
#pragma unroll
    for (int u = 0; u < kTopK / WAVES; ++u) blks[u] = sel[(size_t)row * kTopK + w + u * WAVES];
  }
  if (threadIdx.x == 0) nan_sh = 0;
  if (FP8MODE) build_fp8_lut(lut);
  __syncthreads();

  // B operand of S^T = K Q^T: lane (Q, head j), k-chunk c = dims 32Q+8c..+7.
  h8 Bq[4];
  {
    const uint32_t wq[8] = {qu0.x, qu0.y, qu0.z, qu0.w, qu1.x, qu1.y, qu1.z, qu1.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const h8 a = fp8x8_to_h8(wq[2 * c], wq[2 * c + 1]);
      Bq[c] = (KT == 2 && FP8MODE) ? reorder_like_lut_a(a) : a;
    }
  }

  const int p = L - T + t;
  const int kp = lane & 7;     // key pair within a V tile (keys 2kp, 2kp+1)
  const int dg = lane >> 3;    // 16-dim group of a V tile
  uint8_t* vt = reinterpret_cast<uint8_t*>(smem) + w * kVtSlotBytes;
  // LDS byte offsets, fixed per lane: where this lane writes its V values
  // (keys 2kp+u, dims 16dg+8hh..) and where its transposing reads point
  // (key lane/4, dims 16dt + 4(lane mod 4)..; the chunk index 2dt + x XORs as
  // a bit field, so dt enters as "^ 32dt")
  int woff[2][2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) woff[u][hh] = vt_offset(2 * kp + u, 2 * dg + hh);
  const int roff = vt_offset(lane >> 2, (lane & 3) >> 1) + 8 * (lane & 1);
  const KvLaneOffsets lo = kv_lane_offsets<KT>(j, Q, kp, dg);
  float m = NEG_INF, l = 0.0f;
  f4 O[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) O[dt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  // shared prefix of this row's sequence (PREFIX): blocks below pfx_blocks are
  // candidates for their staged images
  int pfx_blocks = 0, pfx_base = 0;
  if constexpr (PREFIX) {
    for (int k = 0; k < pa->n; ++k)
      if (b >= pa->start[k] && b < pa->start[k + 1]) {
        pfx_blocks = pa->blocks[k];
        pfx_base = pa->slot_of_base[k] + g * pa->blocks[k];
      }
  }
  const int own_blk = p / kBlock;

#pragma unroll 1
  for (int u = 0; u < kTopK / WAVES; ++u) {
    const int blk = __builtin_amdgcn_readfirstlane(blks[u]);   // one value per wave
    int nkeys = 0;
    size_t rowbase = 0;
    if (blk >= 0) {
      if (blk >= max_blocks) {
        nan_sh = 1;
      } else {
        const int pg = __builtin_amdgcn_readfirstlane(tbl_lds ? tbl_sh[blk] : table[(size_t)b * max_blocks + blk]);
        if (pg < 0 || (int64_t)pg >= kpages || (int64_t)pg >= vpages) {
          nan_sh = 1;
        } else {
          nkeys = min(kBlock, p + 1 - blk * kBlock);
          rowbase = ((size_t)pg * kGroups + g) * kBlock;   // (page, KV head g)
        }
      }
    }
    if (nkeys <= 0) continue;   // uniform per wave

    // PREFIX: a block of the shared prefix older than the row's own block may
    // have been staged; its operands are then read from the slot's images
    bool staged = false;
    const uint8_t* img_base = nullptr;
    if constexpr (PREFIX) {
      if (blk < pfx_blocks && blk < own_blk) {
        const int slot = __builtin_amdgcn_readfirstlane(pa->slot_of[pfx_base + blk]);
        if (slot >= 0) {
          staged = true;
          img_base = pa->staged + (size_t)slot * kStageBytes;
        }
      }
    }
    const bool full = nkeys == kBlock;   // uniform: no key of the block is past p
    float x[8][4];
    const KvRsrc vr = kv_rsrc<KT>(vdata, vscales, rowbase);
    VRaw<KT> vraw[8];
    if (PREFIX && staged) {
      const __amdgpu_buffer_rsrc_t img =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(img_base), (short)0, kStageBytes, kBufferFlags);
      // ---------------- S^T = K Q^T from the K image (a full block: no mask)
#pragma unroll
      for (int kt = 0; kt < 8; ++kt) {
        // one tile's loads at a time (hoisting all 32 would cost 128 registers)
        __builtin_amdgcn_sched_barrier(0);
        h8 Ak[4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
          Ak[c] = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(img, lane * 16, (kt * 4 + c) * 1024, 0));
        f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < 4; ++c) acc = mfma_16x16x32(Ak[c], Bq[c], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) x[kt][r] = acc[r];
      }
    } else {
    // Every K load and the first V tiles are issued before the first product.
    // All 128 rows of the page are read (they exist even when the block is
    // only partly visible), which keeps control flow uniform so that each
    // wait covers exactly the tile it needs.
    const KvRsrc kr = kv_rsrc<KT>(kdata, kscales, rowbase);
    // K tiles in a ring of kKRing slots: tile kt + kKRing is loaded into the
    // slot tile kt leaves once decoded
    KRaw<KT> kraw[kKRing];
#pragma unroll
    for (int kt = 0; kt < kKRing; ++kt) kraw[kt] = load_k_tile<KT>(kr, lo, kt);
#pragma unroll
    for (int kt = 0; kt < kVAhead<KT>; ++kt) vraw[kt] = load_v_tile<KT>(vr, lo, kt);

    // ---------------- S^T = K Q^T, 8 tiles of 16 keys (raw dot products; the
    // softmax scale c_log2 > 0 enters in the exponent's FMA below)
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      h8 Ak[4];
      decode_k_tile<KT, FP8MODE>(kraw[kt % kKRing], lut, Ak);
      if (kt + kKRing < 8) kraw[kt % kKRing] = load_k_tile<KT>(kr, lo, kt + kKRing);
      f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < 4; ++c) acc = mfma_16x16x32(Ak[c], Bq[c], acc);
      // lane (Q, head j) holds keys kt*16 + 4Q + r
#pragma unroll
      for (int r = 0; r < 4; ++r) x[kt][r] = acc[r];
      if (!full) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (kt * 16 + 4 * Q + r >= nkeys) x[kt][r] = NEG_INF;
      }
    }
    }
    // ---------------- online softmax over this wave's blocks
    float mx = NEG_INF;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, x[kt][r]);
    // rounding is monotone and c_log2 > 0, so this is the max of the scaled logits
    mx = max_over_quarters(mx) * c_log2;
    // NVFP4: the running maximum m moves only when a block's maximum exceeds it
    // by more than kRescaleSlack (log2 units): the weights exp2(s*c - m) then
    // stay below 2^kRescaleSlack, well inside f16, and most blocks skip
    // rescaling O -- the same softmax, written in a shifted frame.  FP8 K/V
    // rescale at every new maximum (the extra live value of the lazy form
    // would push the 4-wave FP8 kernel past its register budget).
    if constexpr (KT == 2) {
      if (mx > m + kRescaleSlack) {
        if (m != NEG_INF) {                      // rescale what earlier blocks left
          const float alpha = fast_exp2(m - mx);
          l *= alpha;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) O[dt] *= alpha;
        }
        m = mx;
      }
    } else {
      const float m_new = fmaxf(m, mx);
      if (m != NEG_INF && m_new != m) {
        const float alpha = fast_exp2(m - m_new);
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) O[dt] *= alpha;
      }
      m = m_new;
    }
    float s = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[kt][r] = fast_exp2(fmaf(x[kt][r], c_log2, -m));
        s += x[kt][r];
      }
    l += sum_over_quarters(s);

    // ---------------- O^T += V^T P^T, 4 pairs of 16-key tiles
    // One 16x16x32 MFMA covers two tiles: lane (Q, j) takes keys 4Q..4Q+3 of
    // each tile of the pair, in P^T (from S^T's layout) and in V^T (two
    // transposing reads) alike.
    if (PREFIX && staged) {
      const __amdgpu_buffer_rsrc_t img =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(img_base), (short)0, kStageBytes, kBufferFlags);
#pragma unroll
      for (int kt2 = 0; kt2 < 8; kt2 += 2) {
        __builtin_amdgcn_sched_barrier(0);
        h8 ph;
#pragma unroll
        for (int e = 0; e < 8; ++e) ph[e] = (_Float16)x[kt2 + (e >> 2)][e & 3];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const h8 a = __builtin_bit_cast(
              h8, __builtin_amdgcn_raw_buffer_load_b128(img, lane * 16, kStageKBytes + ((kt2 / 2) * 8 + dt) * 1024, 0));
          O[dt] = mfma_16x16x32(a, ph, O[dt]);
        }
      }
      continue;
    }
#pragma unroll
    for (int kt2 = 0; kt2 < 8; kt2 += 2) {
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const int kt = kt2 + t2;
        // keeps the V window at kVAhead tiles (hoisting further costs registers)
        __builtin_amdgcn_sched_barrier(0);
        if (kt + kVAhead<KT> < 8)
          vraw[kt + kVAhead<KT>] = load_v_tile<KT>(vr, lo, kt + kVAhead<KT>);
        const int key0 = kt * 16 + 2 * kp;
        stage_v_tile<KT, FP8MODE, true>(vraw[kt], lut, vt + t2 * kVtBytes, woff, full || key0 < nkeys,
                                        full || key0 + 1 < nkeys);
      }
      lds_wait();
      // P^T operand in f16 (P in (0, 2^kRescaleSlack], rounded to nearest)
      h8 ph;
#pragma unroll
      for (int e = 0; e < 8; ++e) ph[e] = (_Float16)x[kt2 + (e >> 2)][e & 3];
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        // A operand: lane (Q, j) gets dim 16dt + j of keys 4Q .. 4Q+3 of both tiles
        const h4 a0 = lds_read_tr16(vt + (roff ^ (32 * dt)));
        const h4 a1 = lds_read_tr16(vt + kVtBytes + (roff ^ (32 * dt)));
        const h8 a = h8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        O[dt] = mfma_16x16x32(a, ph, O[dt]);
      }
      lds_wait();
    }
  }

  // ---------------- merge the WAVES states in a fixed order
  if (Q == 0) {
    m_sh[w][j] = m;
    l_sh[w][j] = l;
  }
  __syncthreads();   // also: every wave is done with its V^T slice
  __shared__ float inv_sh[16], lse_sh[16];
  {
    float M = NEG_INF;
#pragma unroll
    for (int ww = 0; ww < WAVES; ++ww) M = fmaxf(M, m_sh[ww][j]);
    if (w == 0 && Q == 0) {
      // head j's softmax normaliser and log-sum-exp, once for the whole row
      float Lt = 0.0f;
#pragma unroll
      for (int ww = 0; ww < WAVES; ++ww) {
        const float mw = m_sh[ww][j];
        if (mw != NEG_INF) Lt += l_sh[ww][j] * exp2f(mw - M);
      }
      inv_sh[j] = v_scale / Lt;
      lse_sh[j] = (M + log2f(Lt)) * 0.69314718055994530942f;
    }
    const float f = (m == NEG_INF) ? 0.0f : exp2f(m - M);
    float* red = reinterpret_cast<float*>(smem) + ((size_t)w * 16 + j) * kMergeStride;
    if constexpr (KT == 2 && FP8MODE) {
      // the table decode leaves each 8-dim chunk in the order (0,2,4,6 | 1,3,5,7),
      // so row 4Q + r of a tile is dim 8(Q/2) + (Q%2) + 2r
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[dt * 16 + 8 * (Q >> 1) + (Q & 1) + 2 * r] = O[dt][r] * f;
    } else {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f4*>(red + dt * 16 + 4 * Q) = O[dt] * f;
    }
  }
  __syncthreads();
  const bool bad = nan_sh != 0;
  for (int e = threadIdx.x; e < 16 * 64; e += WAVES * 64) {
    // e -> head hh, dims 2*dl, 2*dl+1
    const int hh = e >> 6, dl = e & 63;
    const float* red = reinterpret_cast<const float*>(smem) + (size_t)hh * kMergeStride + 2 * dl;
    float2 acc = make_float2(0.0f, 0.0f);
#pragma unroll
    for (int ww = 0; ww < WAVES; ++ww) {
      const float2 v = *reinterpret_cast<const float2*>(red + (size_t)ww * 16 * kMergeStride);
      acc.x += v.x;
      acc.y += v.y;
    }
    const float inv = inv_sh[hh];
    float2 o = make_float2(acc.x * inv, acc.y * inv);
    if (bad) o = make_float2(__builtin_nanf(""), __builtin_nanf(""));
    const size_t orow = ((size_t)b * T + t) * kHeads + g * kHeadsPerGroup + hh;
    *reinterpret_cast<float2*>(out + orow * kHeadDim + 2 * dl) = o;
    if (lse != nullptr && dl == 0) lse[orow] = bad ? __builtin_nanf("") : lse_sh[hh];
  }
}

}  // namespace msa
