// Shared-prefix decode attention (msa_sparse_attn_decode_prefix): every
// shared-prefix block that two or more requests of a prefix group selected is
// dequantised once, and all of those requests read it from there.
//
// Source: "vLLM 為 MiniMax-M3.1-Flash 提供 Day-0 支援", section "NVFP4 MSA
// kernel" (AMD): the sparse decode attention decodes a prefix page common to
// as many as 64 requests a single time for all of them.
//
// Three launches, no workgroup waits for another:
//  1. plan: one workgroup per (prefix group, KV head) marks, in LDS bitmaps,
//     the prefix blocks two or more of the group's rows selected as an older
//     block, and numbers them in block order: slot_of[k][g][i] (-1 otherwise)
//     and slot_blk[slot] = i, count[k][g] = the number of slots used.  Slots of
//     (k, g) lie in a fixed region of the workspace whose size the host derives
//     from the call's arguments (min(prefix blocks, 16 x the group's rows)).
//  2. stage: one wave per slot of every region (waves past their region's
//     count return at once) decodes the slot's (page, KV head) slice with the
//     attention's own tile code into the operand images of attn_row.hpp
//     (64 KiB per slot).
//  3. attention: attend_row<..., PREFIX=true> reads staged blocks from their
//     images; every other block is decoded from its page as usual.
// Every slot the attention reads was written by this call's stage launch, and
// every slot_of entry of every group by its plan launch, so nothing from an
// earlier call is read.
#include "attn_row.hpp"
#include "launch.hpp"

namespace msa {

struct PrefixPlanArgs {
  const int32_t* sel;          // [B][T][4][16]
  const int32_t* seq_lens;
  int T;
  int32_t* slot_of;
  int32_t* slot_blk;
  int32_t* count;              // [groups][4]
  PrefixAttnArgs map;          // start, blocks, slot_of_base (staged / slot_of unused here)
  int region[4 * kMaxPrefixGroupsDev + 1];   // slot region of (k, g) = [region[4k+g], region[4k+g+1])
};

__global__ __launch_bounds__(256) void prefix_plan_kernel(PrefixPlanArgs a) {
  __shared__ uint32_t bits[kMaxBlocksSelect / 32];    // selected by at least one row
  __shared__ uint32_t multi[kMaxBlocksSelect / 32];   // selected by at least two rows
  __shared__ uint32_t scan[256];
  const int k = blockIdx.x >> 2, g = blockIdx.x & 3, tid = threadIdx.x;
  const int pb = a.map.blocks[k], s0 = a.map.start[k], s1 = a.map.start[k + 1], T = a.T;
  bits[tid] = 0u;
  multi[tid] = 0u;
  __syncthreads();
  const int entries = (s1 - s0) * T * kTopK;
  for (int e = tid; e < entries; e += 256) {
    const int r = e / kTopK;
    const int s = s0 + r / T, t = r % T;
    const int id = a.sel[((size_t)(s * T + t) * kGroups + g) * kTopK + e % kTopK];
    const int own = (a.seq_lens[s] - T + t) / kBlock;
    if (id >= 0 && id < pb && id < own) {
      const uint32_t m = 1u << (id & 31);
      // a row's ids are distinct, so a bit already set means a second row
      if (atomicOr(&bits[id >> 5], m) & m) atomicOr(&multi[id >> 5], m);
    }
  }
  __syncthreads();
  // Only blocks that two or more rows selected are staged: for a block one row
  // reads, decoding it in place costs no more than decoding it for the image.
  // Exclusive prefix sum of the 256 words' bit counts (Hillis-Steele over LDS).
  const uint32_t mine = multi[tid];
  uint32_t v = __builtin_popcount(mine);
  scan[tid] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const uint32_t add = tid >= off ? scan[tid - off] : 0u;
    __syncthreads();
    scan[tid] += add;
    __syncthreads();
  }
  const uint32_t before = scan[tid] - v;
  const int region = a.region[4 * k + g];
  int32_t* so = a.slot_of + a.map.slot_of_base[k] + g * pb;
  for (int bit = 0; bit < 32; ++bit) {
    const int i = tid * 32 + bit;
    if (i >= pb) break;
    if ((mine >> bit) & 1u) {
      const int slot = region + (int)(before + __builtin_popcount(mine & ((1u << bit) - 1u)));
      so[i] = slot;
      a.slot_blk[slot] = i;
    } else {
      so[i] = -1;
    }
  }
  if (tid == 255) a.count[4 * k + g] = (int)scan[255];
}

struct PrefixStageArgs {
  const uint8_t* kdata;
  const uint8_t* kscales;
  int64_t kpages;
  const uint8_t* vdata;
  const uint8_t* vscales;
  int64_t vpages;
  const int32_t* table;
  int max_blocks;
  const int32_t* slot_blk;
  const int32_t* count;
  uint8_t* staged;
  int nregions;
  int start[kMaxPrefixGroupsDev + 1];
  int region[4 * kMaxPrefixGroupsDev + 1];
};

template <int KT, bool FP8MODE>
__global__ __launch_bounds__(64) void prefix_stage_kernel(PrefixStageArgs a) {
  __shared__ uint32_t lut[FP8MODE ? 512 : 2];
  __shared__ __attribute__((aligned(16))) uint8_t vt[kVtSlotBytes];
  const int slot = blockIdx.x, lane = threadIdx.x;
  // the (group, head) region holding this slot
  int lo_r = 0, hi_r = a.nregions;   // region[lo_r] <= slot < region[hi_r]
  while (hi_r - lo_r > 1) {
    const int mid = (lo_r + hi_r) >> 1;
    if (a.region[mid] <= slot) lo_r = mid; else hi_r = mid;
  }
  const int r = lo_r, k = r >> 2, g = r & 3;
  if (slot - a.region[r] >= a.count[r]) return;   // past the slots the plan used
  const int blk = a.slot_blk[slot];
  const int pg = a.table[(size_t)a.start[k] * a.max_blocks + blk];
  if (pg < 0 || (int64_t)pg >= a.kpages || (int64_t)pg >= a.vpages) return;   // the attention marks such rows NaN
  if (FP8MODE) {
    build_fp8_lut(lut);
    __syncthreads();
  }
  const size_t rowbase = ((size_t)pg * kGroups + g) * kBlock;
  const KvRsrc kr = kv_rsrc<KT>(a.kdata, a.kscales, rowbase);
  const KvRsrc vr = kv_rsrc<KT>(a.vdata, a.vscales, rowbase);
  const int Q = lane >> 4, j = lane & 15, kp = lane & 7, dg = lane >> 3;
  const KvLaneOffsets lo = kv_lane_offsets<KT>(j, Q, kp, dg);
  uint8_t* img = a.staged + (size_t)slot * kStageBytes;
  // K image: the decoded A fragments of every tile
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
    h8 Ak[4];
    decode_k_tile<KT, FP8MODE>(load_k_tile<KT>(kr, lo, kt), lut, Ak);
#pragma unroll
    for (int c = 0; c < 4; ++c) *reinterpret_cast<h8*>(img + ((kt * 4 + c) * 64 + lane) * 16) = Ak[c];
  }
  // V image: each tile pair staged through LDS and read back transposed, as the
  // attention does
  int woff[2][2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) woff[u][hh] = vt_offset(2 * kp + u, 2 * dg + hh);
  const int roff = vt_offset(lane >> 2, (lane & 3) >> 1) + 8 * (lane & 1);
#pragma unroll
  for (int kt2 = 0; kt2 < 8; kt2 += 2) {
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
      stage_v_tile<KT, FP8MODE, false>(load_v_tile<KT>(vr, lo, kt2 + t2), lut, vt + t2 * kVtBytes, woff, true, true);
    lds_wait();
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const h4 a0 = lds_read_tr16(vt + (roff ^ (32 * dt)));
      const h4 a1 = lds_read_tr16(vt + kVtBytes + (roff ^ (32 * dt)));
      const h8 av = h8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      *reinterpret_cast<h8*>(img + kStageKBytes + (((kt2 / 2) * 8 + dt) * 64 + lane) * 16) = av;
    }
    lds_wait();
  }
}

// Slots of a call: region (k, g) holds min(blocks[k], 16 x rows of group k).
int prefix_slot_regions(const PrefixGroups& gr, int T, int* region) {
  int total = 0;
  for (int k = 0; k < gr.n; ++k) {
    const int64_t rows16 = (int64_t)(gr.start[k + 1] - gr.start[k]) * T * kTopK;
    const int per = (int)(gr.blocks[k] < rows16 ? gr.blocks[k] : rows16);
    for (int g = 0; g < kGroups; ++g) {
      region[4 * k + g] = total;
      total += per;
    }
  }
  region[4 * gr.n] = total;
  return total;
}

PrefixWorkspace prefix_workspace_layout(const PrefixGroups& gr, int T) {
  PrefixWorkspace w{};
  int region[4 * kMaxPrefixGroupsDev + 1];
  w.slots = prefix_slot_regions(gr, T, region);
  int64_t nslot_of = 0;
  for (int k = 0; k < gr.n; ++k) nslot_of += 4 * (int64_t)gr.blocks[k];
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  w.staged = 0;
  w.slot_of = up((size_t)w.slots * kStageBytes);
  w.slot_blk = up(w.slot_of + (size_t)nslot_of * 4);
  w.count = up(w.slot_blk + (size_t)w.slots * 4);
  w.bytes = up(w.count + (size_t)(4 * kMaxPrefixGroupsDev) * 4);
  return w;
}

hipError_t launch_attention_prefix(const ProblemArgs& p, const void* q, float q_scale, const CacheArgs& k,
                                   const CacheArgs& v, bool fp8mode, const int32_t* sel, float softmax_scale,
                                   float* out, float* lse, const PrefixGroups& gr, void* workspace, hipStream_t s) {
  const PrefixWorkspace wl = prefix_workspace_layout(gr, p.T);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  PrefixAttnArgs pa{};
  pa.staged = ws + wl.staged;
  pa.slot_of = reinterpret_cast<const int32_t*>(ws + wl.slot_of);
  pa.n = gr.n;
  int base = 0;
  for (int kk = 0; kk < gr.n; ++kk) {
    pa.start[kk] = gr.start[kk];
    pa.blocks[kk] = gr.blocks[kk];
    pa.slot_of_base[kk] = base;
    base += 4 * gr.blocks[kk];
  }
  pa.start[gr.n] = gr.start[gr.n];
  if (gr.n > 0 && wl.slots > 0) {
    PrefixPlanArgs pl{};
    pl.sel = sel;
    pl.seq_lens = p.seq_lens;
    pl.T = p.T;
    pl.slot_of = reinterpret_cast<int32_t*>(ws + wl.slot_of);
    pl.slot_blk = reinterpret_cast<int32_t*>(ws + wl.slot_blk);
    pl.count = reinterpret_cast<int32_t*>(ws + wl.count);
    pl.map = pa;
    prefix_slot_regions(gr, p.T, pl.region);
    hipLaunchKernelGGL(prefix_plan_kernel, dim3(4 * gr.n), dim3(256), 0, s, pl);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    PrefixStageArgs st{};
    st.kdata = k.data;
    st.kscales = k.scales;
    st.kpages = k.num_pages;
    st.vdata = v.data;
    st.vscales = v.scales;
    st.vpages = v.num_pages;
    st.table = p.block_table;
    st.max_blocks = p.max_blocks;
    st.slot_blk = pl.slot_blk;
    st.count = pl.count;
    st.staged = ws + wl.staged;
    st.nregions = 4 * gr.n;
    for (int kk = 0; kk <= gr.n; ++kk) st.start[kk] = gr.start[kk];
    for (int r = 0; r <= 4 * gr.n; ++r) st.region[r] = pl.region[r];
    if (k.dtype == 1)
      hipLaunchKernelGGL((prefix_stage_kernel<1, false>), dim3(wl.slots), dim3(64), 0, s, st);
    else if (fp8mode)
      hipLaunchKernelGGL((prefix_stage_kernel<2, true>), dim3(wl.slots), dim3(64), 0, s, st);
    else
      hipLaunchKernelGGL((prefix_stage_kernel<2, false>), dim3(wl.slots), dim3(64), 0, s, st);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_attention(p, q, 1, q_scale, k, v, fp8mode, sel, softmax_scale, out, lse, s, nullptr, nullptr,
                          gr.n > 0 ? &pa : nullptr);
}

}  // namespace msa
