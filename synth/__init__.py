"""Seeded synthetic inputs for the MSA hot path.

This module only draws numbers: it holds none of the method's arithmetic (no
quantisation, scoring, pooling, selection or attention).  The HIP library
and the CPU oracle both consume what it produces; each quantises and computes
on its own.

Workloads (the shapes of the long-context decode, speculative-decode and
chunked-prefill cases the source pages discuss; the pages measure on a
serving benchmark that these synthetic inputs stand in for):

  c1       batch 1, 4,096-token context, T=1, fp32 everywhere, 3 hot blocks
           (groups 0-2), pages in order.
  c2       batch 32, 32,768 tokens, T=1, FP8 caches and queries (scale 1.0),
           8 hot blocks per sequence (2 per group), shuffled pages.
  c3       batch 64, ragged lengths uniform in [65,536, 163,840], T=1, NVFP4
           caches with 5% N(0,16) outliers, FP8 queries, shuffled pages.
  c3_128k  c3 with every length 131,072 (the decode headline workload).
  c4       batch 16, 262,144 tokens, T=4 (speculative decode), NVFP4, FP8 q.
  c5       batch 2, 65,536 cached + 4,096 new tokens (T=4,096), NVFP4,
           8 hot blocks per sequence in the cached region.
Small variants (``tiny_*``) keep the same structure at sizes the oracle
finishes in seconds.

Values are N(0,1) from torch's seeded generators; an outlier replaces a value
by four times a fresh N(0,1) draw (i.e. N(0,16)).  A hot block of sequence b
for group g gets 2.0 * qhat added to each of its index-key rows, where qhat
is the L2-normalised fp32 index query of group g (for prefill the index
queries are z + m_g with m_g shared by all tokens and qhat = m_g / |m_g|).
"""
from dataclasses import dataclass, field
import math

import numpy as np
import torch

BLOCK = 128
HEAD_DIM = 128
GROUPS = 4
HEADS_PER_GROUP = 16
HEADS = GROUPS * HEADS_PER_GROUP

STREAMS = {"idx_q": 0, "q": 1, "idx_k": 2, "k": 3, "v": 4, "perm": 5, "hot": 6,
           "lens": 7, "outlier": 8, "prefill_m": 9}

# NVFP4 per-tensor scale: a fixed bound on |x| divided by 448, so block
# scales stay <= 448/6 and the FP8-rounded products never saturate.
NVFP4_BOUND = 32.0


@dataclass
class Workload:
    name: str
    B: int
    T: int
    lens: object                 # int, (lo, hi) for uniform ragged lengths, or a list per sequence
    kv_dtype: str                # 'f32' | 'fp8' | 'nvfp4'
    q_dtype: str                 # 'f32' | 'fp8'
    hot_per_seq: int = 0
    hot_groups: list = field(default_factory=list)   # group of hot block n (default n % G)
    outlier_p: float = 0.0
    shuffle_pages: bool = True
    prefill_planting: bool = False

    def tensor_scale(self):
        """Per-tensor scale of the caches, as the fp32 value the library uses."""
        return float(np.float32(NVFP4_BOUND / 448.0)) if self.kv_dtype == "nvfp4" else 1.0


WORKLOADS = {
    "c1": Workload("c1", 1, 1, 4096, "f32", "f32", 3, [0, 1, 2], 0.0, False),
    "c2": Workload("c2", 32, 1, 32768, "fp8", "fp8", 8),
    "c3": Workload("c3", 64, 1, (65536, 163840), "nvfp4", "fp8", 0, [], 0.05),
    "c3_128k": Workload("c3_128k", 64, 1, 131072, "nvfp4", "fp8", 0, [], 0.05),
    "c4": Workload("c4", 16, 4, 262144, "nvfp4", "fp8"),
    # the 128K decode batch verifying 1 + 7 speculative tokens per sequence
    "c3_t8": Workload("c3_t8", 64, 8, 131072, "nvfp4", "fp8", 0, [], 0.05),
    "c5": Workload("c5", 2, 4096, 69632, "nvfp4", "fp8", 8, [], 0.0, True, True),
    # small cases with the same structure (several tiles, ragged tails)
    "tiny_f32": Workload("tiny_f32", 2, 1, (300, 2600), "f32", "f32", 3, [0, 1, 2], 0.0, True),
    "tiny_fp8": Workload("tiny_fp8", 3, 1, (1000, 5000), "fp8", "fp8", 8),
    "tiny_nvfp4": Workload("tiny_nvfp4", 3, 1, (1500, 7000), "nvfp4", "fp8", 4, [], 0.05),
    "tiny_spec": Workload("tiny_spec", 2, 4, (2100, 6000), "nvfp4", "fp8", 4),
    "tiny_prefill": Workload("tiny_prefill", 2, 300, (2500, 4200), "nvfp4", "fp8", 8, [], 0.0, True, True),
    "tiny_prefill_fp8": Workload("tiny_prefill_fp8", 2, 200, (1500, 3000), "fp8", "fp8", 8, [], 0.0, True, True),
    # edge cases: T = 2 and 3; contexts of 1, 128, 129, 2,048 and 2,049 tokens (one key,
    # exact block edges, 16 vs 17 blocks); a prefill with no cached context; a row of
    # more than 2,048 blocks
    "tiny_t2": Workload("tiny_t2", 2, 2, (130, 3000), "nvfp4", "fp8", 4, [], 0.05),
    "tiny_t3": Workload("tiny_t3", 3, 3, (2200, 4000), "fp8", "fp8", 4),
    # speculative decode with 7 speculative tokens (T = 8) and a T = 6 case
    "tiny_spec8": Workload("tiny_spec8", 2, 8, (2100, 6000), "nvfp4", "fp8", 4, [], 0.05),
    "tiny_t6": Workload("tiny_t6", 3, 6, (130, 4000), "fp8", "fp8", 4),
    "tiny_edge": Workload("tiny_edge", 5, 1, [1, 128, 129, 2048, 2049], "nvfp4", "fp8", 2, [], 0.0),
    "tiny_prefill_nocache": Workload("tiny_prefill_nocache", 2, 129, [129, 700], "nvfp4", "fp8", 2, [], 0.0,
                                     True, True),
    "long_rows": Workload("long_rows", 1, 1, 300000, "fp8", "fp8", 8),
    # a row of exactly 2,048 blocks: the largest whose block-table row the selecting
    # attention copies into LDS during its selection
    "rows_2048": Workload("rows_2048", 1, 1, 262144, "nvfp4", "fp8", 4, [], 0.05),
    # speculative decode with the first token's position L - T at and around the scan's
    # 64-key unit edges (62, 63, 64, 127, 128, 129, 255, 1023): the units that need
    # the visibility masks start exactly there
    "spec_edges": Workload("spec_edges", 8, 4, [66, 67, 68, 131, 132, 133, 259, 1027], "nvfp4", "fp8", 0, [], 0.05),
    "spec_edges8": Workload("spec_edges8", 8, 8, [70, 71, 72, 135, 136, 137, 263, 1031], "fp8", "fp8", 0, [], 0.05),
    # more sequences (1,030) than the evenly spread one-token scan takes, short ragged contexts
    "wide_batch": Workload("wide_batch", 1030, 1, (1, 300), "nvfp4", "fp8", 2, [], 0.05),
    # enough query rows (2 x 1,100 x 4) for the many-row attention form
    "tiny_prefill_many": Workload("tiny_prefill_many", 2, 1100, (2300, 3600), "nvfp4", "fp8", 8, [], 0.0, True, True),
}


def _gen(seed, stream, chunk=0, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + stream * 7_919 + chunk * 104_729) & 0x7FFF_FFFF_FFFF)
    return g


@dataclass
class Layout:
    """Page bookkeeping of one batch: lengths, block table, pool size."""
    seq_lens: torch.Tensor       # [B] int32 (CPU)
    block_table: torch.Tensor    # [B, max_blocks] int32 (CPU), -1 past each sequence
    num_pages: int
    max_blocks: int


def make_layout(w: Workload, seed: int) -> Layout:
    g = _gen(seed, STREAMS["lens"])
    if isinstance(w.lens, tuple):
        lo, hi = w.lens
        lens = torch.randint(lo, hi + 1, (w.B,), generator=g, dtype=torch.int64)
    elif isinstance(w.lens, list):
        assert len(w.lens) == w.B
        lens = torch.tensor(w.lens, dtype=torch.int64)
    else:
        lens = torch.full((w.B,), int(w.lens), dtype=torch.int64)
    assert int(lens.min()) >= w.T
    nbs = (lens + BLOCK - 1) // BLOCK
    P = int(nbs.sum())
    maxb = int(nbs.max())
    if w.shuffle_pages:
        perm = torch.randperm(P, generator=_gen(seed, STREAMS["perm"]), dtype=torch.int64)
    else:
        perm = torch.arange(P, dtype=torch.int64)
    table = torch.full((w.B, maxb), -1, dtype=torch.int32)
    off = 0
    for b in range(w.B):
        n = int(nbs[b])
        table[b, :n] = perm[off:off + n].to(torch.int32)
        off += n
    return Layout(lens.to(torch.int32), table, P, maxb)


def queries(w: Workload, seed: int, device="cpu"):
    """fp32 idx_q [B, T, G, 128], q [B, T, 64, 128], and the hot directions
    qhat [B, G, 128] used for planting."""
    gq = _gen(seed, STREAMS["idx_q"], device=device)
    idx_q = torch.randn((w.B, w.T, GROUPS, HEAD_DIM), generator=gq, device=device)
    if w.prefill_planting:
        gm = _gen(seed, STREAMS["prefill_m"], device=device)
        m = torch.randn((w.B, 1, GROUPS, HEAD_DIM), generator=gm, device=device)
        idx_q = idx_q + m
        direction = m[:, 0]
    else:
        direction = idx_q[:, 0]
    qhat = direction / torch.linalg.vector_norm(direction, dim=-1, keepdim=True)
    q = torch.randn((w.B, w.T, HEADS, HEAD_DIM), generator=_gen(seed, STREAMS["q"], device=device),
                    device=device)
    return idx_q, q, qhat


def hot_blocks(w: Workload, lay: Layout, seed: int):
    """List of (b, logical block, group) planted hot blocks.

    Hot blocks are distinct, exclude every query token's own block (for
    prefill: they lie in the cached region before the first new token)."""
    g = _gen(seed, STREAMS["hot"])
    out = []
    for b in range(w.B):
        L = int(lay.seq_lens[b])
        first_own = (L - w.T) // BLOCK
        n = min(w.hot_per_seq, first_own)
        if n <= 0:
            continue
        pick = torch.randperm(first_own, generator=g)[:n]
        for k in range(n):
            grp = w.hot_groups[k] if k < len(w.hot_groups) else k % GROUPS
            out.append((b, int(pick[k]), grp))
    return out


def cache_pages(w: Workload, lay: Layout, seed: int, which: str, first: int, count: int,
                qhat=None, hot=None, device="cpu"):
    """fp32 values of pages [first, first+count) of one cache.

    which: 'idx_k' (one head) or 'k' / 'v' (four heads).  Shape
    [count, heads, 128, 128].  Pages are drawn in chunks of 1024 with their own
    sub-seed, so any page range can be regenerated on its own (on the same
    device type).  Index-key pages of hot blocks get the planted direction.
    """
    heads = 1 if which == "idx_k" else GROUPS
    CH = 1024
    c0, c1 = first // CH, (first + count - 1) // CH
    parts = []
    for c in range(c0, c1 + 1):
        n = min(CH, lay.num_pages - c * CH)
        gen = _gen(seed, STREAMS[which], c, device=device)
        x = torch.randn((n, heads, BLOCK, HEAD_DIM), generator=gen, device=device)
        if w.outlier_p > 0:
            go = _gen(seed, STREAMS["outlier"] + 16 * STREAMS[which], c, device=device)
            u = torch.rand((n, heads, BLOCK, HEAD_DIM), generator=go, device=device)
            z = torch.randn((n, heads, BLOCK, HEAD_DIM), generator=go, device=device)
            x = torch.where(u < w.outlier_p, 4.0 * z, x)
        parts.append(x)
    x = torch.cat(parts)[first - c0 * CH: first - c0 * CH + count]
    if which == "idx_k" and hot:
        for (b, blk, grp) in hot:
            page = int(lay.block_table[b, blk])
            if first <= page < first + count:
                x[page - first, 0] += 2.0 * qhat[b, grp].to(x.device)
    return x


def describe(w: Workload):
    return {"workload": w.name, "batch": w.B, "query_tokens": w.T,
            "context": w.lens if not isinstance(w.lens, tuple) else list(w.lens),
            "kv_dtype": w.kv_dtype, "q_dtype": w.q_dtype}
