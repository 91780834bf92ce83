"""The MSA layer written out step by step, in fp64 on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "vLLM 為 MiniMax-M3.1-Flash 提供 Day-0 支援" (English post),
section "MSA primer" and its Figure 1 caption, in this module's words:
  1. keys are grouped in blocks of 128 tokens (one cache page each);
  2. every visible key gets a score per GQA group: the group's index query
     dotted with the key's row in the single index-key head all groups share;
  3. a block's score is the largest score among its keys;
  4. per group, 16 blocks are kept -- the newest always among them -- so a
     query sees at most 2,048 keys, and attention over those keys is exact;
  5. all query heads of a group use that group's kept blocks.

Readings where the pages are silent (each is also a test):
  * the index score is the plain dot product of the decoded index query and
    index key -- no activation, weight or temperature;
  * query token t of a sequence of length L (L counts the T new tokens) sits
    at position p = L - T + t and sees keys 0..p; its "most recent block" is
    its own block p // 128, which is one of the 16;
  * a block partly beyond p is pooled over its visible keys only; blocks past
    the own block score -inf;
  * with 16 or fewer visible blocks all of them are selected; otherwise the
    own block plus the 15 best other blocks by (score descending, block index
    ascending); the selection is reported ascending, padded with -1;
  * query head h belongs to group h // 16 (contiguous GQA), and attention uses
    softmax(scale * q.k) with max subtraction, all in fp64.
"""
import numpy as np

BLOCK = 128        # tokens per KV block / cache page
TOPK = 16          # blocks attended per query token and group
HEAD_DIM = 128
MAX_KEYS = BLOCK * TOPK


def positions(L, T):
    """Positions of the T query tokens of a sequence of total length L."""
    assert 1 <= T <= L
    return np.arange(L - T, L, dtype=np.int64)


def own_blocks(L, T):
    return positions(L, T) // BLOCK


def num_blocks(L):
    return (L + BLOCK - 1) // BLOCK


# ---------------------------------------------------------------- steps 2-3


def indexer_token_scores(idx_q, idx_k, L, T):
    """Per-key index scores s[t, g, j] = idx_q[t, g] . idx_k[j] for j <= p_t.

    idx_q: [T, G, 128] decoded index queries; idx_k: [L, 128] decoded keys of
    the single shared index-key head.  Keys after p_t get -inf.
    """
    idx_q = np.asarray(idx_q, dtype=np.float64)
    idx_k = np.asarray(idx_k, dtype=np.float64)
    assert idx_k.shape[0] == L
    T_, G, D = idx_q.shape
    s = (idx_q.reshape(T_ * G, D) @ idx_k.T).reshape(T_, G, L)        # library matmul, fp64
    p = positions(L, T)
    visible = np.arange(L)[None, :] <= p[:, None]                      # [T, L]
    return np.where(visible[:, None, :], s, -np.inf)


def block_max_pool(token_scores, L):
    """S[t, g, i] = max of the scores of block i's visible keys (-inf if none)."""
    T, G, _ = token_scores.shape
    nb = num_blocks(L)
    padded = np.full((T, G, nb * BLOCK), -np.inf)
    padded[:, :, :L] = token_scores
    return padded.reshape(T, G, nb, BLOCK).max(axis=-1)


def pooled_scores(idx_q, idx_k, L, T, chunk=128):
    """Steps 2-3 for all T query tokens, scored ``chunk`` tokens at a time so
    that a long prefill never holds every per-key score at once.  Token t of
    the whole sequence keeps its position L - T + t."""
    out = np.empty((T, idx_q.shape[1], num_blocks(L)))
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        # tokens t0..t1-1 are the last (t1 - t0) tokens of a sequence cut at L - T + t1
        Lc = L - T + t1
        s = indexer_token_scores(idx_q[t0:t1], idx_k[:Lc], Lc, t1 - t0)
        S = block_max_pool(s, Lc)
        out[t0:t1] = -np.inf
        out[t0:t1, :, :S.shape[-1]] = S
    return out


# ---------------------------------------------------------------- step 4


def select_blocks(block_scores_row, own, k=TOPK):
    """Top-k block ids for one (token, group) row, own block forced.

    Returns k ints, ascending, padded with -1.
    """
    S = np.asarray(block_scores_row, dtype=np.float64)
    if own + 1 <= k:
        chosen = list(range(own + 1))
    else:
        cand = np.arange(own)
        cs = S[:own]
        assert np.all(np.isfinite(cs)), "visible blocks must have finite scores"
        order = np.lexsort((cand, -cs))          # score descending, then index ascending
        chosen = sorted([int(i) for i in cand[order[: k - 1]]] + [int(own)])
    return np.array(chosen + [-1] * (k - len(chosen)), dtype=np.int32)


def near_tie(block_scores_row, own, k=TOPK, rel=1e-5):
    """True when the k-th and (k+1)-th ranked blocks (own block ranked first)
    are within ``rel`` relative of each other, so that fp32 rounding on the
    GPU may legitimately pick either."""
    if own + 1 <= k:
        return False
    cs = np.sort(np.asarray(block_scores_row[:own], dtype=np.float64))[::-1]
    if len(cs) < k:
        return False
    a, b = cs[k - 2], cs[k - 1]          # ranks k and k+1 overall
    return abs(a - b) <= rel * max(abs(a), abs(b))


def select_all(block_scores, L, T, k=TOPK):
    """sel[t, g, :] for every row of one sequence."""
    Tn, G, _ = block_scores.shape
    own = own_blocks(L, T)
    out = np.empty((Tn, G, k), dtype=np.int32)
    for t in range(Tn):
        for g in range(G):
            out[t, g] = select_blocks(block_scores[t, g], int(own[t]), k)
    return out


# ---------------------------------------------------------------- DCP selection
#
# Source: sections "NVFP4 indexer DCP" (NVIDIA part and AMD part): with
# decode context parallelism each of P GPUs scores all four groups over its
# share of the pages; every GPU sends its local top-16 per group to the GPU
# that owns the group, which merges them into the final top-16, and the
# selection stays exact (on AMD the block scores themselves are written to
# the owner and are bit-identical to a single-GPU run).
# Readings where the pages are silent:
#   * block i of every sequence belongs to shard i % P;
#   * a shard's candidates for a row are its blocks older than the row's own
#     block (the own block is forced by the owner, not sent);
#   * a shard sends its 16 best candidates by (score descending, block index
#     ascending), best first, fewer when it has fewer (padded with block -1,
#     score NaN);
#   * the owner applies the single-GPU rule to the union of the candidates:
#     all blocks when own+1 <= 16, else the own block plus the 15 best
#     candidates, reported ascending.


def shard_blocks(nblocks, shard, num_shards):
    """Logical block ids < nblocks that belong to `shard` of `num_shards`."""
    assert 0 <= shard < num_shards
    return np.arange(shard, nblocks, num_shards, dtype=np.int64)


def shard_candidates(block_scores_row, own, shard, num_shards, k=TOPK):
    """The shard's k best blocks older than `own` for one (token, group) row.

    Returns (scores [k] float64, blocks [k] int32), best first, padded with
    (NaN, -1)."""
    S = np.asarray(block_scores_row, dtype=np.float64)
    blocks = shard_blocks(own, shard, num_shards)
    cs = S[blocks]
    assert np.all(np.isfinite(cs)), "visible blocks must have finite scores"
    order = np.lexsort((blocks, -cs))[:k]     # score descending, then block ascending
    scores = np.full(k, np.nan)
    ids = np.full(k, -1, dtype=np.int32)
    scores[: len(order)] = cs[order]
    ids[: len(order)] = blocks[order]
    return scores, ids


def merge_candidates(cand_scores, cand_blocks, own, k=TOPK):
    """The owner's merge for one row: cand_* [P, k] from shard_candidates.

    Returns k block ids, ascending, padded with -1 -- the same layout as
    select_blocks."""
    if own + 1 <= k:
        chosen = list(range(own + 1))
    else:
        ids = np.asarray(cand_blocks).ravel()
        sc = np.asarray(cand_scores, dtype=np.float64).ravel()
        keep = ids >= 0
        ids, sc = ids[keep].astype(np.int64), sc[keep]
        order = np.lexsort((ids, -sc))[: k - 1]
        chosen = sorted([int(i) for i in ids[order]] + [int(own)])
    return np.array(chosen + [-1] * (k - len(chosen)), dtype=np.int32)


def dcp_select_all(block_scores, L, T, num_shards, k=TOPK):
    """sel[t, g, :] of one sequence by the sharded route: every shard's
    candidates, then the merge."""
    Tn, G, _ = block_scores.shape
    own = own_blocks(L, T)
    out = np.empty((Tn, G, k), dtype=np.int32)
    for t in range(Tn):
        for g in range(G):
            parts = [shard_candidates(block_scores[t, g], int(own[t]), s, num_shards, k)
                     for s in range(num_shards)]
            out[t, g] = merge_candidates(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]),
                                         int(own[t]), k)
    return out


def attended_keys(sel_row, p):
    """Key positions a query at position p attends through one selection row."""
    keys = []
    for i in sel_row:
        if i < 0:
            continue
        lo = int(i) * BLOCK
        hi = min(lo + BLOCK, p + 1)
        keys.extend(range(lo, hi))
    return np.asarray(keys, dtype=np.int64)


# ---------------------------------------------------------------- step 5


def sparse_attention(q, K, V, sel, L, T, softmax_scale):
    """Exact attention over the selected blocks.

    q: [T, H, 128]; K, V: [G, L, 128] per KV head in logical order;
    sel: [T, G, 16].  Head h uses group h // (H // G).
    Returns out [T, H, 128] and the natural-log LSE [T, H] of the scaled logits.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Tn, H, D = q.shape
    G = K.shape[0]
    hpg = H // G
    p = positions(L, T)
    out = np.zeros((Tn, H, D))
    lse = np.zeros((Tn, H))
    for t in range(Tn):
        for g in range(G):
            keys = attended_keys(sel[t, g], int(p[t]))
            assert len(keys) <= MAX_KEYS
            Kg = K[g, keys]                        # [n, D]
            Vg = V[g, keys]
            for h in range(g * hpg, (g + 1) * hpg):
                logits = softmax_scale * (Kg @ q[t, h])
                m = logits.max()
                e = np.exp(logits - m)
                ssum = e.sum()
                out[t, h] = (e @ Vg) / ssum
                lse[t, h] = m + np.log(ssum)
    return out, lse


# ---------------------------------------------------------------- layer step


def layer_step(idx_q, idx_k, q, K, V, L, T, softmax_scale):
    """All four steps for one sequence, on decoded fp64 inputs in logical order.

    idx_q [T, G, 128], idx_k [L, 128], q [T, H, 128], K/V [G, L, 128].
    Returns a dict with token_scores, block_scores, sel, out and lse.
    """
    s = indexer_token_scores(idx_q, idx_k, L, T)
    S = block_max_pool(s, L)
    sel = select_all(S, L, T)
    out, lse = sparse_attention(q, K, V, sel, L, T, softmax_scale)
    return {"token_scores": s, "block_scores": S, "sel": sel, "out": out, "lse": lse}


# ---------------------------------------------------------------- paged caches


def decode_pages(cache, pages, mode="exact"):
    """Decode some pages of a paged cache to fp64 [len(pages), heads, 128, 128].

    ``cache`` is a dict: dtype ('f32' | 'fp8' | 'nvfp4'), data, scales (NVFP4
    only), tensor_scale.  Layout: page, head, token-in-page, then the 128 dims
    (fp32 values, FP8 bytes, or NVFP4 codes two per byte plus one E4M3 scale
    byte per 16 dims in a separate array).
    """
    from . import formats
    pages = np.asarray(pages, dtype=np.int64)
    dt = cache["dtype"]
    S = float(cache.get("tensor_scale", 1.0))
    if dt == "f32":
        return S * np.asarray(cache["data"][pages], dtype=np.float64)
    if dt == "fp8":
        return formats.fp8_dequantize(cache["data"][pages], S)
    if dt == "nvfp4":
        return formats.nvfp4_dequantize(cache["data"][pages], cache["scales"][pages], S, mode)
    raise ValueError(dt)


def decode_query(qarr, dtype, scale):
    """Decoded query values (fp32 array as is, FP8 bytes through E4M3), times scale."""
    from . import formats
    if dtype == "f32":
        return float(scale) * np.asarray(qarr, dtype=np.float64)
    if dtype == "fp8":
        return formats.fp8_dequantize(qarr, scale)
    raise ValueError(dtype)


def cache_insert(cache, x, seq_lens, block_table, T):
    """Quantise-and-insert: the new tokens' rows written into a paged cache.

    Source: section "QKV GEMM + norm + RoPE + KV insert fusion" -- K, V and the
    index key are quantised (to NVFP4) as they are written into their caches.
    x: fp32 [B, T, heads, 128], the rows of the T new tokens of each sequence;
    token t of sequence b sits at position p = seq_lens[b] - T + t, which is
    row p % 128 of page block_table[b][p // 128] (as for every other step).
    Each row is quantised on its own with the cache's tensor scale
    (formats.fp8_quantize / formats.nvfp4_quantize; fp32 rows are copied).
    Returns a new cache dict; rows whose page id is outside the pool are
    skipped, and nothing else changes.
    """
    from . import formats
    out = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in cache.items()}
    dt = cache["dtype"]
    S = float(cache.get("tensor_scale", 1.0))
    P = out["data"].shape[0]
    x = np.asarray(x, dtype=np.float32)
    for b in range(len(seq_lens)):
        for t in range(T):
            p = int(seq_lens[b]) - T + t
            page = int(block_table[b][p // BLOCK])
            if page < 0 or page >= P:
                continue
            r = p % BLOCK
            for h in range(x.shape[2]):
                row = x[b, t, h]
                if dt == "f32":
                    out["data"][page, h, r] = row
                elif dt == "fp8":
                    out["data"][page, h, r] = formats.fp8_quantize(row, S)
                elif dt == "nvfp4":
                    codes, sc = formats.nvfp4_quantize(row, S)
                    out["data"][page, h, r] = codes
                    out["scales"][page, h, r] = sc
                else:
                    raise ValueError(dt)
    return out


def sequence_view(cache, block_table_row, L, mode="exact"):
    """[heads, L, 128] decoded rows of one sequence, logical order."""
    nb = num_blocks(L)
    pages = np.asarray(block_table_row[:nb], dtype=np.int64)
    dec = decode_pages(cache, pages, mode)                 # [nb, heads, 128, 128]
    heads = dec.shape[1]
    return dec.transpose(1, 0, 2, 3).reshape(heads, nb * BLOCK, HEAD_DIM)[:, :L]


def batch_layer(idx_q, q, idx_cache, k_cache, v_cache, seq_lens, block_table, T,
                softmax_scale, mode="exact", idx_q_dtype="f32", idx_q_scale=1.0,
                q_dtype="f32", q_scale=1.0, max_blocks=None, sequences=None,
                with_attention=True):
    """The layer step for a batch of paged sequences.

    idx_q: [B, T, G, 128] and q: [B, T, H, 128] (fp32 values or FP8 bytes);
    caches as in ``decode_pages`` (index-key cache has one head).
    Returns block_scores [B, T, G, max_blocks] (-inf past each row's own block),
    sel [B, T, G, 16], out [B, T, H, 128], lse [B, T, H], near_tie [B, T, G];
    ``sequences`` restricts the work to some batch rows (others stay NaN / -1).
    """
    B = len(seq_lens)
    G = idx_q.shape[2]
    H = q.shape[2]
    if max_blocks is None:
        max_blocks = block_table.shape[1]
    bs = np.full((B, T, G, max_blocks), np.nan)
    sel = np.full((B, T, G, TOPK), -1, dtype=np.int32)
    out = np.full((B, T, H, HEAD_DIM), np.nan)
    lse = np.full((B, T, H), np.nan)
    ties = np.zeros((B, T, G), dtype=bool)
    for b in (range(B) if sequences is None else sequences):
        L = int(seq_lens[b])
        iq = decode_query(idx_q[b], idx_q_dtype, idx_q_scale)
        ik = sequence_view(idx_cache, block_table[b], L, mode)[0]
        S = pooled_scores(iq, ik, L, T)
        nb = S.shape[-1]
        bs[b, :, :, :] = -np.inf
        bs[b, :, :, :nb] = S
        own = own_blocks(L, T)
        for t in range(T):
            for g in range(G):
                sel[b, t, g] = select_blocks(S[t, g], int(own[t]))
                ties[b, t, g] = near_tie(S[t, g], int(own[t]))
        if with_attention:
            qq = decode_query(q[b], q_dtype, q_scale)
            K = sequence_view(k_cache, block_table[b], L, mode)
            V = sequence_view(v_cache, block_table[b], L, mode)
            out[b], lse[b] = sparse_attention(qq, K, V, sel[b], L, T, softmax_scale)
    return {"block_scores": bs, "sel": sel, "out": out, "lse": lse, "near_tie": ties}
