"""Pins of the oracle's layer step against things other than itself:
brute-force loops and subset enumeration on tiny inputs, torch's CPU fp64
scaled_dot_product_attention (dense causal attention, and masked attention
built from a selection), closed forms (q = 0, L = 1), page-order invariance,
and the invariants the source pages state (own block kept, <= 16 blocks,
<= 2,048 keys)."""
import itertools
import json
import os

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import msa as M

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))
SCALE = 1.0 / np.sqrt(128.0)


def test_page_constants():
    assert M.BLOCK == GOLD["block_tokens"]["value"]
    assert M.TOPK == GOLD["selected_blocks"]["value"]
    assert M.MAX_KEYS == GOLD["max_keys_per_query"]["value"]


def test_indexer_scores_and_pool_brute_force():
    rng = np.random.default_rng(3)
    for L, T in [(1, 1), (130, 1), (300, 3), (257, 2), (128, 1), (129, 4)]:
        G, D = 4, 8
        q = rng.normal(size=(T, G, D))
        k = rng.normal(size=(L, D))
        s = M.indexer_token_scores(q, k, L, T)
        S = M.block_max_pool(s, L)
        nb = (L + 127) // 128
        assert S.shape == (T, G, nb)
        for t in range(T):
            p = L - T + t
            for g in range(G):
                for j in range(L):
                    want = sum(q[t, g, d] * k[j, d] for d in range(D)) if j <= p else -np.inf
                    assert s[t, g, j] == pytest.approx(want, abs=1e-12) or (want == -np.inf and s[t, g, j] == -np.inf)
                for i in range(nb):
                    vals = [s[t, g, j] for j in range(i * 128, min((i + 1) * 128, L)) if j <= p]
                    want = max(vals) if vals else -np.inf
                    assert S[t, g, i] == want


def brute_select(S, own, k=16):
    """Enumerate every candidate subset; keep the one with the largest score
    sum, then the smallest index sum (ties go to lower block ids)."""
    if own + 1 <= k:
        return list(range(own + 1))
    best = None
    for sub in itertools.combinations(range(own), k - 1):
        key = (sum(S[i] for i in sub), -sum(sub))
        if best is None or key > best[0]:
            best = (key, sub)
    return sorted(list(best[1]) + [own])


@pytest.mark.parametrize("nb", [1, 5, 16, 17, 18, 19, 20])
def test_selection_matches_subset_enumeration(nb):
    rng = np.random.default_rng(nb)
    for trial in range(3):
        S = np.round(rng.normal(size=nb), 1 if trial == 2 else 6)      # trial 2: many exact ties
        for own in sorted({nb - 1, max(0, nb - 3)}):
            sel = M.select_blocks(S, own)
            got = [int(i) for i in sel if i >= 0]
            assert got == brute_select(S, own)
            assert list(sel[len(got):]) == [-1] * (16 - len(got))


def test_selection_invariants_random_rows():
    rng = np.random.default_rng(5)
    for _ in range(300):
        nb = int(rng.integers(1, 400))
        own = int(rng.integers(0, nb))
        S = rng.normal(size=nb)
        S[own + 1:] = -np.inf
        sel = M.select_blocks(S, own)
        got = [int(i) for i in sel if i >= 0]
        assert own in got                                      # most recent block kept
        assert len(got) == min(16, own + 1)                    # <= 16 blocks
        assert got == sorted(got) and len(set(got)) == len(got)
        p = own * 128 + int(rng.integers(0, 128))
        assert len(M.attended_keys(sel, p)) <= GOLD["max_keys_per_query"]["value"]
        # every unselected older block scores no higher than every selected one
        others = [i for i in range(own) if i not in got]
        chosen = [i for i in got if i != own]
        if others and chosen:
            assert max(S[others]) <= min(S[chosen])


def test_near_tie_flag():
    S = np.arange(40, dtype=float)[::-1].copy()       # strictly decreasing
    assert not M.near_tie(S, 39)
    S[14] = S[15] * (1 + 5e-6)                          # ranks 16/17 overall
    assert M.near_tie(S, 39)
    assert not M.near_tie(S, 10)                        # <= 16 visible blocks


def sdpa_masked(q, K, V, mask):
    """torch fp64 SDPA with GQA expanded; mask [T, L] True = attend."""
    T, H, D = q.shape
    G = K.shape[0]
    Kx = torch.tensor(K).repeat_interleave(H // G, dim=0)          # [H, L, D]
    Vx = torch.tensor(V).repeat_interleave(H // G, dim=0)
    qq = torch.tensor(q).permute(1, 0, 2)                           # [H, T, D]
    m = torch.tensor(mask)[None].expand(H, -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qq, Kx, Vx, attn_mask=m, scale=SCALE)
    logits = (qq @ Kx.transpose(-1, -2)) * SCALE
    lse = torch.logsumexp(logits.masked_fill(~m, -float("inf")), dim=-1)
    return o.permute(1, 0, 2).numpy(), lse.T.numpy()


@pytest.mark.parametrize("L,T", [(1, 1), (77, 1), (128, 1), (1000, 1), (2048, 1), (2048, 4), (1500, 7)])
def test_short_context_equals_dense_causal_attention(L, T):
    rng = np.random.default_rng(L + T)
    G, H, D = 4, 64, 128
    idx_q = rng.normal(size=(T, G, D))
    idx_k = rng.normal(size=(L, D))
    q = rng.normal(size=(T, H, D))
    K = rng.normal(size=(G, L, D))
    V = rng.normal(size=(G, L, D))
    r = M.layer_step(idx_q, idx_k, q, K, V, L, T, SCALE)
    pos = np.arange(L - T, L)
    mask = np.arange(L)[None, :] <= pos[:, None]
    o, lse = sdpa_masked(q, K, V, mask)
    assert np.abs(r["out"] - o).max() < 1e-12
    assert np.abs(r["lse"] - lse).max() < 1e-12


def test_sparse_attention_equals_masked_sdpa_from_selection():
    rng = np.random.default_rng(11)
    G, H, D, L, T = 4, 64, 128, 128 * 40 + 55, 3
    idx_q = rng.normal(size=(T, G, D))
    idx_k = rng.normal(size=(L, D))
    q = rng.normal(size=(T, H, D))
    K = rng.normal(size=(G, L, D))
    V = rng.normal(size=(G, L, D))
    r = M.layer_step(idx_q, idx_k, q, K, V, L, T, SCALE)
    for g in range(G):
        mask = np.zeros((T, L), dtype=bool)
        for t in range(T):
            p = L - T + t
            for i in r["sel"][t, g]:
                if i >= 0:
                    mask[t, i * 128:(i + 1) * 128] = True
            mask[t, p + 1:] = False
        o, lse = sdpa_masked(q[:, g * 16:(g + 1) * 16], K[g:g + 1], V[g:g + 1], mask)
        assert np.abs(r["out"][:, g * 16:(g + 1) * 16] - o).max() < 1e-12
        assert np.abs(r["lse"][:, g * 16:(g + 1) * 16] - lse).max() < 1e-12
        assert mask.sum(axis=1).max() <= 2048


def test_closed_forms_zero_query_and_single_key():
    rng = np.random.default_rng(12)
    G, H, D, L, T = 4, 64, 128, 128 * 20 + 3, 1
    idx_q = rng.normal(size=(T, G, D))
    idx_k = rng.normal(size=(L, D))
    K = rng.normal(size=(G, L, D))
    V = rng.normal(size=(G, L, D))
    r = M.layer_step(idx_q, idx_k, np.zeros((T, H, D)), K, V, L, T, SCALE)
    for g in range(G):
        keys = M.attended_keys(r["sel"][0, g], L - 1)
        assert np.abs(r["out"][0, g * 16] - V[g, keys].mean(axis=0)).max() < 1e-12
        assert r["lse"][0, g * 16] == pytest.approx(np.log(len(keys)), abs=1e-12)
    r1 = M.layer_step(idx_q, idx_k[:1], rng.normal(size=(1, H, D)), K[:, :1], V[:, :1], 1, 1, SCALE)
    for h in range(H):
        assert np.array_equal(r1["out"][0, h], V[h // 16, 0])


def test_paged_batch_is_invariant_to_page_order_and_matches_layer_step():
    rng = np.random.default_rng(13)
    G, H, D = 4, 64, 128
    lens = [128 * 21 + 9, 128 * 5, 700]
    T = 2
    nbs = [(L + 127) // 128 for L in lens]
    P = sum(nbs)
    maxb = max(nbs)
    pools = {w: rng.normal(size=(P, h, 128, D)).astype(np.float32) for w, h in [("i", 1), ("k", 4), ("v", 4)]}
    idx_q = rng.normal(size=(3, T, G, D)).astype(np.float32)
    q = rng.normal(size=(3, T, H, D)).astype(np.float32)
    results = []
    for order in [np.arange(P), rng.permutation(P)]:
        table = np.full((3, maxb), -1, np.int32)
        off = 0
        for b, n in enumerate(nbs):
            table[b, :n] = order[off:off + n]
            off += n
        inv = np.argsort(order)                     # logical slot -> which original page
        caches = {w: {"dtype": "f32", "data": pools[w][inv], "tensor_scale": 1.0} for w in pools}
        results.append(M.batch_layer(idx_q, q, caches["i"], caches["k"], caches["v"], np.array(lens),
                                     table, T, SCALE))
    for key in ["block_scores", "sel", "out", "lse"]:
        a, b = results
        assert np.array_equal(np.nan_to_num(a[key[:]], nan=7.0), np.nan_to_num(b[key], nan=7.0)), key
    # and each sequence equals the unpaged layer step
    off = 0
    for b, L in enumerate(lens):
        n = nbs[b]
        ik = pools["i"][off:off + n, 0].reshape(-1, D)[:L]
        K = pools["k"][off:off + n].transpose(1, 0, 2, 3).reshape(4, -1, D)[:, :L]
        V = pools["v"][off:off + n].transpose(1, 0, 2, 3).reshape(4, -1, D)[:, :L]
        ref = M.layer_step(idx_q[b], ik, q[b], K, V, L, T, SCALE)
        assert np.array_equal(results[0]["sel"][b], ref["sel"])
        assert np.abs(results[0]["out"][b] - ref["out"]).max() < 1e-12
        bs = results[0]["block_scores"][b]
        assert np.array_equal(bs[:, :, :n], ref["block_scores"])
        assert np.all(bs[:, :, n:] == -np.inf)
        off += n


def test_selection_boundary_tie_goes_to_lower_block():
    # 19 older blocks: 14 clear winners, four blocks tied for the last slot,
    # one loser; the lowest-numbered tied block must win the slot
    own = 19
    tied = [3, 7, 11, 16]
    S = np.full(20, 0.1)
    winners = [i for i in range(own) if i not in tied][:14]
    S[winners] = np.linspace(9.0, 2.0, 14)
    S[tied] = 0.5
    sel = [int(i) for i in M.select_blocks(S, own) if i >= 0]
    assert sel == brute_select(S, own) == sorted(winners + [3, own])


def test_chunked_pooling_equals_unchunked():
    rng = np.random.default_rng(21)
    L, T = 128 * 9 + 17, 300
    q = rng.normal(size=(T, 4, 16))
    k = rng.normal(size=(L, 16))
    full = M.block_max_pool(M.indexer_token_scores(q, k, L, T), L)
    for chunk in (1, 7, 128, 1000):
        got = M.pooled_scores(q, k, L, T, chunk=chunk)
        assert np.array_equal(np.isneginf(got), np.isneginf(full))
        fin = np.isfinite(full)
        assert np.abs(got[fin] - full[fin]).max() < 1e-12


def _insert_pool(dtype, P, heads, rng):
    """A page pool filled with arbitrary (valid) bytes, and its tensor scale."""
    S = 0.25
    if dtype == "f32":
        return {"dtype": "f32", "data": rng.normal(size=(P, heads, 128, 128)).astype(np.float32), "tensor_scale": 1.0}
    if dtype == "fp8":
        data = rng.integers(0, 256, size=(P, heads, 128, 128), dtype=np.uint8)
        data[(data & 0x7F) == 0x7F] = 0          # no NaN bytes
        return {"dtype": "fp8", "data": data, "tensor_scale": S}
    return {"dtype": "nvfp4", "data": rng.integers(0, 256, size=(P, heads, 128, 64), dtype=np.uint8),
            "scales": rng.integers(0, 0x7F, size=(P, heads, 128, 8), dtype=np.uint8), "tensor_scale": S}


@pytest.mark.parametrize("dtype", ["f32", "fp8", "nvfp4"])
def test_insert_then_read_back_equals_quantised_rows(dtype):
    """Inserting a whole sequence and reading it back through the (separately pinned)
    paged reader gives the rows quantised and decoded in one piece, in logical order."""
    rng = np.random.default_rng(21)
    heads, L = 4, 128 * 3 + 17
    nb = (L + 127) // 128
    P = nb + 3
    table = np.array([rng.permutation(P)[:nb]], np.int32)
    pool = _insert_pool(dtype, P, heads, rng)
    x = (3.0 * rng.normal(size=(1, L, heads, 128))).astype(np.float32)
    got = M.sequence_view(M.cache_insert(pool, x, [L], table, L), table[0], L)
    rows = x[0].transpose(1, 0, 2)                      # [heads, L, 128]
    S = pool["tensor_scale"]
    if dtype == "f32":
        ref = rows.astype(np.float64)
    elif dtype == "fp8":
        ref = F.fp8_dequantize(F.fp8_quantize(rows, S), S)
    else:
        c, sc = F.nvfp4_quantize(rows, S)
        ref = F.nvfp4_dequantize(c, sc, S)
    assert np.array_equal(got, ref)


def test_insert_in_steps_equals_insert_at_once_and_touches_nothing_else():
    """Growing a sequence token by token (decode) or a chunk at a time (prefill) gives
    the same pool as one insert; pages of other sequences and free slots stay as they
    were; a row whose page id is outside the pool is skipped."""
    rng = np.random.default_rng(22)
    heads, L = 1, 300
    nb = (L + 127) // 128
    P = 6
    table = np.array([[4, 1, 3]], np.int32)
    pool = _insert_pool("nvfp4", P, heads, rng)
    x = rng.normal(size=(1, L, heads, 128)).astype(np.float32)
    once = M.cache_insert(pool, x, [L], table, L)
    step = pool
    for n in [1, 2, 130, 290, 299, 300]:
        prev = step
        T = n - (0 if prev is pool else last)
        step = M.cache_insert(prev, x[:, n - T:n], [n], table, T)
        last = n
    for k in ("data", "scales"):
        assert np.array_equal(step[k], once[k])
        untouched = np.ones(P, bool)
        untouched[table[0]] = False
        assert np.array_equal(once[k][untouched], pool[k][untouched])
        # slots past the sequence in its last page
        assert np.array_equal(once[k][3, :, L - 256:], pool[k][3, :, L - 256:])
    bad = M.cache_insert(pool, x[:, :5], [5], np.array([[P + 2, 0, 0]], np.int32), 5)
    assert all(np.array_equal(bad[k], pool[k]) for k in ("data", "scales"))


# ---------------------------------------------------------------- DCP selection


def test_shards_partition_the_blocks():
    for n in (0, 1, 7, 16, 1000):
        for P in (1, 2, 3, 4, 8):
            parts = [M.shard_blocks(n, s, P) for s in range(P)]
            assert np.array_equal(np.sort(np.concatenate(parts)), np.arange(n))
            sizes = [len(p) for p in parts]
            assert max(sizes) - min(sizes) <= 1


def test_shard_candidates_and_merge_worked_example():
    # Blocks 0..9, own block 9, two shards (even / odd blocks), 4 kept (k = 4).
    # Shard 0 holds blocks 0,2,4,6,8 with scores 5,5,2,0,5: best first by
    # (score desc, block asc) that is 0,2,8,4.  Shard 1 holds 1,3,5,7 with
    # scores 1,3,3,4: 7,3,5,1.  The owner keeps block 9 and the 3 best of the
    # union -- blocks 0, 2 and 8 (score 5) -- and reports 0,2,8,9.
    S = np.array([5, 1, 5, 3, 2, 3, 0, 4, 5, 9], dtype=float)
    s0, b0 = M.shard_candidates(S, 9, 0, 2, k=4)
    s1, b1 = M.shard_candidates(S, 9, 1, 2, k=4)
    assert b0.tolist() == [0, 2, 8, 4] and s0.tolist() == [5, 5, 5, 2]
    assert b1.tolist() == [7, 3, 5, 1] and s1.tolist() == [4, 3, 3, 1]
    sel = M.merge_candidates(np.stack([s0, s1]), np.stack([b0, b1]), 9, k=4)
    assert sel.tolist() == [0, 2, 8, 9]
    assert np.array_equal(sel, M.select_blocks(S, 9, k=4))


def test_shard_candidates_brute_force():
    rng = np.random.default_rng(5)
    for _ in range(300):
        P = int(rng.integers(1, 5))
        shard = int(rng.integers(0, P))
        own = int(rng.integers(0, 60))
        S = rng.integers(0, 4, own + 1).astype(float)
        ranked = sorted((-S[i], i) for i in range(shard, own, P))[:16]
        sc, ids = M.shard_candidates(S, own, shard, P)
        n = len(ranked)
        assert ids[:n].tolist() == [i for _, i in ranked] and np.all(ids[n:] == -1)
        assert sc[:n].tolist() == [-v for v, _ in ranked] and np.all(np.isnan(sc[n:]))


def _dcp_route(S, own, P):
    parts = [M.shard_candidates(S, own, s, P) for s in range(P)]
    return M.merge_candidates(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]), own)


def test_dcp_merge_equals_single_gpu_selection():
    """The pages' claim: merging the shards' local top-16s selects exactly what
    one GPU selects from all the scores -- here against select_blocks."""
    rng = np.random.default_rng(11)
    for P in (1, 2, 3, 4, 5, 8):
        for trial in range(120):
            own = int(rng.integers(0, 400))
            S = rng.integers(0, 6, own + 1).astype(float) if trial % 2 else rng.normal(size=own + 1)
            assert np.array_equal(_dcp_route(S, own, P), M.select_blocks(S, own)), (P, trial)
        # every one of the 15 best older blocks on one shard, the own block scoring highest
        own = 300
        S = rng.normal(size=own + 1)
        S[0:own:P] += 100.0
        S[own] = 1e3
        assert np.array_equal(_dcp_route(S, own, P), M.select_blocks(S, own)), P


def test_dcp_select_all_equals_select_all():
    rng = np.random.default_rng(12)
    L, T = 40 * 128 + 17, 4
    S = rng.integers(0, 8, (T, 4, M.num_blocks(L))).astype(float)
    for P in (2, 4):
        assert np.array_equal(M.dcp_select_all(S, L, T, P), M.select_all(S, L, T))


def test_tensor_scales_enter_where_their_tensors_do():
    """How the four per-tensor scales act on the layer step, from the definition of a
    decoded value (scale times stored element) and of softmax attention:
    * the index-query and index-key scales multiply every block score, so a power-of-
      two scale multiplies the scores exactly and never changes the selection;
    * the V scale multiplies the attention output and leaves the LSE alone;
    * the query and K scales multiply the logits together: only their product counts,
      and the LSE of logits c*l is the LSE of the logits computed with c folded in.
    FP8 caches, K and V on different scales."""
    rng = np.random.default_rng(31)
    lens, T = [2600, 700], 2
    B = len(lens)
    nbs = [(L + 127) // 128 for L in lens]
    P = sum(nbs)
    table = np.full((B, max(nbs)), -1, np.int32)
    perm = rng.permutation(P)
    table[0, :nbs[0]], table[1, :nbs[1]] = perm[:nbs[0]], perm[nbs[0]:]
    idx_q = F.fp8_quantize(rng.normal(0, 1, (B, T, 4, 128)), 1.0)
    q = F.fp8_quantize(rng.normal(0, 1, (B, T, 64, 128)), 1.0)

    def cache(heads, S, seed):
        x = np.random.default_rng(seed).normal(0, 1, (P, heads, 128, 128)).astype(np.float32)
        return {"dtype": "fp8", "data": F.fp8_quantize(x, 1.0), "tensor_scale": S}

    def run(iqs, ks, qs, kS, vS):
        return M.batch_layer(idx_q, q, cache(1, ks, 1), cache(4, kS, 2), cache(4, vS, 3), lens, table, T,
                             1 / np.sqrt(128), idx_q_dtype="fp8", idx_q_scale=iqs, q_dtype="fp8", q_scale=qs)

    base = run(1.0, 1.0, 1.0, 1.0, 1.0)
    r = run(2.0, 0.5 * 8, 0.75, 0.4, 3.0)        # index scales multiply to 8, a power of two
    fin = np.isfinite(base["block_scores"])
    assert np.array_equal(np.isfinite(r["block_scores"]), fin)
    assert np.array_equal(r["block_scores"][fin], 8.0 * base["block_scores"][fin])
    assert np.array_equal(r["sel"], base["sel"])
    # only q_scale * k_scale matters for the logits; V's scale multiplies the output
    a = run(1.0, 1.0, 0.75, 0.4, 1.0)
    b = run(1.0, 1.0, 0.3, 1.0, 3.0)
    assert np.allclose(3.0 * a["out"], b["out"], rtol=1e-12, atol=1e-12)
    assert np.allclose(a["lse"], b["lse"], rtol=1e-12, atol=1e-12)
    assert not np.allclose(a["out"], base["out"], atol=1e-3)      # the logit scale does act
    # shrinking the logits to zero leaves the mean of V over the attended keys
    z = run(1.0, 1.0, 1e-30, 1.0, 1.0)
    for bb, L in enumerate(lens):
        V = M.sequence_view(cache(4, 1.0, 3), table[bb], L)
        for t in range(T):
            p = L - T + t
            for h in (0, 37):
                keys = M.attended_keys(z["sel"][bb, t, h // 16], p)
                assert np.allclose(z["out"][bb, t, h], V[h // 16, keys].mean(axis=0), atol=1e-12)
