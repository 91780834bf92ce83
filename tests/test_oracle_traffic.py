"""Pins of the bytes model against the numbers the source pages print
(tests/golden/page_facts.json)."""
import json
import os

import pytest

from oracle import traffic as TR

GOLD = {k: v["value"] for k, v in json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json"))).items()
        if isinstance(v, dict)}


def test_per_token_bytes_fp8():
    assert TR.index_key_bytes_per_token("fp8") == GOLD["index_key_bytes_fp8"]
    assert TR.kv_bytes_per_token("fp8", GOLD["kv_heads"]) == GOLD["kv_bytes_fp8"]
    assert TR.index_key_bytes_per_token("fp8") / TR.kv_bytes_per_token("fp8") == GOLD["index_to_kv_fraction"]


@pytest.mark.parametrize("dtype", ["fp8", "nvfp4", "f32"])
def test_long_context_traffic_tends_to_an_eighth(dtype):
    # closed form: 1/8 + 2048 / L for L >= 2048, for every storage format
    for L in [4096, 32768, 131072, 1 << 20]:
        assert TR.sparse_to_dense_ratio(L, dtype) == pytest.approx(0.125 + 2048 / L, rel=1e-12)
    assert TR.sparse_to_dense_ratio(1 << 30, dtype) == pytest.approx(GOLD["long_context_traffic"], abs=1e-5)
    assert TR.sparse_to_dense_ratio(4096, "f32") == pytest.approx(0.625)


def test_nvfp4_is_four_and_a_half_bits():
    ratio = TR.kv_bytes_per_token("nvfp4") / TR.kv_bytes_per_token("fp8")
    assert ratio == GOLD["model_bytes_nvfp4"] / GOLD["model_bytes_fp8"]
    assert 1 - ratio == GOLD["nvfp4_saving"]
    assert TR.ROW_BYTES["nvfp4"] * 8 / 128 == 4.5


def test_dense_is_never_cheaper_past_2048():
    for L in [2049, 5000, 10 ** 6]:
        assert TR.sparse_decode_bytes(L, "fp8") < TR.dense_decode_bytes(L, "fp8") * (0.125 + 2048 / L + 1e-12)


def test_bench_bytes_model_matches_the_oracle_model():
    """bench.py restates the algorithmic bytes model (it may not import the oracle);
    both must give the same figures for the same selection."""
    import types
    import numpy as np
    import bench
    from oracle import traffic as TR
    rng = np.random.default_rng(4)
    for kv, qd, T in (("nvfp4", "fp8", 1), ("fp8", "fp8", 4), ("f32", "f32", 1)):
        lens = [1000, 3001, 129]
        maxb = 24
        B = len(lens)
        sel = np.full((B, T, 4, 16), -1, np.int32)
        for b, L in enumerate(lens):
            nb = (L + 127) // 128
            for t in range(T):
                for g in range(4):
                    k = min(16, nb)
                    sel[b, t, g, :k] = np.sort(rng.choice(nb, k, replace=False))
        w = types.SimpleNamespace(B=B, T=T, kv_dtype=kv, q_dtype=qd)
        lay = types.SimpleNamespace(seq_lens=np.array(lens), max_blocks=maxb)
        wl = types.SimpleNamespace(w=w, lay=lay)
        idx, topk, attn = bench.algorithmic_bytes(wl, sel)
        assert idx == TR.indexer_bytes(lens, T, kv, qd, 4, maxb)
        assert topk == TR.topk_bytes(B, T, 4, maxb)
        keys = sum(min(128, lens[b] - 128 * i) for b in range(B) for g in range(4)
                   for i in set(int(x) for x in sel[b, :, g].reshape(-1) if x >= 0))
        assert attn == TR.attention_bytes(keys, kv, qd, B, T, 64)


def test_flop_model_counts_the_oracles_products():
    """indexer_flops and attention_flops, and bench.py's restatement of them, against
    the products the oracle forms on a small seeded case: 2*128 flops per finite
    per-key index score (one 128-dim dot product each), and 2*(2*128) per (query
    head, attended key) -- one QK dot product and one PV accumulation."""
    import types
    import numpy as np
    import bench
    from oracle import msa as OM
    rng = np.random.default_rng(5)
    lens, T = [700, 3000, 2049], 3
    idx_pairs = attn_pairs = 0
    sels = []
    for L in lens:
        iq = rng.normal(0, 1, (T, 4, 128))
        ik = rng.normal(0, 1, (L, 128))
        s = OM.indexer_token_scores(iq, ik, L, T)
        idx_pairs += int(np.isfinite(s).sum()) // 4           # (token, key) pairs, per group
        sel = OM.select_all(OM.block_max_pool(s, L), L, T)
        sels.append(sel)
        p = OM.positions(L, T)
        for t in range(T):
            for g in range(4):
                attn_pairs += 16 * len(OM.attended_keys(sel[t, g], int(p[t])))
    w = types.SimpleNamespace(B=len(lens), T=T, kv_dtype="fp8", q_dtype="fp8")
    lay = types.SimpleNamespace(seq_lens=np.array(lens), max_blocks=24)
    f_idx, f_attn = bench.algorithmic_flops(types.SimpleNamespace(w=w, lay=lay), np.stack(sels))
    assert f_idx == TR.indexer_flops(idx_pairs, 4) == 2 * 128 * 4 * idx_pairs
    assert f_attn == TR.attention_flops(attn_pairs) == 4 * 128 * attn_pairs
