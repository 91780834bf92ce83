"""Planted mistakes in the oracle (on the CPU) must be caught by its pins.

Each case swaps one oracle function for a plausibly wrong variant and checks
that the pin meant to guard it fails."""
import numpy as np
import pytest

import oracle.msa as M
import oracle.formats as F
from tests import test_oracle_msa as TM
from tests import test_oracle_formats as TF


def _select_ties_to_higher_index(S, own, k=16):
    S = np.asarray(S, float)
    if own + 1 <= k:
        return np.array(list(range(own + 1)) + [-1] * (k - own - 1), np.int32)
    cand = np.arange(own)
    order = np.lexsort((-cand, -S[:own]))
    ch = sorted([int(i) for i in cand[order[: k - 1]]] + [own])
    return np.array(ch + [-1] * (k - len(ch)), np.int32)


def _select_without_forcing_own(S, own, k=16):
    S = np.asarray(S, float)
    cand = np.arange(own + 1)
    order = np.lexsort((cand, -S[:own + 1]))
    ch = sorted(int(i) for i in cand[order[:k]])
    return np.array(ch + [-1] * (k - len(ch)), np.int32)


def _attended_keys_ignoring_causality(sel_row, p):
    return np.concatenate([np.arange(i * 128, i * 128 + 128) for i in sel_row if i >= 0]).astype(np.int64)


def _e4m3_ties_away(x):
    x = np.asarray(x, float)
    pos = F._E4M3_POS
    a = np.abs(x)
    idx = np.array([int(np.argmin(np.abs(pos - v) - 1e-300 * np.arange(len(pos)))) for v in np.minimum(a, 448.0)])
    return (idx | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)


def _sparse_attention_wrong_gqa(q, K, V, sel, L, T, scale):
    # heads assigned round-robin instead of contiguously
    q = np.asarray(q, float)
    qq = q.reshape(q.shape[0], 16, 4, q.shape[2]).transpose(0, 2, 1, 3).reshape(q.shape)
    return _orig_attention(qq, K, V, sel, L, T, scale)


_orig_attention = M.sparse_attention
_orig_insert = M.cache_insert


def _insert_one_token_late(cache, x, seq_lens, block_table, T):
    # the new tokens placed one position too far
    return _orig_insert(cache, x, [int(L) + 1 for L in seq_lens], block_table, T)


def _insert_one_scale_per_row(cache, x, seq_lens, block_table, T):
    # NVFP4 with one scale byte for the whole 128-dim row instead of one per 16 dims
    if cache["dtype"] != "nvfp4":
        return _orig_insert(cache, x, seq_lens, block_table, T)
    out = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in cache.items()}
    S = np.float32(cache["tensor_scale"])
    x = np.asarray(x, np.float32)
    for b in range(len(seq_lens)):
        for t in range(T):
            p = int(seq_lens[b]) - T + t
            page, r = int(block_table[b][p // 128]), p % 128
            for h in range(x.shape[2]):
                row = x[b, t, h]
                sb = F.e4m3_encode(np.float64(np.abs(row).max() / (np.float32(6.0) * S)))
                denom = np.float32(F.e4m3_value(sb)) * S
                codes = F.e2m1_encode((row / denom).astype(np.float64)) if denom > 0 else np.zeros(128, np.int64)
                out["data"][page, h, r] = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
                out["scales"][page, h, r] = sb
    return out


_orig_decode_query = M.decode_query


def _fp8_dequantize_dividing(b, tensor_scale):
    # mirrors the quantiser's division instead of undoing it
    return F.e4m3_value(b) / float(tensor_scale)


def _decode_query_ignoring_scale(qarr, dtype, scale):
    return _orig_decode_query(qarr, dtype, 1.0)


def _decode_pages_without_fp8_scale(cache, pages, mode="exact"):
    # FP8 pages read without their tensor scale
    c = dict(cache)
    if c["dtype"] == "fp8":
        c["tensor_scale"] = 1.0
    return _orig_decode_pages(c, pages, mode)


_orig_decode_pages = M.decode_pages
_orig_shard_candidates = M.shard_candidates
_orig_merge = M.merge_candidates


def _shard_sends_top8(S, own, shard, P, k=16):
    sc, ids = _orig_shard_candidates(S, own, shard, P, k)
    sc[8:], ids[8:] = np.nan, -1
    return sc, ids


def _shard_includes_own_block(S, own, shard, P, k=16):
    S = np.asarray(S, float)
    blocks = np.arange(shard, own + 1, P)
    order = np.lexsort((blocks, -S[blocks]))[:k]
    sc, ids = np.full(k, np.nan), np.full(k, -1, np.int32)
    sc[: len(order)], ids[: len(order)] = S[blocks][order], blocks[order]
    return sc, ids


def _merge_ties_to_higher_block(cs, cb, own, k=16):
    if own + 1 <= k:
        return _orig_merge(cs, cb, own, k)
    ids, sc = np.asarray(cb).ravel(), np.asarray(cs, float).ravel()
    keep = ids >= 0
    ids, sc = ids[keep], sc[keep]
    order = np.lexsort((-ids, -sc))[: k - 1]
    ch = sorted([int(i) for i in ids[order]] + [own])
    return np.array(ch + [-1] * (k - len(ch)), np.int32)


@pytest.mark.parametrize("target,mutant,pin", [
    (M, ("select_blocks", _select_ties_to_higher_index), TM.test_selection_boundary_tie_goes_to_lower_block),
    (M, ("select_blocks", _select_without_forcing_own), TM.test_selection_invariants_random_rows),
    (M, ("attended_keys", _attended_keys_ignoring_causality), lambda: TM.test_short_context_equals_dense_causal_attention(2048, 4)),
    (M, ("sparse_attention", _sparse_attention_wrong_gqa), TM.test_sparse_attention_equals_masked_sdpa_from_selection),
    (F, ("e4m3_encode", _e4m3_ties_away), TF.test_e4m3_encode_matches_torch_rne_in_range),
    (M, ("cache_insert", _insert_one_token_late), lambda: TM.test_insert_then_read_back_equals_quantised_rows("fp8")),
    (M, ("cache_insert", _insert_one_scale_per_row), lambda: TM.test_insert_then_read_back_equals_quantised_rows("nvfp4")),
    (M, ("shard_candidates", _shard_sends_top8), TM.test_dcp_merge_equals_single_gpu_selection),
    (M, ("shard_candidates", _shard_includes_own_block), TM.test_dcp_merge_equals_single_gpu_selection),
    (M, ("merge_candidates", _merge_ties_to_higher_block), TM.test_dcp_merge_equals_single_gpu_selection),
    (F, ("fp8_dequantize", _fp8_dequantize_dividing), lambda: TF.test_fp8_tensor_scale_round_trip_bound(0.37)),
    (F, ("fp8_dequantize", _fp8_dequantize_dividing), lambda: TF.test_decode_query_applies_its_scale(4.0)),
    (M, ("decode_query", _decode_query_ignoring_scale), lambda: TF.test_decode_query_applies_its_scale(4.0)),
    (M, ("decode_query", _decode_query_ignoring_scale), TM.test_tensor_scales_enter_where_their_tensors_do),
    (M, ("decode_pages", _decode_pages_without_fp8_scale), TM.test_tensor_scales_enter_where_their_tensors_do),
])
def test_planted_mistake_is_caught(monkeypatch, target, mutant, pin):
    name, fn = mutant
    monkeypatch.setattr(target, name, fn)
    with pytest.raises(AssertionError):
        pin()
