"""HIP path against the CPU fp64 oracle, through the C ABI.

Bars: pack/unpack bit-exact; block scores within 1e-5 relative (1 + |s|);
selected block ids bit-exact except rows the oracle flags as near-ties
(16th/17th scores within 1e-5 relative), which must still be a valid top-16;
attention within max-abs 2e-3 and mean-abs 2e-4 of the oracle run on the
GPU's selection; LSE within 1e-4."""
import os

import numpy as np
import pytest
import torch

import synth
from oracle import formats as OF
from oracle import msa as OM
from tests import harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import block_sparse_attention_indexer_amd as M
    assert os.path.exists(M.LIB_PATH), "libmsa.so must be built before the GPU tests"
    return M


def _say(*a):
    print("[gpu-test]", *a, flush=True)


# ------------------------------------------------------------------ pack / unpack

def _edge_values(rng):
    pos = OF.e4m3_value(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2
    return np.concatenate([rng.normal(0, 1, 60000), rng.normal(0, 100, 20000), mids, -mids, pos, -pos,
                           [0.0, -0.0, 448.0, 460.0, 470.0, 1e5, -1e5, 2.0 ** -10, 3 * 2.0 ** -11]]).astype(np.float32)


@pytest.mark.parametrize("scale", [1.0, float(np.float32(0.37)), float(np.float32(32.0 / 448.0))])
def test_pack_fp8_bit_exact(M, scale):
    x = _edge_values(np.random.default_rng(1))
    x = x[: (len(x) // 4) * 4]
    d = torch.from_numpy(x).cuda()
    out = torch.empty(len(x), dtype=torch.uint8, device="cuda")
    M.msa_pack_fp8(d, scale, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), OF.fp8_quantize(x, scale))


@pytest.mark.parametrize("S", [float(np.float32(32.0 / 448.0)), 1.0, float(np.float32(0.0123)), 5.0])
def test_pack_nvfp4_bit_exact(M, S):
    rng = np.random.default_rng(2)
    x = rng.normal(0, 1, (2048, 128)).astype(np.float32)
    x[rng.random(x.shape) < 0.05] *= 4.0
    x[5, 16:32] = 0.0                      # an all-zero group
    x[6] = _edge_values(rng)[:128]
    x[7, :16] = np.float32(1e-7)           # scale underflows to zero
    d = torch.from_numpy(x).cuda()
    codes = torch.empty((2048, 64), dtype=torch.uint8, device="cuda")
    sc = torch.empty((2048, 8), dtype=torch.uint8, device="cuda")
    M.msa_pack_nvfp4(d, S, codes, sc)
    torch.cuda.synchronize()
    oc, os_ = OF.nvfp4_quantize(x, S)
    assert np.array_equal(sc.cpu().numpy(), os_)
    assert np.array_equal(codes.cpu().numpy(), oc)


def _tie_sweep(lo_exp, hi_exp):
    """Every float32 of both signs with biased exponent in [lo_exp, hi_exp], any of the
    top 11 mantissa bits and the low 12 bits in {0, 1, 0x7FF, 0x800, 0x801, 0xFFF}: all
    the E4M3 and E2M1 rounding ties of that range and their float neighbours."""
    e = np.arange(lo_exp, hi_exp + 1, dtype=np.uint32)
    top = np.arange(2048, dtype=np.uint32) << 12
    low = np.array([0, 1, 0x7FF, 0x800, 0x801, 0xFFF], dtype=np.uint32)
    bits = ((e[:, None, None] << 23) | top[None, :, None] | low[None, None, :]).ravel()
    bits = np.concatenate([bits, bits | np.uint32(0x80000000), np.array([0, 0x80000000], dtype=np.uint32)])
    return bits.view(np.float32)


def test_pack_fp8_rounding_ties(M):
    """Magnitudes 2^-27 .. 2^14 (past the saturation point) at and beside every tie."""
    x = _tie_sweep(100, 141)
    d = torch.from_numpy(x).cuda()
    out = torch.empty(len(x), dtype=torch.uint8, device="cuda")
    M.msa_pack_fp8(d, 1.0, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), OF.fp8_quantize(x, 1.0))


def test_pack_nvfp4_rounding_ties(M):
    """Groups whose largest magnitude is 6 * 2^k (scale byte exactly 2^k) around values
    at and beside every E2M1 tie, and groups whose scale rounds down (codes saturate)."""
    v = _tie_sweep(100, 129)
    v = v[np.abs(v) < 6.0]
    groups = []
    for k in (-3, 0, 4):
        f = np.float32(2.0 ** k)
        body = v * f
        body = np.concatenate([body, np.zeros((-len(body)) % 15, dtype=np.float32)]).reshape(-1, 15)
        groups.append(np.concatenate([np.full((len(body), 1), 6 * f, dtype=np.float32), body], axis=1))
        sat = np.array([6.375, 6.2, -6.375, 6.0, 5.9, -6.1, 0.25, -0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0, 0.0, -0.0],
                       dtype=np.float32) * f                 # amax/6 = 1.0625: the scale rounds down to 1
        groups.append(sat[None, :])
    g = np.concatenate(groups)
    g = np.concatenate([g, np.zeros(((-len(g)) % 8, 16), dtype=np.float32)])
    x = np.ascontiguousarray(g.reshape(-1, 128))
    d = torch.from_numpy(x).cuda()
    codes = torch.empty((len(x), 64), dtype=torch.uint8, device="cuda")
    sc = torch.empty((len(x), 8), dtype=torch.uint8, device="cuda")
    M.msa_pack_nvfp4(d, 1.0, codes, sc)
    torch.cuda.synchronize()
    oc, os_ = OF.nvfp4_quantize(x, 1.0)
    assert np.array_equal(sc.cpu().numpy(), os_)
    assert np.array_equal(codes.cpu().numpy(), oc)


@pytest.mark.parametrize("mode", ["exact", "fp8"])
def test_unpack_nvfp4_every_scale_and_code(M, mode):
    scales = np.array([s for s in range(256) if not (s & 0x80) and s != 0x7F], dtype=np.uint8)
    codes16 = np.arange(16, dtype=np.uint8)
    row = (codes16[0::2] | (codes16[1::2] << 4)).astype(np.uint8)       # 16 codes
    codes = np.tile(row, (len(scales), 1))                               # [n, 8] -> 16 elements per row
    sb = scales[:, None].copy()
    for S in [1.0, float(np.float32(32.0 / 448.0))]:
        out = torch.empty((len(scales), 16), dtype=torch.float32, device="cuda")
        M.msa_unpack_nvfp4(torch.from_numpy(codes).cuda(), torch.from_numpy(sb).cuda(), 16, S, mode, out)
        torch.cuda.synchronize()
        ref = OF.nvfp4_dequantize(codes, sb, S, OF.EXACT if mode == "exact" else OF.FP8_ROUNDED)
        assert np.array_equal(out.cpu().numpy(), ref.astype(np.float32))


def test_unpack_fp8_every_code(M):
    b = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    for S in [1.0, float(np.float32(0.37))]:
        out = torch.empty(len(b), dtype=torch.float32, device="cuda")
        M.msa_unpack_fp8(torch.from_numpy(b).cuda(), S, out)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), OF.fp8_dequantize(b, S).astype(np.float32))


# ------------------------------------------------------------------ small cases, full comparison

SMALL = [("c1", "exact"), ("tiny_f32", "exact"), ("tiny_fp8", "exact"), ("tiny_nvfp4", "exact"),
         ("tiny_nvfp4", "fp8"), ("tiny_spec", "exact"), ("tiny_spec", "fp8"),
         ("tiny_prefill", "exact"), ("tiny_prefill", "fp8"), ("tiny_prefill_fp8", "exact"),
         ("tiny_prefill_many", "exact"), ("tiny_t2", "exact"), ("tiny_t2", "fp8"), ("tiny_t3", "exact"),
         ("tiny_edge", "exact"), ("tiny_prefill_nocache", "exact"), ("long_rows", "exact"),
         # 7 speculative tokens (T = 8) and T = 6: the two-row-tile speculative scan and the decode attention
         ("tiny_spec8", "exact"), ("tiny_spec8", "fp8"), ("tiny_t6", "exact"),
         # first token's position at the speculative scan's unit edges (T = 4 NVFP4, T = 8 FP8)
         ("spec_edges", "exact"), ("spec_edges", "fp8"), ("spec_edges8", "exact")]
SMALL = [(w, m, False) for w, m in SMALL]
# per-tensor scales other than 1 (index query, query, index keys, K and V all different)
SMALL += [(w, m, True) for w, m in [
    ("c1", "exact"), ("tiny_f32", "exact"), ("tiny_fp8", "exact"), ("tiny_nvfp4", "exact"), ("tiny_nvfp4", "fp8"),
    ("tiny_spec", "exact"), ("tiny_spec", "fp8"), ("tiny_spec8", "fp8"), ("tiny_t3", "exact"),
    ("tiny_prefill", "exact"), ("tiny_prefill", "fp8"), ("tiny_prefill_fp8", "exact"),
    ("tiny_prefill_many", "fp8")]]


@pytest.mark.parametrize("wname,mode,scaled", SMALL)
def test_layer_parity_small(M, wname, mode, scaled):
    _say("small case", wname, mode, "scaled" if scaled else "unit scales")
    case = H.HostCase(wname, scaled=scaled).upload()
    w, lay = case.w, case.lay
    res = H.to_host(H.run_path(case, mode, token_scores=True))
    seq_lens, table = lay.seq_lens.numpy(), lay.block_table.numpy()
    ora = H.oracle_scores(case.caches, case.idx_q, seq_lens, table, w.T, mode, w.q_dtype,
                          idx_q_scale=case.idx_q_scale)
    H.compare_scores(res["block_scores"], ora["block_scores"])
    # per-key scores
    for b in range(w.B):
        L = int(seq_lens[b])
        iq = OM.decode_query(case.idx_q[b], w.q_dtype, case.idx_q_scale)
        ik = OM.sequence_view(case.caches["idx_k"], table[b], L, mode)[0]
        s = OM.indexer_token_scores(iq, ik, L, w.T)
        full = np.full((w.T, 4, lay.max_blocks * 128), -np.inf)
        full[:, :, :L] = s
        H.compare_scores(res["token_scores"][b], full)
    nties = H.compare_selection(res["sel"], ora["sel"], ora["block_scores"], ora["near_tie"], seq_lens, w.T)
    for b in range(w.B):
        o, lse = H.oracle_attention(case.caches, case.q, seq_lens, table, w.T, res["sel"][b], mode, w.q_dtype, b,
                                    q_scale=case.q_scale)
        H.compare_out(res["out"][b], o)
        assert np.abs(res["lse"][b] - lse).max() <= 1e-4
    _say(wname, mode, "ok; near-tie rows that differ:", nties)


def test_deterministic_and_page_order_invariant(M):
    case = H.HostCase("tiny_nvfp4").upload()
    r1 = H.to_host(H.run_path(case, "exact"))
    r2 = H.to_host(H.run_path(case, "exact"))
    for k in ("block_scores", "sel", "out", "lse"):
        assert np.array_equal(r1[k], r2[k]), k
    # permute the physical pages and the table consistently
    P = case.lay.num_pages
    perm = np.random.default_rng(9).permutation(P)            # new page id of old page p: perm[p]
    inv = np.argsort(perm)
    for name, (data, scales, _) in list(case.d_caches.items()):
        nd = data[torch.from_numpy(inv).cuda()].contiguous()
        ns = scales[torch.from_numpy(inv).cuda()].contiguous() if scales is not None else None
        heads = 1 if name == "idx_k" else 4
        case.d_caches[name] = (nd, ns, M.cache("nvfp4", nd, ns, case.S, heads))
    tab = case.lay.block_table.numpy()
    new_tab = np.where(tab >= 0, perm[np.maximum(tab, 0)], -1).astype(np.int32)
    case.d_table = torch.from_numpy(new_tab).cuda()
    r3 = H.to_host(H.run_path(case, "exact"))
    for k in ("block_scores", "sel", "out", "lse"):
        assert np.array_equal(r1[k], r3[k]), k


@pytest.mark.parametrize("wname", ["tiny_fp8", "tiny_spec", "tiny_prefill"])
def test_out_of_range_page_gives_nan_not_a_fault(M, wname):
    # decode scan, speculative scan and the prefill GEMM (built without NaN semantics,
    # so its NaN mark must survive as a bit pattern)
    case = H.HostCase(wname).upload()
    tab = case.lay.block_table.numpy().copy()
    tab[0, 2] = case.lay.num_pages + 5            # never dereferenced by the kernels
    case.d_table = torch.from_numpy(tab).cuda()
    res = H.to_host(H.run_path(case, "exact", attention=False))
    bs = res["block_scores"]
    seq = case.lay.seq_lens.numpy()
    T = case.w.T
    visible = (seq[0] - T + np.arange(T)) // 128 >= 2        # tokens whose own block is at or past 2
    assert visible.any()
    assert np.isnan(bs[0, visible, :, 2]).all()
    assert not np.isnan(bs[0, ~visible, :, 2]).any()          # -inf: block 2 is in their future
    assert not np.isnan(np.delete(bs[0], 2, axis=-1)).any()
    assert not np.isnan(bs[1]).any()


@pytest.mark.parametrize("wname,mode", [("tiny_fp8", "exact"), ("tiny_nvfp4", "exact"), ("tiny_nvfp4", "fp8"),
                                        ("tiny_edge", "exact"), ("long_rows", "exact"), ("c3", "exact")])
def test_flat_scan_equals_per_sequence_chunks(M, wname, mode):
    """The one-token scan spread evenly over all sequences' blocks (used when no
    per-key scores are asked for) writes every block score -- -inf past each
    sequence, NaN for an unreadable page -- bit for bit as the per-sequence
    chunked scan (the form that also writes per-key scores), on ragged batches up
    to c3's 64 contexts of 64K-160K tokens."""
    _say("flat scan", wname, mode)
    case = H.DeviceCase(wname) if wname == "c3" else H.HostCase(wname).upload()
    w, lay = case.w, case.lay
    tab = lay.block_table.numpy().copy()
    bb = int(np.argmax(lay.seq_lens.numpy()))      # a sequence with at least 4 blocks
    tab[bb, 3] = lay.num_pages + 9                 # one unreadable page
    d_tab = torch.from_numpy(tab).cuda()
    prob = M.problem(case.d_seq, d_tab, w.T)
    shape = (w.B, w.T, 4, lay.max_blocks)
    flat = torch.full(shape, 7.25, dtype=torch.float32, device="cuda")
    chunked = torch.full(shape, -7.25, dtype=torch.float32, device="cuda")
    ts = torch.empty((w.B, w.T, 4, lay.max_blocks * 128), dtype=torch.float32, device="cuda")
    ik = case.d_caches["idx_k"][2]
    M.msa_indexer_scores(prob, case.d_idx_q, w.q_dtype, case.idx_q_scale, ik, mode, flat, None)
    M.msa_indexer_scores(prob, case.d_idx_q, w.q_dtype, case.idx_q_scale, ik, mode, chunked, ts)
    torch.cuda.synchronize()
    a, b = flat.cpu().numpy(), chunked.cpu().numpy()
    assert np.isnan(a[bb, :, :, 3]).all()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("B", [1024, 1025])
def test_flat_scan_at_its_batch_limit(M, B):
    """The even-split scan covers batches of up to 1,024 sequences (its prefix sums
    live in LDS); at 1,024 short ragged contexts (1..700 tokens, a third of them a
    single block or less, pages shared at random) its block scores equal the
    chunked scan's bit for bit, and at 1,025 the call takes the chunked scan."""
    _say("flat scan batch limit", B)
    g = torch.Generator(device="cpu").manual_seed(77 + B)
    maxb = 6
    L = torch.randint(1, 701, (B,), generator=g, dtype=torch.int32)
    L[: B // 3] = torch.randint(1, 129, (B // 3,), generator=g, dtype=torch.int32)
    pages = 300
    table = torch.randint(0, pages, (B, maxb), generator=g, dtype=torch.int32)
    x = torch.randn((pages * 128, 128), generator=g).cuda()
    codes = torch.empty((pages * 128, 64), dtype=torch.uint8, device="cuda")
    scales = torch.empty((pages * 128, 8), dtype=torch.uint8, device="cuda")
    S = 32.0 / 448.0
    M.msa_pack_nvfp4(x, S, codes, scales)
    ik = M.cache("nvfp4", codes, scales, S, heads=1)
    q = torch.empty((B, 1, 4, 128), dtype=torch.uint8, device="cuda")
    M.msa_pack_fp8(torch.randn((B, 1, 4, 128), generator=g).cuda(), 1.0, q)
    prob = M.problem(L.cuda(), table.cuda(), 1)
    flat = torch.full((B, 1, 4, maxb), 7.25, dtype=torch.float32, device="cuda")
    chunked = torch.full((B, 1, 4, maxb), -7.25, dtype=torch.float32, device="cuda")
    ts = torch.empty((B, 1, 4, maxb * 128), dtype=torch.float32, device="cuda")
    M.msa_indexer_scores(prob, q, "fp8", 1.0, ik, "exact", flat, None)
    M.msa_indexer_scores(prob, q, "fp8", 1.0, ik, "exact", chunked, ts)
    torch.cuda.synchronize()
    a, b = flat.cpu().numpy(), chunked.cpu().numpy()
    nb = (L.numpy() + 127) // 128
    assert np.isneginf(a[np.arange(B), 0, 0, np.minimum(nb, maxb - 1)][nb < maxb]).all()   # past each sequence
    assert np.isfinite(a[:, 0, :, 0]).all()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ------------------------------------------------------------------ full sizes, sampled

FULL = [("c2", [0, 17, 31], "exact", False), ("c3", [0, 21, 63], "exact", False),
        ("c3_128k", [5, 40], "exact", False), ("c3_128k", [7], "fp8", False), ("c4", [3, 11], "exact", False),
        ("c5", [1], "exact", False),
        # the FP8-rounded reading on the speculative and prefill workloads
        ("c4", [5], "fp8", False), ("c5", [0], "fp8", False),
        # per-tensor scales other than 1 (K and V on different scales) at full size
        ("c2", [9], "exact", True), ("c3_128k", [33], "exact", True), ("c4", [14], "fp8", True),
        ("c5", [1], "exact", True),
        # 1 + 7 speculative tokens on the 128K batch (two row tiles in the scan)
        ("c3_t8", [2], "exact", False), ("c3_t8", [50], "fp8", True)]


@pytest.mark.parametrize("wname,samples,mode,scaled", FULL)
def test_full_size_sampled(M, wname, samples, mode, scaled):
    _say("full-size case", wname, "samples", samples, mode, "scaled" if scaled else "unit scales")
    case = H.DeviceCase(wname, scaled=scaled)
    w, lay = case.w, case.lay
    res = H.to_host(H.run_path(case, mode))
    T = w.T
    for b in samples:
        gsel = res["sel"][b]
        # oracle scores over the whole sequence, K/V packed for the oracle's and GPU's blocks
        inp = case.oracle_inputs(b, kv_blocks=None if w.kv_dtype == "f32" else [])
        ora = H.oracle_scores(inp["caches"], inp["idx_q"], inp["seq_lens"], inp["idx_table"], T, mode, w.q_dtype,
                              idx_q_scale=case.idx_q_scale)
        H.compare_scores(res["block_scores"][b:b + 1], ora["block_scores"])
        H.compare_selection(gsel[None], ora["sel"], ora["block_scores"], ora["near_tie"], inp["seq_lens"], T)
        rows = np.arange(T) if T <= 8 else np.random.default_rng(b).choice(T, 64, replace=False)
        # K/V packed (by the oracle, from the fp32 sources) for the blocks the sampled rows attend
        blocks = np.unique(gsel[rows][gsel[rows] >= 0])
        inp = case.oracle_inputs(b, kv_blocks=blocks)
        L = int(inp["seq_lens"][0])
        K = OM.sequence_view(inp["caches"]["k"], inp["kv_table"][0], L, mode)       # decoded once per sample
        V = OM.sequence_view(inp["caches"]["v"], inp["kv_table"][0], L, mode)
        _say(wname, "sample", b, "scores and selection ok; attention rows", len(rows))
        for t in rows:
            qq = OM.decode_query(inp["q"][0, t:t + 1], w.q_dtype, case.q_scale)
            # a single query token at position L - T + t: view the sequence as ending there
            Lt = L - T + t + 1
            o, lse = OM.sparse_attention(qq, K[:, :Lt], V[:, :Lt], gsel[t:t + 1], Lt, 1, H.SOFTMAX_SCALE)
            H.compare_out(res["out"][b, t], o[0])
            assert np.abs(res["lse"][b, t] - lse[0]).max() <= 1e-4
        _say(wname, "sample", b, "ok")


# ------------------------------------------------------------------ fused scan + selection

def _fused(M, case, ws, B=None, dequant="exact"):
    w, lay = case.w, case.lay
    B = w.B if B is None else B
    prob = M.problem(case.d_seq[:B], case.d_table[:B], w.T)
    bs = torch.empty((B, w.T, 4, lay.max_blocks), dtype=torch.float32, device="cuda")
    sel = torch.empty((B, w.T, 4, 16), dtype=torch.int32, device="cuda")
    M.msa_indexer_topk(prob, case.d_idx_q[:B], w.q_dtype, case.idx_q_scale, case.d_caches["idx_k"][2], dequant, bs,
                       sel, ws)
    torch.cuda.synchronize()
    return bs.cpu().numpy(), sel.cpu().numpy()


@pytest.mark.parametrize("wname,mode", [("tiny_fp8", "exact"), ("tiny_nvfp4", "exact"), ("tiny_edge", "exact"),
                                        ("long_rows", "exact"), ("tiny_nvfp4", "fp8"), ("tiny_spec", "exact"),
                                        ("c1", "exact")])
def test_indexer_topk_equals_the_separate_calls(M, wname, mode):
    """msa_indexer_topk gives the block scores and selection of msa_indexer_scores +
    msa_block_topk bit for bit, call after call, and leaves its workspace zeroed --
    also when a later call covers fewer sequences."""
    _say("indexer_topk", wname, mode)
    case = H.HostCase(wname).upload()
    ref = H.to_host(H.run_path(case, mode, attention=False))
    B = case.w.B
    ws = torch.zeros(M.msa_workspace_size(M.problem(case.d_seq, case.d_table, case.w.T), M.MSA_CALL_INDEXER_TOPK) // 4,
                     dtype=torch.int32, device="cuda")
    for rep in range(3):
        bs, sel = _fused(M, case, ws, dequant=mode)
        assert np.array_equal(bs, ref["block_scores"], equal_nan=True), rep
        assert np.array_equal(sel, ref["sel"]), rep
        assert int(ws.abs().sum()) == 0
    if B > 1:
        bs, sel = _fused(M, case, ws, B=B - 1, dequant=mode)
        assert np.array_equal(sel, ref["sel"][:B - 1])
        assert int(ws.abs().sum()) == 0


def test_indexer_topk_full_size(M):
    _say("indexer_topk full size c3_128k")
    case = H.DeviceCase("c3_128k", keep_fp32=False)
    ref = H.to_host(H.run_path(case, "exact", attention=False))
    ws = torch.zeros(case.w.B, dtype=torch.int32, device="cuda")
    for rep in range(2):
        bs, sel = _fused(M, case, ws)
        assert np.array_equal(bs, ref["block_scores"]) and np.array_equal(sel, ref["sel"]), rep
    assert int(ws.abs().sum()) == 0


def _step(M, case, B=None, dequant="exact"):
    w, lay = case.w, case.lay
    B = w.B if B is None else B
    prob = M.problem(case.d_seq[:B], case.d_table[:B], w.T)
    bs = torch.empty((B, w.T, 4, lay.max_blocks), dtype=torch.float32, device="cuda")
    sel = torch.empty((B, w.T, 4, 16), dtype=torch.int32, device="cuda")
    out = torch.empty((B, w.T, 64, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, w.T, 64), dtype=torch.float32, device="cuda")
    M.msa_decode_step(prob, case.d_idx_q[:B], w.q_dtype, case.idx_q_scale, case.d_caches["idx_k"][2], case.d_q[:B],
                      w.q_dtype, case.q_scale, case.d_caches["k"][2], case.d_caches["v"][2], dequant, H.SOFTMAX_SCALE,
                      bs, sel, out, lse)
    torch.cuda.synchronize()
    return bs.cpu().numpy(), sel.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("wname,mode,scaled", [
    ("tiny_fp8", "exact", False), ("tiny_nvfp4", "exact", False), ("tiny_edge", "exact", False),
    ("long_rows", "exact", False), ("tiny_nvfp4", "fp8", False), ("tiny_spec", "exact", False), ("c1", "exact", False),
    ("tiny_spec8", "fp8", False), ("tiny_fp8", "exact", True), ("tiny_nvfp4", "fp8", True),
    ("tiny_spec8", "exact", True)])
def test_decode_step_equals_the_separate_calls(M, wname, mode, scaled):
    """msa_decode_step gives the block scores, selection, outputs and LSE of the three
    calls bit for bit, call after call and for a smaller batch; its output also meets
    the oracle bar on the selection it made."""
    _say("decode_step", wname, mode, "scaled" if scaled else "unit scales")
    case = H.HostCase(wname, scaled=scaled).upload()
    w, lay = case.w, case.lay
    ref = H.to_host(H.run_path(case, mode))
    B = w.B
    for rep in range(2):
        bs, sel, out, lse = _step(M, case, dequant=mode)
        assert np.array_equal(bs, ref["block_scores"], equal_nan=True), rep
        assert np.array_equal(sel, ref["sel"]), rep
        assert np.array_equal(out, ref["out"]) and np.array_equal(lse, ref["lse"]), rep
    seq_lens, table = lay.seq_lens.numpy(), lay.block_table.numpy()
    for b in range(B):
        o, _ = H.oracle_attention(case.caches, case.q, seq_lens, table, w.T, sel[b], mode, w.q_dtype, b,
                                  q_scale=case.q_scale)
        H.compare_out(out[b], o)
    if B > 1:
        bs, sel, out, lse = _step(M, case, B=B - 1, dequant=mode)
        assert np.array_equal(sel, ref["sel"][:B - 1]) and np.array_equal(out, ref["out"][:B - 1])


@pytest.mark.parametrize("wname", ["c3_128k", "c2"])
def test_decode_step_full_size(M, wname):
    _say("decode_step full size", wname)
    case = H.DeviceCase(wname, keep_fp32=False)
    ref = H.to_host(H.run_path(case, "exact"))
    bs, sel, out, lse = _step(M, case)
    assert np.array_equal(bs, ref["block_scores"]) and np.array_equal(sel, ref["sel"])
    assert np.array_equal(out, ref["out"]) and np.array_equal(lse, ref["lse"])


@pytest.mark.parametrize("dtype,heads,T,lens", [
    ("nvfp4", 4, 1, [300, 129, 5000, 128]),          # decode: one token per sequence
    ("nvfp4", 1, 130, [300, 700]),                  # a chunk spanning block boundaries
    ("fp8", 4, 5, [127, 128, 129]),
    ("fp8", 1, 1, [1, 64]),
    ("f32", 4, 3, [260]),
    ("nvfp4", 4, 4096, [4096 + 65536, 4096 + 1000]),  # c5-sized prefill chunk, K or V
])
def test_cache_insert_bit_exact(M, dtype, heads, T, lens):
    """msa_cache_insert writes exactly the oracle's quantised rows into exactly their
    slots; every other byte of the pool (arbitrary contents) is left alone, and a
    row whose page id is outside the pool is not written."""
    _say("cache_insert", dtype, heads, T, lens)
    from tests.test_oracle_msa import _insert_pool
    rng = np.random.default_rng(31 + T)
    B = len(lens)
    nbs = [(L + 127) // 128 for L in lens]
    maxb = max(nbs)
    P = sum(nbs) + 3
    perm = rng.permutation(P)
    table = np.full((B, maxb), -1, np.int32)
    off = 0
    for b, n in enumerate(nbs):
        table[b, :n] = perm[off:off + n]
        off += n
    if B > 1:
        table[1, nbs[1] - 1] = P + 7        # the last block of sequence 1 has no page in this pool
    pool = _insert_pool(dtype, P, heads, rng)
    x = (3.0 * rng.normal(size=(B, T, heads, 128))).astype(np.float32)
    want = OM.cache_insert(pool, x, lens, table, T)
    d_data = torch.from_numpy(pool["data"]).cuda()
    d_sc = torch.from_numpy(pool["scales"]).cuda() if dtype == "nvfp4" else None
    c = M.cache(dtype, d_data, d_sc, pool["tensor_scale"], heads)
    prob = M.problem(torch.tensor(lens, dtype=torch.int32, device="cuda"), torch.from_numpy(table).cuda(), T)
    M.msa_cache_insert(prob, torch.from_numpy(x).cuda(), c)
    torch.cuda.synchronize()
    assert np.array_equal(d_data.cpu().numpy(), want["data"])
    if dtype == "nvfp4":
        assert np.array_equal(d_sc.cpu().numpy(), want["scales"])


@pytest.mark.parametrize("specs,T,lens", [
    ((("nvfp4", 4), ("nvfp4", 4), ("nvfp4", 1)), 1, [300, 129, 5000, 128]),     # a decode step's K, V, index keys
    ((("nvfp4", 4), ("nvfp4", 4), ("fp8", 1), ("f32", 1)), 37, [300, 700]),    # mixed dtypes, a chunk
])
def test_cache_insert_many_bit_exact(M, specs, T, lens):
    """msa_cache_insert_many writes what one msa_cache_insert per cache writes -- the
    oracle's quantised rows in their slots and nothing else."""
    _say("cache_insert_many", specs, T, lens)
    from tests.test_oracle_msa import _insert_pool
    rng = np.random.default_rng(77 + T)
    B = len(lens)
    nbs = [(L + 127) // 128 for L in lens]
    maxb = max(nbs)
    P = sum(nbs) + 2
    perm = rng.permutation(P)
    table = np.full((B, maxb), -1, np.int32)
    off = 0
    for b, n in enumerate(nbs):
        table[b, :n] = perm[off:off + n]
        off += n
    prob = M.problem(torch.tensor(lens, dtype=torch.int32, device="cuda"), torch.from_numpy(table).cuda(), T)
    pools, wants, xs, caches, devs = [], [], [], [], []
    for dtype, heads in specs:
        pool = _insert_pool(dtype, P, heads, rng)
        x = (3.0 * rng.normal(size=(B, T, heads, 128))).astype(np.float32)
        wants.append(OM.cache_insert(pool, x, lens, table, T))
        d_data = torch.from_numpy(pool["data"]).cuda()
        d_sc = torch.from_numpy(pool["scales"]).cuda() if dtype == "nvfp4" else None
        caches.append(M.cache(dtype, d_data, d_sc, pool["tensor_scale"], heads))
        devs.append((d_data, d_sc))
        xs.append(torch.from_numpy(x).cuda())
    M.msa_cache_insert_many(prob, xs, caches)
    torch.cuda.synchronize()
    for (d_data, d_sc), want in zip(devs, wants):
        assert np.array_equal(d_data.cpu().numpy(), want["data"])
        if d_sc is not None:
            assert np.array_equal(d_sc.cpu().numpy(), want["scales"])


# ------------------------------------------------------------------ context parallelism (DCP) on one GPU

SENTINEL = 12345.0


def _dcp_run(M, case, P, dequant="exact"):
    """Every shard's scan into one buffer (prefilled with a sentinel), then every
    shard's local top-16 and the merge.  Returns host copies."""
    w, lay = case.w, case.lay
    B, T, maxb = w.B, w.T, lay.max_blocks
    prob = M.problem(case.d_seq, case.d_table, T)
    bs = torch.full((B, T, 4, maxb), SENTINEL, dtype=torch.float32, device="cuda")
    owned = []
    for s in range(P):
        M.msa_indexer_scores_shard(prob, s, P, case.d_idx_q, w.q_dtype, 1.0, case.d_caches["idx_k"][2], dequant, bs)
        torch.cuda.synchronize()
        host = bs.cpu().numpy()
        mine = np.zeros(maxb, bool)
        mine[s::P] = True
        owned.append(mine)
        # no entry of a shard that has not run yet is touched
        later = ~np.any(np.stack(owned), axis=0)
        assert np.all(host[..., later] == SENTINEL), s
    cs = torch.empty((P, B, T, 4, 16), dtype=torch.float32, device="cuda")
    cb = torch.empty((P, B, T, 4, 16), dtype=torch.int32, device="cuda")
    for s in range(P):
        M.msa_shard_topk(prob, s, P, bs, cs[s], cb[s])
    sel = torch.empty((B, T, 4, 16), dtype=torch.int32, device="cuda")
    M.msa_topk_merge(prob, P, cs, cb, sel)
    torch.cuda.synchronize()
    return bs.cpu().numpy(), cs.cpu().numpy(), cb.cpu().numpy(), sel.cpu().numpy()


def _check_dcp(case, ref, bs, cs, cb, sel, P, rows=None):
    w = case.w
    seq = case.lay.seq_lens.numpy()
    # the pages' claim: shard scores are bit-identical to the single-GPU scan ...
    assert np.array_equal(bs, ref["block_scores"], equal_nan=True)
    # ... and the merged selection is the single-GPU selection
    assert np.array_equal(sel, ref["sel"])
    # local lists and merge against the oracle, on the same (GPU) scores
    for b in (range(w.B) if rows is None else rows):
        L = int(seq[b])
        own = OM.own_blocks(L, w.T)
        for t in range(w.T):
            for g in range(4):
                for s in range(P):
                    os_, ob = OM.shard_candidates(bs[b, t, g], int(own[t]), s, P)
                    assert np.array_equal(cb[s, b, t, g], ob), (b, t, g, s)
                    n = int((ob >= 0).sum())
                    assert np.array_equal(cs[s, b, t, g, :n], os_[:n].astype(np.float32)), (b, t, g, s)
                    assert np.all(np.isnan(cs[s, b, t, g, n:]))
                assert np.array_equal(sel[b, t, g], OM.merge_candidates(cs[:, b, t, g], cb[:, b, t, g], int(own[t])))


@pytest.mark.parametrize("wname,mode,P", [("tiny_nvfp4", "exact", 4), ("tiny_nvfp4", "exact", 1),
                                          ("tiny_nvfp4", "fp8", 3), ("tiny_fp8", "exact", 2),
                                          ("tiny_spec", "exact", 4), ("tiny_spec", "fp8", 8),
                                          ("tiny_t3", "exact", 5), ("tiny_edge", "exact", 4),
                                          ("long_rows", "exact", 4), ("long_rows", "exact", 2),
                                          ("tiny_spec8", "exact", 4), ("tiny_spec8", "fp8", 3), ("tiny_t6", "exact", 2)])
def test_dcp_shards_and_merge(M, wname, mode, P):
    """Shard scans write only their own blocks and, together, the unsharded scores bit
    for bit; local top-16s and the merge match the oracle; the merged selection
    equals msa_block_topk's."""
    _say("dcp", wname, mode, P)
    case = H.HostCase(wname).upload()
    ref = H.to_host(H.run_path(case, mode, attention=False))
    _check_dcp(case, ref, *_dcp_run(M, case, P, mode), P)


@pytest.mark.parametrize("wname,rows", [("c3_128k", [0, 33, 63]), ("c4", [2, 15])])
def test_dcp_full_size(M, wname, rows):
    """At full size (one token over 131,072-token contexts; 4 tokens over 262,144):
    four shards against the unsharded scan and selection."""
    _say("dcp full size", wname)
    case = H.DeviceCase(wname, keep_fp32=False)
    ref = H.to_host(H.run_path(case, "exact", attention=False))
    _check_dcp(case, ref, *_dcp_run(M, case, 4), 4, rows=rows)


# ------------------------------------------------------------------ shared-prefix decode (index scan)

def _share_prefixes(case, groups):
    """Make every sequence of each group (first, end, blocks) read the same pages in its first
    `blocks` logical blocks -- those of the group's longest member -- in the host table (the
    oracle's) and its device copy.  Shorter members use only the blocks they reach."""
    tab = case.lay.block_table
    lens = case.lay.seq_lens
    for s, e, pb in groups:
        donor = s + int(torch.argmax(lens[s:e]))
        assert (int(lens[donor]) + 127) // 128 >= pb
        for b in range(s, e):
            tab[b, :pb] = tab[donor, :pb]
    case.d_table = tab.to("cuda")


def _prefix_run(M, case, groups, mode):
    w = case.w
    prob = M.problem(case.d_seq, case.d_table, w.T)
    bs = torch.full((w.B, w.T, 4, case.lay.max_blocks), 777.0, dtype=torch.float32, device="cuda")
    ws = torch.empty(M.msa_workspace_size(prob, M.MSA_CALL_INDEXER_PREFIX) // 4, dtype=torch.int32, device="cuda")
    starts = [g[0] for g in groups] + [groups[-1][1]]
    M.msa_indexer_scores_prefix(prob, starts, [g[2] for g in groups], case.d_idx_q, w.q_dtype, 1.0,
                                case.d_caches["idx_k"][2], mode, bs, ws)
    torch.cuda.synchronize()
    return bs.cpu().numpy()


def _check_prefix(got, ref, groups, B):
    assert not (got == 777.0).any(), "an entry was not written"
    skip = np.zeros(B, int)
    for s, e, pb in groups:
        skip[s:e] = pb
    for b in range(B):   # blocks outside the shared prefix: the decode scan's own bits
        assert np.array_equal(got[b, ..., skip[b]:], ref[b, ..., skip[b]:], equal_nan=True), b
    H.compare_scores(got, ref)   # shared blocks: same -inf pattern, values within summation order


PREFIX = [("tiny_nvfp4", "exact", [(0, 3, 8)]), ("tiny_nvfp4", "fp8", [(0, 2, 12)]),
          ("tiny_fp8", "exact", [(0, 2, 5)]), ("tiny_spec", "exact", [(0, 2, 10)]),
          ("tiny_spec", "fp8", [(0, 2, 17)]), ("tiny_t3", "exact", [(0, 1, 4), (1, 3, 12)]),
          ("tiny_edge", "exact", [(0, 5, 16)]), ("long_rows", "exact", [(0, 1, 2000)]),
          ("tiny_spec8", "exact", [(0, 2, 12)]), ("tiny_t6", "exact", [(0, 3, 1)])]


@pytest.mark.parametrize("wname,mode,groups", PREFIX)
def test_indexer_prefix(M, wname, mode, groups):
    """msa_indexer_scores_prefix writes every block score; blocks outside the shared
    prefixes equal msa_indexer_scores bit for bit, shared ones within fp32 summation
    order, and all of them match the oracle on the sharing block table (including
    sequences whose own block lies inside the shared prefix)."""
    _say("prefix", wname, mode, groups)
    case = H.HostCase(wname).upload()
    _share_prefixes(case, groups)
    w, lay = case.w, case.lay
    ref = H.to_host(H.run_path(case, mode, attention=False))
    got = _prefix_run(M, case, groups, mode)
    _check_prefix(got, ref["block_scores"], groups, w.B)
    ora = H.oracle_scores(case.caches, case.idx_q, lay.seq_lens.numpy(), lay.block_table.numpy(), w.T, mode,
                          w.q_dtype)
    H.compare_scores(got, ora["block_scores"])


@pytest.mark.parametrize("wname,groups,samples", [("c3_128k", [(0, 64, 512)], [0, 37, 63]),
                                                  ("c4", [(0, 8, 1024), (8, 16, 1536)], [5, 12])])
def test_indexer_prefix_full_size(M, wname, groups, samples):
    _say("prefix full size", wname, groups)
    case = H.DeviceCase(wname)
    _share_prefixes(case, groups)
    w = case.w
    ref = H.to_host(H.run_path(case, "exact", attention=False))
    got = _prefix_run(M, case, groups, "exact")
    _check_prefix(got, ref["block_scores"], groups, w.B)
    for b in samples:
        inp = case.oracle_inputs(b, kv_blocks=[])
        ora = H.oracle_scores(inp["caches"], inp["idx_q"], inp["seq_lens"], inp["idx_table"], w.T, "exact", w.q_dtype)
        H.compare_scores(got[b:b + 1], ora["block_scores"])


@pytest.mark.parametrize("mode", ["exact", "fp8"])
def test_wide_batch_scan_and_prefix(M, mode):
    """1,030 one-token sequences, more than the evenly spread scan takes: the
    per-sequence scan and selection against the oracle, then the shared-prefix call
    (there the per-sequence scan with skip counts from the workspace) on a sharing
    table, against the plain call and the oracle."""
    _say("wide batch", mode)
    case = H.HostCase("wide_batch", names=("idx_k",)).upload()
    w, lay = case.w, case.lay
    res = H.to_host(H.run_path(case, mode, attention=False))
    ora = H.oracle_scores(case.caches, case.idx_q, lay.seq_lens.numpy(), lay.block_table.numpy(), w.T, mode,
                          w.q_dtype)
    H.compare_scores(res["block_scores"], ora["block_scores"])
    H.compare_selection(res["sel"], ora["sel"], ora["block_scores"], ora["near_tie"], lay.seq_lens.numpy(), w.T)
    # consecutive groups of up to 64 sequences over the whole batch, sharing 0 .. 3 blocks
    lens = lay.seq_lens.numpy()
    groups = [(s0, min(s0 + 64, w.B), min(k % 4, (int(lens[s0:s0 + 64].max()) + 127) // 128))
              for k, s0 in enumerate(range(0, w.B, 64))]
    _share_prefixes(case, groups)
    ref = H.to_host(H.run_path(case, mode, attention=False))
    got = _prefix_run(M, case, groups, mode)
    _check_prefix(got, ref["block_scores"], groups, w.B)
    ora = H.oracle_scores(case.caches, case.idx_q, lay.seq_lens.numpy(), lay.block_table.numpy(), w.T, mode,
                          w.q_dtype)
    H.compare_scores(got, ora["block_scores"])


# ------------------------------------------------------------------ shared-prefix decode attention

def _force_prefix_blocks(sel, seq_lens, T, groups, per_row=8, seed=0):
    """A selection in which every row of a group also picks the same `per_row`
    shared-prefix blocks older than its own block: the own block is kept, the row's
    other entries are trimmed to make room; rows stay distinct, ascending and -1
    padded.  (The attention takes any such selection.)"""
    rng = np.random.default_rng(seed)
    out = sel.copy()
    for s0, e0, pb in groups:
        common = [int(x) for x in rng.permutation(pb)[:per_row]]
        for b in range(s0, e0):
            for t in range(T):
                own = (int(seq_lens[b]) - T + t) // 128
                for g in range(4):
                    add = [i for i in common if i < own]
                    others = [int(i) for i in out[b, t, g] if 0 <= i != own and int(i) not in add]
                    others = others[:max(0, 15 - len(add))]
                    row = sorted(set(others + add + [own]))
                    out[b, t, g] = np.array(row + [-1] * (16 - len(row)), np.int32)
    return out


def _attn_prefix(M, case, groups, mode, sel):
    w = case.w
    prob = M.problem(case.d_seq, case.d_table, w.T)
    starts = [g[0] for g in groups] + [groups[-1][1]]
    blocks = [g[2] for g in groups]
    nws = M.msa_sparse_attn_prefix_workspace_size(prob, starts, blocks)
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device="cuda")
    d_sel = torch.from_numpy(np.ascontiguousarray(sel)).cuda()
    ref_out = torch.empty((w.B, w.T, 64, 128), dtype=torch.float32, device="cuda")
    ref_lse = torch.empty((w.B, w.T, 64), dtype=torch.float32, device="cuda")
    M.msa_sparse_attn_decode(prob, case.d_q, w.q_dtype, case.q_scale, case.d_caches["k"][2], case.d_caches["v"][2],
                             mode, d_sel, H.SOFTMAX_SCALE, ref_out, ref_lse)
    out = torch.full_like(ref_out, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    M.msa_sparse_attn_decode_prefix(prob, starts, blocks, case.d_q, w.q_dtype, case.q_scale, case.d_caches["k"][2],
                                    case.d_caches["v"][2], mode, d_sel, H.SOFTMAX_SCALE, out, lse, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), ref_out.cpu().numpy(), ref_lse.cpu().numpy()


ATTN_PREFIX = [("tiny_nvfp4", "exact", [(0, 3, 8)], False), ("tiny_nvfp4", "fp8", [(0, 2, 12)], False),
               ("tiny_fp8", "exact", [(0, 2, 5)], False), ("tiny_spec", "exact", [(0, 2, 10)], False),
               ("tiny_spec8", "fp8", [(0, 2, 14)], False), ("tiny_t3", "exact", [(0, 1, 4), (1, 3, 12)], False),
               ("tiny_edge", "exact", [(0, 5, 1)], False), ("long_rows", "exact", [(0, 1, 2000)], False),
               ("tiny_nvfp4", "exact", [(0, 3, 8)], True), ("tiny_fp8", "exact", [(1, 3, 7)], True)]


@pytest.mark.parametrize("wname,mode,groups,scaled", ATTN_PREFIX)
def test_sparse_attn_decode_prefix(M, wname, mode, groups, scaled):
    """msa_sparse_attn_decode_prefix equals msa_sparse_attn_decode bit for bit on the
    same selection -- one where the rows of a group share prefix blocks, so the
    staged images are read -- and then on the plain selection through the same
    workspace (nothing of the first call is reused); the output meets the oracle bar
    on the sharing block table."""
    _say("attn prefix", wname, mode, groups, "scaled" if scaled else "unit scales")
    case = H.HostCase(wname, scaled=scaled).upload()
    _share_prefixes(case, groups)
    w, lay = case.w, case.lay
    seq_lens, table = lay.seq_lens.numpy(), lay.block_table.numpy()
    base = H.to_host(H.run_path(case, mode, attention=False))["sel"]
    forced = _force_prefix_blocks(base, seq_lens, w.T, groups)
    shared = sum(int(((forced[s0:e0] >= 0) & (forced[s0:e0] < pb)).sum()) for s0, e0, pb in groups)
    assert shared > 0
    results = []
    for sel in (forced, base):
        out, lse, ref_out, ref_lse = _attn_prefix(M, case, groups, mode, sel)
        assert np.array_equal(out, ref_out) and np.array_equal(lse, ref_lse)
        results.append((out, lse))
    out, lse = results[0]
    for b in range(w.B):
        o, l_ = H.oracle_attention(case.caches, case.q, seq_lens, table, w.T, forced[b], mode, w.q_dtype, b,
                                   q_scale=case.q_scale)
        H.compare_out(out[b], o)
        assert np.abs(lse[b] - l_).max() <= 1e-4


def test_sparse_attn_decode_prefix_full_size(M):
    """c3_128k with all 64 sequences sharing their first 512 blocks and every row
    also selecting 8 common prefix blocks: bit for bit equal to msa_sparse_attn_decode."""
    _say("attn prefix full size c3_128k")
    case = H.DeviceCase("c3_128k", keep_fp32=False)
    groups = [(0, 64, 512)]
    _share_prefixes(case, groups)
    base = H.to_host(H.run_path(case, "exact", attention=False))["sel"]
    forced = _force_prefix_blocks(base, case.lay.seq_lens.numpy(), case.w.T, groups)
    out, lse, ref_out, ref_lse = _attn_prefix(M, case, groups, "exact", forced)
    assert np.array_equal(out, ref_out) and np.array_equal(lse, ref_lse)


# ------------------------------------------------------------------ selection inside the attention launch

@pytest.mark.parametrize("wname,mode", [("tiny_nvfp4", "exact"), ("tiny_nvfp4", "fp8"), ("tiny_fp8", "exact"),
                                        ("tiny_spec", "exact"), ("tiny_edge", "exact"), ("tiny_prefill", "exact"),
                                        ("tiny_prefill_many", "exact"), ("long_rows", "exact"), ("c1", "exact"),
                                        ("tiny_t3", "exact"), ("rows_2048", "exact")])
def test_topk_sparse_attn_equals_the_two_calls(M, wname, mode):
    """msa_topk_sparse_attn writes msa_block_topk's selection and the attention call's
    out / lse for it, bit for bit (decode and prefill forms, fp32 fallback)."""
    _say("topk_sparse_attn", wname, mode)
    case = H.HostCase(wname).upload()
    w, lay = case.w, case.lay
    ref = H.to_host(H.run_path(case, mode))
    prob = M.problem(case.d_seq, case.d_table, w.T)
    bs = torch.from_numpy(ref["block_scores"]).cuda()
    sel = torch.full((w.B, w.T, 4, 16), -7, dtype=torch.int32, device="cuda")
    out = torch.empty((w.B, w.T, 64, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.T, 64), dtype=torch.float32, device="cuda")
    M.msa_topk_sparse_attn(prob, bs, sel, case.d_q, w.q_dtype, 1.0, case.d_caches["k"][2], case.d_caches["v"][2],
                           mode, H.SOFTMAX_SCALE, out, lse)
    torch.cuda.synchronize()
    assert np.array_equal(sel.cpu().numpy(), ref["sel"])
    assert np.array_equal(out.cpu().numpy(), ref["out"], equal_nan=True)
    assert np.array_equal(lse.cpu().numpy(), ref["lse"], equal_nan=True)


def test_topk_sparse_attn_full_size(M):
    _say("topk_sparse_attn full size c3_128k")
    case = H.DeviceCase("c3_128k", keep_fp32=False)
    w = case.w
    ref = H.to_host(H.run_path(case, "exact"))
    prob = M.problem(case.d_seq, case.d_table, w.T)
    bs = torch.from_numpy(ref["block_scores"]).cuda()
    sel = torch.empty((w.B, w.T, 4, 16), dtype=torch.int32, device="cuda")
    out = torch.empty((w.B, w.T, 64, 128), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.T, 64), dtype=torch.float32, device="cuda")
    M.msa_topk_sparse_attn(prob, bs, sel, case.d_q, w.q_dtype, 1.0, case.d_caches["k"][2], case.d_caches["v"][2],
                           "exact", H.SOFTMAX_SCALE, out, lse)
    torch.cuda.synchronize()
    assert np.array_equal(sel.cpu().numpy(), ref["sel"])
    assert np.array_equal(out.cpu().numpy(), ref["out"]) and np.array_equal(lse.cpu().numpy(), ref["lse"])


# ------------------------------------------------------------------ crafted score rows

def _crafted_scores(rng, B, T, maxb, L, period, width):
    """Score rows for the four groups: random; a "crowded" row whose best scores fill
    the first 14 lanes (or waves) of the selection and whose 15th lane (or wave) sits
    lower, so that more than 64 keys reach the threshold; scores rounded to integers
    (ties, broken by block index); 10% NaN (below every number).  Blocks at or past a
    token's own block hold +inf, which the selection must never read."""
    s = rng.standard_normal((B, T, 4, maxb)).astype(np.float32)
    slot = (np.arange(maxb) % period) // width     # the lane (or wave) that holds each block
    s[:, :, 1, :] += np.where(slot < 14, 200.0, np.where(slot == 14, 100.0, 0.0)).astype(np.float32)
    s[:, :, 2, :] = np.round(s[:, :, 2, :] * 2.0)
    s[:, :, 3, :][rng.random((B, T, maxb)) < 0.1] = np.nan
    for b in range(B):
        for t in range(T):
            s[b, t, :, (L[b] - T + t) // 128:] = np.inf
    return s


def _oracle_sel(scores, L, T):
    """The oracle's selection; NaN scores enter as -1e30 (below every finite score,
    tied among themselves, so block order decides), as the library ranks NaN."""
    B, _, G, _ = scores.shape
    sel = np.empty((B, T, G, 16), dtype=np.int32)
    for b in range(B):
        for t in range(T):
            own = (int(L[b]) - T + t) // 128
            for g in range(G):
                row = np.where(np.isnan(scores[b, t, g]), -1e30, scores[b, t, g]).astype(np.float64)
                sel[b, t, g] = OM.select_blocks(row, own)
    return sel


@pytest.mark.parametrize("T", [1, 64])
def test_block_topk_crafted_rows(M, T):
    """msa_block_topk on crafted rows of up to 1,000 blocks, 256 and 4,096 rows (a wave
    per row: the lane-maximum bound, with the crowded rows taking the radix fallback)."""
    _say("block_topk crafted", T)
    rng = np.random.default_rng(4321 + T)
    B, maxb = (64, 1000) if T == 1 else (16, 1000)
    L = rng.integers(T, maxb * 128 + 1, size=B).astype(np.int32)
    L[:5] = [T, 16 * 128 + T - 1, 17 * 128 + T, 64 * 15 * 128 + 5, maxb * 128]
    scores = _crafted_scores(rng, B, T, maxb, L, 64, 1)
    seq = torch.from_numpy(L).cuda()
    table = torch.zeros((B, maxb), dtype=torch.int32, device="cuda")
    prob = M.problem(seq, table, T)
    sel = torch.full((B, T, 4, 16), -7, dtype=torch.int32, device="cuda")
    M.msa_block_topk(prob, torch.from_numpy(scores).cuda(), sel)
    torch.cuda.synchronize()
    assert np.array_equal(sel.cpu().numpy(), _oracle_sel(scores, L, T))


def test_block_topk_wave_bound_edges(M):
    """msa_block_topk's one-wave form (4,096 rows of up to 1,000 blocks; block i sits in
    lane i mod 64) at the edges of its bound-then-rank selection: exactly 64 keys at the
    bound (the ranked list full); 65 (the radix fallback); 15 winners alone in their
    16-bit prefix above a crowd one prefix lower; every score equal; scores 1,000 apart
    from zero with a spread of 0.01 or 1 (the top 16 bits agree, so the bound's low bits
    are set in a second pass), negative and positive; 97% NaN (fewer than 15 lanes hold a
    number); -3e38 everywhere but 20 blocks.  Equal to the oracle."""
    _say("block_topk wave bound edges")
    rng = np.random.default_rng(808)
    B, T, maxb = 16, 64, 1000
    L = rng.integers(T + 40 * 128, maxb * 128 + 1, size=B).astype(np.int32)
    L[0] = maxb * 128
    s = (-100.0 + 0.01 * rng.standard_normal((B, T, 4, maxb))).astype(np.float32)
    ev, od = s[:, 0::2], s[:, 1::2]              # views: even and odd tokens
    ev[:, :, 0, 0:64] = 5.0                       # 64 ties, one per lane
    ev[:, :, 1, 0:65] = 5.0                       # 65 ties
    ev[:, :, 2, :] = -1000.0 - np.abs(rng.standard_normal((B, T // 2, maxb)))
    ev[:, :, 3, :] = rng.standard_normal((B, T // 2, maxb))
    ev[:, :, 3, :][rng.random((B, T // 2, maxb)) < 0.97] = np.nan
    od[:, :, 0, 100:115] = 7.0                    # 15 winners in 15 lanes
    od[:, :, 0, 200:400] = 6.99                   # a crowd one 16-bit prefix lower
    od[:, :, 1, :] = 1.0                          # every key tied
    od[:, :, 2, :] = 1000.0 + 0.01 * rng.standard_normal((B, T // 2, maxb))
    od[:, :, 3, :] = -3.0e38                      # the oracle takes finite scores only
    for b in range(B):
        for t in range(1, T, 2):
            od[b, t // 2, 3, rng.permutation(40)[:20]] = rng.standard_normal(20)   # 20 lanes
    for b in range(B):
        for t in range(T):
            s[b, t, :, (L[b] - T + t) // 128:] = np.inf
    seq = torch.from_numpy(L).cuda()
    table = torch.zeros((B, maxb), dtype=torch.int32, device="cuda")
    prob = M.problem(seq, table, T)
    sel = torch.full((B, T, 4, 16), -7, dtype=torch.int32, device="cuda")
    M.msa_block_topk(prob, torch.from_numpy(s).cuda(), sel)
    torch.cuda.synchronize()
    want = _oracle_sel(s, L, T)
    assert list(want[0, 0, 0]) == list(range(15)) + [(int(L[0]) - T) // 128]
    assert list(want[0, 1, 0]) == list(range(100, 115)) + [(int(L[0]) - T + 1) // 128]
    assert np.array_equal(sel.cpu().numpy(), want)


def test_selecting_attention_crafted_rows(M):
    """The attention launch that selects its own rows (a 16-wave workgroup per row,
    radix select) on crafted score rows of 2,344 blocks -- crowded, tied and NaN rows:
    the selection equals the oracle's and msa_block_topk's."""
    _say("selecting attention crafted")
    case = H.HostCase("long_rows").upload()
    w, lay = case.w, case.lay
    rng = np.random.default_rng(99)
    L = lay.seq_lens.numpy()
    scores = _crafted_scores(rng, w.B, w.T, lay.max_blocks, L, 1024, 64)
    prob = M.problem(case.d_seq, case.d_table, w.T)
    bs = torch.from_numpy(scores).cuda()
    sel = torch.full((w.B, w.T, 4, 16), -7, dtype=torch.int32, device="cuda")
    sel2 = torch.full((w.B, w.T, 4, 16), -7, dtype=torch.int32, device="cuda")
    out = torch.empty((w.B, w.T, 64, 128), dtype=torch.float32, device="cuda")
    M.msa_topk_sparse_attn(prob, bs, sel, case.d_q, w.q_dtype, 1.0, case.d_caches["k"][2], case.d_caches["v"][2],
                           "exact", H.SOFTMAX_SCALE, out, None)
    M.msa_block_topk(prob, bs, sel2)
    torch.cuda.synchronize()
    got = sel.cpu().numpy()
    assert np.array_equal(got, _oracle_sel(scores, L, w.T))
    assert np.array_equal(got, sel2.cpu().numpy())


def test_selecting_attention_bound_edges(M):
    """The selecting attention's bound-then-rank selection at its edges (2,344-block
    rows, three keys per thread): exactly 64 keys at the bound (all tied, the ranked
    list is full), 65 (the radix fallback), 15 winners alone in their 16-bit prefix
    above a crowd one prefix lower, and a row of equal scores (every key at the
    bound).  Ties are broken by block order; the selection equals the oracle's and
    msa_block_topk's."""
    _say("selecting attention bound edges")
    case = H.HostCase("long_rows").upload()
    w, lay = case.w, case.lay
    rng = np.random.default_rng(5)
    L = lay.seq_lens.numpy()
    maxb = lay.max_blocks
    s = (-100.0 + 0.01 * rng.standard_normal((w.B, w.T, 4, maxb))).astype(np.float32)
    s[:, :, 0, 0:64] = 5.0          # 64 ties, all held by wave 0
    s[:, :, 1, 0:65] = 5.0          # 65 ties: wave 0 and one key of wave 1
    s[:, :, 2, 100:115] = 7.0       # 15 winners in wave 1
    s[:, :, 2, 200:300] = 6.99      # a crowd in the next-lower prefix (waves 3 and 4)
    s[:, :, 3, :] = 1.0             # every key tied
    for b in range(w.B):
        for t in range(w.T):
            s[b, t, :, (L[b] - w.T + t) // 128:] = np.inf
    prob = M.problem(case.d_seq, case.d_table, w.T)
    bs = torch.from_numpy(s).cuda()
    sel = torch.full((w.B, w.T, 4, 16), -7, dtype=torch.int32, device="cuda")
    sel2 = torch.full((w.B, w.T, 4, 16), -7, dtype=torch.int32, device="cuda")
    out = torch.empty((w.B, w.T, 64, 128), dtype=torch.float32, device="cuda")
    M.msa_topk_sparse_attn(prob, bs, sel, case.d_q, w.q_dtype, 1.0, case.d_caches["k"][2], case.d_caches["v"][2],
                           "exact", H.SOFTMAX_SCALE, out, None)
    M.msa_block_topk(prob, bs, sel2)
    torch.cuda.synchronize()
    got = sel.cpu().numpy()
    want = _oracle_sel(s, L, w.T)
    own = (int(L[0]) - w.T) // 128
    assert list(want[0, 0, 0]) == list(range(15)) + [own] and list(want[0, 0, 2]) == list(range(100, 115)) + [own]
    assert np.array_equal(got, want)
    assert np.array_equal(got, sel2.cpu().numpy())


def test_selecting_attention_offset_rows(M):
    """The selecting attention's selection on rows whose scores share a common offset
    far larger than their spread (the top 16 bits of every score agree, so the bound's
    low bits are set in a second pass): 1,000 + 0.01 N(0,1), -1,000 - |N(0,1)|, 3 + 0.001
    N(0,1), and 1,000 + 0.01 N(0,1) rounded to 0.05 (ties: the radix cut decides).  The
    selection equals the oracle's and msa_block_topk's."""
    _say("selecting attention offset rows")
    case = H.HostCase("long_rows").upload()
    w, lay = case.w, case.lay
    rng = np.random.default_rng(17)
    L = lay.seq_lens.numpy()
    maxb = lay.max_blocks
    z = rng.standard_normal((w.B, w.T, 4, maxb))
    s = np.empty((w.B, w.T, 4, maxb), np.float32)
    s[:, :, 0] = 1000.0 + 0.01 * z[:, :, 0]
    s[:, :, 1] = -1000.0 - np.abs(z[:, :, 1])
    s[:, :, 2] = 3.0 + 0.001 * z[:, :, 2]
    s[:, :, 3] = 1000.0 + np.round(0.2 * z[:, :, 3]) * 0.05
    for b in range(w.B):
        for t in range(w.T):
            s[b, t, :, (L[b] - w.T + t) // 128:] = np.inf
    prob = M.problem(case.d_seq, case.d_table, w.T)
    bs = torch.from_numpy(s).cuda()
    sel = torch.full((w.B, w.T, 4, 16), -7, dtype=torch.int32, device="cuda")
    sel2 = torch.full((w.B, w.T, 4, 16), -7, dtype=torch.int32, device="cuda")
    out = torch.empty((w.B, w.T, 64, 128), dtype=torch.float32, device="cuda")
    M.msa_topk_sparse_attn(prob, bs, sel, case.d_q, w.q_dtype, 1.0, case.d_caches["k"][2], case.d_caches["v"][2],
                           "exact", H.SOFTMAX_SCALE, out, None)
    M.msa_block_topk(prob, bs, sel2)
    torch.cuda.synchronize()
    got = sel.cpu().numpy()
    assert np.array_equal(got, _oracle_sel(s, L, w.T))
    assert np.array_equal(got, sel2.cpu().numpy())


def test_decode_step_graph_replays(M):
    """The decode layer step (index scan, then the selecting attention) captured in a HIP
    graph: three replays, each followed by an eager step, all bit-identical to eager."""
    _say("graph replays tiny_nvfp4")
    case = H.HostCase("tiny_nvfp4").upload()
    w, lay = case.w, case.lay
    prob = M.problem(case.d_seq, case.d_table, w.T)
    bs = torch.empty((w.B, w.T, 4, lay.max_blocks), dtype=torch.float32, device="cuda")
    sel = torch.empty((w.B, w.T, 4, 16), dtype=torch.int32, device="cuda")
    out = torch.empty((w.B, w.T, 64, 128), dtype=torch.float32, device="cuda")

    def step():
        M.msa_indexer_scores(prob, case.d_idx_q, w.q_dtype, 1.0, case.d_caches["idx_k"][2], "exact", bs, None)
        M.msa_topk_sparse_attn(prob, bs, sel, case.d_q, w.q_dtype, 1.0, case.d_caches["k"][2],
                               case.d_caches["v"][2], "exact", H.SOFTMAX_SCALE, out, None)

    step()
    torch.cuda.synchronize()
    ref = (bs.clone(), sel.clone(), out.clone())
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        bs.zero_(), sel.zero_(), out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bs, ref[0]) and torch.equal(sel, ref[1]) and torch.equal(out, ref[2]), rep
        step()
        torch.cuda.synchronize()
    del g


def test_probes_run(M):
    """The benchmark's measurement probes (bench_probes, not part of libmsa) launch and
    finish: a streaming read leaves its sink untouched for zero-filled data, and the
    MFMA probe writes finite sums."""
    import bench_probes as BP
    _say("probes")
    buf = torch.zeros(1 << 24, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(BP.SINK_WORDS, dtype=torch.int32, device="cuda")
    BP.stream_read(buf, sink)
    out = torch.full((4 * 256,), float("nan"), dtype=torch.float32, device="cuda")
    BP.mfma_f16(out, 4, 10)
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0
    assert bool(torch.isfinite(out).all())
