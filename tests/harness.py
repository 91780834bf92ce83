"""Test harness: builds seeded cases, runs the HIP path through the C ABI and
the CPU oracle, and compares them.

Two ways of feeding the two sides:
* small cases ("host"): synth draws fp32 on the CPU, the oracle's quantiser
  packs it, and the same bytes are uploaded for the HIP path;
* full-size cases ("device"): synth draws fp32 on the GPU and the library's
  pack kernels quantise it there; for the sampled sequences the fp32 source
  pages are copied back and the oracle quantises them itself (the pack
  kernels are separately shown bit-identical to the oracle's quantiser).
No oracle input is ever read from a HIP-path output.
"""
import math

import numpy as np
import torch

import synth
from oracle import formats as OF
from oracle import msa as OM

SOFTMAX_SCALE = 1.0 / math.sqrt(128.0)


def msa_lib():
    import block_sparse_attention_indexer_amd as M
    return M


# ------------------------------------------------------------------ oracle-side packing

def oracle_pack(x, dtype, S):
    """fp32 numpy [..., 128] -> oracle cache dict (same layout as the library).  An
    fp32 cache keeps x as stored elements, so its decoded values are S * x."""
    if dtype == "f32":
        return {"dtype": "f32", "data": np.asarray(x, np.float32), "tensor_scale": S}
    if dtype == "fp8":
        return {"dtype": "fp8", "data": OF.fp8_quantize(x, S), "tensor_scale": S}
    codes, sc = OF.nvfp4_quantize(x, S)
    return {"dtype": "nvfp4", "data": codes, "scales": sc, "tensor_scale": S}


def oracle_query(x, dtype, scale=1.0):
    """Query bytes: FP8 of x / scale (so they decode to about x), or fp32 x itself."""
    return np.asarray(x, np.float32) if dtype == "f32" else OF.fp8_quantize(x, scale)


# Per-tensor scales other than 1, with the index keys, K and V all on different
# scales: large enough that no NVFP4 block scale of the workloads' data (|x| up to
# about 26) saturates, and not powers of two, so a scale applied twice, dropped or
# taken from the wrong tensor shows in the results.
SCALED = {"idx_q": float(np.float32(0.37)), "q": float(np.float32(1.9)), "idx_k": float(np.float32(0.093)),
          "k": float(np.float32(0.061)), "v": float(np.float32(0.113))}


def case_scales(w, scaled):
    """Query and cache scales of a case: the workload's defaults, or SCALED."""
    if scaled:
        return dict(SCALED)
    S = w.tensor_scale()
    return {"idx_q": 1.0, "q": 1.0, "idx_k": S, "k": S, "v": S}


# ------------------------------------------------------------------ small cases

class HostCase:
    """All inputs drawn on the CPU and packed by the oracle.  scaled=True packs the
    queries and the three caches with the per-tensor scales of SCALED; names: the
    caches to draw (the index keys alone for a scan-only case)."""

    def __init__(self, wname, seed=0, scaled=False, names=("idx_k", "k", "v")):
        w = synth.WORKLOADS[wname]
        self.w, self.seed = w, seed
        self.lay = lay = synth.make_layout(w, seed)
        idx_q, q, qhat = synth.queries(w, seed)
        hot = synth.hot_blocks(w, lay, seed)
        P = lay.num_pages
        self.scales = sc = case_scales(w, scaled)
        self.S = sc["k"]
        self.idx_q_scale, self.q_scale = sc["idx_q"], sc["q"]
        self.caches = {}
        for name in names:
            x = synth.cache_pages(w, lay, seed, name, 0, P, qhat, hot).numpy()
            self.caches[name] = oracle_pack(x, w.kv_dtype, sc[name])
        self.idx_q = oracle_query(idx_q.numpy(), w.q_dtype, sc["idx_q"])
        self.q = oracle_query(q.numpy(), w.q_dtype, sc["q"])

    # device copies of the same bytes
    def upload(self):
        M = msa_lib()
        dev = "cuda"
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        self.d_seq = t(self.lay.seq_lens.numpy())
        self.d_table = t(self.lay.block_table.numpy())
        self.d_idx_q = t(self.idx_q)
        self.d_q = t(self.q)
        self.d_caches = {}
        for name, c in self.caches.items():
            heads = 1 if name == "idx_k" else 4
            data = t(c["data"])
            scales = t(c["scales"]) if "scales" in c else None
            self.d_caches[name] = (data, scales, M.cache(c["dtype"], data, scales, c["tensor_scale"], heads))
        return self


# ------------------------------------------------------------------ full-size cases

class DeviceCase:
    """Inputs drawn on the GPU and packed by the library's pack kernels (scaled: as
    for HostCase)."""

    def __init__(self, wname, seed=0, keep_fp32=True, scaled=False):
        M = msa_lib()
        w = synth.WORKLOADS[wname]
        self.w, self.seed = w, seed
        self.lay = lay = synth.make_layout(w, seed)
        dev = "cuda"
        idx_q, q, qhat = synth.queries(w, seed, device=dev)
        self.idx_q32, self.q32 = idx_q, q
        hot = synth.hot_blocks(w, lay, seed)
        P = lay.num_pages
        self.scales = scl = case_scales(w, scaled)
        self.S = scl["k"]
        self.idx_q_scale, self.q_scale = scl["idx_q"], scl["q"]
        self.d_seq = lay.seq_lens.to(dev)
        self.d_table = lay.block_table.to(dev)
        self.fp32 = {}
        self.d_caches = {}
        for name in ("idx_k", "k", "v"):
            heads = 1 if name == "idx_k" else 4
            S = scl[name]
            x = synth.cache_pages(w, lay, seed, name, 0, P, qhat, hot, device=dev)
            if keep_fp32:
                self.fp32[name] = x
            if w.kv_dtype == "nvfp4":
                codes = torch.empty(x.shape[:-1] + (64,), dtype=torch.uint8, device=dev)
                sc = torch.empty(x.shape[:-1] + (8,), dtype=torch.uint8, device=dev)
                M.msa_pack_nvfp4(x, S, codes, sc)
                self.d_caches[name] = (codes, sc, M.cache("nvfp4", codes, sc, S, heads))
            elif w.kv_dtype == "fp8":
                data = torch.empty(x.shape, dtype=torch.uint8, device=dev)
                M.msa_pack_fp8(x, S, data)
                self.d_caches[name] = (data, None, M.cache("fp8", data, None, S, heads))
            else:
                self.d_caches[name] = (x, None, M.cache("f32", x, None, S, heads))
            if not keep_fp32:
                del x
        if w.q_dtype == "fp8":
            self.d_idx_q = torch.empty(idx_q.shape, dtype=torch.uint8, device=dev)
            self.d_q = torch.empty(q.shape, dtype=torch.uint8, device=dev)
            M.msa_pack_fp8(idx_q, scl["idx_q"], self.d_idx_q)
            M.msa_pack_fp8(q, scl["q"], self.d_q)
        else:
            self.d_idx_q, self.d_q = idx_q, q
        torch.cuda.synchronize()

    def oracle_inputs(self, b, kv_blocks=None):
        """Oracle-packed inputs of sequence b, quantised by the oracle from the
        fp32 sources.  The index keys of the whole sequence are packed; K/V only
        for ``kv_blocks`` (logical ids; all blocks when None) -- the others map to
        a zero page the attention never reads."""
        w, lay = self.w, self.lay
        L = int(lay.seq_lens[b])
        nb = (L + 127) // 128
        pages = lay.block_table[b, :nb].long()
        ik = self.fp32["idx_k"][pages.to(self.fp32["idx_k"].device)].cpu().numpy()
        caches = {"idx_k": oracle_pack(ik, w.kv_dtype, self.scales["idx_k"])}
        blocks = list(range(nb)) if kv_blocks is None else sorted(set(int(i) for i in kv_blocks if 0 <= i < nb))
        kv_table = np.zeros((1, lay.max_blocks), np.int32)        # default: zero page 0
        for slot, i in enumerate(blocks):
            kv_table[0, i] = slot + 1
        sel_pages = pages[blocks] if blocks else pages[:0]
        for n in ("k", "v"):
            src = self.fp32[n][sel_pages.to(self.fp32[n].device)].cpu().numpy()
            src = np.concatenate([np.zeros((1,) + src.shape[1:], np.float32), src])
            caches[n] = oracle_pack(src, w.kv_dtype, self.scales[n])
        idx_table = np.full((1, lay.max_blocks), -1, np.int32)
        idx_table[0, :nb] = np.arange(nb)
        idx_q = oracle_query(self.idx_q32[b:b + 1].cpu().numpy(), w.q_dtype, self.idx_q_scale)
        q = oracle_query(self.q32[b:b + 1].cpu().numpy(), w.q_dtype, self.q_scale)
        return {"caches": caches, "idx_q": idx_q, "q": q, "seq_lens": np.array([L]),
                "idx_table": idx_table, "kv_table": kv_table}


# ------------------------------------------------------------------ HIP path

def run_path(case, dequant="exact", token_scores=False, attention=True, stream=None):
    M = msa_lib()
    w, lay = case.w, case.lay
    B, T, maxb = w.B, w.T, lay.max_blocks
    prob = M.problem(case.d_seq, case.d_table, T)
    dev = "cuda"
    bs = torch.empty((B, T, 4, maxb), dtype=torch.float32, device=dev)
    ts = torch.empty((B, T, 4, maxb * 128), dtype=torch.float32, device=dev) if token_scores else None
    M.msa_indexer_scores(prob, case.d_idx_q, w.q_dtype, case.idx_q_scale, case.d_caches["idx_k"][2], dequant, bs,
                         ts, stream=stream)
    sel = torch.empty((B, T, 4, 16), dtype=torch.int32, device=dev)
    M.msa_block_topk(prob, bs, sel, stream=stream)
    res = {"block_scores": bs, "sel": sel, "token_scores": ts}
    if attention:
        out = torch.empty((B, T, 64, 128), dtype=torch.float32, device=dev)
        lse = torch.empty((B, T, 64), dtype=torch.float32, device=dev)
        fn = M.msa_sparse_attn_decode if T <= 8 else M.msa_sparse_attn_prefill
        fn(prob, case.d_q, w.q_dtype, case.q_scale, case.d_caches["k"][2], case.d_caches["v"][2], dequant, sel,
           SOFTMAX_SCALE, out, lse, stream=stream)
        res.update(out=out, lse=lse)
    torch.cuda.synchronize()
    return res


def to_host(res):
    return {k: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for k, v in res.items()}


# ------------------------------------------------------------------ oracle side

def oracle_scores(caches, idx_q, seq_lens, table, T, mode, q_dtype, sequences=None, idx_q_scale=1.0):
    """Oracle block scores, selection and near-tie flags (no attention)."""
    dummy_q = np.zeros((len(seq_lens), T, 64, 128), np.float32)
    return OM.batch_layer(idx_q, dummy_q, caches["idx_k"], caches.get("k"), caches.get("v"), seq_lens, table, T,
                          SOFTMAX_SCALE, mode=mode, idx_q_dtype=q_dtype, idx_q_scale=idx_q_scale, q_dtype=q_dtype,
                          sequences=sequences, with_attention=False)


def oracle_attention(caches, q, seq_lens, table, T, sel, mode, q_dtype, b, q_scale=1.0):
    L = int(seq_lens[b])
    qq = OM.decode_query(q[b], q_dtype, q_scale)
    K = OM.sequence_view(caches["k"], table[b], L, mode)
    V = OM.sequence_view(caches["v"], table[b], L, mode)
    return OM.sparse_attention(qq, K, V, sel, L, T, SOFTMAX_SCALE)


# ------------------------------------------------------------------ comparisons

SCORE_RTOL = 1e-5
OUT_MAX_ABS = 2e-3
OUT_MEAN_ABS = 2e-4


def compare_scores(gpu_bs, ora_bs, rows_mask=None):
    """Same -inf pattern, finite values within SCORE_RTOL * (1 + |oracle|)."""
    g, o = np.asarray(gpu_bs, np.float64), np.asarray(ora_bs, np.float64)
    assert not np.isnan(g).any(), "NaN block score"
    assert np.array_equal(np.isneginf(g), np.isneginf(o)), "-inf pattern differs"
    fin = np.isfinite(o)
    err = np.abs(g[fin] - o[fin]) / (1.0 + np.abs(o[fin]))
    assert err.max(initial=0.0) <= SCORE_RTOL, f"block score rel err {err.max():.3g}"
    return float(err.max(initial=0.0))


NEAR_TIE_BAND = 2e-5      # relative half-width of the band a near-tie choice may fall in


def check_valid_top16(row_sel, scores, own):
    """A selection row that differs from the oracle's on a near-tie must still be a
    top-16 of the oracle's scores up to the tie band: distinct ids, ascending, the own
    block in, 16 of them (or every block up to own); every older block it keeps scores
    at least thr - eps, and every older block scoring above thr + eps is kept, where
    thr is the oracle's 15th-best older score and eps = NEAR_TIE_BAND * |thr| + 1e-6."""
    ids = [int(i) for i in row_sel]
    row = [i for i in ids if i >= 0]
    assert all(i == -1 for i in ids[len(row):]), f"padding not at the end: {ids}"
    assert len(set(row)) == len(row), f"repeated block id: {row}"
    assert row == sorted(row) and own in row and len(row) == min(16, own + 1), (row, own)
    assert all(0 <= i <= own for i in row), (row, own)
    if own + 1 <= 16:
        return                                   # every visible block, nothing to rank
    older = np.asarray(scores[:own], np.float64)
    thr = np.sort(older)[::-1][14]
    eps = NEAR_TIE_BAND * abs(thr) + 1e-6
    kept = set(row)
    for i in kept - {own}:
        assert older[i] >= thr - eps, f"block {i} ({older[i]}) is below the 15th-best older score {thr}"
    missing = [int(i) for i in np.flatnonzero(older > thr + eps) if int(i) not in kept]
    assert not missing, f"blocks {missing} clearly above the 15th-best older score {thr} are not selected"


def compare_selection(gpu_sel, ora_sel, ora_bs, near_tie, seq_lens, T):
    """Bit-exact except near-tie rows; near-tie rows must still be a valid top-16."""
    gs, os_ = np.asarray(gpu_sel), np.asarray(ora_sel)
    mism = np.any(gs != os_, axis=-1)
    bad = mism & ~near_tie
    assert not bad.any(), f"{int(bad.sum())} selection rows differ outside near-ties, e.g. {np.argwhere(bad)[:3].tolist()}"
    for idx in np.argwhere(mism):
        b, t, g = idx
        L = int(seq_lens[b])
        own = (L - T + t) // 128
        check_valid_top16(gs[b, t, g], ora_bs[b, t, g], own)
    return int(mism.sum())


def compare_out(gpu_out, ora_out):
    d = np.abs(np.asarray(gpu_out, np.float64) - np.asarray(ora_out, np.float64))
    assert not np.isnan(d).any(), "NaN in attention output"
    assert d.max() <= OUT_MAX_ABS, f"attention max-abs {d.max():.3g}"
    assert d.mean() <= OUT_MEAN_ABS, f"attention mean-abs {d.mean():.3g}"
    return float(d.max()), float(d.mean())
