"""The C-ABI library loads on a host without a GPU, exports every function
include/msa.h declares, and rejects bad arguments before any HIP call."""
import ctypes
import math
import os
import re

import pytest

import block_sparse_attention_indexer_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if h.endswith(".h"):
            text = open(os.path.join(ROOT, "include", h)).read()
            names |= set(re.findall(r"^\s*(?:msa_status|size_t|const char\*|int)\s+(msa_\w+)\s*\(", text, re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(M.LIB_PATH):
        pytest.skip("libmsa.so not built")
    return M._lib()


def test_header_declares_the_binding_surface():
    assert declared_functions() == sorted(M.EXPORTED)


# The calls the boundary must carry, with their parameter types in order: the four
# steps of the method and the FP8 / NVFP4 pack and unpack helpers, plus the workspace
# query, the status string and the version.
REQUIRED = {
    "msa_indexer_scores": ("const msa_problem*", "const void*", "msa_dtype", "float", "const msa_cache*",
                           "msa_dequant", "float*", "float*", "hipStream_t"),
    "msa_block_topk": ("const msa_problem*", "const float*", "int32_t*", "void*", "size_t", "hipStream_t"),
    "msa_sparse_attn_decode": ("const msa_problem*", "const void*", "msa_dtype", "float", "const msa_cache*",
                               "const msa_cache*", "msa_dequant", "const int32_t*", "float", "float*", "float*",
                               "void*", "size_t", "hipStream_t"),
    "msa_workspace_size": ("const msa_problem*", "msa_call"),
    "msa_pack_fp8": ("const float*", "int64_t", "float", "uint8_t*", "hipStream_t"),
    "msa_unpack_fp8": ("const uint8_t*", "int64_t", "float", "float*", "hipStream_t"),
    "msa_pack_nvfp4": ("const float*", "int64_t", "int32_t", "float", "uint8_t*", "uint8_t*", "hipStream_t"),
    "msa_unpack_nvfp4": ("const uint8_t*", "const uint8_t*", "int64_t", "int32_t", "float", "msa_dequant",
                         "float*", "hipStream_t"),
    "msa_status_string": ("msa_status",),
    "msa_abi_version": ("void",),
}
REQUIRED["msa_sparse_attn_prefill"] = REQUIRED["msa_sparse_attn_decode"]


def header_signatures():
    text = open(os.path.join(ROOT, "include", "msa.h")).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    sigs = {}
    for name, params in re.findall(r"(?:msa_status|size_t|const char\*|int)\s+(msa_\w+)\s*\(([^)]*)\)\s*;", text):
        types = []
        for prm in params.split(","):
            prm = " ".join(prm.split())
            prm = re.sub(r"\s*\*\s*", "* ", prm).strip()
            toks = prm.split()
            if len(toks) > 1 and re.fullmatch(r"\w+", toks[-1]) and toks[-1] not in ("void",):
                toks = toks[:-1]                      # drop the parameter name
            types.append(" ".join(toks).replace("* ", "*").replace(" *", "*"))
        sigs[name] = tuple(types)
    return sigs


def test_header_carries_the_boundary_calls():
    sigs = header_signatures()
    for name, types in REQUIRED.items():
        assert name in sigs, name
        assert sigs[name] == types, (name, sigs[name])
    text = open(os.path.join(ROOT, "include", "msa.h")).read()
    assert re.search(r"MSA_DQ_FP8\s*=\s*0\s*,\s*MSA_DQ_EXACT\s*=\s*1", text)
    assert re.search(r"MSA_F32\s*=\s*0\s*,\s*MSA_FP8_E4M3\s*=\s*1\s*,\s*MSA_NVFP4\s*=\s*2", text)
    assert (M.MSA_DQ_FP8, M.MSA_DQ_EXACT) == (0, 1)
    # include/ declares the method's library only
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == ["msa.h"]


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.msa_abi_version() == 2
    # the benchmark's probes live in their own library, outside the product ABI
    assert not hasattr(lib, "msa_probe_stream_read") and not hasattr(lib, "msa_probe_mfma_f16")
    for s in range(5):
        assert lib.msa_status_string(s)


def _prob(**kw):
    d = dict(batch=2, tokens=1, groups=4, heads_per_group=16, head_dim=128, block_size=128, topk=16,
             seq_lens=64, block_table=128, max_blocks=8)
    d.update(kw)
    return M.msa_problem(**d)


def _cache(**kw):
    d = dict(dtype=M.MSA_NVFP4, data=256, scales=512, tensor_scale=0.5, heads=1, head_dim=128, num_pages=4)
    d.update(kw)
    return M.msa_cache(**d)


def idx(lib, prob, cache, q=1024, qd=M.MSA_FP8_E4M3, qs=1.0, dq=M.MSA_DQ_EXACT, bs=2048):
    return lib.msa_indexer_scores(ctypes.byref(prob) if prob is not None else None, q, qd, qs,
                                  ctypes.byref(cache) if cache is not None else None, dq, bs, None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(groups=8), M.MSA_ERR_UNSUPPORTED), (dict(head_dim=64), M.MSA_ERR_UNSUPPORTED),
    (dict(block_size=64), M.MSA_ERR_UNSUPPORTED), (dict(topk=8), M.MSA_ERR_UNSUPPORTED),
    (dict(heads_per_group=8), M.MSA_ERR_UNSUPPORTED), (dict(batch=0), M.MSA_ERR_INVALID_ARG),
    (dict(tokens=0), M.MSA_ERR_INVALID_ARG), (dict(max_blocks=0), M.MSA_ERR_INVALID_ARG),
    (dict(max_blocks=9000), M.MSA_ERR_UNSUPPORTED), (dict(seq_lens=None), M.MSA_ERR_INVALID_ARG),
    (dict(block_table=None), M.MSA_ERR_INVALID_ARG), (dict(seq_lens=66), M.MSA_ERR_INVALID_ARG),
])
def test_problem_validation(lib, kw, status):
    assert idx(lib, _prob(**kw), _cache()) == status


@pytest.mark.parametrize("kw,status", [
    (dict(data=None), M.MSA_ERR_INVALID_ARG), (dict(scales=None), M.MSA_ERR_INVALID_ARG),
    (dict(heads=4), M.MSA_ERR_INVALID_ARG), (dict(head_dim=64), M.MSA_ERR_UNSUPPORTED),
    (dict(tensor_scale=0.0), M.MSA_ERR_INVALID_ARG), (dict(tensor_scale=-1.0), M.MSA_ERR_INVALID_ARG),
    (dict(tensor_scale=math.inf), M.MSA_ERR_INVALID_ARG), (dict(num_pages=0), M.MSA_ERR_INVALID_ARG),
    (dict(dtype=7), M.MSA_ERR_UNSUPPORTED), (dict(data=257), M.MSA_ERR_INVALID_ARG),
])
def test_cache_validation(lib, kw, status):
    assert idx(lib, _prob(), _cache(**kw)) == status


def test_dtype_pairs_and_scalars(lib):
    assert idx(lib, None, _cache()) == M.MSA_ERR_INVALID_ARG
    assert idx(lib, _prob(), None) == M.MSA_ERR_INVALID_ARG
    assert idx(lib, _prob(), _cache(), qd=M.MSA_F32) == M.MSA_ERR_UNSUPPORTED          # f32 q, nvfp4 keys
    assert idx(lib, _prob(), _cache(dtype=M.MSA_F32), qd=M.MSA_FP8_E4M3) == M.MSA_ERR_UNSUPPORTED
    assert idx(lib, _prob(), _cache(), qs=0.0) == M.MSA_ERR_INVALID_ARG
    assert idx(lib, _prob(), _cache(), dq=5) == M.MSA_ERR_INVALID_ARG
    assert idx(lib, _prob(), _cache(), q=None) == M.MSA_ERR_INVALID_ARG
    assert idx(lib, _prob(), _cache(), bs=None) == M.MSA_ERR_INVALID_ARG


def test_attention_and_topk_validation(lib):
    p = _prob()
    kc = _cache(heads=4)
    args = lambda **o: dict(dict(q=1024, qd=M.MSA_FP8_E4M3, qs=1.0, k=kc, v=kc, dq=0, sel=4096, sm=0.088, out=8192), **o)

    def call(fn, a, prob=p):
        return fn(ctypes.byref(prob), a["q"], a["qd"], a["qs"], ctypes.byref(a["k"]), ctypes.byref(a["v"]),
                  a["dq"], a["sel"], a["sm"], a["out"], None, None, 0, None)
    assert call(lib.msa_sparse_attn_decode, args(sel=None)) == M.MSA_ERR_INVALID_ARG
    assert call(lib.msa_sparse_attn_decode, args(out=None)) == M.MSA_ERR_INVALID_ARG
    assert call(lib.msa_sparse_attn_decode, args(sm=0.0)) == M.MSA_ERR_INVALID_ARG
    # each scale valid, but their product (the logit scale) underflows or overflows a float
    assert call(lib.msa_sparse_attn_decode, args(sm=1e-30, qs=1e-30)) == M.MSA_ERR_INVALID_ARG
    assert call(lib.msa_sparse_attn_decode, args(sm=1e30, qs=1e30)) == M.MSA_ERR_INVALID_ARG
    assert call(lib.msa_sparse_attn_decode, args(v=_cache(heads=4, dtype=M.MSA_FP8_E4M3))) == M.MSA_ERR_UNSUPPORTED
    assert call(lib.msa_sparse_attn_decode, args(k=_cache(heads=1))) == M.MSA_ERR_INVALID_ARG
    assert call(lib.msa_sparse_attn_decode, args(), prob=_prob(tokens=9)) == M.MSA_ERR_UNSUPPORTED
    assert lib.msa_block_topk(ctypes.byref(p), None, 4096, None, 0, None) == M.MSA_ERR_INVALID_ARG
    assert lib.msa_block_topk(ctypes.byref(p), 4096, None, None, 0, None) == M.MSA_ERR_INVALID_ARG
    assert lib.msa_workspace_size(ctypes.byref(p), M.MSA_CALL_TOPK) == 0
    assert lib.msa_workspace_size(ctypes.byref(p), M.MSA_CALL_ATTN) == 0


def test_pack_validation(lib):
    assert lib.msa_pack_nvfp4(None, 1, 128, 1.0, 64, 64, None) == M.MSA_ERR_INVALID_ARG
    assert lib.msa_pack_nvfp4(64, 1, 100, 1.0, 64, 64, None) == M.MSA_ERR_INVALID_ARG
    assert lib.msa_pack_nvfp4(64, 1, 128, 0.0, 64, 64, None) == M.MSA_ERR_INVALID_ARG
    assert lib.msa_pack_nvfp4(64, 0, 128, 1.0, 64, 64, None) == M.MSA_OK          # empty: no launch
    assert lib.msa_unpack_nvfp4(64, 64, 1, 128, 1.0, 9, 64, None) == M.MSA_ERR_INVALID_ARG
    assert lib.msa_pack_fp8(None, 4, 1.0, 64, None) == M.MSA_ERR_INVALID_ARG
    assert lib.msa_pack_fp8(64, -1, 1.0, 64, None) == M.MSA_ERR_INVALID_ARG
    assert lib.msa_pack_fp8(64, 0, 1.0, 64, None) == M.MSA_OK
    assert lib.msa_unpack_fp8(64, 4, float("nan"), 64, None) == M.MSA_ERR_INVALID_ARG


def test_indexer_topk_validation(lib):
    p = _prob()
    c = _cache()
    def call(prob=p, sel=4096, ws=8192, ws_bytes=64):
        return lib.msa_indexer_topk(ctypes.byref(prob), 1024, M.MSA_FP8_E4M3, 1.0, ctypes.byref(c), 0, 2048, sel,
                                    ws, ws_bytes, None)
    assert lib.msa_workspace_size(ctypes.byref(p), M.MSA_CALL_INDEXER_TOPK) == 2 * 4
    assert call(sel=None) == M.MSA_ERR_INVALID_ARG
    assert call(ws=None) == M.MSA_ERR_WORKSPACE
    assert call(ws_bytes=4) == M.MSA_ERR_WORKSPACE
    assert call(ws=8193) == M.MSA_ERR_WORKSPACE
    assert call(prob=_prob(topk=8)) == M.MSA_ERR_UNSUPPORTED


def test_indexer_topk_noalloc_validation(lib):
    """The allocation-free call rejects a batch beyond its scratch before any HIP call."""
    c = _cache()

    def call(prob, sel=4096):
        return lib.msa_indexer_topk_noalloc(ctypes.byref(prob), 1024, M.MSA_FP8_E4M3, 1.0, ctypes.byref(c), 0, 2048,
                                            sel, None)
    assert call(_prob(batch=M.MSA_NOALLOC_MAX_BATCH + 1)) == M.MSA_ERR_UNSUPPORTED
    assert call(_prob(), sel=None) == M.MSA_ERR_INVALID_ARG
    assert call(_prob(topk=8)) == M.MSA_ERR_UNSUPPORTED


def test_decode_step_validation(lib):
    p = _prob()
    ik = _cache()
    kv = _cache(heads=4)
    def call(prob=p, idx_k=ik, k=kv, v=kv, sel=4096, out=8192, ws=16384, ws_bytes=64, qs=1.0, sm=0.1,
             q_dtype=M.MSA_FP8_E4M3):
        return lib.msa_decode_step(ctypes.byref(prob), 1024, M.MSA_FP8_E4M3, 1.0, ctypes.byref(idx_k), 3072,
                                   q_dtype, qs, ctypes.byref(k), ctypes.byref(v), M.MSA_DQ_EXACT, sm, 2048, sel,
                                   out, None, ws, ws_bytes, None)
    assert lib.msa_workspace_size(ctypes.byref(p), M.MSA_CALL_DECODE_STEP) == 0   # no workspace needed
    assert call(sel=None) == M.MSA_ERR_INVALID_ARG
    assert call(out=None) == M.MSA_ERR_INVALID_ARG
    assert call(out=8196) == M.MSA_ERR_INVALID_ARG          # misaligned
    assert call(qs=0.0) == M.MSA_ERR_INVALID_ARG
    assert call(sm=float("nan")) == M.MSA_ERR_INVALID_ARG
    assert call(prob=_prob(tokens=9)) == M.MSA_ERR_UNSUPPORTED
    assert call(v=_cache(heads=4, dtype=M.MSA_FP8_E4M3)) == M.MSA_ERR_UNSUPPORTED   # K and V differ
    assert call(k=_cache(heads=1)) == M.MSA_ERR_INVALID_ARG                          # K/V need 4 heads
    assert call(q_dtype=M.MSA_F32) == M.MSA_ERR_UNSUPPORTED


def test_cache_insert_validation(lib):
    p = _prob()
    def call(prob=p, x=1024, c=None):
        c = _cache(heads=4) if c is None else c
        return lib.msa_cache_insert(ctypes.byref(prob), x, ctypes.byref(c), None)
    assert call(x=None) == M.MSA_ERR_INVALID_ARG
    assert call(x=1032) == M.MSA_ERR_INVALID_ARG                       # rows need 16-byte alignment
    assert call(c=_cache(heads=2)) == M.MSA_ERR_INVALID_ARG            # 1 (index keys) or 4 (K, V)
    assert call(c=_cache(heads=4, scales=None)) == M.MSA_ERR_INVALID_ARG
    assert call(c=_cache(heads=4, tensor_scale=0.0)) == M.MSA_ERR_INVALID_ARG
    assert call(prob=_prob(block_size=64)) == M.MSA_ERR_UNSUPPORTED


def test_dcp_validation(lib):
    p = _prob()
    c = _cache()

    def shard_scan(prob=p, shard=0, n=4, q=1024, cache=c, bs=2048, qd=M.MSA_FP8_E4M3):
        return lib.msa_indexer_scores_shard(ctypes.byref(prob), shard, n, q, qd, 1.0, ctypes.byref(cache),
                                            M.MSA_DQ_EXACT, bs, None)

    assert shard_scan(n=0) == M.MSA_ERR_INVALID_ARG
    assert shard_scan(n=M.MSA_MAX_SHARDS + 1) == M.MSA_ERR_INVALID_ARG
    assert shard_scan(shard=4) == M.MSA_ERR_INVALID_ARG
    assert shard_scan(shard=-1) == M.MSA_ERR_INVALID_ARG
    assert shard_scan(prob=_prob(tokens=9)) == M.MSA_ERR_UNSUPPORTED          # decode and speculative only
    assert shard_scan(cache=_cache(dtype=M.MSA_F32, scales=None), qd=M.MSA_F32) == M.MSA_ERR_UNSUPPORTED
    assert shard_scan(bs=None) == M.MSA_ERR_INVALID_ARG
    assert shard_scan(q=1032) == M.MSA_ERR_INVALID_ARG

    def local(prob=p, shard=1, n=4, bs=2048, cs=4096, cb=8192):
        return lib.msa_shard_topk(ctypes.byref(prob), shard, n, bs, cs, cb, None)

    assert local(shard=4) == M.MSA_ERR_INVALID_ARG
    assert local(cs=None) == M.MSA_ERR_INVALID_ARG
    assert local(cb=8194) == M.MSA_ERR_INVALID_ARG
    assert local(prob=_prob(topk=8)) == M.MSA_ERR_UNSUPPORTED

    def merge(prob=p, n=4, cs=4096, cb=8192, sel=16384):
        return lib.msa_topk_merge(ctypes.byref(prob), n, cs, cb, sel, None)

    assert merge(n=0) == M.MSA_ERR_INVALID_ARG
    assert merge(n=9) == M.MSA_ERR_INVALID_ARG
    assert merge(sel=None) == M.MSA_ERR_INVALID_ARG
    assert merge(prob=_prob(batch=0)) == M.MSA_ERR_INVALID_ARG


def test_indexer_prefix_validation(lib):
    p = _prob(batch=4)
    ws_need = lib.msa_workspace_size(ctypes.byref(p), M.MSA_CALL_INDEXER_PREFIX)
    assert ws_need == 16

    def call(prob=p, gs=(0, 2, 4), pb=(3, 1), ws=4096, wsb=16, cache=None, qd=M.MSA_FP8_E4M3):
        n = len(pb)
        g = (ctypes.c_int32 * (n + 1))(*gs) if gs is not None else None
        b = (ctypes.c_int32 * max(n, 1))(*pb) if pb is not None else None
        c = _cache() if cache is None else cache
        return lib.msa_indexer_scores_prefix(ctypes.byref(prob), n, ctypes.cast(g, ctypes.c_void_p) if g else None,
                                             ctypes.cast(b, ctypes.c_void_p) if b else None, 1024, qd, 1.0,
                                             ctypes.byref(c), M.MSA_DQ_EXACT, 2048, ws, wsb, None)

    assert call(gs=(0, 2, 2)) == M.MSA_ERR_INVALID_ARG              # empty group
    assert call(gs=(0, 2, 5)) == M.MSA_ERR_INVALID_ARG              # past the batch
    assert call(gs=(1, 0, 4)) == M.MSA_ERR_INVALID_ARG              # decreasing
    assert call(pb=(3, 9)) == M.MSA_ERR_INVALID_ARG                 # more blocks than max_blocks
    assert call(pb=(-1, 1)) == M.MSA_ERR_INVALID_ARG
    assert call(gs=None) == M.MSA_ERR_INVALID_ARG
    assert call(wsb=12) == M.MSA_ERR_WORKSPACE
    assert call(ws=None) == M.MSA_ERR_WORKSPACE
    assert call(prob=_prob(batch=4, tokens=9)) == M.MSA_ERR_UNSUPPORTED
    assert call(cache=_cache(dtype=M.MSA_F32, scales=None), qd=M.MSA_F32) == M.MSA_ERR_UNSUPPORTED
    big = _prob(batch=70)
    gs = (0, 65)
    assert call(prob=big, gs=gs, pb=(1,), wsb=4 * 70) == M.MSA_ERR_INVALID_ARG   # more than 64 sequences


def test_sparse_attn_decode_prefix_validation(lib):
    p = _prob(batch=4)
    k = _cache(heads=4)
    gs = (ctypes.c_int32 * 3)(0, 2, 4)
    pb = (ctypes.c_int32 * 2)(3, 1)
    need = lib.msa_sparse_attn_prefix_workspace_size(ctypes.byref(p), 2, ctypes.cast(gs, ctypes.c_void_p),
                                                     ctypes.cast(pb, ctypes.c_void_p))
    # 4 heads x (3 + 1) slots of 64 KiB, plus the slot map, ids and counts
    assert need >= 4 * 4 * 65536

    def call(prob=p, n=2, g=gs, b=pb, kk=None, ws=1 << 20, wsb=None, sel=4096, qs=1.0):
        kk = k if kk is None else kk
        wsb = need if wsb is None else wsb
        return lib.msa_sparse_attn_decode_prefix(ctypes.byref(prob), n, ctypes.cast(g, ctypes.c_void_p) if g else None,
                                                 ctypes.cast(b, ctypes.c_void_p) if b else None, 8192,
                                                 M.MSA_FP8_E4M3, qs, ctypes.byref(kk), ctypes.byref(kk),
                                                 M.MSA_DQ_EXACT, sel, 0.088, 16384, None, ws, wsb, None)
    assert call(wsb=need - 1) == M.MSA_ERR_WORKSPACE
    assert call(ws=None) == M.MSA_ERR_WORKSPACE
    assert call(ws=(1 << 20) + 16) == M.MSA_ERR_WORKSPACE                 # not 256-byte aligned
    assert call(g=(ctypes.c_int32 * 3)(0, 2, 2)) == M.MSA_ERR_INVALID_ARG  # empty group
    assert call(b=(ctypes.c_int32 * 2)(3, 99)) == M.MSA_ERR_INVALID_ARG    # past max_blocks
    assert call(g=None) == M.MSA_ERR_INVALID_ARG
    assert call(n=65) == M.MSA_ERR_INVALID_ARG
    assert call(sel=None) == M.MSA_ERR_INVALID_ARG
    assert call(qs=0.0) == M.MSA_ERR_INVALID_ARG
    assert call(prob=_prob(batch=4, tokens=9)) == M.MSA_ERR_UNSUPPORTED
    assert call(kk=_cache(heads=4, dtype=M.MSA_F32, scales=None)) == M.MSA_ERR_UNSUPPORTED
    assert lib.msa_sparse_attn_prefix_workspace_size(ctypes.byref(p), 65, None, None) == 0


def test_topk_sparse_attn_validation(lib):
    p = _prob()
    k = _cache(heads=4)

    def call(bs=2048, sel=4096, q=8192, out=16384, kk=None, vv=None, prob=p):
        kk = k if kk is None else kk
        vv = k if vv is None else vv
        return lib.msa_topk_sparse_attn(ctypes.byref(prob), bs, sel, q, M.MSA_FP8_E4M3, 1.0, ctypes.byref(kk),
                                        ctypes.byref(vv), M.MSA_DQ_EXACT, 0.088, out, None, None)

    assert call(bs=None) == M.MSA_ERR_INVALID_ARG
    assert call(bs=2050) == M.MSA_ERR_INVALID_ARG
    assert call(sel=None) == M.MSA_ERR_INVALID_ARG
    assert call(out=16388) == M.MSA_ERR_INVALID_ARG
    assert call(kk=_cache(heads=1)) == M.MSA_ERR_INVALID_ARG
    assert call(vv=_cache(heads=4, dtype=M.MSA_FP8_E4M3, scales=None)) == M.MSA_ERR_UNSUPPORTED


def test_cache_insert_many_validation(lib):
    p = _prob()

    def call(n=2, xs=(1024, 2048), caches=None, prob=p):
        cs = caches if caches is not None else [_cache(heads=4), _cache(heads=1)]
        xa = (ctypes.c_void_p * max(len(xs), 1))(*xs) if xs is not None else None
        ca = (M.msa_cache * max(len(cs), 1))(*cs)
        return lib.msa_cache_insert_many(ctypes.byref(prob), n, ctypes.cast(xa, ctypes.c_void_p) if xa else None,
                                         ctypes.cast(ca, ctypes.c_void_p), None)

    assert call(n=0) == M.MSA_ERR_INVALID_ARG
    assert call(n=5, xs=(1024,) * 5, caches=[_cache(heads=4)] * 5) == M.MSA_ERR_INVALID_ARG
    assert call(xs=None) == M.MSA_ERR_INVALID_ARG
    assert call(xs=(1024, 2056)) == M.MSA_ERR_INVALID_ARG                   # misaligned rows
    assert call(caches=[_cache(heads=4), _cache(heads=2)]) == M.MSA_ERR_INVALID_ARG
    assert call(caches=[_cache(heads=4), _cache(heads=1, tensor_scale=0.0)]) == M.MSA_ERR_INVALID_ARG
    assert call(prob=_prob(block_size=64)) == M.MSA_ERR_UNSUPPORTED


def test_library_binds_to_torchs_hip_runtime():
    # loading the library first must not pull in a second HIP runtime next to torch's
    import subprocess
    import sys
    code = ("import os, sys; sys.path.insert(0, %r); import block_sparse_attention_indexer_amd as M; M._lib(); "
            "m = open('/proc/%%d/maps' %% os.getpid()).read(); "
            "print(len(set(l.split()[-1] for l in m.splitlines() if 'amdhip64' in l)))") % ROOT
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "1"


def test_bench_probe_library_validation():
    import bench_probes as BP
    if not os.path.exists(BP.LIB_PATH):
        pytest.skip("libmsa_probe.so not built")
    lib = BP._lib()
    assert lib.msa_probe_stream_read(None, 64, 4096, None) == M.MSA_ERR_INVALID_ARG
    assert lib.msa_probe_stream_read(64, 0, 4096, None) == M.MSA_ERR_INVALID_ARG
    assert lib.msa_probe_stream_read(64, 100, 4096, None) == M.MSA_ERR_INVALID_ARG     # not a multiple of 16
    assert lib.msa_probe_stream_read(72, 64, 4096, None) == M.MSA_ERR_INVALID_ARG      # not 16-byte aligned
    assert lib.msa_probe_stream_read(64, 64, None, None) == M.MSA_ERR_INVALID_ARG
    assert lib.msa_probe_mfma_f16(None, 1, 1, None) == M.MSA_ERR_INVALID_ARG
    assert lib.msa_probe_mfma_f16(64, 0, 1, None) == M.MSA_ERR_INVALID_ARG
    assert lib.msa_probe_mfma_f16(64, 1, 0, None) == M.MSA_ERR_INVALID_ARG
