"""Python binding of libmsa, the MI355X (gfx950) MSA hot path.

Argument marshalling only: every step runs in the HIP kernels of libmsa.so
(see include/msa.h for the contract of each call).  torch supplies device
memory and the current stream; nothing here computes on the CPU, and if the
library is missing every call raises instead of falling back.

The functions keep the C names: msa_indexer_scores, msa_indexer_topk, msa_block_topk,
msa_sparse_attn_decode, msa_sparse_attn_prefill, msa_decode_step, msa_cache_insert,
msa_indexer_scores_shard, msa_shard_topk, msa_topk_merge, msa_indexer_scores_prefix,
msa_topk_sparse_attn, msa_cache_insert_many, msa_pack_fp8,
msa_unpack_fp8, msa_pack_nvfp4, msa_unpack_nvfp4, msa_workspace_size.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmsa.so")

MSA_OK, MSA_ERR_INVALID_ARG, MSA_ERR_UNSUPPORTED, MSA_ERR_WORKSPACE, MSA_ERR_HIP = range(5)
MSA_F32, MSA_FP8_E4M3, MSA_NVFP4 = 0, 1, 2
MSA_DQ_FP8, MSA_DQ_EXACT = 0, 1
MSA_MAX_SHARDS = 8
MSA_CALL_INDEXER, MSA_CALL_TOPK, MSA_CALL_ATTN, MSA_CALL_INDEXER_TOPK, MSA_CALL_DECODE_STEP = 0, 1, 2, 3, 4
MSA_CALL_INDEXER_PREFIX = 5
MSA_MAX_PREFIX_GROUPS = MSA_MAX_PREFIX_SEQS = 64
MSA_MAX_INSERTS = 4

EXPORTED = ("msa_indexer_scores", "msa_indexer_topk", "msa_block_topk", "msa_sparse_attn_decode",
            "msa_decode_step", "msa_cache_insert", "msa_indexer_scores_shard", "msa_shard_topk",
            "msa_topk_merge", "msa_indexer_scores_prefix", "msa_topk_sparse_attn", "msa_cache_insert_many",
            "msa_sparse_attn_prefill", "msa_workspace_size", "msa_pack_fp8", "msa_unpack_fp8",
            "msa_pack_nvfp4", "msa_unpack_nvfp4", "msa_status_string", "msa_abi_version",
            "msa_indexer_topk_noalloc", "msa_sparse_attn_decode_prefix", "msa_sparse_attn_prefix_workspace_size")
MSA_NOALLOC_MAX_BATCH = 4096

DTYPES = {"f32": MSA_F32, "fp8": MSA_FP8_E4M3, "nvfp4": MSA_NVFP4}
DEQUANT = {"exact": MSA_DQ_EXACT, "fp8": MSA_DQ_FP8}


class MsaError(RuntimeError):
    def __init__(self, status, call):
        self.status = status
        super().__init__(f"{call}: {_lib().msa_status_string(status).decode()} (status {status})")


class msa_cache(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("data", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("tensor_scale", ctypes.c_float), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("num_pages", ctypes.c_int64)]


class msa_problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("tokens", ctypes.c_int32), ("groups", ctypes.c_int32),
                ("heads_per_group", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("seq_lens", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("max_blocks", ctypes.c_int32)]


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                               "python -m block_sparse_attention_indexer_amd.build")
        # torch first: its bundled HIP runtime is then the one libmsa binds to.  Loaded
        # the other way round, the process would hold two HIP runtimes, and torch's
        # streams and device pointers would be foreign to the library's launches.
        import torch  # noqa: F401
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        P = ctypes.POINTER
        sig = {
            "msa_indexer_scores": [P(msa_problem), vp, ctypes.c_int, f32, P(msa_cache), ctypes.c_int, vp, vp, vp],
            "msa_indexer_topk": [P(msa_problem), vp, ctypes.c_int, f32, P(msa_cache), ctypes.c_int, vp, vp, vp,
                                 sz, vp],
            "msa_block_topk": [P(msa_problem), vp, vp, vp, sz, vp],
            "msa_indexer_topk_noalloc": [P(msa_problem), vp, ctypes.c_int, f32, P(msa_cache), ctypes.c_int, vp, vp,
                                         vp],
            "msa_sparse_attn_decode": [P(msa_problem), vp, ctypes.c_int, f32, P(msa_cache), P(msa_cache),
                                       ctypes.c_int, vp, f32, vp, vp, vp, sz, vp],
            "msa_sparse_attn_prefill": [P(msa_problem), vp, ctypes.c_int, f32, P(msa_cache), P(msa_cache),
                                        ctypes.c_int, vp, f32, vp, vp, vp, sz, vp],
            "msa_decode_step": [P(msa_problem), vp, ctypes.c_int, f32, P(msa_cache), vp, ctypes.c_int, f32,
                                P(msa_cache), P(msa_cache), ctypes.c_int, f32, vp, vp, vp, vp, vp, sz, vp],
            "msa_cache_insert": [P(msa_problem), vp, P(msa_cache), vp],
            "msa_cache_insert_many": [P(msa_problem), i32, vp, vp, vp],
            "msa_indexer_scores_shard": [P(msa_problem), i32, i32, vp, ctypes.c_int, f32, P(msa_cache),
                                         ctypes.c_int, vp, vp],
            "msa_shard_topk": [P(msa_problem), i32, i32, vp, vp, vp, vp],
            "msa_topk_merge": [P(msa_problem), i32, vp, vp, vp, vp],
            "msa_indexer_scores_prefix": [P(msa_problem), i32, vp, vp, vp, ctypes.c_int, f32, P(msa_cache),
                                          ctypes.c_int, vp, vp, sz, vp],
            "msa_sparse_attn_decode_prefix": [P(msa_problem), i32, vp, vp, vp, ctypes.c_int, f32, P(msa_cache),
                                              P(msa_cache), ctypes.c_int, vp, f32, vp, vp, vp, sz, vp],
            "msa_sparse_attn_prefix_workspace_size": [P(msa_problem), i32, vp, vp],
            "msa_topk_sparse_attn": [P(msa_problem), vp, vp, vp, ctypes.c_int, f32, P(msa_cache), P(msa_cache),
                                     ctypes.c_int, f32, vp, vp, vp],
            "msa_workspace_size": [P(msa_problem), ctypes.c_int],
            "msa_pack_fp8": [vp, i64, f32, vp, vp],
            "msa_unpack_fp8": [vp, i64, f32, vp, vp],
            "msa_pack_nvfp4": [vp, i64, i32, f32, vp, vp, vp],
            "msa_unpack_nvfp4": [vp, vp, i64, i32, f32, ctypes.c_int, vp, vp],
            "msa_status_string": [ctypes.c_int],
            "msa_abi_version": [],
        }
        for name, args in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        lib.msa_workspace_size.restype = sz
        lib.msa_sparse_attn_prefix_workspace_size.restype = sz
        lib.msa_status_string.restype = ctypes.c_char_p
        _LIB = lib
    return _LIB


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmsa must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status, call):
    if status != MSA_OK:
        raise MsaError(status, call)


def problem(seq_lens, block_table, tokens):
    """msa_problem for device int32 seq_lens [B] and block_table [B, max_blocks]."""
    p = msa_problem(batch=int(seq_lens.shape[0]), tokens=int(tokens), groups=4, heads_per_group=16,
                    head_dim=128, block_size=128, topk=16, seq_lens=_ptr(seq_lens),
                    block_table=_ptr(block_table), max_blocks=int(block_table.shape[1]))
    p._keep = (seq_lens, block_table)
    return p


def cache(dtype, data, scales=None, tensor_scale=1.0, heads=1):
    """msa_cache over a device page pool (data: floats, FP8 bytes or NVFP4 codes)."""
    per_page = heads * 128 * (128 * 4 if dtype == "f32" else 128 if dtype == "fp8" else 64)
    nbytes = data.numel() * data.element_size()
    c = msa_cache(dtype=DTYPES[dtype], data=_ptr(data), scales=_ptr(scales),
                  tensor_scale=float(tensor_scale), heads=int(heads), head_dim=128,
                  num_pages=int(nbytes // per_page))
    c._keep = (data, scales)
    return c


def msa_indexer_scores(prob, idx_q, q_dtype, q_scale, idx_k, dequant, block_scores,
                       token_scores=None, stream=None):
    _check(_lib().msa_indexer_scores(ctypes.byref(prob), _ptr(idx_q), DTYPES[q_dtype], float(q_scale),
                                     ctypes.byref(idx_k), DEQUANT[dequant], _ptr(block_scores),
                                     _ptr(token_scores), _stream(stream)), "msa_indexer_scores")


def msa_indexer_topk(prob, idx_q, q_dtype, q_scale, idx_k, dequant, block_scores, sel, workspace,
                     stream=None):
    """Steps 1-3 in one call; `workspace`: a zero-filled device tensor of at least
    msa_workspace_size(prob, MSA_CALL_INDEXER_TOPK) bytes (left zero-filled)."""
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib().msa_indexer_topk(ctypes.byref(prob), _ptr(idx_q), DTYPES[q_dtype], float(q_scale),
                                   ctypes.byref(idx_k), DEQUANT[dequant], _ptr(block_scores), _ptr(sel),
                                   _ptr(workspace), ws_bytes, _stream(stream)), "msa_indexer_topk")


def msa_indexer_topk_noalloc(prob, idx_q, q_dtype, q_scale, idx_k, dequant, block_scores, sel, stream=None):
    """msa_indexer_topk without a workspace: the library's own per-GPU scratch array
    holds the arrival counters (at most MSA_NOALLOC_MAX_BATCH sequences; calls that
    overlap on one GPU race on it)."""
    _check(_lib().msa_indexer_topk_noalloc(ctypes.byref(prob), _ptr(idx_q), DTYPES[q_dtype], float(q_scale),
                                           ctypes.byref(idx_k), DEQUANT[dequant], _ptr(block_scores), _ptr(sel),
                                           _stream(stream)), "msa_indexer_topk_noalloc")


def msa_indexer_scores_shard(prob, shard, num_shards, idx_q, q_dtype, q_scale, idx_k, dequant, block_scores,
                             stream=None):
    _check(_lib().msa_indexer_scores_shard(ctypes.byref(prob), int(shard), int(num_shards), _ptr(idx_q),
                                           DTYPES[q_dtype], float(q_scale), ctypes.byref(idx_k),
                                           DEQUANT[dequant], _ptr(block_scores), _stream(stream)),
           "msa_indexer_scores_shard")


def msa_shard_topk(prob, shard, num_shards, block_scores, cand_scores, cand_blocks, stream=None):
    _check(_lib().msa_shard_topk(ctypes.byref(prob), int(shard), int(num_shards), _ptr(block_scores),
                                 _ptr(cand_scores), _ptr(cand_blocks), _stream(stream)), "msa_shard_topk")


def msa_topk_merge(prob, num_shards, cand_scores, cand_blocks, sel, stream=None):
    _check(_lib().msa_topk_merge(ctypes.byref(prob), int(num_shards), _ptr(cand_scores), _ptr(cand_blocks),
                                 _ptr(sel), _stream(stream)), "msa_topk_merge")


def msa_indexer_scores_prefix(prob, group_start, prefix_blocks, idx_q, q_dtype, q_scale, idx_k, dequant,
                              block_scores, workspace, stream=None):
    """group_start / prefix_blocks: host sequences of ints (num_groups + 1 and num_groups
    entries); workspace: a device tensor of at least
    msa_workspace_size(prob, MSA_CALL_INDEXER_PREFIX) bytes."""
    n = len(prefix_blocks)
    gs = (ctypes.c_int32 * (n + 1))(*[int(x) for x in group_start])
    pb = (ctypes.c_int32 * max(n, 1))(*[int(x) for x in prefix_blocks])
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(_lib().msa_indexer_scores_prefix(ctypes.byref(prob), n, ctypes.cast(gs, ctypes.c_void_p),
                                            ctypes.cast(pb, ctypes.c_void_p), _ptr(idx_q), DTYPES[q_dtype],
                                            float(q_scale), ctypes.byref(idx_k), DEQUANT[dequant],
                                            _ptr(block_scores), _ptr(workspace), ws_bytes, _stream(stream)),
           "msa_indexer_scores_prefix")


def _groups(group_start, prefix_blocks):
    n = len(prefix_blocks)
    gs = (ctypes.c_int32 * (n + 1))(*[int(x) for x in group_start])
    pb = (ctypes.c_int32 * max(n, 1))(*[int(x) for x in prefix_blocks])
    return n, gs, pb


def msa_sparse_attn_prefix_workspace_size(prob, group_start, prefix_blocks):
    n, gs, pb = _groups(group_start, prefix_blocks)
    return int(_lib().msa_sparse_attn_prefix_workspace_size(ctypes.byref(prob), n, ctypes.cast(gs, ctypes.c_void_p),
                                                             ctypes.cast(pb, ctypes.c_void_p)))


def msa_sparse_attn_decode_prefix(prob, group_start, prefix_blocks, q, q_dtype, q_scale, k, v, dequant, sel,
                                  softmax_scale, out, lse=None, workspace=None, stream=None):
    """Decode attention with shared-prefix blocks dequantised once per group (see
    include/msa.h); workspace: a 256-byte aligned device tensor of at least
    msa_sparse_attn_prefix_workspace_size(prob, group_start, prefix_blocks) bytes."""
    n, gs, pb = _groups(group_start, prefix_blocks)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib().msa_sparse_attn_decode_prefix(ctypes.byref(prob), n, ctypes.cast(gs, ctypes.c_void_p),
                                                ctypes.cast(pb, ctypes.c_void_p), _ptr(q), DTYPES[q_dtype],
                                                float(q_scale), ctypes.byref(k), ctypes.byref(v), DEQUANT[dequant],
                                                _ptr(sel), float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                                ws_bytes, _stream(stream)), "msa_sparse_attn_decode_prefix")


def msa_topk_sparse_attn(prob, block_scores, sel, q, q_dtype, q_scale, k, v, dequant, softmax_scale, out,
                         lse=None, stream=None):
    _check(_lib().msa_topk_sparse_attn(ctypes.byref(prob), _ptr(block_scores), _ptr(sel), _ptr(q), DTYPES[q_dtype],
                                       float(q_scale), ctypes.byref(k), ctypes.byref(v), DEQUANT[dequant],
                                       float(softmax_scale), _ptr(out), _ptr(lse), _stream(stream)),
           "msa_topk_sparse_attn")


def msa_block_topk(prob, block_scores, sel, workspace=None, stream=None):
    """Step 3; msa_workspace_size(prob, MSA_CALL_TOPK) is 0, so workspace may be None."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib().msa_block_topk(ctypes.byref(prob), _ptr(block_scores), _ptr(sel), _ptr(workspace), ws_bytes,
                                 _stream(stream)), "msa_block_topk")


def _attn(name, prob, q, q_dtype, q_scale, k, v, dequant, sel, softmax_scale, out, lse=None,
          workspace=None, stream=None):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    fn = getattr(_lib(), name)
    _check(fn(ctypes.byref(prob), _ptr(q), DTYPES[q_dtype], float(q_scale), ctypes.byref(k),
              ctypes.byref(v), DEQUANT[dequant], _ptr(sel), float(softmax_scale), _ptr(out),
              _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)), name)


def msa_sparse_attn_decode(*args, **kw):
    _attn("msa_sparse_attn_decode", *args, **kw)


def msa_sparse_attn_prefill(*args, **kw):
    _attn("msa_sparse_attn_prefill", *args, **kw)


def msa_decode_step(prob, idx_q, idx_q_dtype, idx_q_scale, idx_k, q, q_dtype, q_scale, k, v, dequant,
                    softmax_scale, block_scores, sel, out, lse=None, workspace=None, stream=None):
    """One decode layer step (steps 1-4) in one call (two launches); no workspace is needed."""
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib().msa_decode_step(ctypes.byref(prob), _ptr(idx_q), DTYPES[idx_q_dtype], float(idx_q_scale),
                                  ctypes.byref(idx_k), _ptr(q), DTYPES[q_dtype], float(q_scale), ctypes.byref(k),
                                  ctypes.byref(v), DEQUANT[dequant], float(softmax_scale), _ptr(block_scores),
                                  _ptr(sel), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)),
           "msa_decode_step")


def msa_cache_insert_many(prob, xs, caches, stream=None):
    """Several quantise-and-inserts in one launch: xs[i] into caches[i] (msa_cache objects)."""
    n = len(xs)
    ptrs = (ctypes.c_void_p * n)(*[_ptr(x) for x in xs])
    arr = (msa_cache * n)(*caches)
    _check(_lib().msa_cache_insert_many(ctypes.byref(prob), n, ctypes.cast(ptrs, ctypes.c_void_p),
                                        ctypes.cast(arr, ctypes.c_void_p), _stream(stream)), "msa_cache_insert_many")


def msa_cache_insert(prob, x, cache_, stream=None):
    """Quantise the fp32 rows x [B, T, heads, 128] of the T new tokens and write them
    into their slots of the paged cache `cache_` (its data and scales are written)."""
    _check(_lib().msa_cache_insert(ctypes.byref(prob), _ptr(x), ctypes.byref(cache_), _stream(stream)),
           "msa_cache_insert")


def msa_workspace_size(prob, which):
    return int(_lib().msa_workspace_size(ctypes.byref(prob), int(which)))


def msa_pack_fp8(x, scale, out, stream=None):
    _check(_lib().msa_pack_fp8(_ptr(x), x.numel(), float(scale), _ptr(out), _stream(stream)), "msa_pack_fp8")


def msa_unpack_fp8(x, scale, out, stream=None):
    _check(_lib().msa_unpack_fp8(_ptr(x), x.numel(), float(scale), _ptr(out), _stream(stream)), "msa_unpack_fp8")


def msa_pack_nvfp4(x, tensor_scale, codes, scales, stream=None):
    row_len = int(x.shape[-1])
    rows = x.numel() // row_len
    _check(_lib().msa_pack_nvfp4(_ptr(x), rows, row_len, float(tensor_scale), _ptr(codes), _ptr(scales),
                                 _stream(stream)), "msa_pack_nvfp4")


def msa_unpack_nvfp4(codes, scales, row_len, tensor_scale, dequant, out, stream=None):
    rows = out.numel() // row_len
    _check(_lib().msa_unpack_nvfp4(_ptr(codes), _ptr(scales), rows, int(row_len), float(tensor_scale),
                                   DEQUANT[dequant], _ptr(out), _stream(stream)), "msa_unpack_nvfp4")


def abi_version():
    return int(_lib().msa_abi_version())
