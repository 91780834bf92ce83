"""The allocation-free entry point msa_indexer_topk_noalloc against msa_indexer_topk
(the same call with a caller workspace), through the C ABI: block scores and
selection bit for bit, on two calls in a row with the second on a smaller batch
(the library's scratch keeps the previous call's contents), for the fused
one-token scan and for shapes that run the two kernels."""
import numpy as np
import pytest
import torch

from tests import harness as H

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[gpu-test]", *a, flush=True)


def _run(M, case, B, dequant, noalloc, ws=None):
    w, lay = case.w, case.lay
    prob = M.problem(case.d_seq[:B], case.d_table[:B], w.T)
    bs = torch.full((B, w.T, 4, lay.max_blocks), float("nan"), dtype=torch.float32, device="cuda")
    sel = torch.full((B, w.T, 4, 16), -7, dtype=torch.int32, device="cuda")
    if noalloc:
        M.msa_indexer_topk_noalloc(prob, case.d_idx_q[:B], w.q_dtype, case.idx_q_scale, case.d_caches["idx_k"][2],
                                   dequant, bs, sel)
    else:
        M.msa_indexer_topk(prob, case.d_idx_q[:B], w.q_dtype, case.idx_q_scale, case.d_caches["idx_k"][2], dequant,
                           bs, sel, ws)
    torch.cuda.synchronize()
    return bs.cpu().numpy(), sel.cpu().numpy()


@pytest.mark.parametrize("wname,mode,scaled", [("tiny_nvfp4", "exact", False), ("tiny_fp8", "exact", True),
                                               ("tiny_edge", "exact", False), ("long_rows", "exact", False),
                                               ("tiny_nvfp4", "fp8", False), ("tiny_spec", "exact", False)])
def test_noalloc_equals_the_workspace_call(wname, mode, scaled):
    import block_sparse_attention_indexer_amd as M
    _say("noalloc", wname, mode, "scaled" if scaled else "unit scales")
    case = H.HostCase(wname, scaled=scaled).upload()
    B = case.w.B
    ws = torch.zeros(max(1, B), dtype=torch.int32, device="cuda")
    for nb in (B, max(1, B - 1)):        # two calls in a row, the second on a smaller batch
        ref = _run(M, case, nb, mode, noalloc=False, ws=ws)
        got = _run(M, case, nb, mode, noalloc=True)
        assert np.array_equal(got[0], ref[0], equal_nan=True), (wname, nb)
        assert np.array_equal(got[1], ref[1]), (wname, nb)
    assert int(ws.abs().sum()) == 0


def test_noalloc_full_size_then_small():
    """c3_128k (64 sequences of 131,072 tokens), then a 3-sequence batch: both equal
    the workspace call."""
    import block_sparse_attention_indexer_amd as M
    _say("noalloc c3_128k then tiny_nvfp4")
    big = H.DeviceCase("c3_128k", keep_fp32=False)
    ws = torch.zeros(big.w.B, dtype=torch.int32, device="cuda")
    ref = _run(M, big, big.w.B, "exact", noalloc=False, ws=ws)
    got = _run(M, big, big.w.B, "exact", noalloc=True)
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
    del big
    small = H.HostCase("tiny_nvfp4").upload()
    ws = torch.zeros(small.w.B, dtype=torch.int32, device="cuda")
    ref = _run(M, small, small.w.B, "exact", noalloc=False, ws=ws)
    got = _run(M, small, small.w.B, "exact", noalloc=True)
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
