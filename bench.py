"""Benchmark of the MSA decode layer step on one MI355X.

One step = msa_indexer_scores (index scan and block max-pool) ->
msa_topk_sparse_attn (each attention workgroup selects its row's top-16 blocks,
then attends over them) for the whole batch (one MSA layer).  --path calls runs
the selection as its own launch (msa_block_topk, then msa_sparse_attn_decode);
--path fused runs the scan and selection as msa_indexer_topk; --path step runs
the step as msa_decode_step.  Inputs are seeded synthetic data drawn and packed
on the GPU before the timed region (resident in HBM).

    python bench.py [--steps K] [--warmup W] [--workload c3_128k]
                    [--dequant exact|fp8] [--no-cpu-baseline] [--no-prefill]
                    [--path select|calls|fused|step] [--only insert|dcp|prefix]

Prints one JSON line.  ``value`` is layer-steps/s over the timed steps (wall
clock, synchronised on both sides); ``roofline`` describes the dominant kernel
(the index-key scan) from HIP events recorded around its launch in every fifth
step of the timed region, on the stream it runs on, and ``traffic`` from the rocprofv3
counter summary under profiles/ (null once the kernel sources changed);
``dcp``, ``prefix``, ``prefill`` and ``insert`` time the side sections
(context-parallel shards, shared-prefix scan, the chunked-prefill workload,
the cache insert); ``ragged_c3``, ``spec_c4``, ``fp8_c2`` and ``spec8_c3_128k`` run the default
step on the other decode workloads; ``ceilings`` measures a streaming read and
the f16 MFMA rate with the benchmark's probe library; ``timing`` gives the step's
median / p10 / p90 and its HIP-graph replay; ``cpu_baseline`` is the CPU fp64
oracle timed on a bounded sample.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MSA decode layer-steps/s at 128K ctx NVFP4; achieved HBM TB/s as % of peak"
HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 * 2 ** 20          # MI355X Infinity Cache


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # defaults: 200 warm-up steps (~30 ms) bring the GPU to its working clocks (5 left
    # the first timed steps ~2% slow); 300 timed steps take ~45 ms
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="c3_128k")
    ap.add_argument("--dequant", default="exact", choices=["exact", "fp8"])
    ap.add_argument("--seed", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the chunked-prefill section")
    ap.add_argument("--no-sides", action="store_true",
                    help="skip the dcp and prefix sections (which launch the scan kernel on other shapes)")
    ap.add_argument("--path", default="select", choices=["select", "calls", "fused", "step"],
                    help="select: msa_indexer_scores + msa_topk_sparse_attn (the selection inside the "
                         "attention launch); calls: the three calls msa_indexer_scores, msa_block_topk, "
                         "msa_sparse_attn_decode; fused: msa_indexer_topk + attention; step: msa_decode_step")
    ap.add_argument("--cpu-sample", type=int, default=4, help="sequences the oracle leg runs")
    ap.add_argument("--only", choices=["insert", "dcp", "prefix"], default=None,
                    help="run one side section alone and print its JSON (for profiling), not the step line")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


class Workload:
    """A decode workload drawn and packed on the GPU."""

    def __init__(self, name, seed, keep_sequences=()):
        import torch
        import synth
        import block_sparse_attention_indexer_amd as M
        self.M = M
        w = synth.WORKLOADS[name]
        self.w = w
        self.lay = lay = synth.make_layout(w, seed)
        dev = "cuda"
        idx_q, q, qhat = synth.queries(w, seed, device=dev)
        hot = synth.hot_blocks(w, lay, seed)
        S = w.tensor_scale()
        self.S = S
        P = lay.num_pages
        self.seq = lay.seq_lens.to(dev)
        self.table = lay.block_table.to(dev)
        # pages of the sequences the CPU leg will use: their fp32 sources are kept on the host
        keep_pages = {}
        for b in keep_sequences:
            nb = (int(lay.seq_lens[b]) + 127) // 128
            keep_pages[b] = lay.block_table[b, :nb].long()
        self.kept = {b: {} for b in keep_sequences}
        self.caches = {}
        chunk = 2048
        for name_ in ("idx_k", "k", "v"):
            heads = 1 if name_ == "idx_k" else 4
            if w.kv_dtype == "nvfp4":
                data = torch.empty((P, heads, 128, 64), dtype=torch.uint8, device=dev)
                sc = torch.empty((P, heads, 128, 8), dtype=torch.uint8, device=dev)
            elif w.kv_dtype == "fp8":
                data = torch.empty((P, heads, 128, 128), dtype=torch.uint8, device=dev)
                sc = None
            else:
                data = torch.empty((P, heads, 128, 128), dtype=torch.float32, device=dev)
                sc = None
            keep_host = {b: torch.empty((len(pg), heads, 128, 128)) for b, pg in keep_pages.items()}
            for first in range(0, P, chunk):
                n = min(chunk, P - first)
                x = synth.cache_pages(w, lay, seed, name_, first, n, qhat, hot, device=dev)
                if w.kv_dtype == "nvfp4":
                    M.msa_pack_nvfp4(x, S, data[first:first + n], sc[first:first + n])
                elif w.kv_dtype == "fp8":
                    M.msa_pack_fp8(x, S, data[first:first + n])
                else:
                    data[first:first + n].copy_(x)
                for b, pg in keep_pages.items():
                    m = (pg >= first) & (pg < first + n)
                    if m.any():
                        keep_host[b][m] = x[(pg[m] - first).to(dev)].cpu()
                del x
            for b in keep_pages:
                self.kept[b][name_] = keep_host[b].numpy()
            self.caches[name_] = (data, sc, M.cache(w.kv_dtype, data, sc, S if w.kv_dtype != "f32" else 1.0, heads))
        if w.q_dtype == "fp8":
            self.idx_q = torch.empty(idx_q.shape, dtype=torch.uint8, device=dev)
            self.q = torch.empty(q.shape, dtype=torch.uint8, device=dev)
            M.msa_pack_fp8(idx_q, 1.0, self.idx_q)
            M.msa_pack_fp8(q, 1.0, self.q)
        else:
            self.idx_q, self.q = idx_q, q
        self.idx_q32 = {b: idx_q[b].cpu().numpy() for b in keep_sequences}
        self.q32 = {b: q[b].cpu().numpy() for b in keep_sequences}
        B, T, maxb = w.B, w.T, lay.max_blocks
        self.prob = M.problem(self.seq, self.table, T)
        self.bs = torch.empty((B, T, 4, maxb), dtype=torch.float32, device=dev)
        self.sel = torch.empty((B, T, 4, 16), dtype=torch.int32, device=dev)
        self.out = torch.empty((B, T, 64, 128), dtype=torch.float32, device=dev)
        # arrival counters of msa_indexer_topk: zero-filled once, left zero-filled by every call
        self.ws = torch.zeros(max(1, M.msa_workspace_size(self.prob, M.MSA_CALL_INDEXER_TOPK) // 4),
                              dtype=torch.int32, device=dev)
        torch.cuda.synchronize()

    def copies(self, n):
        """n sets of the three caches: the originals and n - 1 device copies of them
        (same bytes at other addresses), as msa_cache triples for step(caches=...)."""
        import torch
        sets = [tuple(self.caches[k][2] for k in ("idx_k", "k", "v"))]
        self._copies = []
        for _ in range(n - 1):
            trip = []
            for name_ in ("idx_k", "k", "v"):
                data, sc, c = self.caches[name_]
                d2 = data.clone()
                s2 = sc.clone() if sc is not None else None
                self._copies.append((d2, s2))
                trip.append(self.M.cache(self.w.kv_dtype, d2, s2, c.tensor_scale, c.heads))
            sets.append(tuple(trip))
        torch.cuda.synchronize()
        return sets

    def step(self, dequant, ev=None, scan_only=False, path="calls", caches=None):
        """One layer step on torch's current stream.  path "select": msa_indexer_scores
        then msa_topk_sparse_attn; "calls": the three separate calls; "fused":
        msa_indexer_topk (scan + selection) then attention; "step": msa_decode_step.
        `ev` events are recorded before the first call and after each call (after the
        first only, when scan_only).  `caches`: an (index keys, K, V) triple from
        copies() in place of the workload's own caches."""
        M, w = self.M, self.w
        ik, kc, vc = caches if caches is not None else (self.caches["idx_k"][2], self.caches["k"][2],
                                                        self.caches["v"][2])
        if ev is not None:
            ev[0].record()
        if path == "step":
            M.msa_decode_step(self.prob, self.idx_q, w.q_dtype, 1.0, ik, self.q, w.q_dtype,
                              1.0, kc, vc, dequant, 1.0 / math.sqrt(128.0),
                              self.bs, self.sel, self.out, None)
            if ev is not None:
                ev[1].record()
            return
        if path == "select":
            # the scan, then one launch that selects each row's blocks and attends over them
            M.msa_indexer_scores(self.prob, self.idx_q, w.q_dtype, 1.0, ik, dequant,
                                 self.bs, None)
            if ev is not None:
                ev[1].record()
            M.msa_topk_sparse_attn(self.prob, self.bs, self.sel, self.q, w.q_dtype, 1.0, kc,
                                   vc, dequant, 1.0 / math.sqrt(128.0), self.out, None)
            if ev is not None and not scan_only:
                ev[2].record()
            return
        fused = path == "fused"
        if fused:
            M.msa_indexer_topk(self.prob, self.idx_q, w.q_dtype, 1.0, ik, dequant, self.bs,
                               self.sel, self.ws)
            calls_done = 1
        else:
            M.msa_indexer_scores(self.prob, self.idx_q, w.q_dtype, 1.0, ik, dequant,
                                 self.bs, None)
            if ev is not None:
                ev[1].record()
            M.msa_block_topk(self.prob, self.bs, self.sel)
            calls_done = 2
        if ev is not None and (fused or not scan_only):
            ev[calls_done].record()
        fn = M.msa_sparse_attn_decode if w.T <= 8 else M.msa_sparse_attn_prefill
        fn(self.prob, self.q, w.q_dtype, 1.0, kc, vc, dequant, self.sel,
           1.0 / math.sqrt(128.0), self.out, None)
        if ev is not None and not scan_only:
            ev[calls_done + 1].record()


# Algorithmic bytes per element row of 128 dims (NVFP4: 64 B of E2M1 codes + 8 E4M3 scales).
ROW_BYTES = {"f32": 512, "fp8": 128, "nvfp4": 72}
F16_MFMA_PEAK_TFLOPS = 2500.0


def algorithmic_bytes(wl, sel_host):
    """Bytes the method itself must move in one layer step: every index key of every
    sequence once, the index queries, the block scores written (and read back by the
    top-16), K and V rows of each distinct selected (sequence, group, block) once, the
    queries, the fp32 outputs and the small tables.  Repeat reads are not counted."""
    w, lay = wl.w, wl.lay
    lens = [int(x) for x in lay.seq_lens]
    maxb = lay.max_blocks
    qb = 4 if w.q_dtype == "f32" else 1
    rows = w.B * w.T * 4
    idx = (sum(lens) * ROW_BYTES[w.kv_dtype] + rows * 128 * qb + rows * maxb * 4 + w.B * maxb * 4 + w.B * 4)
    topk = rows * maxb * 4 + rows * 16 * 4
    keys = 0   # distinct selected keys, summed over (sequence, group)
    for b in range(w.B):
        L = lens[b]
        for g in range(4):
            for i in set(int(i) for i in sel_host[b, :, g].reshape(-1) if i >= 0):
                keys += min(128, L - 128 * i)
    attn = 2 * keys * ROW_BYTES[w.kv_dtype] + w.B * w.T * 64 * 128 * (qb + 4)
    return idx, topk, attn


def algorithmic_flops(wl, sel_host):
    """Index scores: 2*128 flops per (token, group, visible key); attention: 4*128 flops
    per (token, head, attended key) -- QK^T and PV."""
    w, lay = wl.w, wl.lay
    idx = attn = 0
    for b in range(w.B):
        L = int(lay.seq_lens[b])
        p = np.arange(L - w.T, L, dtype=np.int64)                         # token positions
        idx += 2 * 128 * 4 * int((p + 1).sum())
        s = sel_host[b].astype(np.int64)                                   # [T, 4, 16]
        nk = np.where(s >= 0, np.clip(p[:, None, None] + 1 - 128 * s, 0, 128), 0)
        attn += 4 * 128 * 16 * int(nk.sum())
    return idx, attn


def indexer_kernel_name(w, dequant, path="calls", max_blocks=None, cus=256, skip=False):
    """The first kernel of the step (the index scan) that
    libmsa launches for this workload, as rocprofv3 names it: for one token the
    evenly spread scan (its SKIP form when a shared prefix is skipped) unless the
    selection is fused into it (then, as for speculative decode, the pages-per-wave
    template argument follows the launcher's rule: the largest of its three sizes
    whose grid gives every CU one workgroup (one token) or two (speculative decode))."""
    kt = {"fp8": 1, "nvfp4": 2}.get(w.kv_dtype)
    if kt is None:
        return "msa::indexer_f32_kernel"
    fp8mode = kt == 2 and dequant == "fp8"
    fused = path == "fused" and not fp8mode
    nb = max_blocks if max_blocks is not None else -(-max(np.atleast_1d(w.lens)) // 128)

    def ppw(big, per_cu):
        for p_ in (big, big // 2):
            if w.B * -(-nb // (4 * p_)) >= per_cu * cus:
                return p_
        return big // 4
    b = lambda x: str(x).lower()
    if w.T == 1 and not fused and w.B <= 1024:
        return f"msa::indexer_decode1_flat_kernel<{kt}, {b(fp8mode)}, {b(skip)}>"
    if w.T == 1:
        return f"msa::indexer_decode1_kernel<{kt}, false, {b(fused)}, {ppw(16, 1)}, {b(fp8mode)}>"
    if w.T <= 8:
        return (f"msa::indexer_decode_kernel<{kt}, {b(fp8mode)}, false, {4 if kt == 2 else 2}, true, {ppw(8, 2)}, "
                f"{1 if w.T <= 4 else 2}>")
    return f"msa::indexer_prefill_kernel<{kt}, {b(fp8mode)}, false>"


def measured_traffic(workload, kernel=None, role=None):
    """Calibrated HBM bytes per launch (read + write) of one kernel -- named, or the
    only kernel of a role ("indexer", "topk", "attention") -- from the rocprofv3
    counter summary under profiles/; None when there is none or when the kernel
    sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"layer_step_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    import profile_step
    with open(path) as fh:
        d = json.load(fh)
    if d.get("sources_sha256") != profile_step.sources_hash():
        return None
    if kernel is None:
        names = [n for n, e in d["kernels"].items() if e.get("role") == role]
        if len(names) != 1:
            return None
        kernel = names[0]
    e = d["kernels"].get(kernel)
    if e is None or "fetch_bytes" not in e or "write_bytes" not in e:
        return None
    return round(e["fetch_bytes"] + e["write_bytes"])


def prefill_section(wl, dequant, steps=5, warmup=2):
    """The chunked-prefill workload (c5, drawn once as `wl`) through the same three
    calls: per-call event timings (medians) and the MFMA rate of the two
    contractions (f16 MFMAs, exact products) against the f16 dense peak."""
    import torch
    w = wl.w
    for _ in range(warmup):
        wl.step(dequant)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for k in range(steps):
        wl.step(dequant, evs[k])
    torch.cuda.synchronize()
    t = np.median(np.array([[evs[k][i].elapsed_time(evs[k][i + 1]) for i in range(3)] for k in range(steps)]),
                  axis=0)
    f_idx, f_attn = algorithmic_flops(wl, wl.sel.cpu().numpy())
    tf_idx = f_idx / (t[0] * 1e-3) / 1e12
    tf_attn = f_attn / (t[2] * 1e-3) / 1e12
    # msa_topk_sparse_attn on the same block scores (for this many rows: the top-16 kernel, then attention)
    M = wl.M
    ev2 = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for k in range(steps):
        ev2[k][0].record()
        M.msa_topk_sparse_attn(wl.prob, wl.bs, wl.sel, wl.q, w.q_dtype, 1.0, wl.caches["k"][2], wl.caches["v"][2],
                               dequant, 1.0 / math.sqrt(128.0), wl.out, None)
        ev2[k][1].record()
    torch.cuda.synchronize()
    t_sel = float(np.median([e[0].elapsed_time(e[1]) for e in ev2]))
    return {"workload": f"c5: chunked prefill, batch {w.B}, {w.T} new query tokens per sequence on "
                        f"{w.lens - w.T} cached ({w.lens} total), NVFP4 K/V and index keys, FP8 queries",
            "dequant": dequant,
            "ms_per_step": round(float(t.sum()), 4),
            "indexer": {"kernel": "msa::indexer_prefill_kernel", "ms": round(float(t[0]), 4),
                        "gflop": round(f_idx / 1e9, 1), "tflops": round(tf_idx, 1),
                        "frac_of_f16_mfma_peak": round(tf_idx / F16_MFMA_PEAK_TFLOPS, 4),
                        "traffic": measured_traffic("c5", role="indexer")},
            "topk_ms": round(float(t[1]), 4),
            "topk_sparse_attn_ms": round(t_sel, 4),
            "attention": {"kernel": "msa::attn_mfma_kernel (4 waves per row)", "ms": round(float(t[2]), 4),
                          "gflop": round(f_attn / 1e9, 1), "tflops": round(tf_attn, 1),
                          "frac_of_f16_mfma_peak": round(tf_attn / F16_MFMA_PEAK_TFLOPS, 4),
                          "traffic": measured_traffic("c5", role="attention")}}


def decode_section(name, dequant, seed, steps=100, warmup=100, ev_steps=20):
    """Another decode workload through the default step (scan, then the selecting
    attention): after `warmup` steps (the clocks settle over the first milliseconds
    of work), the step from `steps` steps back to back (one event pair around
    them), the calls from `ev_steps` steps with each call bracketed by HIP events (medians),
    with the step's algorithmic bytes and HBM rate; reported beside the
    uniform-128K headline.  c3: 64 sequences,
    ragged contexts uniform in [64K, 160K] tokens, NVFP4 with 5% outliers; c4: 16
    sequences of 262,144 tokens, 4 query tokens each (speculative decode), NVFP4;
    c3_t8: the 128K batch with 8 query tokens each (1 verified + 7 speculative);
    c2: 32 sequences of 32,768 tokens, FP8.  A step whose bytes fit the 256 MB
    Infinity Cache (c2: 203 MB) is reported cold (caches rotated, cold_timing) as its
    headline figures, with the back-to-back (cache-resident) figures beside them."""
    import torch
    wl = Workload(name, seed)
    w = wl.w
    for _ in range(warmup):
        wl.step(dequant, path="select")
    step_ms = unbracketed_ms(lambda k: wl.step(dequant, path="select"), steps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(ev_steps)]
    for k in range(ev_steps):
        wl.step(dequant, evs[k], path="select")
    torch.cuda.synchronize()
    t = np.array([[evs[k][i].elapsed_time(evs[k][i + 1]) for i in range(2)] for k in range(ev_steps)])
    b_idx, b_topk, b_attn = algorithmic_bytes(wl, wl.sel.cpu().numpy())
    scan_ms = float(np.median(t[:, 0]))
    total = b_idx + b_topk + b_attn
    lens = [int(x) for x in wl.lay.seq_lens]
    hot = None
    if total < MALL_BYTES:   # step_ms above is the back-to-back (cache-resident) figure
        hot = {"step_ms": round(step_ms, 5), "indexer_ms": round(scan_ms, 5),
               "layer_steps_per_s": round(1e3 / step_ms, 2),
               "note": "back to back: the step's bytes stay resident in the Infinity Cache"}
        cold = cold_timing(wl, dequant, total, steps=ev_steps)
        step_ms, scan_ms = cold["step_ms"], cold["indexer_ms"]
        t = np.array([[cold["indexer_ms"], cold["topk_attention_ms"]]])
    res = {"workload": f"{name}: decode, batch {w.B}, {w.T} query token(s) per sequence, contexts "
                       f"{min(lens)}..{max(lens)} tokens (sum {sum(lens)}), {w.kv_dtype} K/V and index keys, "
                       f"{w.q_dtype} queries, shuffled pages",
           "timing": "cold (caches rotated)" if hot else "back to back",
           "step_ms": round(step_ms, 5), "layer_steps_per_s": round(1e3 / step_ms, 2),
           "sequence_layer_steps_per_s": round(w.B * 1e3 / step_ms, 1),
           "indexer_ms": round(scan_ms, 5), "topk_attention_ms": round(float(np.median(t[:, 1])), 5),
           "bytes_per_step": {"indexer": b_idx, "topk": b_topk, "attention": b_attn},
           "indexer_GBps": round(b_idx / (scan_ms * 1e-3) / 1e9, 1),
           "hbm_TBps_step": round(total / (step_ms * 1e-3) / 1e12, 3),
           "pct_of_peak_hbm_step": round(100 * total / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 1)}
    if hot:
        res["cold"] = {"cache_copies": cold["cache_copies"]}
        res["hot"] = hot
    return res


def reading_section(wl, dequant, steps=100, warmup=100, ev_steps=20):
    """The default decode step of `wl` in another NVFP4 reading (the FP8-rounded one
    beside the exact headline): after `warmup` steps, the step back to back (one
    event pair around `steps` steps), the calls bracketed by HIP events in a second
    pass of `ev_steps` steps (medians)."""
    import torch
    for _ in range(warmup):
        wl.step(dequant, path="select")
    step_ms = unbracketed_ms(lambda k: wl.step(dequant, path="select"), steps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(ev_steps)]
    torch.cuda.synchronize()
    for k in range(ev_steps):
        wl.step(dequant, evs[k], path="select")
    torch.cuda.synchronize()
    t = np.array([[evs[k][i].elapsed_time(evs[k][i + 1]) for i in range(2)] for k in range(ev_steps)])
    b_idx, b_topk, b_attn = algorithmic_bytes(wl, wl.sel.cpu().numpy())
    scan_ms = float(np.median(t[:, 0]))
    return {"dequant": dequant, "kernels": {"scan": indexer_kernel_name(wl.w, dequant, "select", wl.lay.max_blocks)},
            "step_ms": round(step_ms, 5), "layer_steps_per_s": round(1e3 / step_ms, 2),
            "indexer_ms": round(scan_ms, 5), "topk_attention_ms": round(float(np.median(t[:, 1])), 5),
            "indexer_GBps": round(b_idx / (scan_ms * 1e-3) / 1e9, 1),
            "pct_of_peak_hbm_step": round(100 * (b_idx + b_topk + b_attn) / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                                          1)}


def cold_timing(wl, dequant, footprint_bytes, steps=20, warmup=3):
    """The default step with the caches cold: ceil(1 GB / footprint) + 1 copies of the
    three caches are used in rotation, so between two uses of one copy at least 1 GB
    of other data has streamed through the caches (the 256 MB Infinity Cache
    included).  The step from the rotation run back to back (one event pair around
    it); the calls from a second pass with each call bracketed (medians)."""
    import torch
    n = int(math.ceil(1e9 / footprint_bytes)) + 1
    sets = wl.copies(n)
    for k in range(warmup):
        wl.step(dequant, path="select", caches=sets[k % n])
    step_ms = unbracketed_ms(lambda k: wl.step(dequant, path="select", caches=sets[k % n]), steps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        wl.step(dequant, evs[k], path="select", caches=sets[k % n])
    torch.cuda.synchronize()
    t = np.array([[evs[k][i].elapsed_time(evs[k][i + 1]) for i in range(2)] for k in range(steps)])
    wl._copies = []
    torch.cuda.empty_cache()
    return {"cache_copies": n, "step_ms": round(step_ms, 5),
            "indexer_ms": round(float(np.median(t[:, 0])), 5),
            "topk_attention_ms": round(float(np.median(t[:, 1])), 5)}


def unbracketed_ms(run_step, steps):
    """Milliseconds per step of `steps` steps run back to back with one HIP event pair
    around them all (an event between the calls of every step would slow the steps)."""
    import torch
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    e[0].record()
    for k in range(steps):
        run_step(k)
    e[1].record()
    torch.cuda.synchronize()
    return e[0].elapsed_time(e[1]) / steps


def ceilings_section(reps=7):
    """Ceilings measured on this GPU with the benchmark's probe library
    (bench_probes/libmsa_probe.so, not part of libmsa): one streaming read of a 2 GiB
    buffer and the dense 16x16x32 f16 MFMA issue rate with no memory traffic, each the
    median of `reps` event-timed launches, beside the published peaks the roofline
    fractions use."""
    import torch
    import bench_probes as BP

    def median_ms(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    nbytes = 2 << 30
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(BP.SINK_WORDS, dtype=torch.int32, device="cuda")
    ms_read = median_ms(lambda: BP.stream_read(buf, sink))
    del buf
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs, iters = 8 * cus, 2000
    out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    ms_mfma = median_ms(lambda: BP.mfma_f16(out, wgs, iters))
    flops = wgs * 4 * iters * 16 * 16 * 16 * 32 * 2
    gbps = nbytes / (ms_read * 1e-3) / 1e9
    tflops = flops / (ms_mfma * 1e-3) / 1e12
    return {"stream_read": {"bytes": nbytes, "ms": round(ms_read, 4), "GBps": round(gbps, 1),
                            "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4)},
            "mfma_f16": {"workgroups": wgs, "ms": round(ms_mfma, 4), "TFLOPs": round(tflops, 1),
                         "frac_of_f16_peak": round(tflops / F16_MFMA_PEAK_TFLOPS, 4)},
            "compute_units": cus}


def insert_section(seed, steps=50):
    """Quantise-and-insert of the new tokens' K, V and index-key rows (NVFP4): c5's
    2 x 4,096-token prefill chunk and one decode token of c3_128k, as one
    msa_cache_insert_many launch and as three msa_cache_insert launches.  Each is
    launched `steps` times back to back in five groups, each between two HIP events
    on the stream, and the median group's time per repetition is reported (for the decode token the kernels are a few
    microseconds, so there it is bounded by the host's launch rate; the
    rocprofv3 summary has the kernel durations).  Algorithmic bytes: each row read
    once in fp32 (512 B) and written once in NVFP4 (64 B codes + 8 B scales)."""
    import numpy as np
    import torch
    import block_sparse_attention_indexer_amd as M
    out = {}

    def per_rep_ms(run, groups=5):
        # `steps` launches in `groups` back-to-back groups, each between two events;
        # the median group's time per launch (one host stall cannot skew it)
        for _ in range(3):
            run()
        torch.cuda.synchronize()
        n = max(1, steps // groups)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(groups + 1)]
        ev[0].record()
        for gi in range(groups):
            for _ in range(n):
                run()
            ev[gi + 1].record()
        torch.cuda.synchronize()
        return float(np.median([ev[gi].elapsed_time(ev[gi + 1]) / n for gi in range(groups)]))

    for name, B, T, L in (("prefill_c5", 2, 4096, 69632), ("decode_c3_128k", 64, 1, 131072)):
        g = torch.Generator(device="cuda").manual_seed(seed)
        nb = (L + 127) // 128
        table = torch.arange(B * nb, dtype=torch.int32, device="cuda").reshape(B, nb)
        seq = torch.full((B,), L, dtype=torch.int32, device="cuda")
        prob = M.problem(seq, table, T)
        caches, xs = [], []
        for heads in (4, 4, 1):                      # K, V, index keys
            codes = torch.zeros((B * nb, heads, 128, 64), dtype=torch.uint8, device="cuda")
            sc = torch.zeros((B * nb, heads, 128, 8), dtype=torch.uint8, device="cuda")
            caches.append((codes, sc, M.cache("nvfp4", codes, sc, 32.0 / 448.0, heads)))
            xs.append(torch.randn((B, T, heads, 128), generator=g, device="cuda"))
        cs = [c for _, _, c in caches]

        def three():
            for c, x in zip(cs, xs):
                M.msa_cache_insert(prob, x, c)

        def one():
            M.msa_cache_insert_many(prob, xs, cs)
        ms1, ms3 = per_rep_ms(one), per_rep_ms(three)
        rows = B * T * 9
        nbytes = rows * (512 + 72)
        out[name] = {"tokens": B * T, "rows": rows, "ms": round(ms1, 5), "three_launches_ms": round(ms3, 5),
                     "bytes": nbytes, "GBps": round(nbytes / (ms1 * 1e-3) / 1e9, 1),
                     "frac_of_hbm_peak": round(nbytes / (ms1 * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
        del caches, xs
    return {"kernel": "msa::insert_many_kernel (K, V and index keys in one launch)", **out}


def dcp_section(wl, dequant, P=4, steps=20):
    """Decode context parallelism on one GPU: the P shard scans of the index cache
    (each the work one of P GPUs would do), every shard's local top-16 and the
    owner's merge, each bracketed by HIP events on the launching stream, against the
    unsharded scan + top-16 of the same batch (medians over `steps` steps).  The
    exchange between GPUs is not part of it.  Algorithmic bytes of a shard scan: the index keys of its blocks, the
    index queries and the block scores it writes."""
    import torch
    M, w, lay = wl.M, wl.w, wl.lay
    B, T, maxb = w.B, w.T, lay.max_blocks
    ik = wl.caches["idx_k"][2]
    bs = torch.empty_like(wl.bs)
    cs = torch.empty((P, B, T, 4, 16), dtype=torch.float32, device="cuda")
    cb = torch.empty((P, B, T, 4, 16), dtype=torch.int32, device="cuda")
    sel = torch.empty_like(wl.sel)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def once(t=None):
        rec = t is not None
        for s_ in range(P):
            if rec: t[s_].record()
            M.msa_indexer_scores_shard(wl.prob, s_, P, wl.idx_q, w.q_dtype, 1.0, ik, dequant, bs)
        if rec: t[P].record()
        for s_ in range(P):
            M.msa_shard_topk(wl.prob, s_, P, bs, cs[s_], cb[s_])
            if rec: t[P + 1 + s_].record()
        M.msa_topk_merge(wl.prob, P, cs, cb, sel)
        if rec: t[2 * P + 1].record()
        return t

    for _ in range(3):
        once()
    # every event is created before the first timed launch; each figure is the median
    # over the steps (a single host stall cannot move it)
    runs = [[ev() for _ in range(2 * P + 2)] for _ in range(steps)]
    full_ev = [[ev() for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        once(runs[k])
        e = full_ev[k]
        e[0].record()
        M.msa_indexer_scores(wl.prob, wl.idx_q, w.q_dtype, 1.0, ik, dequant, wl.bs, None)
        e[1].record()
        M.msa_block_topk(wl.prob, wl.bs, wl.sel)
        e[2].record()
    torch.cuda.synchronize()
    scan = np.median(np.array([[r[s_].elapsed_time(r[s_ + 1]) for s_ in range(P)] for r in runs]), axis=0)
    local = np.median(np.array([[r[P + s_].elapsed_time(r[P + 1 + s_]) for s_ in range(P)] for r in runs]), axis=0)
    merge = float(np.median([r[2 * P].elapsed_time(r[2 * P + 1]) for r in runs]))
    full_scan = float(np.median([e[0].elapsed_time(e[1]) for e in full_ev]))
    full_topk = float(np.median([e[1].elapsed_time(e[2]) for e in full_ev]))
    exact = bool(torch.equal(bs, wl.bs)) and bool(torch.equal(sel, wl.sel))
    lens = [int(x) for x in lay.seq_lens]
    shard_keys = np.zeros(P)
    for L in lens:
        nb = (L + 127) // 128
        for s_ in range(P):
            blocks = np.arange(s_, nb, P)
            shard_keys[s_] += np.minimum(128, L - 128 * blocks).sum()
    qb = 4 if w.q_dtype == "f32" else 1
    shard_bytes = shard_keys * ROW_BYTES[w.kv_dtype] + B * T * 4 * 128 * qb + \
        np.array([B * T * 4 * len(range(s_, maxb, P)) * 4 for s_ in range(P)])
    gbps = shard_bytes / (scan * 1e-3) / 1e9
    return {"workload": w.name, "shards": P,
            "kernels": {"scan": indexer_kernel_name(w, dequant, max_blocks=-(-maxb // P)),
                        "local_top16": "msa::shard_topk_kernel<4>" if -(-maxb // P) <= 1024 else
                        "msa::shard_topk_kernel<32>",
                        "merge": "msa::topk_merge_kernel"},
            "shard_scan_ms": [round(float(x), 5) for x in scan],
            "shard_scan_GBps": [round(float(x), 1) for x in gbps],
            "shard_scan_frac_of_hbm_peak": round(float(gbps.mean()) / HBM_PEAK_GBPS, 4),
            "local_top16_ms": [round(float(x), 5) for x in local], "merge_ms": round(merge, 5),
            "unsharded_scan_ms": round(full_scan, 5), "unsharded_top16_ms": round(full_topk, 5),
            "per_gpu_ms": round(float(scan.max() + local.max() + merge), 5),
            "scan_speedup_per_gpu": round(full_scan / float(scan.max()), 3),
            "bit_identical_scores_and_selection": exact}


def prefix_section(wl, dequant, shared_blocks=512, steps=20):
    """Shared-prefix decode of the index scan: every sequence of the decode workload
    reads the same pages in its first `shared_blocks` blocks (one prefix group per 64
    sequences).  Times msa_indexer_scores on that block table (each sequence scans
    the shared pages itself; repeated pages may hit in L2 / Infinity Cache) against
    msa_indexer_scores_prefix (shared blocks scored once per group), both bracketed by
    HIP events.  Algorithmic bytes of the prefix call: the shared index keys once per
    group, every other visible key once, queries and scores."""
    import torch
    M, w, lay = wl.M, wl.w, wl.lay
    B, T, maxb = w.B, w.T, lay.max_blocks
    lens = [int(x) for x in lay.seq_lens]
    sb = min(shared_blocks, min((L - T) // 128 for L in lens))
    tab = lay.block_table.clone()
    groups = [(s_, min(s_ + 64, B)) for s_ in range(0, B, 64)]
    for s_, e_ in groups:
        tab[s_:e_, :sb] = tab[s_, :sb]
    d_tab = tab.to("cuda")
    prob = M.problem(wl.seq, d_tab, T)
    ik = wl.caches["idx_k"][2]
    bs_u = torch.empty_like(wl.bs)
    bs_p = torch.empty_like(wl.bs)
    ws = torch.empty(M.msa_workspace_size(prob, M.MSA_CALL_INDEXER_PREFIX) // 4, dtype=torch.int32, device="cuda")
    starts = [g[0] for g in groups] + [groups[-1][1]]
    blocks = [sb] * len(groups)
    for _ in range(3):
        M.msa_indexer_scores(prob, wl.idx_q, w.q_dtype, 1.0, ik, dequant, bs_u, None)
        M.msa_indexer_scores_prefix(prob, starts, blocks, wl.idx_q, w.q_dtype, 1.0, ik, dequant, bs_p, ws)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for k in range(steps):
        ev[k][0].record()
        M.msa_indexer_scores(prob, wl.idx_q, w.q_dtype, 1.0, ik, dequant, bs_u, None)
        ev[k][1].record()
        M.msa_indexer_scores_prefix(prob, starts, blocks, wl.idx_q, w.q_dtype, 1.0, ik, dequant, bs_p, ws)
        ev[k][2].record()
    torch.cuda.synchronize()
    t_u = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
    t_p = float(np.median([e[1].elapsed_time(e[2]) for e in ev]))
    fin = torch.isfinite(bs_u)
    same_inf = bool(torch.equal(torch.isneginf(bs_u), torch.isneginf(bs_p)))
    rel = float(((bs_p[fin] - bs_u[fin]).abs() / (1 + bs_u[fin].abs())).max()) if bool(fin.any()) else 0.0
    qb = 4 if w.q_dtype == "f32" else 1
    other = B * T * 4 * (128 * qb + maxb * 4)
    keys_shared = len(groups) * sb * 128 + sum(L - sb * 128 for L in lens)
    b_prefix = keys_shared * ROW_BYTES[w.kv_dtype] + other
    b_plain = sum(lens) * ROW_BYTES[w.kv_dtype] + other
    attn = prefix_attention(wl, dequant, prob, starts, blocks, sb, steps)
    return {"workload": w.name, "shared_blocks": sb, "groups": len(groups), "attention": attn,
            "kernels": {"shared": f"msa::indexer_prefill_kernel<{2 if w.kv_dtype == 'nvfp4' else 1}, "
                                  f"{str(dequant == 'fp8' and w.kv_dtype == 'nvfp4').lower()}, false, true, C>",
                        "rest": indexer_kernel_name(w, dequant, max_blocks=maxb, skip=True)},
            "unshared_scan_ms": round(t_u, 5), "prefix_scan_ms": round(t_p, 5),
            "speedup": round(t_u / t_p, 3),
            "prefix_algorithmic_bytes": int(b_prefix), "unshared_algorithmic_bytes": int(b_plain),
            "prefix_GBps": round(b_prefix / (t_p * 1e-3) / 1e9, 1),
            "max_rel_diff_vs_unshared": rel, "same_inf_pattern": same_inf}


def shared_prefix_selection(sel, seq_lens, T, starts, sb, per_row=8, seed=0):
    """A selection in which every row of a prefix group also picks the same `per_row`
    shared-prefix blocks (older than its own block): the rows' own blocks are kept
    and their other entries trimmed to make room; rows stay distinct, ascending and
    -1 padded.  This is the access pattern of requests that share a prompt prefix
    and attend into it (a sparse attention takes any such selection)."""
    rng = np.random.default_rng(seed)
    out = sel.copy()
    for gi in range(len(starts) - 1):
        common = [int(x) for x in rng.permutation(sb)[:per_row]]
        for b in range(starts[gi], starts[gi + 1]):
            for t in range(T):
                own = (int(seq_lens[b]) - T + t) // 128
                for g in range(4):
                    add = [i for i in common if i < own]
                    others = [int(i) for i in out[b, t, g] if 0 <= i != own and int(i) not in add]
                    others = others[:max(0, 15 - len(add))]
                    row = sorted(set(others + add + [own]))
                    out[b, t, g] = np.array(row + [-1] * (16 - len(row)), np.int32)
    return out


def prefix_attention(wl, dequant, prob, starts, blocks, sb, steps):
    """The shared-prefix decode attention (msa_sparse_attn_decode_prefix: every selected
    shared-prefix block dequantised once per group and KV head) against
    msa_sparse_attn_decode on the same sharing block table and the same selection
    (each row's own top-16 blocks with 8 common prefix blocks forced in), both
    bracketed by HIP events (medians); outputs must be bit-identical."""
    import torch
    M, w = wl.M, wl.w
    M.msa_indexer_scores(prob, wl.idx_q, w.q_dtype, 1.0, wl.caches["idx_k"][2], dequant, wl.bs, None)
    M.msa_block_topk(prob, wl.bs, wl.sel)
    sel = shared_prefix_selection(wl.sel.cpu().numpy(), wl.lay.seq_lens.numpy(), w.T, starts, sb)
    d_sel = torch.from_numpy(sel).cuda()
    nws = M.msa_sparse_attn_prefix_workspace_size(prob, starts, blocks)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    out_u, out_p = torch.empty_like(wl.out), torch.empty_like(wl.out)
    sm = 1.0 / math.sqrt(128.0)
    kc, vc = wl.caches["k"][2], wl.caches["v"][2]

    def plain():
        M.msa_sparse_attn_decode(prob, wl.q, w.q_dtype, 1.0, kc, vc, dequant, d_sel, sm, out_u, None)

    def shared():
        M.msa_sparse_attn_decode_prefix(prob, starts, blocks, wl.q, w.q_dtype, 1.0, kc, vc, dequant, d_sel, sm, out_p,
                                        None, ws)
    for _ in range(3):
        plain()
        shared()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        ev[k][0].record()
        plain()
        ev[k][1].record()
        shared()
        ev[k][2].record()
    torch.cuda.synchronize()
    t_u = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
    t_p = float(np.median([e[1].elapsed_time(e[2]) for e in ev]))
    in_prefix = int(((sel >= 0) & (sel < sb)).sum())
    return {"call": "msa_sparse_attn_decode_prefix",
            "kernels": ["msa::prefix_plan_kernel", "msa::prefix_stage_kernel", "msa::attn_prefix_kernel"],
            "selected_prefix_entries": in_prefix, "selected_entries": int((sel >= 0).sum()),
            "workspace_bytes": nws, "unshared_ms": round(t_u, 5), "shared_ms": round(t_p, 5),
            "speedup": round(t_u / t_p, 3), "bit_identical": bool(torch.equal(out_u, out_p))}


def cpu_baseline(wl, dequant, sample, cores):
    """The oracle on the sequences `sample` (kept when the workload was drawn) of the
    same workload, packed by the oracle itself from the fp32 sources; timed from
    decode to attention with the BLAS thread pool limited to `cores` threads."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import formats as OF
    from oracle import msa as OM
    w, lay = wl.w, wl.lay
    mode = "exact" if dequant == "exact" else "fp8"
    total = 0.0
    with threadpool_limits(cores):
        for b in sample:
            src = wl.kept[b]
            L = int(lay.seq_lens[b])
            nb = (L + 127) // 128
            caches = {}
            for n, x in src.items():
                if w.kv_dtype == "nvfp4":
                    c, s = OF.nvfp4_quantize(x, wl.S)
                    caches[n] = {"dtype": "nvfp4", "data": c, "scales": s, "tensor_scale": wl.S}
                elif w.kv_dtype == "fp8":
                    caches[n] = {"dtype": "fp8", "data": OF.fp8_quantize(x, wl.S), "tensor_scale": wl.S}
                else:
                    caches[n] = {"dtype": "f32", "data": x, "tensor_scale": 1.0}
            qd = w.q_dtype
            idx_q = OF.fp8_quantize(wl.idx_q32[b], 1.0)[None] if qd == "fp8" else wl.idx_q32[b][None]
            q = OF.fp8_quantize(wl.q32[b], 1.0)[None] if qd == "fp8" else wl.q32[b][None]
            table = np.arange(nb, dtype=np.int32)[None]
            t0 = time.perf_counter()
            OM.batch_layer(idx_q, q, caches["idx_k"], caches["k"], caches["v"], np.array([L]), table, w.T,
                           1.0 / math.sqrt(128.0), mode=mode, idx_q_dtype=qd, q_dtype=qd)
            total += time.perf_counter() - t0
    per_seq = total / max(1, len(sample))
    return {"value": 1.0 / (per_seq * w.B), "unit": "layer-steps/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(sample)} of {w.B} sequences of {w.name} (full layer step each: dequant, "
                      f"score, pool, select, attend) with the BLAS pool at {cores} thread(s); rate scaled "
                      f"to the {w.B}-sequence step; {total:.1f} s of wall time"}


def graph_timing(wl, dequant, path, steps):
    """The same layer step captured once in a HIP graph and replayed: ms per replay
    over `steps` back-to-back replays between two HIP events.  Before timing, three
    replays, each followed by an eager step, must leave outputs bit-identical to the
    eager step's (the path records no memset nodes)."""
    import torch
    ref_sel, ref_out = wl.sel.clone(), wl.out.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        wl.step(dequant, path=path)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        wl.step(dequant, path=path)
    identical = True
    for _ in range(3):
        wl.out.zero_()
        g.replay()
        torch.cuda.synchronize()
        identical &= bool(torch.equal(wl.sel, ref_sel) and torch.equal(wl.out, ref_out))
        wl.step(dequant, path=path)
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del g
    return {"ms_per_step": round(ms, 5), "layer_steps_per_s": round(1e3 / ms, 2),
            "replays_identical_to_eager": identical}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the library runs on one "
              "GPU (how the path would shard is a design note, not code).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    torch.cuda.set_device(0)
    if args.calib_copy_mib:
        # a plain elementwise copy kernel (reads and writes calib_copy_mib MiB each) whose
        # FETCH_SIZE / WRITE_SIZE counter readings calibrate the counters of the MSA kernels
        n = args.calib_copy_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        bbuf = torch.empty_like(a)
        for _ in range(3):
            torch.mul(a, 1.0, out=bbuf)
        torch.cuda.synchronize()
        del a, bbuf
    if args.only == "insert":
        print(json.dumps({"insert": insert_section(args.seed, steps=args.steps)}), flush=True)
        return
    if args.only in ("dcp", "prefix"):
        wl = Workload(args.workload, args.seed)
        fn = dcp_section if args.only == "dcp" else prefix_section
        print(json.dumps({args.only: fn(wl, args.dequant, steps=args.steps)}), flush=True)
        return
    sample = [] if args.no_cpu_baseline else list(range(0, 64, 64 // max(1, args.cpu_sample)))[: args.cpu_sample]
    wl = Workload(args.workload, args.seed, keep_sequences=sample)
    w = wl.w
    print(f"[bench] workload {w.name} ready: B={w.B} T={w.T} pages={wl.lay.num_pages}", file=sys.stderr, flush=True)

    path = args.path
    for _ in range(args.warmup):
        wl.step(args.dequant, path=path)
    torch.cuda.synchronize()

    K = args.steps
    fused = path == "fused"
    ncalls = {"calls": 3, "fused": 2, "step": 1, "select": 2}[path]
    # Timed region: K whole steps.  HIP events on the launching stream bracket the
    # first call (the index scan, with the selection when fused: the roofline kernel)
    # in every EV_EVERY-th step only: an event pair costs ~6 us per step (each record
    # waits for the work before it), so bracketing every step would slow the step
    # being measured by ~4%.  One more pair brackets the whole region.
    EV_EVERY = 5
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(ncalls + 1)] if k % EV_EVERY == 0 else None
           for k in range(K)]
    e_all = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_all[0].record()
    for k in range(K):
        wl.step(args.dequant, evs[k], scan_only=True, path=path)
    e_all[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / K
    k_idx = [evs[k][0].elapsed_time(evs[k][1]) for k in range(K) if evs[k] is not None]
    region_event_ms = e_all[0].elapsed_time(e_all[1]) / K
    # after the timed region: every call bracketed, for the per-call breakdown
    Kb = min(K, 20)
    evb = [[torch.cuda.Event(enable_timing=True) for _ in range(ncalls + 1)] for _ in range(Kb)]
    for k in range(Kb):
        wl.step(args.dequant, evb[k], path=path)
    torch.cuda.synchronize()
    per_call = np.array([[evb[k][i].elapsed_time(evb[k][i + 1]) for i in range(ncalls)] for k in range(Kb)]).mean(axis=0)

    step_ev = np.array([evb[k][0].elapsed_time(evb[k][ncalls]) for k in range(Kb)])
    timing = {"timed_region_event_ms_per_step": round(region_event_ms, 5),
              "scan_launches_bracketed": len(k_idx),
              "step_event_ms": {"median": round(float(np.median(step_ev)), 5),
                                "p10": round(float(np.percentile(step_ev, 10)), 5),
                                "p90": round(float(np.percentile(step_ev, 90)), 5), "steps": Kb},
              "graph": graph_timing(wl, args.dequant, path, K)}

    sel = wl.sel.cpu().numpy()
    b_idx, b_topk, b_attn = algorithmic_bytes(wl, sel)
    total_bytes = b_idx + b_topk + b_attn
    if path == "select" and not args.no_sides:
        # the same step with the caches rotated so that no step finds its bytes in a cache
        timing["cold"] = cold_timing(wl, args.dequant, total_bytes, steps=Kb)
    idx_ms = float(np.mean(k_idx))
    # bytes of the first (roofline) call
    b_first = total_bytes if path == "step" else b_idx + b_topk if fused else b_idx
    achieved_idx = b_first / (idx_ms * 1e-3) / 1e9
    step_tbps = total_bytes / (ms_step * 1e-3) / 1e12

    out = {
        "metric": METRIC,
        "value": round(1e3 / ms_step, 2),
        "unit": "layer-steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "sequence_layer_steps_per_s": round(w.B * 1e3 / ms_step, 1),
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: decode, batch {w.B}, context {w.lens} tokens, NVFP4 K/V and index "
                               f"keys, FP8 queries, shuffled 128-token pages",
                   "batch": w.B, "query_tokens": w.T, "context": w.lens, "kv_storage": w.kv_dtype,
                   "q_storage": w.q_dtype, "dequant": args.dequant, "compute": "f16 MFMA, fp32 accumulate"},
        "hbm_TBps_step": round(step_tbps, 3),
        "pct_of_peak_hbm_step": round(100 * step_tbps * 1e3 / HBM_PEAK_GBPS, 1),
        "bytes_per_step": {"indexer": b_idx, "topk": b_topk, "attention": b_attn},
        "call_ms": ({"decode_step": round(idx_ms, 5)} if path == "step" else
                    {"indexer_topk": round(idx_ms, 5), "attention": round(float(per_call[1]), 5)} if fused else
                    {"indexer": round(idx_ms, 5), "topk_attention": round(float(per_call[1]), 5)}
                    if path == "select" else
                    {"indexer": round(idx_ms, 5), "topk": round(float(per_call[1]), 5),
                     "attention": round(float(per_call[2]), 5)}),
        "roofline": {"bound": "hbm", "kernel": indexer_kernel_name(w, args.dequant, path, wl.lay.max_blocks) +
                     {                      "fused": " (index-key scan + block max-pool + top-16)",
                      "calls": " (index-key scan + block max-pool)",
                      "step": " (index-key scan + block max-pool)",
                      "select": " (index-key scan + block max-pool)"}[path],
                     "achieved": round(achieved_idx, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved_idx / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(w.name, indexer_kernel_name(w, args.dequant, path,
                                                                              wl.lay.max_blocks))},
        "cpu_baseline": None,
        "timing": timing,
    }
    if w.T <= 4 and w.kv_dtype != "f32" and not args.no_sides:
        out["dcp"] = dcp_section(wl, args.dequant)
        out["prefix"] = prefix_section(wl, args.dequant)
        if w.kv_dtype == "nvfp4":
            other = "fp8" if args.dequant == "exact" else "exact"
            out["other_reading"] = reading_section(wl, other)
            out["other_reading"]["vs_headline_step"] = round(ms_step / out["other_reading"]["step_ms"], 3)
    if args.workload == "c3_128k" and not args.no_sides:
        out["ragged_c3"] = decode_section("c3", args.dequant, args.seed)
        out["spec_c4"] = decode_section("c4", args.dequant, 4)
        out["fp8_c2"] = decode_section("c2", args.dequant, 2)
        out["spec8_c3_128k"] = decode_section("c3_t8", args.dequant, 5)
        out["ceilings"] = ceilings_section()
        out["roofline"]["frac_of_measured_stream_read"] = round(
            achieved_idx / out["ceilings"]["stream_read"]["GBps"], 4)
    if not args.no_prefill and args.workload != "c5":
        wl5 = Workload("c5", args.seed)
        out["prefill"] = prefill_section(wl5, args.dequant)
        other = "fp8" if args.dequant == "exact" else "exact"
        out["prefill_other_reading"] = prefill_section(wl5, other)
        del wl5
        torch.cuda.empty_cache()
        out["insert"] = insert_section(args.seed)
    if sample:
        cores = len(os.sched_getaffinity(0))
        out["cpu_baseline"] = cpu_baseline(wl, args.dequant, sample, cores)
        out["cpu_baseline"]["one_core"] = cpu_baseline(wl, args.dequant, sample[:2], 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
