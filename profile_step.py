"""Collect the rocprofv3 figures that bench.py reports, for one workload.

    python profile_step.py [--workload c3_128k] [--only insert|dcp|prefix] [--out DIR]

Runs bench.py five times as a child process under rocprofv3 (this process
never touches the GPU):

  1. --kernel-trace --stats      bench.py --steps 10 --warmup 2 --no-cpu-baseline --no-prefill --no-sides
  2. --pmc FETCH_SIZE            bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-prefill --no-sides
                                 --calib-copy-mib 512
  3. --pmc WRITE_SIZE            (same)
  4. --pmc SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VALU
           SQ_INSTS_VALU SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE   (same bench.py)
  5. --pmc SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_LDS SQ_INSTS_LDS SQ_INST_LEVEL_VMEM
           SQ_ACTIVE_INST_ANY GRBM_GUI_ACTIVE                                  (same bench.py)

FETCH_SIZE / WRITE_SIZE readings are per dispatch, in KiB.  Each is scaled by
what the same counter reads for the 512 MiB elementwise copy that bench.py
launches with --calib-copy-mib (which reads and writes exactly 512 MiB), so the
reported bytes are calibrated HBM bytes per launch.  The SQ counters give, per
kernel: VALU and MFMA instructions per wave, the VALU and MFMA pipes' busy
fractions, the share of wave time spent waiting, and LDS bank-conflict cycles
per LDS instruction (formulas in the summary).  Writes, into --out:

With --only, bench.py runs that side section alone (bench.py --only ...) and the
files are named cache_insert_c5_chunk_and_c3_decode.*, dcp_<workload>.* or prefix_<workload>.*
instead.

  layer_step_<workload>.md           per-kernel launches and durations, calibrated HBM
                          bytes per launch, the calibration factors and the
                          commands that produced them;
  layer_step_<workload>_traffic.json the same numbers for bench.py, with a hash of the
                          kernel sources they were measured on.
Raw rocprofv3 output is deleted once summarised.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "block_sparse_attention_indexer_amd", "csrc")
CALIB_MIB = 512
# SQ counter passes (at most 8 SQ and 2 GRBM counters each, which one rocprofv3 pass can hold)
SQ_PASSES = {
    "SQ1": ["SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU",
            "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"],
    "SQ2": ["SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS", "SQ_INSTS_LDS", "SQ_INST_LEVEL_VMEM",
            "SQ_ACTIVE_INST_ANY", "GRBM_GUI_ACTIVE"],
}
XCDS = 8          # MI355X: GRBM_GUI_ACTIVE sums the active cycles of its 8 XCDs
CUS = 256         # MI355X compute units (4 SIMDs each)


def sources_hash():
    """sha256 over the library's kernel and host sources (sorted by name)."""
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(CSRC, "*"))):
        h.update(os.path.basename(p).encode())
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def role_of(name):
    """Which step of the layer a kernel belongs to."""
    for key, role in (("indexer", "indexer"), ("topk", "topk"), ("attn", "attention")):
        if key in name:
            return role
    return None


def short(name):
    """Kernel name without the argument list."""
    n = name.replace("void ", "")
    depth = 0
    for i, ch in enumerate(n):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return n[:i]
    return n


def derive(c):
    """Per-kernel figures from the SQ counters of one dispatch (whole-GPU sums).
    SIMD-cycles = 4 SIMDs x CUs x (GRBM_GUI_ACTIVE / XCDS) -- the kernel's active
    cycles on every SIMD; a wave64 VALU instruction occupies its SIMD 4 cycles and
    SQ_VALU_MFMA_BUSY_CYCLES counts MFMA pipe cycles directly."""
    out = {}
    waves = c.get("SQ_WAVES", 0)
    gui = c.get("GRBM_GUI_ACTIVE", 0) / XCDS
    simd_cycles = 4 * CUS * gui
    if waves:
        if "SQ_INSTS_VALU" in c:
            out["valu_per_wave"] = c["SQ_INSTS_VALU"] / waves
        if "SQ_INSTS_MFMA" in c:
            out["mfma_per_wave"] = c["SQ_INSTS_MFMA"] / waves
        if "SQ_INSTS_LDS" in c:
            out["lds_per_wave"] = c["SQ_INSTS_LDS"] / waves
    if simd_cycles:
        if "SQ_ACTIVE_INST_VALU" in c:
            out["valu_busy"] = 4 * c["SQ_ACTIVE_INST_VALU"] / simd_cycles
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
            out["mfma_busy"] = c["SQ_VALU_MFMA_BUSY_CYCLES"] / simd_cycles
    if c.get("SQ_WAVE_CYCLES"):
        out["wait_share"] = c.get("SQ_WAIT_INST_ANY", 0) / c["SQ_WAVE_CYCLES"]
    if c.get("SQ_INSTS_LDS"):
        out["lds_conflict_cycles_per_lds_inst"] = c.get("SQ_LDS_BANK_CONFLICT", 0) / c["SQ_INSTS_LDS"]
    return out


def run(cmd, log):
    env = dict(os.environ, TMPDIR="/tmp")
    print("[profile] " + " ".join(cmd), flush=True)
    with open(log, "w") as fh:
        r = subprocess.run(cmd, cwd="/tmp", env=env, stdout=fh, stderr=subprocess.STDOUT, timeout=300)
    print(f"[profile] exit {r.returncode}", flush=True)
    return r.returncode


def read_counters(d):
    """{(kernel, counter): [values]} and {kernel: grid sizes} from counter_collection CSVs."""
    vals, grids = {}, {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                name = row.get("Kernel_Name", "")
                if "msa::" not in name and "MulFunctor" not in name:
                    continue
                vals.setdefault((name, row["Counter_Name"]), []).append(
                    (int(row.get("Grid_Size", 0) or 0), float(row["Counter_Value"])))
    return vals


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="c3_128k")
    ap.add_argument("--only", choices=["insert", "dcp", "prefix"], default=None)
    ap.add_argument("--out", default=os.path.join(ROOT, "profile_out"))
    args = ap.parse_args()
    args.out = os.path.abspath(args.out)   # rocprofv3 runs from /tmp
    os.makedirs(args.out, exist_ok=True)
    py = sys.executable
    bench = os.path.join(ROOT, "bench.py")
    w = args.workload
    raw = os.path.join(args.out, "raw")
    shutil.rmtree(raw, ignore_errors=True)

    only = ["--only", args.only] if args.only else []
    tag = {None: f"layer_step_{w}", "insert": "cache_insert_c5_chunk_and_c3_decode", "dcp": f"dcp_{w}",
           "prefix": f"prefix_{w}"}[args.only]
    title = {None: f"MSA layer step, workload {w}",
             "insert": "quantise-and-insert (msa_cache_insert_many, msa_cache_insert), c5 prefill chunk and "
                       "c3_128k decode token",
             "dcp": f"single-GPU DCP (4 shard scans, local top-16s, merge), workload {w}",
             "prefix": f"shared-prefix index scan against the unshared scan, workload {w}"}[args.only]
    trace_cmd = ["rocprofv3", "--kernel-trace", "--stats", "-d", os.path.join(raw, "trace"), "-o", "run",
                 "-f", "csv", "--", py, bench, "--workload", w, "--steps", "10", "--warmup", "2",
                 "--no-cpu-baseline", "--no-prefill", "--no-sides"] + only
    pmc_bench = [py, bench, "--workload", w, "--steps", "3", "--warmup", "1", "--no-cpu-baseline", "--no-prefill",
                 "--no-sides", "--calib-copy-mib", str(CALIB_MIB)] + only
    cmds = {"trace": trace_cmd}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        cmds[c] = ["rocprofv3", "--pmc", c, "-d", os.path.join(raw, c), "-o", "run", "-f", "csv", "--"] + pmc_bench
    for tagp, cs in SQ_PASSES.items():
        cmds[tagp] = ["rocprofv3", "--pmc"] + cs + ["-d", os.path.join(raw, tagp), "-o", "run", "-f", "csv",
                                                   "--"] + pmc_bench
    for k, cmd in cmds.items():
        if run(cmd, os.path.join(args.out, f"{tag}_{k}.log")) != 0:
            sys.exit(f"rocprofv3 pass {k} failed; see {args.out}/{tag}_{k}.log")

    # per-dispatch durations by launch shape (grid size), for kernels launched with several shapes
    shapes = {}
    for f in glob.glob(os.path.join(raw, "trace", "**", "*kernel_trace.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                name = row.get("Kernel_Name", "")
                if "msa::" not in name:
                    continue
                grid = "x".join(row[k] for k in sorted(row) if k.startswith("Grid_Size"))
                dur = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
                shapes.setdefault((short(name), grid), []).append(dur)
    # kernel trace statistics
    stats = {}
    for f in glob.glob(os.path.join(raw, "trace", "**", "*kernel_stats.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if "msa::" in row["Name"]:
                    stats[short(row["Name"])] = {"calls": int(row["Calls"]), "avg_us": float(row["AverageNs"]) / 1e3,
                                                 "min_us": float(row["MinNs"]) / 1e3, "max_us": float(row["MaxNs"]) / 1e3}
    # counters
    kib = {}
    calib = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        vals = read_counters(os.path.join(raw, c))
        copy = [v for (name, cn), lst in vals.items() if "MulFunctor" in name and cn == c for v in lst]
        gmax = max(g for g, _ in copy)
        copy_kib = [v for g, v in copy if g == gmax]
        calib[c] = CALIB_MIB * 1024.0 / (sum(copy_kib) / len(copy_kib))
        for (name, cn), lst in vals.items():
            if "msa::" in name and cn == c:
                kib.setdefault(short(name), {})[c] = sum(v for _, v in lst) / len(lst)
    sq = {}
    for tagp, cs in SQ_PASSES.items():
        vals = read_counters(os.path.join(raw, tagp))
        for (name, cn), lst in vals.items():
            if "msa::" in name:
                sq.setdefault(short(name), {})[cn] = sum(v for _, v in lst) / len(lst)
    shutil.rmtree(raw, ignore_errors=True)

    kernels = {}
    for name in sorted(set(stats) | set(kib)):
        if "pack" in name:
            continue
        e = dict(stats.get(name, {}))
        k = kib.get(name, {})
        if "FETCH_SIZE" in k:
            e["fetch_bytes"] = k["FETCH_SIZE"] * 1024.0 * calib["FETCH_SIZE"]
        if "WRITE_SIZE" in k:
            e["write_bytes"] = k["WRITE_SIZE"] * 1024.0 * calib["WRITE_SIZE"]
        e["role"] = role_of(name)
        c = sq.get(name)
        if c:
            e["sq"] = c
            e["derived"] = derive(c)
        kernels[name] = e
    out = {"workload": w, "sources_sha256": sources_hash(), "calibration": calib,
           "commands": {k: " ".join(v) for k, v in cmds.items()}, "kernels": kernels}
    with open(os.path.join(args.out, f"{tag}_traffic.json"), "w") as fh:
        json.dump(out, fh, indent=1)

    lines = [f"# rocprofv3 summary: {title}", "",
             "Produced by `python profile_step.py --workload " + w + " ".join([""] + only) +
             " --out " + os.path.relpath(args.out, ROOT) + "` on one MI355X, which runs:", ""]
    lines += ["    " + " ".join(c if not c.startswith(ROOT) else os.path.relpath(c, ROOT) for c in v)
              .replace(py, "python3") for v in cmds.values()]
    lines += ["", "(rocprofv3 runs from /tmp with TMPDIR=/tmp; raw output is summarised and deleted.)", "",
              f"Counter calibration: the 512 MiB elementwise copy reads FETCH_SIZE x {calib['FETCH_SIZE']:.4f} and "
              f"WRITE_SIZE x {calib['WRITE_SIZE']:.4f} of its true bytes' KiB, so per-kernel readings are "
              "multiplied by these factors.", "",
              f"Kernel sources sha256: `{out['sources_sha256']}`", "",
              "| kernel | launches | avg us | min us | max us | HBM read B/launch | HBM write B/launch |",
              "|---|---|---|---|---|---|---|"]
    for name, e in kernels.items():
        lines.append(f"| `{name}` | {e.get('calls', '')} | {e.get('avg_us', 0):.2f} | {e.get('min_us', 0):.2f} | "
                     f"{e.get('max_us', 0):.2f} | {e.get('fetch_bytes', 0):,.0f} | {e.get('write_bytes', 0):,.0f} |")
    with_sq = [(n, e) for n, e in kernels.items() if "derived" in e]
    if with_sq:
        lines += ["", "SQ counters (passes SQ1 and SQ2, whole-GPU sums per dispatch).  VALU busy = 4 x "
                  "SQ_ACTIVE_INST_VALU / SIMD-cycles and MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / SIMD-cycles, "
                  f"with SIMD-cycles = 4 x {CUS} x GRBM_GUI_ACTIVE / {XCDS}; wait = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES; "
                  "LDS conflict = SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS.", "",
                  "| kernel | waves | VALU / wave | MFMA / wave | LDS / wave | VALU busy | MFMA busy | wait | "
                  "LDS conflict cycles / LDS inst |", "|---|---|---|---|---|---|---|---|---|"]
        for name, e in with_sq:
            d, c = e["derived"], e["sq"]
            f = lambda k, fmt: format(d[k], fmt) if k in d else ""
            lines.append(f"| `{name}` | {c.get('SQ_WAVES', 0):,.0f} | {f('valu_per_wave', ',.0f')} | "
                         f"{f('mfma_per_wave', ',.1f')} | {f('lds_per_wave', ',.1f')} | {f('valu_busy', '.3f')} | "
                         f"{f('mfma_busy', '.3f')} | {f('wait_share', '.3f')} | "
                         f"{f('lds_conflict_cycles_per_lds_inst', '.3f')} |")
        lines += ["", "Raw SQ counters:", "", "| kernel | counter | value |", "|---|---|---|"]
        for name, e in with_sq:
            for cn, v in sorted(e["sq"].items()):
                lines.append(f"| `{name}` | {cn} | {v:,.0f} |")
    grids_of = {}
    for name, grid in shapes:
        grids_of.setdefault(name, set()).add(grid)
    multi = sorted(name for name, grids in grids_of.items() if len(grids) > 1)
    if multi:
        lines += ["", "Kernels launched with several grid sizes, by launch shape (kernel trace):", "",
                  "| kernel | grid (threads) | launches | avg us | min us |", "|---|---|---|---|---|"]
        for (name, grid), durs in sorted(shapes.items()):
            if name in multi:
                lines.append(f"| `{name}` | {grid} | {len(durs)} | {sum(durs) / len(durs):.2f} | {min(durs):.2f} |")
    with open(os.path.join(args.out, f"{tag}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines), flush=True)


if __name__ == "__main__":
    main()
