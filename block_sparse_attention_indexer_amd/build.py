"""Build libmsa.so for gfx950 in-tree with hipcc (cross-compiles without a GPU),
and the benchmark's probe library bench_probes/libmsa_probe.so beside it.

    python -m block_sparse_attention_indexer_amd.build
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libmsa.so")
BUILD = os.path.join(ROOT, "_build", "msa")
PROBE_SRC = os.path.join(ROOT, "bench_probes", "probe.hip")
PROBE_OUT = os.path.join(ROOT, "bench_probes", "libmsa_probe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 instructions are kept out of the device code on purpose.
COMMON = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
          "-I", os.path.join(ROOT, "include"), "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
SOURCES = ["pack.hip", "insert.hip", "indexer.hip", "indexer_prefill.hip", "topk.hip", "attn.hip",
           "dcp.hip", "prefix_attn.hip", "noalloc.hip", "api.cpp"]
# Per-file flags.  The prefill index GEMM only takes maxima of MFMA results, which
# hold no NaN (an unreadable page is marked through the NaN bit pattern, stored as
# an integer); with NaN semantics every fmaxf of an MFMA result is preceded by a
# canonicalising max, ~6% of that kernel's time.
# The decode scans read their MFMA results straight from ordinary vector
# registers: left to itself the compiler puts the speculative scan's
# accumulators in AGPRs and copies every result out (32 extra VALU per unit).
EXTRA = {"indexer_prefill.hip": ["-fno-honor-nans"],
         "indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src):
    path = src if os.path.isabs(src) else os.path.join(CSRC, src)
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + EXTRA.get(src, []) + (["-x", "hip"] if src.endswith(".hip") else []) + \
        ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    return obj, msgs


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4)) as ex:
        results = list(ex.map(_compile, SOURCES + [PROBE_SRC]))
    for _, msgs in results:
        if msgs.strip() and verbose:
            print(msgs)
    objs = [o for o, _ in results]
    _link(objs[:-1], OUT)
    _link(objs[-1:], PROBE_OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
