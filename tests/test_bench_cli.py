"""bench.py's command line without a GPU: it measures one GPU and says so when asked
for more (it exits before touching torch or the library)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
