"""bench.py's command line on a host without a GPU: more than one GPU is
refused with a message (the library has no multi-GPU path), before torch or
the library is touched."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "measures one GPU" in r.stderr
    assert r.stdout == ""
