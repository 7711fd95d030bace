"""CPU checks of bench.py's command line: the benchmark measures one GPU's
share of the layer, so a multi-GPU request exits with a message before any
GPU work (and without importing torch)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus 2 is not supported" in r.stderr
    assert r.stdout == ""
