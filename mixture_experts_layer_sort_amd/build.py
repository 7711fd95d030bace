"""Build libmoe_mi355x.so (the HIP library) in-tree with hipcc for gfx950.

    python -m mixture_experts_layer_sort_amd.build
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libmoe_mi355x.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
ARCH = "gfx950"

FLAGS = [
    "-O3",
    "-std=c++17",
    f"--offload-arch={ARCH}",
    "-shared",
    "-fPIC",
    # packed fp32 arithmetic off: the compiler must not emit v_pk_{add,mul,fma}_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # fp32 division and sqrt correctly rounded (quantisation decisions depend on it)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fvisibility=hidden",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the MoE library)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed with status {r.returncode}")


def _compile(srcs, out, verbose):
    """Each source to an object in parallel (the translation units share no
    device code), then one link."""
    inc = ["-I", os.path.join(PKG_DIR, "..", "include")]
    cflags = [f for f in FLAGS if f not in ("-shared",)]
    with tempfile.TemporaryDirectory(prefix="moe_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in srcs]
        jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
        with ThreadPoolExecutor(jobs) as pool:
            for f in [pool.submit(_run, [hipcc(), *cflags, *inc, "-c", "-o", o, src], verbose)
                      for src, o in zip(srcs, objs)]:
                f.result()
        tmp = out + ".tmp"
        _run([hipcc(), *FLAGS, "-o", tmp, *objs], verbose)
        os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every HIP source under csrc/ into LIB_PATH; returns LIB_PATH."""
    _compile(sorted(glob.glob(os.path.join(CSRC, "*.hip"))), LIB_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
