"""Build the HIP library ``libawq_mi355x.so`` in-tree for gfx950 with hipcc.

Every source is compiled to an object in parallel, then linked into one
shared library next to this file. Flags:
  -O3 --offload-arch=gfx950          CDNA4 only
  -ffp-contract=off                  the quantiser's float32 steps round once each
  -fhip-fp32-correctly-rounded-divide-sqrt   IEEE float32 division for the codes
  -Xclang -target-feature -Xclang -packed-fp32-ops   no packed fp32 instructions
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libawq_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = ["abi.cpp", "validate.cpp", "stats.hip", "scale.hip", "transform.hip", "gemm.hip",
           "reduce.hip", "pack.hip", "fold.hip", "w4a16.hip",
           "gram.hip", "fused.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-ffp-contract=off",
          "-fhip-fp32-correctly-rounded-divide-sqrt",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the AWQ HIP library)")


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, extra=()) -> str:
    """Compile every source and link ``libawq_mi355x.so``; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra)), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}", file=sys.stderr)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
