"""Build the gfx950 HIP libraries in-tree with hipcc.

Every source under ``csrc/`` is compiled for ``--offload-arch=gfx950`` only,
with packed fp32 instructions disabled (``-packed-fp32-ops``), and linked into
``libotsinkhorn.so`` next to this file (the solver library). The instruction
rate microbenchmarks the benchmark uses for its ceilings,
``ratebench/rates.hip``, become ``ratebench/librates.so``. Run ``python -m
log_domain_sinkhorn_amd.build`` or call :func:`build`.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libotsinkhorn.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
BUILD_DIR = os.path.join(ROOT, "_build")
RATES_SRC = os.path.join(HERE, "ratebench", "rates.hip")
RATES_LIB = os.path.join(HERE, "ratebench", "librates.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, path):
    tmp = path + f".tmp{os.getpid()}"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link ``libotsinkhorn.so`` (and the rate
    microbenchmarks' ``librates.so``); returns the solver library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources() + [RATES_SRC]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:-1], LIB_PATH)
    _link(objs[-1:], RATES_LIB)
    if verbose:
        print(f"built {LIB_PATH} and {RATES_LIB}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
