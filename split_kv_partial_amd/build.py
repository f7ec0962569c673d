"""Build libsplitkv.so in-tree with hipcc for gfx950.

Usage: python split_kv_partial_amd/build.py  (or load this file and call
build(); importing it as a submodule of the package would first load the
library it builds).
Every source is compiled on each call; objects go to _build/ next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libsplitkv.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = [
    "api.cpp",
    "planner.cpp",
    "noalloc.cpp",
    "kernels/gqa_valu.hip",
    "kernels/gqa_mfma.hip",
    "kernels/mla_mfma.hip",
    "kernels/merge.hip",
    "kernels/probe.hip",
]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    # no contraction of separate multiplies and adds: the planner's doubles must
    # match the reference simulation bit for bit
    "-ffp-contract=off",
    # keep the compiler from forming packed fp32 instructions on the device
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


def _compile(src: str, obj_dir: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(obj_dir, src.replace("/", "_") + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else ["-x", "hip"]
    cmd = [HIPCC, *COMMON, *lang, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp, "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
