"""Build liblocks.so (HIP kernels for gfx950 + the C-ABI host code) in-tree.

    python -m sparse_kv_page_amd.build [--jobs N]

Each source is compiled with hipcc for gfx950 only, then linked into
sparse_kv_page_amd/liblocks.so next to this file.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "liblocks.so")
BUILD_DIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["locks_api.cpp", "page_score.hip", "page_score_i4.hip", "select.hip", "sparse_decode.hip",
           "build_summaries.hip", "hot_cache.hip"]
HEADERS = ["common.h", "kernels.h", "score_lds.h", "select_unit.h", "decode_split.h",
           os.path.join("..", "..", "include", "locks.h")]

FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-fno-gpu-rdc",
         # packed fp32 VALU instructions are kept out of the generated code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I" + os.path.join(ROOT, "include")]


# Kernel sources only (not the host validation in locks_api.cpp): no NaN
# operands reach the reductions, which lets max fuse with DPP lane moves.
# Infinities stay honoured (-inf marks masked logits and empty pages).
KERNEL_FLAGS = ["-fno-honor-nans"]


def _compile(src: str) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + KERNEL_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC] + FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every source (always) and link liblocks.so. Returns its path."""
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        raise RuntimeError("hipcc not found; ROCm is required to build liblocks.so")
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    args = ap.parse_args()
    build(args.jobs, verbose=True)
    sys.exit(0)
