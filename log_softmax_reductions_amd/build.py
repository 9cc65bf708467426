"""Build liblse.so (the C-ABI library) from csrc/ with hipcc for gfx950.

Each .hip file is compiled to an object with hipcc; the objects are linked
into one shared library whose only exported symbols are the entry points of
include/lse.h.  No PyTorch headers or libraries are involved.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liblse.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["lse_axis.hip", "lse_cols.hip", "lse_blocks.hip", "lse_rows.hip", "conv_chain.hip", "lse_noalloc.hip", "lse_api.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


BENCH_COPY_SRC = os.path.join(ROOT, "bench_copy.hip")
BENCH_COPY_LIB = os.path.join(ROOT, "libbench_copy.so")


def build_bench_copy() -> str:
    """The benchmark's copy kernels (bench_copy.hip, not part of liblse.so)."""
    tmp = BENCH_COPY_LIB + ".tmp"
    cmd = [HIPCC, *CFLAGS, "-shared", BENCH_COPY_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on bench_copy.hip:\n{r.stderr}")
    os.replace(tmp, BENCH_COPY_LIB)
    return BENCH_COPY_LIB


def build() -> str:
    """Compile every source and link liblse.so in-tree; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
