"""Builds libdd.so (the C-ABI HIP library) in-tree for gfx950.

    python -m sparse_kv_retrieval_dual_amd.build

Each source is compiled by hipcc into _build/ in parallel, then linked into
sparse_kv_retrieval_dual_amd/libdd.so.  Every call compiles from scratch.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdd.so")

SOURCES = ["score.hip", "topk.hip", "gather.hip", "attn.hip", "landmark.hip", "util.hip", "abi.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # Packed fp32 arithmetic stays off: the compiler must not form
    # v_pk_{add,mul,fma}_f32 on this target.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-result",
    "-I", INCLUDE, "-I", CSRC,
]


# Flags of single sources.  topk.hip: the backend's atomic optimizer turns
# an atomic at a uniform address into a wave-wide reduction loop; the only
# such atomics there are the per-layer counters, added by one lane, and the
# loop's register reuse made that lane wait for each atomic to complete
# before the workgroup's next barrier (a device-scope round trip on the
# selection's critical path).  Without it the three adds are issued back to
# back and nothing waits for them.
SOURCE_FLAGS = {
    "topk.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, *SOURCE_FLAGS.get(src, []), "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build_library(verbose: bool = True) -> str:
    if os.path.isdir(BUILD_DIR):
        shutil.rmtree(BUILD_DIR)
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build_library()
    sys.exit(0)
