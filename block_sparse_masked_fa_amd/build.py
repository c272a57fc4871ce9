"""Build libflexattn.so for gfx950 with hipcc, in-tree.

Usage: ``python -m block_sparse_masked_fa_amd.build [--jobs N] [--verbose]``.
Objects go to ``_build/`` at the repository root; the library is written
next to this file. Every HIP translation unit is compiled with packed fp32
arithmetic disabled (the kernels use plain float code only).
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libflexattn.so")

SOURCES = [
    "api.cpp",
    "validate.cpp",
    "block_mask.hip",
    "fwd_bf16_d64.hip",
    "fwd_bf16_d128.hip",
    "fwd_fp32.hip",
    "fwd_combine.hip",
    "fwd_noalloc.hip",
    "bwd_prepare.hip",
    "bwd_bf16_d64.hip",
    "bwd_bf16_d128.hip",
    "decode_bf16.hip",
    "masked_softmax.hip",
]

# Per-source extra flags. The backward kernels keep two fp32 tiles, two
# accumulator sets and their operands live at one wave per SIMD; LLVM's
# iterative ILP scheduler keeps their LDS reads ahead of the MFMAs that use
# them where the default scheduler serialises read, wait and MFMA (measured:
# about 20% less time for the dK / dV kernel). VGPR-form MFMAs: left to its
# heuristic, the compiler gives every MFMA of the dK / dV kernel accumulation
# registers (AGPRs), so the S and dP tiles that the VALU works on are copied
# out of them each stage (64 moves per stage); in VGPR form they stay put and
# the resident K^T and V^T operands move to AGPRs, which MFMA reads directly.
BWD_FLAGS = ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp",
             "-mllvm", "--amdgpu-mfma-vgpr-form"]
EXTRA_FLAGS = {
    "bwd_bf16_d64.hip": BWD_FLAGS,
    "bwd_bf16_d128.hip": BWD_FLAGS,
}

ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *CFLAGS, *EXTRA_FLAGS.get(src, []), "-c",
           os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    t = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"  {src}: {time.time() - t:.1f}s", flush=True)
        if r.stderr.strip():
            print(r.stderr, flush=True)
    return obj


def build(jobs: int = 0, verbose: bool = False) -> str:
    """Compile every source and link the shared library. Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
           *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.verbose))
    return 0


if __name__ == "__main__":
    sys.exit(main())
