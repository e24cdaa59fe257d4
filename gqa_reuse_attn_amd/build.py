"""Build libgqa_av.so (HIP, gfx950) in-tree with hipcc.

    python -m gqa_reuse_attn_amd.build          # or: python gqa_reuse_attn_amd/build.py

Every csrc/*.hip is one translation unit: the host side (gqa_av.hip, with the
score step's host code) and one unit per engine and element type
(launch_*.hip) that instantiates only that engine's kernels. They compile in
parallel to objects for gfx950 only and are linked into one shared library.
Packed fp32 instructions are disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
HEADERS = sorted(glob.glob(os.path.join(CSRC, "*.hpp"))) + sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))
LIB = os.path.join(PKG, "libgqa_av.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libgqa_av.so)")


def flags(extra=None):
    """Compile flags of every translation unit."""
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        *(extra or []),
    ]


def _compile(src: str, obj: str, extra, verbose: bool) -> str:
    cmd = [hipcc(), *flags(extra), "-c", "-o", obj, src]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {os.path.basename(src)} failed:\n{r.stdout}{r.stderr}")
    return obj


def build(out: str = LIB, extra=None, verbose: bool = False, jobs: int = 0) -> str:
    """Compile every csrc/*.hip (in parallel) and link them into `out`; always recompiles."""
    jobs = jobs or min(len(SOURCES), max(1, len(os.sched_getaffinity(0))))
    with tempfile.TemporaryDirectory(prefix="gqa_av_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(src)[:-4] + ".o") for src in SOURCES]
        with cf.ThreadPoolExecutor(jobs) as ex:
            list(ex.map(lambda so: _compile(so[0], so[1], extra, verbose), zip(SOURCES, objs)))
        tmp_lib = out + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib, *objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp_lib, out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)
    sys.exit(0)
