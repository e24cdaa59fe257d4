"""Build libgqa_av.so (HIP, gfx950) in-tree with hipcc.

    python -m gqa_reuse_attn_amd.build          # or: python gqa_reuse_attn_amd/build.py

The library is a single translation unit (csrc/gqa_av.hip includes the kernel
header) compiled for gfx950 only. Packed fp32 instructions are disabled for all
device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "gqa_av.hip")
HEADERS = [os.path.join(PKG, "csrc", f) for f in ("av_kernels.hpp", "qk_kernels.hpp", "qk_host.hpp")] + \
    [os.path.join(ROOT, "include", f) for f in ("gqa_av.h", "gqa_qk.h", "gqa_softmax_av.h", "gqa_paged_av.h", "gqa_fp8_av.h")]
LIB = os.path.join(PKG, "libgqa_av.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libgqa_av.so)")


def flags(extra=None):
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
        *(extra or []),
    ]


def build(out: str = LIB, extra=None, verbose: bool = False) -> str:
    """Compile csrc/gqa_av.hip into `out`; always recompiles."""
    tmp = out + ".tmp"
    cmd = [hipcc(), *flags(extra), "-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)
    sys.exit(0)
