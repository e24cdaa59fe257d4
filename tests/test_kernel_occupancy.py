"""Register budgets of the kernels the decode workloads run (CPU; needs hipcc).

The planner runs two workgroups per CU for the VALU engine (4 waves each), for
the bf16 matrix engine's eight-wave plans (one workgroup), and for its fp8
fused softmax and fused attention (4 waves each): two waves per SIMD. A
kernel whose registers (VGPRs + AGPRs) pass 256 runs one wave per SIMD and
halves that parallelism without any error (fp8 fused attention at B = 64,
C = 8192, G = 8 once went from 178 to 209 us that way). This test compiles
those translation units to gfx950 assembly and checks the compiler's
occupancy for each instantiation the workloads use."""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from gqa_reuse_attn_amd import build as B

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")

# translation unit -> [(kernel name pattern, waves per SIMD the plans need)]
NEED = {
    "launch_valu_bf16_plain.hip": [(r"av_pass1_valuILi2ELi16ELi[24]ELi4ELb0ELb0E", 2)],
    "launch_valu_f16_plain.hip": [(r"av_pass1_valuILi1ELi16ELi3ELi8ELb0ELb0E", 2)],
    "launch_valu_bf16_sm.hip": [(r"av_pass1_valuILi2ELi16ELi[24]ELi4ELb1ELb0E", 2)],
    "launch_mfma_bf16_bf16_sm.hip": [(r"av_pass1_mfma_bf16ILi16ELi1ELi1ELi8ELb1ELi2ELb0ELb0ELi8E", 2)],
    "launch_mfma_bf16_bf16_plain.hip": [(r"av_pass1_mfma_bf16ILi16ELi1ELi1ELi[18]ELb0ELi2ELb0ELb0ELi8E", 2),
                                        (r"av_pass1_mfma_bf16ILi16ELi1ELi1ELi4ELb0ELi2ELb0ELb0ELi4E", 1)],
    "launch_mfma_bf16_fp8_attn.hip": [(r"av_pass1_mfma_bf16ILi16ELi1ELi1ELi[124]ELb1ELi3ELb0ELb1ELi4E", 2)],
    "launch_mfma_bf16_fp8_sm.hip": [(r"av_pass1_mfma_bf16ILi16ELi1ELi1ELi[124]ELb1ELi3ELb0ELb0ELi4E", 2)],
}


def _occupancy(asm: str) -> dict:
    occ = {}
    for m in re.finditer(r"^(_Z\S+):\s*;", asm, re.M):
        end = asm.find(".Lfunc_end", m.start())
        o = re.search(r"; Occupancy: (\d+)", asm[end:end + 6000])
        if o:
            occ[m.group(1)] = int(o.group(1))
    return occ


def _compile(tu: str, out: str) -> str:
    flags = B.flags()
    cmd = [HIPCC, *flags, "--cuda-device-only", "-S", "-o", out, os.path.join(B.CSRC, tu)]
    subprocess.run(cmd, check=True, capture_output=True)
    return open(out).read()


def test_hot_kernels_keep_the_waves_their_plans_need():
    with tempfile.TemporaryDirectory() as d:
        with ThreadPoolExecutor(len(NEED)) as ex:
            asm = dict(zip(NEED, ex.map(lambda tu: _compile(tu, os.path.join(d, tu + ".s")), NEED)))
    for tu, needs in NEED.items():
        occ = _occupancy(asm[tu])
        for pat, need in needs:
            hits = {k: v for k, v in occ.items() if re.search(pat, k)}
            assert hits, f"{tu}: no kernel matches {pat}"
            low = {k: v for k, v in hits.items() if v < need}
            assert not low, f"{tu}: waves per SIMD below {need}: {low}"
