"""GPU parity of the product over a capacity-strided V cache
(gqa_av_decode_strided): V is [B][C_max][Hkv][D] with any capacity
C_max >= C, and rows c < C of every sequence take part. The rows past C hold
NaN, so a kernel that touched them would fail. Each call is checked against
the fp64 oracle on the first C rows (gathered by torch slicing) and against
the dense call on those rows made contiguous, with the same plan, bit for bit.
Needs an MI355X; marked ``gpu``."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import gqa_reuse_attn_amd as ga
from tests.parity import assert_parity
from workloads import WORKLOADS, make_inputs, make_random

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ga.load()
    yield
    torch.cuda.synchronize()


def _strided(V, C_max):
    """V [B, C, Hkv, D] placed at the start of each sequence's C_max rows; the rest NaN."""
    B, C, Hkv, D = V.shape
    full = torch.full((B, C_max, Hkv, D), float("nan"), dtype=V.dtype)
    full[:, :C] = V
    return full


def _plans(B, C, Hq, Hkv, D, dt):
    plans = [("auto", None), ("auto/3", ga.make_plan(B, C, Hq, Hkv, D, dt, nsplit=3)),
             ("auto/1", ga.make_plan(B, C, Hq, Hkv, D, dt, nsplit=1)),
             ("contiguous/5", ga.make_plan(B, C, Hq, Hkv, D, dt, nsplit=5, split_order="contiguous"))]
    if Hq // Hkv >= 2:
        plans.append(("per_head", ga.make_plan(B, C, Hq, Hkv, D, dt, "per_head", nsplit=4)))
        for eng in ("valu", "mfma", "mfma_bf16"):
            try:
                plans.append((eng, ga.make_plan(B, C, Hq, Hkv, D, dt, "reuse", engine=eng, nsplit=4)))
            except ga.GqaAvError as e:
                assert e.name == "UNSUPPORTED"
    return plans


@pytest.mark.parametrize("B,C,C_max,Hq,Hkv,D,dt", [
    (2, 300, 301, 8, 2, 128, "bf16"), (3, 1000, 1537, 16, 1, 128, "bf16"), (2, 777, 1000, 24, 8, 96, "f16"),
    (2, 65, 129, 8, 8, 64, "f32"), (1, 500, 500, 32, 4, 64, "f32"), (2, 129, 1000, 64, 8, 128, "bf16"),
    (2, 1, 7, 16, 2, 256, "bf16")])
def test_strided_sweep(B, C, C_max, Hq, Hkv, D, dt, oracle_lib):
    attn, V = make_random(B, C, Hq, Hkv, D, dt, seed=C + C_max, attn_kind="signed")
    ref = oracle_lib.full(attn, V, dt)
    a, vs, vd = attn.to(DEV), _strided(V, C_max).to(DEV), V.to(DEV)
    for name, plan in _plans(B, C, Hq, Hkv, D, dt):
        got = ga.gqa_av_decode_strided(a, vs, C, plan=plan)
        want = ga.gqa_av_decode(a, vd, plan=plan)
        torch.cuda.synchronize()
        label = f"{(B, C, C_max, Hq, Hkv, D, dt)} {name}"
        assert torch.equal(got, want), f"{label}: strided call differs from the dense call"
        assert_parity(got.cpu().numpy().astype(np.float64), ref, dt, C, label)


@pytest.mark.parametrize("wname", ["g2-b4-c32768-hq16-hkv8-d128-bf16", "mqa16-b4-c32768-hq16-hkv1-d128-bf16",
                                   "g3-b8-c16384-hq24-hkv8-d96-f16"])
def test_strided_workloads(wname, oracle_lib):
    """Full-size workloads in a cache of capacity C + C / 3 (not a power of two)."""
    w = WORKLOADS[wname]
    C_max = w.C + w.C // 3
    print(f"[strided] {wname} C_max={C_max}", flush=True)
    sys.stdout.flush()
    attn, V = make_inputs(w, seed=2)
    ref = oracle_lib.full(attn, V, w.v_dtype)
    a, vs, vd = attn.to(DEV), _strided(V, C_max).to(DEV), V.to(DEV)
    got = ga.gqa_av_decode_strided(a, vs, w.C)
    want = ga.gqa_av_decode(a, vd)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    assert_parity(got.cpu().numpy().astype(np.float64), ref, w.v_dtype, w.C, f"strided {wname}")


def test_strided_refusals():
    a = torch.zeros(2, 100, 8, device=DEV)
    v = torch.zeros(2, 100, 2, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        ga.gqa_av_decode_strided(a, v[:, :50].contiguous(), 100)      # capacity below C
    lib = ga.load()
    out = torch.zeros(2, 8, 64, device=DEV)
    rc = lib.gqa_av_decode_strided(a.data_ptr(), v.data_ptr(), out.data_ptr(), 2, 100, 99, 8, 2, 64, 2, -1, None)
    assert rc == 1 and b"capacity" in lib.gqa_av_last_error()
