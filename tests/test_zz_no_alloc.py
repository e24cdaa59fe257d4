"""GPU test of gqa_av_decode_noalloc, the entry point that allocates nothing:
called through the C ABI, it must give what gqa_av_decode gives on the same
inputs (same plan, same kernels, so the same bits) and pass the acceptance
gate against the fp64 oracle, on two calls in a row of which the second is
smaller; a problem whose split partials exceed the fixed scratch array is
refused before anything is launched. Needs an MI355X; marked ``gpu``.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import gqa_reuse_attn_amd as ga
from tests.parity import assert_parity
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCRATCH = 8 << 20            # GQA_AV_NOALLOC_SCRATCH_BYTES


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ga.load()
    yield
    torch.cuda.synchronize()


def _c_call(fn, a, v, out, dt):
    B, C, Hq = a.shape
    Hkv, D = v.shape[2], v.shape[3]
    rc = getattr(ga.load(), fn)(a.data_ptr(), v.data_ptr(), out.data_ptr(), B, C, Hq, Hkv, D, ga.DTYPES[dt], -1,
                                torch.cuda.current_stream().cuda_stream)
    return rc


@pytest.mark.parametrize("first,second", [
    ("g2-b4-c32768-hq16-hkv8-d128-bf16", "llama3-8b-b1-c4096-hq32-hkv8-d128-bf16"),
    ("batch64-b64-c8192-hq64-hkv8-d128-bf16", "mqa16-b4-c32768-hq16-hkv1-d128-bf16"),
])
def test_noalloc_matches_decode(first, second, oracle_lib):
    """Two calls in a row, the second on a smaller problem: each equals the
    allocating entry point bit for bit and passes the gate."""
    for name in (first, second):
        w = WORKLOADS[name]
        print(f"[noalloc] {name}", flush=True)
        sys.stdout.flush()
        plan = ga.make_plan(w.B, w.C, w.Hq, w.Hkv, w.D, w.v_dtype,
                            cu_count=torch.cuda.get_device_properties(0).multi_processor_count)
        assert plan.nsplit > 1 and 0 < plan.workspace_bytes <= SCRATCH   # the scratch array is used
        attn, V = make_inputs(w, seed=3)
        a, v = attn.to(DEV), V.to(DEV)
        got = torch.full((w.B, w.Hq, w.D), float("nan"), device=DEV)
        want = torch.full((w.B, w.Hq, w.D), float("nan"), device=DEV)
        assert _c_call("gqa_av_decode_noalloc", a, v, got, w.v_dtype) == 0, ga.load().gqa_av_last_error()
        assert _c_call("gqa_av_decode", a, v, want, w.v_dtype) == 0
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"{name}: noalloc differs from gqa_av_decode"
        if w.B <= 8:                                 # the oracle on the whole output (small problems)
            ref = oracle_lib.full(attn, V, w.v_dtype)
            assert_parity(got.cpu().numpy().astype(np.float64), ref, w.v_dtype, w.C, f"noalloc {name}")
        else:                                        # sequences 0 and B-1 one by one
            for b in (0, w.B - 1):
                ref = oracle_lib.full(attn[b:b + 1], V[b:b + 1], w.v_dtype)
                assert_parity(got[b:b + 1].cpu().numpy().astype(np.float64), ref, w.v_dtype, w.C,
                              f"noalloc {name} b={b}")


def test_noalloc_refuses_partials_past_the_scratch():
    """A plan whose split partials exceed the scratch array (one long sequence,
    16 heads of D = 2048: 128 splits of 16 x 2048 floats): UNSUPPORTED, and
    nothing runs (the output keeps its contents)."""
    B, C, Hq, Hkv, D = 1, 16384, 16, 1, 2048
    plan = ga.make_plan(B, C, Hq, Hkv, D, "bf16", cu_count=torch.cuda.get_device_properties(0).multi_processor_count)
    assert plan.workspace_bytes > SCRATCH
    a = torch.zeros(B, C, Hq, device=DEV)
    v = torch.zeros(B, C, Hkv, D, dtype=torch.bfloat16, device=DEV)
    out = torch.full((B, Hq, D), 7.0, device=DEV)
    rc = _c_call("gqa_av_decode_noalloc", a, v, out, "bf16")
    torch.cuda.synchronize()
    assert rc == 3 and b"scratch" in ga.load().gqa_av_last_error()
    assert (out == 7.0).all()
