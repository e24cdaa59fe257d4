"""GPU parity at the full large-batch size (B = 64, C = 8192, Hq = 64, Hkv = 8,
D = 128, bf16) in the launch configurations the bench times, for the products
whose other tests cut that workload to 8 sequences: the fused softmax product,
the score step (bf16 and fp8 K), paged V (16-row pages, shuffled, full
lengths), fp8 V (per-KV-head scales) and fused decode attention (bf16, fp8 K and V, and both paged). The GPU computes all 64 sequences with the plan the
bench uses; sequences are independent, so the oracle checks a sample of them
one by one, with the same gates as the per-product tests. All tests need an
MI355X and are marked ``gpu``.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import gqa_reuse_attn_amd as ga
from tests.parity import assert_parity
from workloads import WORKLOADS, make_qk_random, make_scores

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
W = WORKLOADS["batch64-b64-c8192-hq64-hkv8-d128-bf16"]
SAMPLE = (0, 21, 42, 63)


def _say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ga.load()
    yield
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def inputs():
    """The workload's logits (scores) and V, and the softmax weights, on the host."""
    _say(f"[full] drawing {W.name}")
    s, V = make_scores(W, seed=0)
    attn = torch.softmax(s.double(), dim=1).float().contiguous()
    return s, V, attn


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


@pytest.mark.parametrize("softmax", [False, True])
def test_full_size_paged(inputs, softmax, oracle_lib):
    from tests.test_gpu_paged_av import _bound_ok
    s, V, attn = inputs
    x = s if softmax else attn
    P = 16
    maxp = W.C // P
    perm = torch.randperm(W.B * maxp, generator=torch.Generator().manual_seed(0))
    pages = torch.empty((W.B * maxp, P, W.Hkv, W.D), dtype=V.dtype)
    pages[perm] = V.reshape(W.B * maxp, P, W.Hkv, W.D)
    bt = perm.to(torch.int32).view(W.B, maxp).contiguous()
    lens = torch.full((W.B,), W.C, dtype=torch.int32)
    plan = ga.make_plan(W.B, W.C, W.Hq, W.Hkv, W.D, W.v_dtype, cu_count=_cus(), softmax=softmax, page_size=P)
    _say(f"[full] paged softmax={softmax} plan={plan.as_dict()}")
    out = ga.gqa_av_paged_decode(x.to(DEV), pages.to(DEV), bt.to(DEV), lens.to(DEV), softmax=softmax, plan=plan)
    out = out.cpu().numpy().astype(np.float64)
    for b in SAMPLE:
        ref = oracle_lib.paged(x[b:b + 1], pages, bt[b:b + 1], lens[b:b + 1], W.v_dtype, softmax=softmax)
        _bound_ok(out[b:b + 1], ref, x[b:b + 1], V[b:b + 1], lens[b:b + 1], W.v_dtype, softmax,
                  f"full-size paged b={b} softmax={softmax}")


def test_full_size_softmax(inputs, oracle_lib):
    from tests.test_gpu_softmax_av import _check
    s, V, _ = inputs
    plan = ga.make_plan(W.B, W.C, W.Hq, W.Hkv, W.D, W.v_dtype, cu_count=_cus(), softmax=True)
    _say(f"[full] softmax plan={plan.as_dict()}")
    out = ga.gqa_softmax_av_decode(s.to(DEV), V.to(DEV), plan=plan).cpu().numpy().astype(np.float64)
    for b in SAMPLE:
        ref = oracle_lib.softmax_av(s[b:b + 1], V[b:b + 1], W.v_dtype)
        _check(out[b:b + 1], ref, s[b:b + 1], V[b:b + 1], W.v_dtype, f"full-size softmax b={b}")


@pytest.mark.parametrize("softmax", [False, True])
def test_full_size_fp8(inputs, softmax, oracle_lib):
    from tests.test_gpu_fp8_av import _check, _quantize
    s, V, attn = inputs
    x = s if softmax else attn
    q, scale = _quantize(V)
    plan = ga.make_plan(W.B, W.C, W.Hq, W.Hkv, W.D, "fp8", cu_count=_cus(), softmax=softmax)
    _say(f"[full] fp8 softmax={softmax} plan={plan.as_dict()}")
    out = ga.gqa_av_fp8_decode(x.to(DEV), q.to(DEV), scale.to(DEV), softmax=softmax, plan=plan)
    out = out.cpu().numpy().astype(np.float64)
    for b in SAMPLE:
        ref = oracle_lib.fp8(x[b:b + 1], q[b:b + 1], scale, softmax=softmax)
        _check(out[b:b + 1], ref, x[b:b + 1], q[b:b + 1], scale, softmax, f"full-size fp8 b={b} softmax={softmax}")


def test_full_size_qk(oracle_lib):
    q, K = make_qk_random(W.B, W.C, W.Hq, W.Hkv, W.D, W.v_dtype, seed=0)
    scale = W.D ** -0.5
    plan = ga.qk_make_plan(W.B, W.C, W.Hq, W.Hkv, W.D, W.v_dtype, cu_count=_cus())
    _say(f"[full] qk plan={plan.as_dict()}")
    out = ga.gqa_qk_decode(q.to(DEV), K.to(DEV), scale=scale, plan=plan).cpu().numpy().astype(np.float64)
    for b in SAMPLE:
        ref = oracle_lib.qk(q[b:b + 1], K[b:b + 1], W.v_dtype, scale)
        assert_parity(out[b:b + 1], ref, W.v_dtype, W.D, f"full-size qk b={b}")


def test_full_size_qk_fp8(oracle_lib):
    from tests.test_gpu_qk import _quantize_k
    q, K = make_qk_random(W.B, W.C, W.Hq, W.Hkv, W.D, W.v_dtype, seed=0)
    K8, ks = _quantize_k(K)
    scale = W.D ** -0.5
    plan = ga.qk_make_plan(W.B, W.C, W.Hq, W.Hkv, W.D, "fp8", cu_count=_cus())
    _say(f"[full] qk fp8 plan={plan.as_dict()}")
    out = ga.gqa_qk_decode(q.to(DEV), K8.to(DEV), scale=scale, plan=plan, k_scale=ks.to(DEV))
    out = out.cpu().numpy().astype(np.float64)
    for b in SAMPLE:
        ref = oracle_lib.qk_fp8(q[b:b + 1], K8[b:b + 1], ks, scale)
        assert_parity(out[b:b + 1], ref, "bf16", W.D, f"full-size qk fp8 b={b}")


def test_full_size_attention(oracle_lib):
    from tests.test_gpu_attention import _check
    q, K = make_qk_random(W.B, W.C, W.Hq, W.Hkv, W.D, "bf16", seed=0)
    _, V = make_qk_random(W.B, W.C, W.Hq, W.Hkv, W.D, "bf16", seed=1)
    scale = W.D ** -0.5
    plan = ga.make_plan(W.B, W.C, W.Hq, W.Hkv, W.D, "bf16", cu_count=_cus(), attention=True)
    _say(f"[full] attention plan={plan.as_dict()}")
    out = ga.gqa_attention_decode(q.to(DEV), K.to(DEV), V.to(DEV), scale=scale, plan=plan)
    out = out.cpu().numpy().astype(np.float64)
    for b in SAMPLE:
        ref = oracle_lib.attention(q[b:b + 1], K[b:b + 1], V[b:b + 1], "bf16", scale)
        _check(out[b:b + 1], ref, q[b:b + 1], K[b:b + 1], V[b:b + 1], scale, f"full-size attention b={b}")


def test_full_size_attention_fp8(oracle_lib):
    from tests.test_gpu_attention import _check, _quantize
    q, K = make_qk_random(W.B, W.C, W.Hq, W.Hkv, W.D, "bf16", seed=0)
    _, V = make_qk_random(W.B, W.C, W.Hq, W.Hkv, W.D, "bf16", seed=1)
    K8, ks = _quantize(K)
    V8, vs = _quantize(V)
    scale = W.D ** -0.5
    plan = ga.make_plan(W.B, W.C, W.Hq, W.Hkv, W.D, "fp8", cu_count=_cus(), attention=True)
    _say(f"[full] attention fp8 plan={plan.as_dict()}")
    out = ga.gqa_attention_decode(q.to(DEV), K8.to(DEV), V8.to(DEV), scale=scale, plan=plan,
                                  k_scale=ks.to(DEV), v_scale=vs.to(DEV))
    out = out.cpu().numpy().astype(np.float64)
    kd = K8.float() * ks.view(1, 1, -1, 1)
    vd = V8.float() * vs.view(1, 1, -1, 1)
    for b in SAMPLE:
        ref = oracle_lib.attention_fp8(q[b:b + 1], K8[b:b + 1], V8[b:b + 1], ks, vs, scale)
        _check(out[b:b + 1], ref, q[b:b + 1], kd[b:b + 1], vd[b:b + 1], scale, f"full-size attention fp8 b={b}")


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_full_size_attention_paged(dt, oracle_lib):
    """Paged K and V in 16-row pages (shuffled, full lengths), as the bench runs it."""
    from tests.test_gpu_attention import _check, _page, _quantize
    q, K = make_qk_random(W.B, W.C, W.Hq, W.Hkv, W.D, "bf16", seed=0)
    _, V = make_qk_random(W.B, W.C, W.Hq, W.Hkv, W.D, "bf16", seed=1)
    ks = vs = None
    if dt == "fp8":
        K, ks = _quantize(K)
        V, vs = _quantize(V)
    kp, vp, bt = _page(K, V, 16, seed=0, spare=0)
    lens = torch.full((W.B,), W.C, dtype=torch.int32)
    scale = W.D ** -0.5
    plan = ga.make_plan(W.B, W.C, W.Hq, W.Hkv, W.D, dt, cu_count=_cus(), attention=True, page_size=16)
    _say(f"[full] attention paged {dt} plan={plan.as_dict()}")
    out = ga.gqa_attention_paged_decode(q.to(DEV), kp.to(DEV), vp.to(DEV), bt.to(DEV), lens.to(DEV), scale=scale,
                                        plan=plan, k_scale=None if ks is None else ks.to(DEV),
                                        v_scale=None if vs is None else vs.to(DEV))
    out = out.cpu().numpy().astype(np.float64)
    kd = K.float() * (ks.view(1, 1, -1, 1) if ks is not None else 1.0)
    vd = V.float() * (vs.view(1, 1, -1, 1) if vs is not None else 1.0)
    for b in SAMPLE:
        ref = oracle_lib.attention_paged(q[b:b + 1], kp, vp, bt[b:b + 1], lens[b:b + 1], dt, scale, ks, vs, C=W.C)
        _check(out[b:b + 1], ref, q[b:b + 1], kd[b:b + 1], vd[b:b + 1], scale, f"full-size attention paged {dt} b={b}")
