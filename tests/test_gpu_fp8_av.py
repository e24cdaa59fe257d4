"""GPU parity of the AV product and the fused softmax product over an fp8 V
cache (OCP FP8 E4M3 with a float32 scale per KV head) through the C ABI,
against the fp64 fp8 oracle.

Both sides read the same fp8 bytes and scales; the widening is exact, so only
the fp32 sums (and, for the fused form, the weights) differ: the gate of
tests/parity.py plus the accumulation bound for the plain product and the
softmax bound of tests/test_gpu_softmax_av.py for the fused one, with the
scale applied once (one more rounding, 2^-24 relative). All tests need an
MI355X and are marked ``gpu``.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import gqa_reuse_attn_amd as ga
from tests.parity import accum_bound, gate, rel_l2
from workloads import WORKLOADS, make_scores, make_scores_random

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
U32 = 2.0 ** -24


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


def _quantize(V: torch.Tensor):
    """Per-KV-head scale max|V| / 448 and the E4M3 bytes of V / scale (torch's
    round-to-nearest cast): input preparation, not part of the product."""
    Vf = V.float()
    amax = Vf.abs().amax(dim=(0, 1, 3)).clamp_min(1e-30)
    scale = (amax / 448.0).float().contiguous()
    q = (Vf / scale.view(1, 1, -1, 1)).to(torch.float8_e4m3fn).contiguous()
    return q, scale


def _check(out, ref, w, q, scale, softmax, label):
    ok, msg = gate(out, ref, "bf16")            # fp8 V: the 16-bit gate
    assert ok, f"{label}: gate failed: {msg}"
    C = w.shape[1]
    r = rel_l2(out, ref)
    if not softmax:
        assert r <= accum_bound(C) + 2 * U32, f"{label}: relL2={r:.3e} above {accum_bound(C):.3e}"
        return
    B, _, Hq = w.shape
    Hkv, D = q.shape[2], q.shape[3]
    x = w.double().numpy()
    p = np.exp(x - x.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    a = np.abs(q.float().numpy()) * scale.numpy().reshape(1, 1, -1, 1)
    A = np.einsum("bckg,bckd->bkgd", p.reshape(B, C, Hkv, Hq // Hkv), a).reshape(B, Hq, D)
    fin = w[torch.isfinite(w)]
    rng = float(fin.max() - fin.min()) if fin.numel() else 0.0
    eps = (2.0 * rng + 512.0 + 8.0 * math.sqrt(C) + 2.0) * U32
    err = np.linalg.norm((out - ref).ravel())
    assert err <= eps * np.linalg.norm(A.ravel()) + 1e-30, f"{label}: ||err||={err:.3e} above the bound"


def _run(w, q, scale, softmax, plan=None, mode="auto"):
    out = ga.gqa_av_fp8_decode(w.to(DEV), q.to(DEV), None if scale is None else scale.to(DEV), softmax=softmax,
                               plan=plan, mode=mode)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("wname", list(WORKLOADS))
def test_fp8_workloads(wname, oracle_lib):
    """The decode shapes with V quantized per KV head (large batch cut to 8
    sequences), plain (softmax weights) and fused (logits), reuse and per-head."""
    w = WORKLOADS[wname]
    if w.B > 8:
        w = w.replace(B=8)
    if w.D % 2:
        pytest.skip("fp8 V needs an even D")
    _say(f"[fp8] {w.name}")
    s, V = make_scores(w, seed=0)
    q, scale = _quantize(V)
    attn = torch.softmax(s.double(), dim=1).float().contiguous()
    for softmax, x in ((False, attn), (True, s)):
        ref = oracle_lib.fp8(x, q, scale, softmax=softmax)
        for mode in ("auto", "per_head"):
            out = _run(x, q, scale, softmax, mode=mode)
            _check(out, ref, x, q, scale, softmax, f"fp8 {w.name} softmax={softmax} {mode}")


def _cases():
    cases, k = [], 0
    for G in (1, 2, 3, 4, 5, 8, 16, 17):
        for D in (2, 46, 64, 96, 128, 256):
            for C in (1, 63, 65, 700):
                if (G + D + C) % 3:
                    continue
                Hkv = (1, 2, 4)[k % 3]
                cases.append((1 + k % 2, C, G * Hkv, Hkv, D, (1.0, 3.0)[k % 2]))
                k += 1
    return cases + [(2, 700, 64, 8, 128, 1.0)]      # eight KV heads


@pytest.mark.parametrize("B,C,Hq,Hkv,D,std", _cases())
def test_fp8_sweep(B, C, Hq, Hkv, D, std, oracle_lib):
    """G 1..17, D 2..256 (2-, 4- and 8-byte lane loads), ragged C, forced splits,
    1/2/4 KV heads per workgroup, with and without scales."""
    s, V = make_scores_random(B, C, Hq, Hkv, D, "f32", seed=B * 1000 + C + D, score_std=std)
    q, scale = _quantize(V)
    attn = torch.softmax(s.double(), dim=1).float().contiguous()
    modes = ("auto", "per_head") if Hq // Hkv >= 2 else ("auto",)
    for softmax, x in ((False, attn), (True, s)):
        for sc in (scale, None):
            ref = oracle_lib.fp8(x, q, sc, softmax=softmax)
            plans = [ga.make_plan(B, C, Hq, Hkv, D, "fp8", m, nsplit=ns, softmax=softmax)
                     for m in modes for ns in (0, 1, 7)]
            for ht in (2, 4):
                if Hq // Hkv >= 2 and Hkv % ht == 0:
                    plans.append(ga.make_plan(B, C, Hq, Hkv, D, "fp8", "reuse", kv_tile=ht, nsplit=3,
                                              softmax=softmax))
            if Hq // Hkv >= 2 and D in (64, 128, 256):        # the bf16 matrix engine at any G
                for ht in (1, 2, 8):
                    if Hkv % ht == 0:
                        plans.append(ga.make_plan(B, C, Hq, Hkv, D, "fp8", "reuse", engine="mfma_bf16", kv_tile=ht,
                                                  nsplit=2, softmax=softmax))
            for plan in plans:
                out = _run(x, q, sc, softmax, plan=plan)
                _check(out, ref, x, q, sc if sc is not None else torch.ones(Hkv), softmax,
                       f"fp8 {(B, C, Hq, Hkv, D)} scale={sc is not None} {plan.as_dict()}")


@pytest.mark.parametrize("Hq", [8, 16])
def test_fp8_every_byte_and_dense_entry_points(Hq, oracle_lib):
    """Every E4M3 byte but NaN appears in V; one-hot weights return V * scale
    exactly where the product is exact (scale a power of two); gqa_av_decode
    with fp8 V equals the fp8 entry point with unit scales bit for bit. G = 4
    runs on the VALU engine, G = 8 on the bf16 matrix engine."""
    B, C, Hkv, D = 2, 254, 2, 64
    g = torch.Generator().manual_seed(7)
    vals = torch.tensor([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=torch.uint8)
    raw = vals[torch.randint(0, vals.numel(), (B, C, Hkv, D), generator=g)]
    raw[0, :vals.numel(), 0, 0] = vals
    q = raw.view(torch.float8_e4m3fn).contiguous()
    scale = torch.tensor([0.5, 4.0])
    w = torch.zeros(B, C, Hq)
    pick = {}
    for b in range(B):
        for h in range(Hq):
            c = (13 * b + 29 * h + 5) % C
            w[b, c, h] = 1.0
            pick[b, h] = c
    out = _run(w, q, scale, False)
    dec = oracle_lib.decode_fp8(raw)
    G = Hq // Hkv
    for (b, h), c in pick.items():
        assert np.array_equal(out[b, h], dec[b, c, h // G] * float(scale[h // G])), (b, h)
    s, _ = make_scores_random(B, C, Hq, Hkv, D, "f32", seed=9)
    for softmax, x in ((False, torch.softmax(s.double(), 1).float().contiguous()), (True, s)):
        plan = ga.make_plan(B, C, Hq, Hkv, D, "fp8", softmax=softmax)
        a = _run(x, q, None, softmax, plan=plan)
        fn = ga.gqa_softmax_av_decode if softmax else ga.gqa_av_decode
        b2 = fn(x.to(DEV), q.to(DEV), plan=plan).cpu().numpy().astype(np.float64)
        assert np.array_equal(a, b2)
        _check(a, oracle_lib.fp8(x, q, None, softmax=softmax), x, q, torch.ones(Hkv), softmax, "fp8 dense entry")


@pytest.mark.parametrize("softmax", [False, True])
def test_fp8_pass1_then_combine_is_the_call(softmax):
    """gqa_av_fp8_decode_pass1 then _combine on one stream equals
    gqa_av_fp8_decode_plan bit for bit (VALU at G=2, bf16 matrix engine at G=8,
    one split and several)."""
    for Hq, ns in ((16, 0), (64, 0), (64, 1)):
        B, C, Hkv, D = 3, 3000, 8, 128
        s, V = make_scores_random(B, C, Hq, Hkv, D, "f32", seed=99 + Hq)
        q, scale = _quantize(V)
        x = s if softmax else torch.softmax(s.double(), dim=1).float().contiguous()
        plan = ga.make_plan(B, C, Hq, Hkv, D, "fp8", nsplit=ns, softmax=softmax)
        call = ga.bind_fp8(x.to(DEV), q.to(DEV), scale.to(DEV), plan=plan)
        whole = call().clone()
        call.out.fill_(float("nan"))
        call.pass1()
        got = call.combine()
        torch.cuda.synchronize()
        assert torch.equal(whole, got), (Hq, ns, softmax)
