"""GPU parity of the fused softmax and attention-times-V product through the C
ABI, against the fp64 CPU oracle (softmax over c of the scores, times V).

Gate: the acceptance gate of tests/parity.py (max-abs for fp32 V, relative L2
for bf16/fp16 V), plus a bound derived from the kernel's arithmetic. Each
weight is exp2(fl(fl(s - r) log2 e)) times rescale factors
exp2(fl(fl(r_old - r_new) log2 e)), with r a running maximum. The two
roundings of the exponent cost at most 2 |s - r| u of relative error (u =
2^-24), each exp2 a few u, and every rescale event the same again; the
rescale factors multiply a lane's weighted sum and weight sum alike, so they
only shift the balance between lanes. With R the range of the finite scores,
eps_w = (2 R + 512) u covers the exponents and exp2 calls of up to about a
hundred rescale events per lane. The fp32 sums over c add the accumulation
term of tests/parity.py. So, with A[b,q,d] = sum_c p[b,c,q] |V[b,c,kv,d]| (p
the exact softmax):

    ||out - ref||_2 <= (eps_w + 8 sqrt(C) u) ||A||_2

and elementwise on small shapes |out - ref| <= (eps_w + 2 C u) A.
A kernel that rounded the weights to bf16 (relative error ~2^-9) fails both.
All tests need an MI355X and are marked ``gpu``.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import gqa_reuse_attn_amd as ga
from tests.parity import gate
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


def _run(s, V, mode="auto", plan=None):
    out = ga.gqa_softmax_av_decode(s.to(DEV), V.to(DEV), mode=mode, plan=plan)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _abs_weighted(s: torch.Tensor, V: torch.Tensor) -> np.ndarray:
    """A[b, q, d] = sum_c p[b, c, q] |V[b, c, q // G, d]| with p the softmax over c
    (numpy, fp32 is enough for a bound)."""
    B, C, Hq = s.shape
    Hkv, D = V.shape[2], V.shape[3]
    x = s.double().numpy()
    if C:
        x = x - x.max(axis=1, keepdims=True)
    p = np.exp(x)
    p = (p / p.sum(axis=1, keepdims=True)).astype(np.float32).reshape(B, C, Hkv, Hq // Hkv)
    a = np.abs(V.float().numpy())
    return np.einsum("bckg,bckd->bkgd", p, a, optimize=True).reshape(B, Hq, D).astype(np.float64)


def _check(out, ref, s, V, dt, label, elementwise=False):
    ok, msg = gate(out, ref, dt)
    assert ok, f"{label}: gate failed: {msg}"
    C = s.shape[1]
    finite = s[torch.isfinite(s)]
    rng = float(finite.max() - finite.min()) if finite.numel() else 0.0
    A = _abs_weighted(s, V)
    eps_w = (2.0 * rng + 512.0) * U32
    err = np.linalg.norm((out - ref).ravel())
    bound = (eps_w + 8.0 * math.sqrt(max(C, 1)) * U32) * np.linalg.norm(A.ravel()) + 1e-30
    assert err <= bound, f"{label}: ||err||={err:.3e} above the arithmetic bound {bound:.3e}"
    if elementwise:
        b2 = (eps_w + 2.0 * C * U32) * A + 1e-30
        bad = np.abs(out - ref) > b2
        assert not bad.any(), f"{label}: {int(bad.sum())} elements above the elementwise bound"


@pytest.mark.parametrize("wname", list(WORKLOADS))
@pytest.mark.parametrize("mode", ["auto", "per_head"])
def test_softmax_workload_shapes(wname, mode, oracle_lib):
    """The six decode shapes with their logits as scores (the large batch cut to
    8 sequences so the oracle stays in seconds; the bench runs the full size)."""
    w = WORKLOADS[wname]
    if w.B > 8:
        w = w.replace(B=8)
    _say(f"[softmax] {w.name} B={w.B} mode={mode}")
    s, V = make_scores(w, seed=0)
    ref = oracle_lib.softmax_av(s, V, w.v_dtype)
    out = _run(s, V, mode)
    _check(out, ref, s, V, w.v_dtype, f"softmax {w.name} {mode}")


def _cases():
    cases, k = [], 0
    for G in (1, 2, 3, 4, 5, 8, 16, 17, 32):
        for D in (32, 64, 96, 128, 256):
            for C in (1, 63, 65, 300, 1000):
                if (G + D + C) % 4:
                    continue
                dt = ("bf16", "f16", "f32")[k % 3]
                Hkv = (1, 2, 4)[k % 3]
                std = (1.0, 4.0, 0.25)[k % 3]
                cases.append((1 + k % 2, C, G * Hkv, Hkv, D, dt, std))
                k += 1
    # eight KV heads (the bf16 engine's eight-head tiles)
    return cases + [(2, 700, 64, 8, 128, "bf16", 1.0), (1, 1000, 64, 8, 64, "bf16", 4.0),
                    (2, 65, 128, 8, 256, "bf16", 0.25), (1, 300, 128, 16, 128, "bf16", 1.0)]


@pytest.mark.parametrize("B,C,Hq,Hkv,D,dt,std", _cases())
def test_softmax_sweep(B, C, Hq, Hkv, D, dt, std, oracle_lib):
    """Small shapes: G 1..32, D 32..256, ragged C, all dtypes, every engine that
    takes the shape, forced splits (1, 2, 7, auto) and 1/2/4/8 KV heads per tile."""
    s, V = make_scores_random(B, C, Hq, Hkv, D, dt, seed=B * 1000 + C + D, score_std=std)
    ref = oracle_lib.softmax_av(s, V, dt)
    modes = ("auto", "per_head") if Hq // Hkv >= 2 else ("auto",)
    plans = []
    for mode in modes:
        for ns in (0, 1, 2, 7, 12):                 # 12: the grouped combine (more than 8 splits)
            plans.append(ga.make_plan(B, C, Hq, Hkv, D, dt, mode, nsplit=ns, softmax=True))
        for ns in (2, 7, 12):                       # splits cut into interleaved blocks of one step
            p = ga.make_plan(B, C, Hq, Hkv, D, dt, mode, nsplit=ns, softmax=True, split_order="interleaved")
            assert p.interleave == (p.nsplit > 1)
            plans.append(p)
    if Hq // Hkv >= 2:
        for eng in ("valu", "mfma_bf16"):
            for ht in (1, 2, 4, 8):
                if Hkv % ht:
                    continue
                try:
                    plans.append(ga.make_plan(B, C, Hq, Hkv, D, dt, "reuse", engine=eng, kv_tile=ht, nsplit=3,
                                              softmax=True))
                except ga.GqaAvError as e:
                    assert e.name == "UNSUPPORTED"
    for plan in plans:
        out = _run(s, V, plan=plan)
        _check(out, ref, s, V, dt, f"softmax {(B, C, Hq, Hkv, D, dt)} plan={plan.as_dict()}", elementwise=True)


@pytest.mark.parametrize("dt,Hq,Hkv", [("bf16", 16, 2), ("bf16", 32, 2), ("f16", 6, 2), ("f32", 8, 8)])
def test_softmax_masks(dt, Hq, Hkv, oracle_lib):
    """-inf scores: random rows masked; one head masked everywhere (NaN, as the
    definition gives); a whole split masked for one head (still finite)."""
    B, C, D = 2, 700, 64
    s, V = make_scores_random(B, C, Hq, Hkv, D, dt, seed=41, score_std=2.0)
    g = torch.Generator().manual_seed(43)
    s[torch.rand(s.shape, generator=g) < 0.3] = float("-inf")
    s[1, :, 3] = float("-inf")
    s[0, :350, 5] = float("-inf")                  # with 2+ splits, whole splits of head 5 are masked
    ref = oracle_lib.softmax_av(s, V, dt)
    assert np.isnan(ref[1, 3]).all() and np.isfinite(ref[0]).all()
    for ns in (0, 1, 2, 7, 100):                    # 100: several load batches per split group
        for mode in ("auto", "per_head"):
            plan = ga.make_plan(B, C, Hq, Hkv, D, dt, mode, nsplit=ns, softmax=True)
            out = _run(s, V, plan=plan)
            assert np.isnan(out[1, 3]).all(), f"all -inf head must give NaN ({plan.as_dict()})"
            keep = np.ones((B, Hq, 1), bool)
            keep[1, 3] = False
            assert np.isfinite(np.where(keep, out, 0.0)).all(), f"masked rows leaked a NaN ({plan.as_dict()})"
            sk = s.clone()
            sk[1, :, 3] = 0.0                          # only for the bound's weights
            _check(np.where(keep, out, 0.0), np.where(keep, ref, 0.0), sk, V, dt, f"masks {dt} {plan.as_dict()}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_softmax_large_and_shifted_scores(dt, oracle_lib):
    """Scores near 3000 (exp without the maximum overflows) and ramps that raise
    the running maximum at every step (rising) or never after the first (falling)."""
    B, C, Hq, Hkv, D = 2, 5000, 16, 2, 128
    s, V = make_scores_random(B, C, Hq, Hkv, D, dt, seed=47, score_std=1.0)
    ramp = torch.linspace(0.0, 30.0, C).view(1, C, 1)
    for label, x in (("offset", s + 3000.0), ("rising", s + ramp), ("falling", s - ramp)):
        ref = oracle_lib.softmax_av(x, V, dt)
        for eng in ("valu", "auto"):
            plan = ga.make_plan(B, C, Hq, Hkv, D, dt, "reuse", engine=eng, softmax=True)
            out = _run(x, V, plan=plan)
            _check(out, ref, x, V, dt, f"{label} {dt} {plan.as_dict()}")


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_softmax_one_hot_is_exact(dt):
    """One score per (b, q_h) 200 above the others: every other weight is
    exp2(-288) = 0 in fp32 and the winner's is exp2(0) = 1, so the output is
    that V row bit for bit (the bf16 engine splits 1.0 exactly)."""
    B, C, Hq, Hkv, D = 2, 900, 32, 2, 128
    s, V = make_scores_random(B, C, Hq, Hkv, D, dt, seed=53)
    G = Hq // Hkv
    pick = {}
    for b in range(B):
        for h in range(Hq):
            c = (37 * b + 101 * h + 11) % C
            s[b, c, h] = 200.0 + float(s[b].max())
            pick[b, h] = c
    engines = ("valu", "mfma_bf16") if dt == "bf16" else ("valu",)
    Vd = V.double().numpy()
    for eng in engines:
        for ns in (1, 4):
            plan = ga.make_plan(B, C, Hq, Hkv, D, dt, "reuse", engine=eng, nsplit=ns, softmax=True)
            out = _run(s, V, plan=plan)
            for (b, h), c in pick.items():
                assert np.array_equal(out[b, h], Vd[b, c, h // G]), (dt, eng, ns, b, h)


def test_softmax_edges():
    # C = 0: zeros; B = 0: nothing
    out = ga.gqa_softmax_av_decode(torch.zeros(2, 0, 4, device=DEV),
                                   torch.zeros(2, 0, 2, 64, dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    assert out.shape == (2, 4, 64) and (out == 0).all()
    out = ga.gqa_softmax_av_decode(torch.zeros(0, 9, 4, device=DEV),
                                   torch.zeros(0, 9, 2, 64, dtype=torch.bfloat16, device=DEV))
    assert out.shape == (0, 4, 64)
    # C = 1: the V row itself
    s, V = make_scores_random(2, 1, 8, 2, 96, "f16", seed=59)
    out = _run(s, V)
    assert np.array_equal(out, np.repeat(V.double().numpy()[:, 0], 4, axis=1))
    # forced fp32 matrix engine is refused
    with pytest.raises(ga.GqaAvError) as ei:
        ga.make_plan(1, 100, 16, 1, 128, "f16", "reuse", engine="mfma", softmax=True)
    assert ei.value.name == "UNSUPPORTED"


def test_softmax_deterministic():
    s, V = make_scores_random(4, 6000, 16, 8, 128, "bf16", seed=61, score_std=3.0)
    sd, Vd = s.to(DEV), V.to(DEV)
    a = [ga.gqa_softmax_av_decode(sd, Vd).cpu() for _ in range(3)]
    torch.cuda.synchronize()
    assert all(torch.equal(a[0], x) for x in a[1:])


def test_softmax_matches_unfused_path(oracle_lib):
    """score step -> fused softmax x V equals score step -> softmax -> AV on the
    GPU and the oracles composed the same way."""
    from workloads import make_qk_random
    B, C, Hq, Hkv, D = 2, 3000, 16, 4, 128
    q, K = make_qk_random(B, C, Hq, Hkv, D, "bf16", seed=21)
    _, V = make_qk_random(B, C, Hq, Hkv, D, "bf16", seed=22)
    scale = D ** -0.5
    sc = ga.gqa_qk_decode(q.to(DEV), K.to(DEV), scale=scale)
    fused = ga.gqa_softmax_av_decode(sc, V.to(DEV))
    attn = torch.softmax(sc.double(), dim=1).float().contiguous()
    unfused = ga.gqa_av_decode(attn, V.to(DEV))
    torch.cuda.synchronize()
    f, u = fused.cpu().numpy().astype(np.float64), unfused.cpu().numpy().astype(np.float64)
    ref = oracle_lib.softmax_av(sc.cpu(), V, "bf16")
    _check(f, ref, sc.cpu(), V, "bf16", "qk -> fused softmax x V")
    assert np.linalg.norm((f - u).ravel()) <= 1e-5 * np.linalg.norm(u.ravel())
