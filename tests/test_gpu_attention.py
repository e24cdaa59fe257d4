"""GPU parity of fused decode attention (scores, softmax and product in one
pass over K and V: bf16, fp8 with per-KV-head scales, dense or paged) through
the C ABI, against the fp64 attention oracles.

Bound: the scores carry the score step's fp32 error, |ds_c| <= 2 D 2^-24
scale sum_d |q K| (every product exact, fp32 sums); a softmax weight moves by
at most a factor exp(2 max |ds|); on top comes the fused softmax product's
own arithmetic bound (tests/test_gpu_softmax_av.py). So
||err|| <= ((2 rng + 512) 2^-24 + 2 max|ds| + 8 sqrt(C) 2^-24) ||A|| with
A = sum_c p_c |V_c| and rng the range of the exact scores; plus the gate of
tests/parity.py. All tests need an MI355X and are marked ``gpu``.
"""
from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import gqa_reuse_attn_amd as ga
from tests.parity import gate
from workloads import WORKLOADS, make_qk_random

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


def _inputs(B, C, Hq, Hkv, D, seed, qscale=1.0):
    q, K = make_qk_random(B, C, Hq, Hkv, D, "bf16", seed=seed)
    _, V = make_qk_random(B, C, Hq, Hkv, D, "bf16", seed=seed + 1)
    return (q * qscale).contiguous(), K, V


def _check(out, ref, q, K, V, scale, label):
    ok, msg = gate(out, ref, "bf16")
    assert ok, f"{label}: gate failed: {msg}"
    B, Hq, D = q.shape
    C, Hkv = K.shape[1], K.shape[2]
    if C == 0:
        assert (out == 0).all()
        return
    G = Hq // Hkv
    qd, kd, vd = q.double().numpy(), K.double().numpy(), V.double().numpy()
    kq = np.repeat(kd, G, axis=2)                          # [B, C, Hq, D]
    s = scale * np.einsum("bhd,bchd->bch", qd, kq)
    ds = 2 * D * U32 * abs(scale) * np.einsum("bhd,bchd->bch", np.abs(qd), np.abs(kq))
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    A = np.einsum("bch,bchd->bhd", p, np.abs(np.repeat(vd, G, axis=2)))
    rng = float(s.max() - s.min())
    eps = (2.0 * rng + 512.0) * U32 + 2.0 * float(ds.max()) + 8.0 * math.sqrt(C) * U32
    err = np.linalg.norm((out - ref).ravel())
    assert err <= eps * np.linalg.norm(A.ravel()) + 1e-30, f"{label}: ||err||={err:.3e} above {eps:.3e} ||A||"


def _run(q, K, V, scale, plan=None):
    out = ga.gqa_attention_decode(q.to(DEV), K.to(DEV), V.to(DEV), scale=scale, plan=plan)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("wname", [n for n, w in WORKLOADS.items() if w.D in (64, 128, 256) and w.v_dtype == "bf16"])
def test_attention_workloads(wname, oracle_lib):
    """The bf16 workload shapes (the large batch cut to 8 sequences; the full
    size is in test_gpu_full_size), scale 1/sqrt(D)."""
    w = WORKLOADS[wname]
    if w.B > 8:
        w = w.replace(B=8)
    _say(f"[attention] {w.name}")
    q, K, V = _inputs(w.B, w.C, w.Hq, w.Hkv, w.D, seed=11)
    scale = w.D ** -0.5
    _check(_run(q, K, V, scale), oracle_lib.attention(q, K, V, "bf16", scale), q, K, V, scale, f"attention {w.name}")


def _cases():
    cases, k = [], 0
    for G in (2, 3, 4, 5, 8, 16, 17, 32):
        for D in (64, 128, 256):
            for C in (1, 63, 65, 700):
                if (G + D // 64 + C) % 3 or (G > 16 and D > 128):
                    continue
                Hkv = (1, 2, 4)[k % 3]
                cases.append((1 + k % 2, C, G * Hkv, Hkv, D, (0.125, 1.0, 4.0)[k % 3]))
                k += 1
    return cases


@pytest.mark.parametrize("B,C,Hq,Hkv,D,qscale", _cases())
def test_attention_sweep(B, C, Hq, Hkv, D, qscale, oracle_lib):
    """G 2..32, D 64..256, ragged C, forced splits, 1/2/4 KV heads per
    workgroup, flat to peaky score distributions."""
    q, K, V = _inputs(B, C, Hq, Hkv, D, seed=B * 1000 + C + D, qscale=qscale)
    scale = D ** -0.5
    ref = oracle_lib.attention(q, K, V, "bf16", scale)
    plans = [ga.make_plan(B, C, Hq, Hkv, D, "bf16", nsplit=ns, attention=True) for ns in (0, 1, 5)]
    plans += [ga.make_plan(B, C, Hq, Hkv, D, "bf16", kv_tile=ht, nsplit=3, attention=True)
              for ht in (2, 4) if Hkv % ht == 0]
    for plan in plans:
        _check(_run(q, K, V, scale, plan=plan), ref, q, K, V, scale, f"attention {(B, C, Hq, Hkv, D)} {plan.as_dict()}")


def test_attention_pass1_then_combine_is_the_call():
    B, C, Hq, Hkv, D = 3, 3000, 64, 8, 128
    q, K, V = _inputs(B, C, Hq, Hkv, D, seed=21)
    for ns in (0, 1):
        plan = ga.make_plan(B, C, Hq, Hkv, D, "bf16", nsplit=ns, attention=True)
        call = ga.BoundAttention(q.to(DEV), K.to(DEV), V.to(DEV), scale=0.1, plan=plan)
        whole = call().clone()
        call.out.fill_(float("nan"))
        call.pass1()
        got = call.combine()
        torch.cuda.synchronize()
        assert torch.equal(whole, got), ns


def test_attention_matches_unfused_composition(oracle_lib):
    """Fused attention against the score step followed by the fused softmax
    product: both within the oracle's bound, and close to each other."""
    B, C, Hq, Hkv, D = 2, 2000, 32, 4, 128
    q, K, V = _inputs(B, C, Hq, Hkv, D, seed=31)
    scale = D ** -0.5
    fused = _run(q, K, V, scale)
    s = ga.gqa_qk_decode(q.to(DEV), K.to(DEV), scale=scale)
    two = ga.gqa_softmax_av_decode(s, V.to(DEV)).cpu().numpy().astype(np.float64)
    ref = oracle_lib.attention(q, K, V, "bf16", scale)
    _check(fused, ref, q, K, V, scale, "fused")
    _check(two, ref, q, K, V, scale, "score step + fused softmax")


def test_attention_edges():
    q, K, V = _inputs(2, 0, 16, 2, 128, seed=41)
    out = torch.full((2, 16, 128), float("nan"), device=DEV)
    ga.gqa_attention_decode(q.to(DEV), K.to(DEV), V.to(DEV), out=out, scale=1.0)
    torch.cuda.synchronize()
    assert (out == 0).all(), "C = 0 writes zeros"
    qq, KK, VV = _inputs(1, 10, 4, 4, 64, seed=42)
    with pytest.raises(ga.GqaAvError) as e:                # G = 1: no group to reuse over
        ga.gqa_attention_decode(qq.to(DEV), KK.to(DEV), VV.to(DEV))
    assert e.value.name == "UNSUPPORTED"
    with pytest.raises(ga.GqaAvError) as e:
        ga.gqa_attention_decode(qq.to(DEV), KK.to(DEV), VV.to(DEV), mode="reuse")
    assert e.value.name == "INELIGIBLE"


# ---- fp8 K and V (OCP FP8 E4M3 with a float32 scale per KV head) ---------------

def _quantize(X: torch.Tensor):
    """Per-KV-head scale max|X| / 448 and the E4M3 bytes of X / scale (torch's
    round-to-nearest cast): input preparation."""
    Xf = X.float()
    sc = (Xf.abs().amax(dim=(0, 1, 3)).clamp_min(1e-30) / 448.0).contiguous()
    return (Xf / sc.view(1, 1, -1, 1)).to(torch.float8_e4m3fn).contiguous(), sc


def _run_fp8(q, K8, ks, V8, vs, scale, plan=None):
    out = ga.gqa_attention_decode(q.to(DEV), K8.to(DEV), V8.to(DEV), scale=scale, plan=plan,
                                  k_scale=None if ks is None else ks.to(DEV), v_scale=None if vs is None else vs.to(DEV))
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _fp8_cases():
    cases, k = [], 0
    for G in (2, 4, 5, 8, 16, 17):
        for D in (64, 128, 256):
            for C in (1, 65, 700):
                if (G + D // 64 + C) % 3 or (G > 16 and D > 128):
                    continue
                Hkv = (1, 2, 4)[k % 3]
                cases.append((1 + k % 2, C, G * Hkv, Hkv, D))
                k += 1
    return cases


@pytest.mark.parametrize("B,C,Hq,Hkv,D", _fp8_cases())
def test_attention_fp8_sweep(B, C, Hq, Hkv, D, oracle_lib):
    """fp8 K and V quantized per KV head: G 2..17, D 64..256, ragged C,
    forced splits, 1/2 KV heads per workgroup, with and without scales,
    against the fp8 attention oracle (same bound, on the decoded values)."""
    q, K, V = _inputs(B, C, Hq, Hkv, D, seed=B * 100 + C + D)
    K8, ks = _quantize(K)
    V8, vs = _quantize(V)
    scale = D ** -0.5
    plans = [ga.make_plan(B, C, Hq, Hkv, D, "fp8", nsplit=ns, attention=True) for ns in (0, 1, 4)]
    plans += [ga.make_plan(B, C, Hq, Hkv, D, "fp8", kv_tile=2, nsplit=3, attention=True)] if Hkv % 2 == 0 else []
    for k_s, v_s in ((ks, vs), (None, None)):
        ref = oracle_lib.attention_fp8(q, K8, V8, k_s, v_s, scale)
        kd = K8.float() * (k_s.view(1, 1, -1, 1) if k_s is not None else 1.0)
        vd = V8.float() * (v_s.view(1, 1, -1, 1) if v_s is not None else 1.0)
        for plan in plans:
            out = _run_fp8(q, K8, k_s, V8, v_s, scale, plan=plan)
            _check(out, ref, q, kd, vd, scale, f"attention fp8 {(B, C, Hq, Hkv, D)} scales={k_s is not None} "
                                               f"{plan.as_dict()}")


def test_attention_fp8_equals_bf16_on_widened_values():
    """With unit scales, fp8 K and V give the bf16 call's output on the same
    values bit for bit (exact widening, same products and sums)."""
    B, C, Hq, Hkv, D = 2, 900, 32, 4, 128
    q, K, V = _inputs(B, C, Hq, Hkv, D, seed=51)
    K8, _ = _quantize(K)
    V8, _ = _quantize(V)
    for ns in (0, 1):
        p8 = ga.make_plan(B, C, Hq, Hkv, D, "fp8", nsplit=ns, kv_tile=1, attention=True)
        p16 = ga.make_plan(B, C, Hq, Hkv, D, "bf16", nsplit=ns, kv_tile=1, attention=True)
        assert p8.rows_per_split == p16.rows_per_split
        a = _run_fp8(q, K8, None, V8, None, 0.1, plan=p8)
        b = _run(q, K8.to(torch.bfloat16), V8.to(torch.bfloat16), 0.1, plan=p16)
        assert np.array_equal(a, b), ns


# ---- paged K and V (two page pools sharing one block table) ---------------------

def _page(K, V, P, seed, spare=3, lens=None):
    """K and V [B,C,Hkv,D] cut into pages of P rows, both pools in one shuffled
    order with spare pages (filled with NaN: never read), and the block table.
    With lens, every row of sequence b at or past lens[b] (the padding past C
    included) holds NaN in both pools as well."""
    B, C, Hkv, D = K.shape
    maxp = -(-C // P)
    npg = B * maxp + spare
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(npg, generator=g)[:B * maxp]
    pools = []
    for X in (K, V):
        pool = torch.empty((npg, P, Hkv, D), dtype=X.dtype)
        raw = pool.view(torch.uint8) if X.element_size() == 1 else pool.view(torch.int16)
        raw.fill_(0x7F if X.element_size() == 1 else 0x7FC0)            # NaN in E4M3 / bf16
        pad = torch.zeros((B, maxp * P, Hkv, D), dtype=X.dtype)
        pad[:, :C] = X
        if lens is not None:
            padraw = pad.view(torch.uint8) if X.element_size() == 1 else pad.view(torch.int16)
            for b in range(B):
                padraw[b, int(lens[b]):] = 0x7F if X.element_size() == 1 else 0x7FC0
        pool[perm] = pad.reshape(B * maxp, P, Hkv, D)
        pools.append(pool)
    return pools[0], pools[1], perm.to(torch.int32).view(B, maxp).contiguous()


def _paged_cases():
    cases, k = [], 0
    for dt in ("bf16", "fp8"):
        for G, D, C, P in ((2, 128, 700, 16), (4, 64, 1000, 1), (8, 128, 2100, 64), (16, 256, 333, 8),
                           (5, 128, 257, 256), (17, 64, 1500, 32)):
            cases.append((dt, 1 + k % 3, C, G * (1, 2, 4)[k % 3], (1, 2, 4)[k % 3], D, P))
            k += 1
    return cases


@pytest.mark.parametrize("dt,B,C,Hq,Hkv,D,P", _paged_cases())
def test_attention_paged_sweep(dt, B, C, Hq, Hkv, D, P, oracle_lib):
    """Paged K and V, bf16 and fp8 (per-KV-head scales): G 2..17, D 64..256,
    pages of 1..256 rows, shuffled pools with NaN spare pages and NaN in every
    row at or past a sequence's length, lengths from 0 to the capacity, forced
    splits; against the paged attention oracle with the dense bound on each
    sequence's first len rows."""
    q, K, V = _inputs(B, C, Hq, Hkv, D, seed=B * 7 + C + P)
    ks = vs = None
    if dt == "fp8":
        K, ks = _quantize(K)
        V, vs = _quantize(V)
    g = torch.Generator().manual_seed(C)
    lens = torch.randint(0, C + 1, (B,), generator=g, dtype=torch.int32)
    lens[0] = C
    if B > 2:
        lens[2] = 0
    kp, vp, bt = _page(K, V, P, seed=C + P, lens=lens)
    scale = D ** -0.5
    ref = oracle_lib.attention_paged(q, kp, vp, bt, lens, dt, scale, ks, vs, C=C)
    plans = [ga.make_plan(B, C, Hq, Hkv, D, dt, nsplit=ns, attention=True, page_size=P) for ns in (0, 1, 3)]
    if Hkv % 2 == 0:
        plans.append(ga.make_plan(B, C, Hq, Hkv, D, dt, nsplit=2, kv_tile=2, attention=True, page_size=P))
    kd = K.float() * (ks.view(1, 1, -1, 1) if ks is not None else 1.0)
    vd = V.float() * (vs.view(1, 1, -1, 1) if vs is not None else 1.0)
    for plan in plans:
        out = ga.gqa_attention_paged_decode(q.to(DEV), kp.to(DEV), vp.to(DEV), bt.to(DEV), lens.to(DEV), scale=scale,
                                            C=C, plan=plan, k_scale=None if ks is None else ks.to(DEV),
                                            v_scale=None if vs is None else vs.to(DEV))
        out = out.cpu().numpy().astype(np.float64)
        for b in range(B):
            n = int(lens[b])
            label = f"paged attention {dt} {(B, C, Hq, Hkv, D)} P={P} b={b} len={n} {plan.as_dict()}"
            if n == 0:
                assert (out[b] == 0).all(), label
                continue
            _check(out[b:b + 1], ref[b:b + 1], q[b:b + 1], kd[b:b + 1, :n], vd[b:b + 1, :n], scale, label)


def test_attention_paged_in_order_equals_dense():
    """Pages in order at full length give the dense call's output bit for bit
    (same splits, same arithmetic)."""
    B, C, Hq, Hkv, D, P = 2, 1024, 32, 4, 128, 16
    q, K, V = _inputs(B, C, Hq, Hkv, D, seed=61)
    kp, vp = K.reshape(-1, P, Hkv, D).contiguous(), V.reshape(-1, P, Hkv, D).contiguous()
    bt = torch.arange(B * C // P, dtype=torch.int32).view(B, C // P).contiguous()
    lens = torch.full((B,), C, dtype=torch.int32)
    for ns, ht in ((1, 1), (4, 2)):
        pd = ga.make_plan(B, C, Hq, Hkv, D, "bf16", nsplit=ns, kv_tile=ht, attention=True)
        pp = ga.make_plan(B, C, Hq, Hkv, D, "bf16", nsplit=ns, kv_tile=ht, attention=True, page_size=P)
        assert pd.rows_per_split == pp.rows_per_split
        a = _run(q, K, V, 0.1, plan=pd)
        b = ga.gqa_attention_paged_decode(q.to(DEV), kp.to(DEV), vp.to(DEV), bt.to(DEV), lens.to(DEV), scale=0.1,
                                          plan=pp).cpu().numpy().astype(np.float64)
        assert np.array_equal(a, b), (ns, ht)


def test_attention_paged_pass1_then_combine_is_the_call():
    B, C, Hq, Hkv, D, P = 3, 3000, 64, 8, 128, 16
    q, K, V = _inputs(B, C, Hq, Hkv, D, seed=71)
    kp, vp, bt = _page(K, V, P, seed=72)
    lens = torch.tensor([3000, 17, 2048], dtype=torch.int32)
    call = ga.BoundAttentionPaged(q.to(DEV), kp.to(DEV), vp.to(DEV), bt.to(DEV), lens.to(DEV), scale=0.1, C=C)
    whole = call().clone()
    call.out.fill_(float("nan"))
    call.pass1()
    got = call.combine()
    torch.cuda.synchronize()
    assert torch.equal(whole, got)
