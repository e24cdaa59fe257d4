"""GPU parity with V, K or the page pool larger than 4 GiB, so that the byte
offsets of later sequences (and of high page numbers) do not fit in 32 bits:
the plain and fused products on both engines, the score step, paged V, fp8
V and paged fused attention. Inputs are drawn on the GPU from a seeded generator (torch's, not this
library); the oracle checks the first, a middle and the last sequence one by
one, after copying only those slices to the host. All tests need an MI355X
and are marked ``gpu``.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import gqa_reuse_attn_amd as ga
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
C, Hkv, D = 131072, 8, 128          # one sequence of bf16 V: 268 MB


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


def _gen(seed):
    return torch.Generator(device=DEV).manual_seed(seed)


def _big(shape, dtype, seed):
    return torch.randn(shape, generator=_gen(seed), device=DEV, dtype=dtype)


def _sample(B):
    return (0, B // 2, B - 1)


def _scores(B, Hq, seed):
    return _big((B, C, Hq), torch.float32, seed) * 2.0


@pytest.mark.parametrize("Hq", [16, 64])            # G = 2 (VALU), G = 8 (bf16 matrix engine)
@pytest.mark.parametrize("softmax", [False, True])
def test_dense_beyond_4gib(Hq, softmax, oracle_lib):
    from tests.test_gpu_softmax_av import _check
    B = 17                                           # V: 4.56 GB
    V = _big((B, C, Hkv, D), torch.bfloat16, 1)
    s = _scores(B, Hq, 2)
    x = s if softmax else torch.softmax(s, dim=1)
    assert V.numel() * 2 > 2 ** 32
    plan = ga.make_plan(B, C, Hq, Hkv, D, "bf16", softmax=softmax,
                        cu_count=torch.cuda.get_device_properties(0).multi_processor_count)
    _say(f"[4GiB] dense Hq={Hq} softmax={softmax} plan={plan.as_dict()}")
    fn = ga.gqa_softmax_av_decode if softmax else ga.gqa_av_decode
    out = fn(x, V, plan=plan)
    torch.cuda.synchronize()
    for b in _sample(B):
        xb, Vb = x[b:b + 1].cpu(), V[b:b + 1].cpu()
        ob = out[b:b + 1].cpu().numpy().astype(np.float64)
        if softmax:
            _check(ob, oracle_lib.softmax_av(xb, Vb, "bf16"), xb, Vb, "bf16", f"4GiB softmax Hq={Hq} b={b}")
        else:
            assert_parity(ob, oracle_lib.full(xb, Vb, "bf16"), "bf16", C, f"4GiB av Hq={Hq} b={b}")
    del V, s, x, out


def test_qk_beyond_4gib(oracle_lib):
    B, Hq = 17, 16
    K = _big((B, C, Hkv, D), torch.bfloat16, 3)
    q = _big((B, Hq, D), torch.float32, 4)
    scale = D ** -0.5
    _say("[4GiB] qk")
    out = ga.gqa_qk_decode(q, K, scale=scale)
    torch.cuda.synchronize()
    for b in _sample(B):
        ref = oracle_lib.qk(q[b:b + 1].cpu(), K[b:b + 1].cpu(), "bf16", scale)
        assert_parity(out[b:b + 1].cpu().numpy().astype(np.float64), ref, "bf16", D, f"4GiB qk b={b}")
    del K, q, out


@pytest.mark.parametrize("Hq", [16, 64])
def test_paged_beyond_4gib(Hq, oracle_lib):
    """A pool of 16-row pages larger than 4 GiB, each sequence's pages spread
    over the whole pool in a shuffled order, lengths full / partial."""
    from tests.test_gpu_paged_av import _bound_ok
    B, P = 17, 16
    maxp = C // P
    pages = _big((B * maxp, P, Hkv, D), torch.bfloat16, 5)
    perm = torch.randperm(B * maxp, generator=torch.Generator().manual_seed(6)).to(torch.int32)
    bt = perm.view(B, maxp).contiguous()
    lens = torch.full((B,), C, dtype=torch.int32)
    lens[B // 2] = C // 2 + 7
    s = _scores(B, Hq, 7)
    _say(f"[4GiB] paged Hq={Hq}")
    for softmax in (False, True):
        x = s if softmax else torch.softmax(s, dim=1)
        out = ga.gqa_av_paged_decode(x, pages, bt.to(DEV), lens.to(DEV), softmax=softmax)
        torch.cuda.synchronize()
        for b in _sample(B):
            idx = bt[b].long()
            pb = pages[idx.to(DEV)].cpu()                      # this sequence's pages, in its order
            Vb = pb.reshape(1, maxp * P, Hkv, D)
            xb = x[b:b + 1].cpu()
            btb = torch.arange(maxp, dtype=torch.int32).view(1, maxp)
            ref = oracle_lib.paged(xb, pb, btb, lens[b:b + 1], "bf16", softmax=softmax)
            _bound_ok(out[b:b + 1].cpu().numpy().astype(np.float64), ref, xb, Vb, lens[b:b + 1], "bf16", softmax,
                      f"4GiB paged Hq={Hq} b={b} softmax={softmax}")
    del pages, s, out


def test_fp8_beyond_4gib(oracle_lib):
    from tests.test_gpu_fp8_av import _check
    B, Hq = 33, 64                                   # fp8 V: 4.43 GB
    V8 = (_big((B, C, Hkv, D), torch.bfloat16, 8) * 32.0).to(torch.float8_e4m3fn)   # |x| < 448: 14 sigma
    assert V8.numel() > 2 ** 32
    scale = torch.full((Hkv,), 0.125, device=DEV)
    s = _scores(B, Hq, 9)
    _say("[4GiB] fp8")
    for softmax in (False, True):
        x = s if softmax else torch.softmax(s, dim=1)
        out = ga.gqa_av_fp8_decode(x, V8, scale, softmax=softmax)
        torch.cuda.synchronize()
        for b in _sample(B):
            xb, qb = x[b:b + 1].cpu(), V8[b:b + 1].cpu()
            ref = oracle_lib.fp8(xb, qb, scale.cpu(), softmax=softmax)
            _check(out[b:b + 1].cpu().numpy().astype(np.float64), ref, xb, qb, scale.cpu(), softmax,
                   f"4GiB fp8 b={b} softmax={softmax}")
    del V8, s, out


@pytest.mark.parametrize("fp8,P", [(False, 16), (True, 16), (True, 2)])
def test_attention_paged_beyond_4gib(fp8, P, oracle_lib):
    """Paged fused attention over K and V pools each larger than 4 GiB (pages
    shuffled over the whole pool, full and partial lengths), bf16 or fp8 with
    per-KV-head scales. fp8 runs with 16-row pages, where a 64-lane load's
    four rows lie in one page (one page resource per load), and with 2-row
    pages, where they do not and every lane computes its own 64-bit page
    address. Wrong page addressing gives gross errors, so the sampled
    sequences, each holding pages above the 4 GiB mark, are checked with the
    parity gate against the paged attention oracle (the full error bound would
    need 2 GB host arrays here)."""
    from tests.parity import gate
    B, Hq = (33 if fp8 else 17), 16
    maxp = C // P
    shape = (B * maxp, P, Hkv, D)
    ks = vs = None
    if fp8:
        kp = (_big(shape, torch.bfloat16, 11) * 32.0).to(torch.float8_e4m3fn)   # |x| < 448: 14 sigma
        vp = (_big(shape, torch.bfloat16, 12) * 32.0).to(torch.float8_e4m3fn)
        ks = torch.full((Hkv,), 1.0 / 32.0, device=DEV)
        vs = torch.full((Hkv,), 0.125, device=DEV)
    else:
        kp = _big(shape, torch.bfloat16, 11)
        vp = _big(shape, torch.bfloat16, 12)
    assert kp.numel() * kp.element_size() > 2 ** 32 and vp.numel() * vp.element_size() > 2 ** 32
    perm = torch.randperm(B * maxp, generator=torch.Generator().manual_seed(13)).to(torch.int32)
    bt = perm.view(B, maxp).contiguous()
    lens = torch.full((B,), C, dtype=torch.int32)
    lens[B // 2] = C // 2 + 7
    q = _big((B, Hq, D), torch.float32, 14)
    scale = D ** -0.5
    page_bytes = P * Hkv * D * kp.element_size()
    for b in _sample(B):
        assert ((bt[b].long() + 1) * page_bytes > 2 ** 32).any(), "a sampled sequence has pages past 4 GiB"
    _say(f"[4GiB] attention paged fp8={fp8} P={P}")
    out = ga.gqa_attention_paged_decode(q, kp, vp, bt.to(DEV), lens.to(DEV), scale=scale, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    for b in _sample(B):
        idx = bt[b].long().to(DEV)
        kb, vb = kp[idx].cpu(), vp[idx].cpu()                 # this sequence's pages, in its order
        btb = torch.arange(maxp, dtype=torch.int32).view(1, maxp)
        ref = oracle_lib.attention_paged(q[b:b + 1].cpu(), kb, vb, btb, lens[b:b + 1], "fp8" if fp8 else "bf16",
                                         scale, None if ks is None else ks.cpu(), None if vs is None else vs.cpu(),
                                         C=C)
        ok, msg = gate(out[b:b + 1].cpu().numpy().astype(np.float64), ref, "bf16")
        assert ok, f"4GiB attention paged fp8={fp8} P={P} b={b}: {msg}"
    del kp, vp, out
