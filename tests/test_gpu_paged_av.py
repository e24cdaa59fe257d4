"""GPU parity of the AV product and the fused softmax product over a paged V
cache (block table, per-sequence lengths) through the C ABI, against the fp64
paged oracle.

Gate: the acceptance gate of tests/parity.py plus the same arithmetic bounds
as the dense paths: fp32 accumulation (relative L2 <= 8 sqrt(len) 2^-24) for
the plain product, and for the fused one the bound derived in
tests/test_gpu_softmax_av.py, with A computed over each sequence's own rows.
All tests need an MI355X and are marked ``gpu``.
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
TD = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


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


def _paged_from_dense(V: torch.Tensor, P: int, seed: int, spare: int = 5):
    """Scatter a dense V [B, C, Hkv, D] into a shuffled pool of P-row pages with
    spare pages (filled with large values that must never be read: 3e4, or
    the E4M3 byte of 448 for uint8 V) and return (pages, block_table). Rows
    past C in a sequence's last page are padding."""
    B, C, Hkv, D = V.shape
    maxp = -(-C // P)
    g = torch.Generator().manual_seed(seed)
    npg = B * maxp + spare
    if V.dtype == torch.uint8:
        pages = torch.full((npg, P, Hkv, D), 0x7E, dtype=torch.uint8)
    else:
        pages = torch.full((npg, P, Hkv, D), 3.0e4).to(V.dtype)
    perm = torch.randperm(npg, generator=g)[:B * maxp].to(torch.int32).view(B, maxp).contiguous()
    for b in range(B):
        for k in range(maxp):
            rows = V[b, k * P:(k + 1) * P]
            pages[int(perm[b, k]), :rows.shape[0]] = rows
    return pages, perm


def _poison_tails(pages: torch.Tensor, bt: torch.Tensor, lens: torch.Tensor, P: int) -> torch.Tensor:
    """NaN (0x7F for E4M3 bytes) in every row of a sequence's pages at or past
    its length, the padding past C included: a kernel that let such a row reach
    an output would return NaN there."""
    pages = pages.clone()
    nan = 0x7F if pages.dtype == torch.uint8 else float("nan")
    for b in range(bt.shape[0]):
        c = torch.arange(int(lens[b]), bt.shape[1] * P)
        pages[bt[b].long()[c // P], c % P] = nan
    return pages


def _poison_rows(w: torch.Tensor, lens: torch.Tensor) -> torch.Tensor:
    """NaN in the weights (or scores) of every row at or past a sequence's length."""
    w = w.clone()
    for b in range(w.shape[0]):
        w[b, int(lens[b]):] = float("nan")
    return w


def _bound_ok(out, ref, w, V, lens, dt, softmax, label):
    keep = np.isfinite(ref)
    ok, msg = gate(np.where(keep, out, 0.0), np.where(keep, ref, 0.0), dt)
    assert ok, f"{label}: gate failed: {msg}"
    Cmax = max(int(lens.max()), 1)
    if not softmax:
        r = rel_l2(out, ref)
        assert r <= accum_bound(Cmax), f"{label}: relL2={r:.3e} above {accum_bound(Cmax):.3e}"
        return
    # A[b, q, d] = sum over the sequence's rows of p |V|
    B, C, Hq = w.shape
    Hkv, D = V.shape[2], V.shape[3]
    A = np.zeros((B, Hq, D))
    rng = 0.0
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            continue
        x = w[b, :n].double().numpy()
        fin = x[np.isfinite(x)]
        if fin.size:
            rng = max(rng, float(fin.max() - fin.min()))
        p = np.exp(x - x.max(axis=0, keepdims=True))
        p /= p.sum(axis=0, keepdims=True)
        a = np.abs(V[b, :n].double().numpy())
        A[b] = np.einsum("ckg,ckd->kgd", p.reshape(n, Hkv, Hq // Hkv), a).reshape(Hq, D)
    eps = (2.0 * rng + 512.0) * U32 + 8.0 * math.sqrt(Cmax) * U32
    err = np.linalg.norm(np.where(keep, out - ref, 0.0).ravel())
    assert err <= eps * np.linalg.norm(A.ravel()) + 1e-30, f"{label}: ||err||={err:.3e} above the bound"


def _run(w, pages, bt, lens, softmax, plan=None, mode="auto"):
    out = ga.gqa_av_paged_decode(w.to(DEV), pages.to(DEV), bt.to(DEV), lens.to(DEV), softmax=softmax,
                                 plan=plan, mode=mode)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _cases():
    cases, k = [], 0
    for G in (1, 2, 3, 4, 8, 16):
        for D in (64, 128, 256):
            for P in (1, 16, 64, 256):
                if (G + D // 64 + P) % 3:
                    continue
                dt = ("bf16", "f16", "f32")[k % 3]
                Hkv = (1, 2, 4)[k % 3]
                C = (300, 1000, 77)[k % 3]
                cases.append((2 + k % 2, C, G * Hkv, Hkv, D, P, dt))
                k += 1
    # eight KV heads (the bf16 engine's eight-head tiles)
    return cases + [(2, 1000, 64, 8, 128, 16, "bf16"), (3, 300, 16, 8, 64, 1, "bf16"),
                    (2, 500, 128, 16, 128, 16, "bf16")]


@pytest.mark.parametrize("B,C,Hq,Hkv,D,P,dt", _cases())
def test_paged_sweep(B, C, Hq, Hkv, D, P, dt, oracle_lib):
    """G 1..16, D 64..256, pages of 1..256 rows, all dtypes, ragged lengths
    (full, partial, 1 and 0), plain and fused, automatic and forced splits.
    Every V row, weight and score at or past a sequence's length holds NaN."""
    s, V = make_scores_random(B, C, Hq, Hkv, D, dt, seed=C + D + P, score_std=2.0)
    pages, bt = _paged_from_dense(V, P, seed=P + B)
    # full, partial, 1 and 0 rows over the cases (a length of 0 under split plans too)
    lens = torch.tensor([C, 0] if B == 2 else [C // 2 + 3, 1, 0], dtype=torch.int32)
    pages = _poison_tails(pages, bt, lens, P)
    attn = _poison_rows(torch.softmax(s.double(), dim=1).float(), lens).contiguous()
    s = _poison_rows(s, lens).contiguous()
    modes = ("auto", "per_head") if Hq // Hkv >= 2 else ("auto",)
    for softmax, w in ((False, attn), (True, s)):
        ref = oracle_lib.paged(w, pages, bt, lens, dt, softmax=softmax)
        plans = [ga.make_plan(B, C, Hq, Hkv, D, dt, mode, nsplit=ns, softmax=softmax, page_size=P)
                 for mode in modes for ns in (0, 1, 7)]
        if dt == "bf16" and Hq // Hkv >= 2:          # the bf16 matrix engine at any G
            for ht, ns in ((1, 0), (2, 5), (4, 1), (8, 3)):
                if Hkv % ht == 0 and (ns != 1 or C <= 1023 * P):
                    plans.append(ga.make_plan(B, C, Hq, Hkv, D, dt, "reuse", engine="mfma_bf16", kv_tile=ht,
                                              nsplit=ns, softmax=softmax, page_size=P))
        for plan in plans:
            out = _run(w, pages, bt, lens, softmax, plan=plan)
            _bound_ok(out, ref, w, V, lens, dt, softmax, f"paged {(B, C, Hq, Hkv, D, P, dt)} {plan.as_dict()}")
            assert (out[lens.numpy() == 0] == 0).all(), "a sequence of length 0 gives zeros"


@pytest.mark.parametrize("wname,P", [("g2-b4-c32768-hq16-hkv8-d128-bf16", 16),
                                     ("g3-b8-c16384-hq24-hkv8-d96-f16", 64),
                                     ("batch64-b64-c8192-hq64-hkv8-d128-bf16", 256),
                                     ("mqa16-b4-c32768-hq16-hkv1-d128-bf16", 32)])
def test_paged_workloads(wname, P, oracle_lib):
    """Workload shapes (the large batch cut to 8 sequences) as paged caches with
    lengths between half and all of the capacity, plain and fused; rows past
    each length hold NaN in V, the weights and the scores."""
    w = WORKLOADS[wname]
    if w.B > 8:
        w = w.replace(B=8)
    _say(f"[paged] {w.name} P={P}")
    s, V = make_scores(w, seed=0)
    pages, bt = _paged_from_dense(V, P, seed=1)
    g = torch.Generator().manual_seed(2)
    lens = torch.randint(w.C // 2, w.C + 1, (w.B,), generator=g, dtype=torch.int32)
    lens[0] = w.C
    pages = _poison_tails(pages, bt, lens, P)
    attn = _poison_rows(torch.softmax(s.double(), dim=1).float(), lens).contiguous()
    s = _poison_rows(s, lens).contiguous()
    for softmax, x in ((False, attn), (True, s)):
        ref = oracle_lib.paged(x, pages, bt, lens, w.v_dtype, softmax=softmax)
        out = _run(x, pages, bt, lens, softmax)
        _bound_ok(out, ref, x, V, lens, w.v_dtype, softmax, f"paged {w.name} softmax={softmax}")


@pytest.mark.parametrize("dt,engine", [("bf16", "valu"), ("f32", "valu"), ("bf16", "mfma_bf16"),
                                       ("fp8", "mfma_bf16")])
def test_paged_dense_layout_matches_dense_call(dt, engine):
    """One page per sequence (P = C, block_table[b] = b, full lengths) is the
    dense layout: the paged call equals the dense call on the same engine with
    the same splits and tiles bit for bit (same arithmetic, same order; rows
    past a split weigh 0 on both sides). C = 500 leaves a partial last step."""
    B, C, Hq, Hkv, D = 3, 500, 32, 4, 128
    s, V = make_scores_random(B, C, Hq, Hkv, D, "f32" if dt == "fp8" else dt, seed=91)
    if dt == "fp8":
        V = (V / V.abs().max() * 400.0).to(torch.float8_e4m3fn).contiguous()
    attn = torch.softmax(s.double(), dim=1).float().contiguous()
    P = 512                                          # a power of two >= C
    bt = torch.arange(B, dtype=torch.int32).view(B, 1)
    lens = torch.full((B,), C, dtype=torch.int32)
    pages = torch.zeros((B, P, Hkv, D), dtype=V.dtype)
    pages[:, :C] = V
    for softmax, x in ((False, attn), (True, s)):
        pp = ga.make_plan(B, C, Hq, Hkv, D, dt, "reuse", engine=engine, page_size=P, softmax=softmax, nsplit=4,
                          kv_tile=2)
        dp = ga.make_plan(B, C, Hq, Hkv, D, dt, "reuse", engine=engine, softmax=softmax, nsplit=4, kv_tile=2,
                          split_order="contiguous")
        assert pp.engine == dp.engine and pp.rows_per_split == dp.rows_per_split and pp.interleave == dp.interleave
        a = _run(x, pages, bt, lens, softmax, plan=pp)
        fn = ga.gqa_softmax_av_decode if softmax else ga.gqa_av_decode
        b = fn(x.to(DEV), V.to(DEV), plan=dp).cpu().numpy().astype(np.float64)
        assert np.array_equal(a, b), f"paged dense layout != dense call ({dt}, {engine}, softmax={softmax})"


@pytest.mark.parametrize("P,Hq", [(1, 32), (16, 32), (128, 32), (16, 8), (64, 16)])
def test_paged_fp8_matches_fp8_oracle(P, Hq, oracle_lib):
    """fp8 pages (unit scale), G = 8 on the bf16 matrix engine and G = 2 or 4
    on the VALU engine (16-byte lane loads): the gathered rows of each sequence
    against the fp8 oracle, with the weights (plain) or scores (fused, -inf)
    of rows past its length removed on the oracle's side."""
    B, C, Hkv, D = 3, 700, 4, 128
    s, Vf = make_scores_random(B, C, Hq, Hkv, D, "f32", seed=95 + P)
    V = (Vf / Vf.abs().max() * 400.0).to(torch.float8_e4m3fn).contiguous()
    pages, bt = _paged_from_dense(V.view(torch.uint8), P, seed=P)
    pages = pages.view(torch.float8_e4m3fn)
    lens = torch.tensor([C, 333, 1], dtype=torch.int32)
    keep = torch.arange(C).view(1, C, 1) < lens.view(B, 1, 1)
    attn = torch.softmax(s.double(), dim=1).float().contiguous()
    for softmax, x in ((False, attn), (True, s)):
        xo = torch.where(keep, x, torch.tensor(float("-inf") if softmax else 0.0)).contiguous()
        ref = oracle_lib.fp8(xo, V, None, softmax=softmax)
        for ns in (0, 3):
            plan = ga.make_plan(B, C, Hq, Hkv, D, "fp8", "reuse", nsplit=ns, softmax=softmax, page_size=P)
            assert plan.engine == (3 if Hq // Hkv >= 5 else 1)
            out = _run(x, pages, bt, lens, softmax, plan=plan)
            _bound_ok(out, ref, x, V.float(), lens, "fp8", softmax, f"paged fp8 P={P} softmax={softmax} ns={ns}")


def test_paged_deterministic_and_side_stream():
    B, C, Hq, Hkv, D, P = 4, 3000, 32, 8, 128, 16
    s, V = make_scores_random(B, C, Hq, Hkv, D, "bf16", seed=93)
    pages, bt = _paged_from_dense(V, P, seed=3)
    lens = torch.tensor([3000, 2999, 17, 1500], dtype=torch.int32)
    args = [t.to(DEV) for t in (s, pages, bt, lens)]
    a = [ga.gqa_av_paged_decode(*args, softmax=True).cpu() for _ in range(3)]
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        c = ga.gqa_av_paged_decode(*args, softmax=True, stream=st)
    st.synchronize()
    torch.cuda.synchronize()
    assert all(torch.equal(a[0], x) for x in a[1:]) and torch.equal(a[0], c.cpu())


@pytest.mark.parametrize("softmax", [False, True])
def test_paged_pass1_then_combine_is_the_call(softmax):
    """gqa_av_paged_decode_pass1 then _combine on one stream equals
    gqa_av_paged_decode_plan bit for bit (VALU at G=2, bf16 matrix engine at
    G=8, one split and several)."""
    for Hq, ns in ((16, 0), (64, 0), (64, 1)):
        B, C, Hkv, D, P = 3, 3000, 8, 128, 16
        s, V = make_scores_random(B, C, Hq, Hkv, D, "bf16", seed=97 + Hq)
        pages, bt = _paged_from_dense(V, P, seed=4)
        lens = torch.tensor([3000, 2048, 5], dtype=torch.int32)
        x = s if softmax else torch.softmax(s.double(), dim=1).float().contiguous()
        plan = ga.make_plan(B, C, Hq, Hkv, D, "bf16", nsplit=ns, softmax=softmax, page_size=P)
        call = ga.bind_paged(x.to(DEV), pages.to(DEV), bt.to(DEV), lens.to(DEV), plan=plan)
        whole = call().clone()
        call.out.fill_(float("nan"))
        call.pass1()
        got = call.combine()
        torch.cuda.synchronize()
        assert torch.equal(whole, got), (Hq, ns, softmax)
