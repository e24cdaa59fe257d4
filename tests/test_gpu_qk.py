"""GPU parity of the decode score step (scores = scale * q . K, K shared by each
head group) through the C ABI, against the fp64 CPU oracle.

Gate: the acceptance gate of tests/parity.py (max-abs for fp32 K, relative L2
for bf16/fp16 K) with the fp32-accumulation bound over the D terms of each dot
product, plus an elementwise bound on small shapes: |err| <= 2 D 2^-24 scale
sum_d |q K|. All tests need an MI355X and are marked ``gpu``.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import gqa_reuse_attn_amd as ga
from oracle.brute import abs_sum_qk
from tests.parity import assert_parity
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


def _run(q, K, scale, mode="auto", plan=None):
    s = ga.gqa_qk_decode(q.to(DEV), K.to(DEV), scale=scale, mode=mode, plan=plan)
    torch.cuda.synchronize()
    return s.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("wname", list(WORKLOADS))
@pytest.mark.parametrize("mode", ["auto", "per_head"])
def test_qk_workload_shapes(wname, mode, oracle_lib):
    """The six decode shapes (K of the workload's V dtype), scale 1/sqrt(D)."""
    w = WORKLOADS[wname]
    if w.B * w.C * w.Hkv * w.D > 2 ** 28:
        w = w.replace(B=8)                     # the large batch: 8 sequences keep the oracle in seconds
    _say(f"[qk] {w.name} B={w.B} mode={mode}")
    q, K = make_qk_random(w.B, w.C, w.Hq, w.Hkv, w.D, w.v_dtype, seed=3)
    scale = w.D ** -0.5
    ref = oracle_lib.qk(q, K, w.v_dtype, scale)
    out = _run(q, K, scale, mode)
    assert_parity(out, ref, w.v_dtype, w.D, f"qk {w.name} {mode}")


def _qk_cases():
    cases = []
    k = 0
    for G in (1, 2, 3, 4, 5, 8, 16, 17, 32):
        for D in (32, 64, 96, 128, 160, 256):
            for C in (1, 63, 65, 300):
                if (G + D + C) % 3:
                    continue                    # a spread subset of the grid
                dt = ("bf16", "f16", "f32")[k % 3]
                Hkv = (1, 2, 4)[k % 3]
                rows = (0, 64, 128)[k % 3]
                cases.append((1 + k % 2, C, G * Hkv, Hkv, D, dt, rows))
                k += 1
    return cases


@pytest.mark.parametrize("B,C,Hq,Hkv,D,dt,rows", _qk_cases())
def test_qk_sweep(B, C, Hq, Hkv, D, dt, rows, oracle_lib):
    """Small shapes: G 1..32, D 32..256, ragged C, all dtypes, forced row blocks."""
    q, K = make_qk_random(B, C, Hq, Hkv, D, dt, seed=B * 1000 + C + D)
    scale = 0.375
    ref = oracle_lib.qk(q, K, dt, scale)
    bound = 2 * D * U32 * scale * abs_sum_qk(q, K) + 1e-30
    modes = ("auto", "per_head") if Hq // Hkv >= 2 else ("auto",)
    plans = [ga.qk_make_plan(B, C, Hq, Hkv, D, dt, mode, rows_per_block=rows) for mode in modes]
    plans += [ga.qk_make_plan(B, C, Hq, Hkv, D, dt, "reuse", rows_per_block=rows, kv_tile=ht)
              for ht in (2, 4) if Hq // Hkv >= 2 and Hkv % ht == 0]
    for plan in plans:
        out = _run(q, K, scale, plan=plan)
        assert_parity(out, ref, dt, D, f"qk {(B, C, Hq, Hkv, D, dt)} plan={plan.as_dict()}")
        assert (np.abs(out - ref) <= bound).all(), f"qk elementwise bound {(B, C, Hq, Hkv, D, dt)} {plan.as_dict()}"


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
def test_qk_single_term_is_exact(dt):
    """One nonzero q element per head and K a power of two: each score is
    scale * q * K exactly (bf16 K: the three-term split of q loses no bit)."""
    B, C, Hq, Hkv, D = 2, 200, 32, 2, 128
    G = Hq // Hkv
    gen = torch.Generator().manual_seed(5)
    q = torch.zeros(B, Hq, D)
    pick = {}
    for b in range(B):
        for h in range(Hq):
            j = (7 * b + 11 * h + 3) % D
            val = (torch.rand(1, generator=gen).item() + 1.0) * 2.0 ** int(torch.randint(-30, 10, (1,), generator=gen))
            q[b, h, j] = val
            pick[b, h] = j
    kt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dt]
    K = torch.pow(2.0, torch.randint(-10, 10, (B, C, Hkv, D), generator=gen).float()).to(kt)
    out = _run(q, K, 0.5)
    Kd = K.double().numpy()
    for (b, h), j in pick.items():
        want = (0.5 * q[b, h, j].double().item() * Kd[b, :, h // G, j]).astype(np.float32)
        assert np.array_equal(out[b, :, h].astype(np.float32), want), (dt, b, h)


def test_qk_deterministic():
    q, K = make_qk_random(4, 5000, 16, 8, 128, "bf16", seed=9)
    a = [ga.gqa_qk_decode(q.to(DEV), K.to(DEV), scale=0.1).cpu() for _ in range(3)]
    torch.cuda.synchronize()
    assert all(torch.equal(a[0], x) for x in a[1:])


def test_qk_edges(oracle_lib):
    # C = 0 and B = 0: nothing to do
    s = ga.gqa_qk_decode(torch.zeros(2, 4, 64, device=DEV), torch.zeros(2, 0, 2, 64, dtype=torch.bfloat16, device=DEV))
    assert s.shape == (2, 0, 4)
    s = ga.gqa_qk_decode(torch.zeros(0, 4, 64, device=DEV), torch.zeros(0, 9, 2, 64, dtype=torch.bfloat16, device=DEV))
    assert s.shape == (0, 9, 4)
    # D not a multiple of 32 is refused, not run
    with pytest.raises(ga.GqaAvError) as ei:
        ga.gqa_qk_decode(torch.zeros(1, 4, 48, device=DEV), torch.zeros(1, 8, 2, 48, dtype=torch.bfloat16, device=DEV))
    assert ei.value.name == "UNSUPPORTED"
    # K not 16-byte aligned is refused
    buf = torch.zeros(1 * 8 * 2 * 64 + 8, dtype=torch.bfloat16, device=DEV)
    k_off = buf[1:1 + 8 * 2 * 64].view(1, 8, 2, 64)
    with pytest.raises(ga.GqaAvError) as ei:
        ga.gqa_qk_decode(torch.zeros(1, 4, 64, device=DEV), k_off)
    assert ei.value.name == "UNSUPPORTED"
    # forced reuse with G = 1 is ineligible
    with pytest.raises(ga.GqaAvError) as ei:
        ga.gqa_qk_decode(torch.zeros(1, 2, 64, device=DEV), torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16, device=DEV),
                         mode="reuse")
    assert ei.value.name == "INELIGIBLE"


@pytest.mark.parametrize("B,C,Hq,Hkv,D,dt,ht", [(2, 700, 16, 8, 128, "bf16", 4), (1, 333, 24, 8, 96, "f16", 4),
                                               (2, 129, 16, 1, 64, "bf16", 1), (1, 200, 32, 8, 128, "f32", 2)])
def test_qk_unaligned_scores(B, C, Hq, Hkv, D, dt, ht, oracle_lib):
    """scores 4-byte but not 16-byte aligned (the 4-byte store path on shapes
    that otherwise take 16-byte stores); the floats around it stay untouched."""
    q, K = make_qk_random(B, C, Hq, Hkv, D, dt, seed=C + D)
    ref = oracle_lib.qk(q, K, dt, 0.25)
    n = B * C * Hq
    buf = torch.full((n + 8,), 7.5, dtype=torch.float32, device=DEV)
    sc = buf[1:1 + n].view(B, C, Hq)
    assert sc.data_ptr() % 16 == 4
    plan = ga.qk_make_plan(B, C, Hq, Hkv, D, dt, "auto", kv_tile=ht)
    ga.gqa_qk_decode(q.to(DEV), K.to(DEV), scores=sc, scale=0.25, plan=plan)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert host[0] == 7.5 and (host[1 + n:] == 7.5).all()
    assert_parity(host[1:1 + n].reshape(B, C, Hq).astype(np.float64), ref, dt, D, f"qk unaligned {(B, C, Hq, Hkv, D)}")


def test_qk_then_av_matches_attention(oracle_lib):
    """Scores -> softmax over c -> attention-times-V on the GPU equals the
    oracles composed the same way (the two steps agree on the attn layout)."""
    B, C, Hq, Hkv, D = 2, 3000, 16, 4, 128
    q, K = make_qk_random(B, C, Hq, Hkv, D, "bf16", seed=21)
    _, V = make_qk_random(B, C, Hq, Hkv, D, "bf16", seed=22)
    scale = D ** -0.5
    s = ga.gqa_qk_decode(q.to(DEV), K.to(DEV), scale=scale)
    attn = torch.softmax(s.double(), dim=1).float().contiguous()
    out = ga.gqa_av_decode(attn, V.to(DEV))
    torch.cuda.synchronize()
    ref_s = oracle_lib.qk(q, K, "bf16", scale)
    e = np.exp(ref_s - ref_s.max(axis=1, keepdims=True))
    ref_attn = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    ref = oracle_lib.full(torch.from_numpy(ref_attn), V, "bf16")
    assert_parity(out.cpu().numpy().astype(np.float64), ref, "bf16", C, "qk -> softmax -> av")


# ---- fp8 K (OCP FP8 E4M3 with a float32 scale per KV head) -------------------

def _quantize_k(K: torch.Tensor):
    """Per-KV-head scale max|K| / 448 and the E4M3 bytes of K / scale (torch's
    round-to-nearest cast): input preparation, not part of the step."""
    Kf = K.float()
    amax = Kf.abs().amax(dim=(0, 1, 3)).clamp_min(1e-30)
    scale = (amax / 448.0).float().contiguous()
    return (Kf / scale.view(1, 1, -1, 1)).to(torch.float8_e4m3fn).contiguous(), scale


def _run_fp8(q, K8, k_scale, scale, plan=None, mode="auto"):
    s = ga.gqa_qk_decode(q.to(DEV), K8.to(DEV), scale=scale, mode=mode, plan=plan,
                         k_scale=None if k_scale is None else k_scale.to(DEV))
    torch.cuda.synchronize()
    return s.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("wname", [n for n, w in WORKLOADS.items() if w.D % 64 == 0])
def test_qk_fp8_workloads(wname, oracle_lib):
    """The workload shapes with D a multiple of 64, K quantized per KV head (the
    large batch cut to 8 sequences; the full size is in test_gpu_full_size),
    reuse and per-head."""
    w = WORKLOADS[wname]
    if w.B > 8:
        w = w.replace(B=8)
    _say(f"[qk fp8] {w.name}")
    q, K = make_qk_random(w.B, w.C, w.Hq, w.Hkv, w.D, w.v_dtype, seed=3)
    K8, ks = _quantize_k(K)
    scale = w.D ** -0.5
    ref = oracle_lib.qk_fp8(q, K8, ks, scale)
    for mode in ("auto", "per_head"):
        assert_parity(_run_fp8(q, K8, ks, scale, mode=mode), ref, "bf16", w.D, f"qk fp8 {w.name} {mode}")


def _qk_fp8_cases():
    cases, k = [], 0
    for G in (1, 2, 3, 4, 8, 16, 17):
        for D in (64, 128, 192, 256):
            for C in (1, 63, 65, 300):
                if (G + D // 64 + C) % 3:
                    continue
                cases.append((1 + k % 2, C, G * (1, 2, 4)[k % 3], (1, 2, 4)[k % 3], D, (0, 64, 128)[k % 3]))
                k += 1
    return cases


@pytest.mark.parametrize("B,C,Hq,Hkv,D,rows", _qk_fp8_cases())
def test_qk_fp8_sweep(B, C, Hq, Hkv, D, rows, oracle_lib):
    """Small shapes: G 1..17, D 64..256, ragged C, forced row blocks, 1/2/4 KV
    heads per workgroup, with and without scales; the gate, the accumulation
    bound and the elementwise bound 2 D 2^-24 scale sum_d |q K|."""
    q, K = make_qk_random(B, C, Hq, Hkv, D, "f32", seed=B * 1000 + C + D + 7)
    K8, ks = _quantize_k(K)
    scale = 0.375
    modes = ("auto", "per_head") if Hq // Hkv >= 2 else ("auto",)
    plans = [ga.qk_make_plan(B, C, Hq, Hkv, D, "fp8", mode, rows_per_block=rows) for mode in modes]
    plans += [ga.qk_make_plan(B, C, Hq, Hkv, D, "fp8", "reuse", rows_per_block=rows, kv_tile=ht)
              for ht in (2, 4) if Hq // Hkv >= 2 and Hkv % ht == 0]
    for sc in (ks, None):
        ref = oracle_lib.qk_fp8(q, K8, sc, scale)
        kd = K8.float() * (sc.view(1, 1, -1, 1) if sc is not None else 1.0)
        bound = 2 * D * U32 * scale * abs_sum_qk(q, kd) + 1e-30
        for plan in plans:
            out = _run_fp8(q, K8, sc, scale, plan=plan)
            label = f"qk fp8 {(B, C, Hq, Hkv, D)} scale={sc is not None} plan={plan.as_dict()}"
            assert_parity(out, ref, "bf16", D, label)
            assert (np.abs(out - ref) <= bound).all(), f"elementwise bound: {label}"


def test_qk_fp8_equals_bf16_on_widened_k():
    """With unit scales, fp8 K gives the scores of bf16 K holding the same
    values, bit for bit (the kernel widens K exactly to bf16 before the same
    products), on every plan shape; every non-NaN E4M3 byte appears in K."""
    B, C, Hq, Hkv, D = 2, 700, 32, 4, 128
    g = torch.Generator().manual_seed(17)
    vals = torch.tensor([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=torch.uint8)
    raw = vals[torch.randint(0, vals.numel(), (B, C, Hkv, D), generator=g)]
    raw[0, 0, 0, :] = vals[:D]
    raw[0, 1, 0, :vals.numel() - D] = vals[D:]
    K8 = raw.view(torch.float8_e4m3fn)
    K16 = K8.to(torch.bfloat16)
    q, _ = make_qk_random(B, C, Hq, Hkv, D, "f32", seed=18)
    for mode, ht in (("auto", 0), ("per_head", 0), ("reuse", 1), ("reuse", 2)):
        p8 = ga.qk_make_plan(B, C, Hq, Hkv, D, "fp8", mode, kv_tile=ht)
        p16 = ga.qk_make_plan(B, C, Hq, Hkv, D, "bf16", mode, kv_tile=ht)
        a = _run_fp8(q, K8, None, 0.25, plan=p8)
        b = _run(q, K16, 0.25, plan=p16)
        assert np.array_equal(a, b), (mode, ht)


# ---- paged K (the paged-V layout and tables) ---------------------------------

SENTINEL = -12345.5


def _paged_k(K: torch.Tensor, P: int, seed: int, spare: int = 3):
    """Scatter a dense K [B, C, Hkv, D] into a shuffled pool of P-row pages
    (spare pages hold a large value that must never be read)."""
    B, C, Hkv, D = K.shape
    maxp = -(-C // P)
    g = torch.Generator().manual_seed(seed)
    npg = B * maxp + spare
    if K.dtype == torch.float8_e4m3fn:
        pages = torch.full((npg, P, Hkv, D), 0x7E, dtype=torch.uint8).view(torch.float8_e4m3fn)
    else:
        pages = torch.full((npg, P, Hkv, D), 3.0e4).to(K.dtype)
    perm = torch.randperm(npg, generator=g)[:B * maxp].to(torch.int32).view(B, maxp).contiguous()
    for b in range(B):
        for k in range(maxp):
            rows = K[b, k * P:(k + 1) * P]
            pages[int(perm[b, k]), :rows.shape[0]] = rows
    return pages, perm


def _run_paged(q, pages, bt, lens, C, scale, k_scale=None, plan=None):
    scores = torch.full((q.shape[0], C, q.shape[1]), SENTINEL, device=DEV)
    ga.gqa_qk_paged_decode(q.to(DEV), pages.to(DEV), bt.to(DEV), lens.to(DEV), scores=scores, scale=scale, plan=plan,
                           k_scale=None if k_scale is None else k_scale.to(DEV))
    torch.cuda.synchronize()
    return scores.cpu().numpy().astype(np.float64)


def _check_paged(out, ref, lens, dt, D, label):
    """Rows below each length: the gate and accumulation bound per sequence;
    rows past it: untouched (the sentinel)."""
    for b, n in enumerate(lens.tolist()):
        if n:
            assert_parity(out[b, :n], ref[b, :n], "bf16" if dt == "fp8" else dt, D, f"{label} b={b}")
        assert (out[b, n:] == SENTINEL).all(), f"{label} b={b}: a row past the length was written"


def _qk_paged_cases():
    cases, k = [], 0
    for G in (1, 2, 3, 8, 16):
        for D in (64, 128, 256):
            for P in (1, 16, 64):
                if (G + D // 64 + P) % 2:
                    continue
                dt = ("bf16", "f16", "f32", "fp8")[k % 4]
                Hkv = (1, 2, 4)[k % 3]
                C = (300, 1000, 77)[k % 3]
                cases.append((2 + k % 3, C, G * Hkv, Hkv, D, P, dt))
                k += 1
    return cases


@pytest.mark.parametrize("B,C,Hq,Hkv,D,P,dt", _qk_paged_cases())
def test_qk_paged_sweep(B, C, Hq, Hkv, D, P, dt, oracle_lib):
    """G 1..16, D 64..256, pages of 1..64 rows, all K types (fp8 with scales),
    lengths full / partial / 1 / 0, reuse and per-head, 1/2/4 KV heads per
    workgroup; rows past each length keep the value they had."""
    q, K = make_qk_random(B, C, Hq, Hkv, D, "f32" if dt == "fp8" else dt, seed=C + D + P)
    ks = None
    if dt == "fp8":
        K, ks = _quantize_k(K)
    pages, bt = _paged_k(K, P, seed=P + B)
    lens = torch.tensor([C, C // 2 + 3, 1, 0][:B], dtype=torch.int32)
    scale = 0.375
    ref = oracle_lib.qk_paged(q, pages, bt, lens, dt, scale, ks, C=C)
    modes = ("auto", "per_head") if Hq // Hkv >= 2 else ("auto",)
    plans = [ga.qk_make_plan(B, C, Hq, Hkv, D, dt, m, page_size=P) for m in modes]
    plans += [ga.qk_make_plan(B, C, Hq, Hkv, D, dt, "reuse", kv_tile=ht, rows_per_block=128, page_size=P)
              for ht in (2, 4) if Hq // Hkv >= 2 and Hkv % ht == 0]
    for plan in plans:
        out = _run_paged(q, pages, bt, lens, C, scale, ks, plan=plan)
        _check_paged(out, ref, lens, dt, D, f"qk paged {(B, C, Hq, Hkv, D, P, dt)} {plan.as_dict()}")


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_qk_paged_dense_layout_matches_dense_call(dt):
    """One page per sequence holding its dense K (P = C, block_table[b] = b,
    full lengths) gives the dense call's scores bit for bit."""
    B, C, Hq, Hkv, D = 3, 512, 32, 4, 128
    q, K = make_qk_random(B, C, Hq, Hkv, D, "f32" if dt == "fp8" else dt, seed=71)
    ks = None
    if dt == "fp8":
        K, ks = _quantize_k(K)
    bt = torch.arange(B, dtype=torch.int32).view(B, 1)
    lens = torch.full((B,), C, dtype=torch.int32)
    for mode in ("auto", "per_head"):
        pp = ga.qk_make_plan(B, C, Hq, Hkv, D, dt, mode, page_size=C)
        dp = ga.qk_make_plan(B, C, Hq, Hkv, D, dt, mode)
        assert pp.rows_per_block == dp.rows_per_block
        a = _run_paged(q, K, bt, lens, C, 0.125, ks, plan=pp)
        b = (_run_fp8(q, K, ks, 0.125, plan=dp) if dt == "fp8" else _run(q, K, 0.125, plan=dp))
        assert np.array_equal(a, b), (dt, mode)


@pytest.mark.parametrize("wname,P", [("g2-b4-c32768-hq16-hkv8-d128-bf16", 16),
                                     ("batch64-b64-c8192-hq64-hkv8-d128-bf16", 256),
                                     ("mqa16-b4-c32768-hq16-hkv1-d128-bf16", 32)])
def test_qk_paged_workloads(wname, P, oracle_lib):
    """Workload shapes (the large batch cut to 8 sequences) as paged K with
    lengths between half and all of the capacity."""
    w = WORKLOADS[wname]
    if w.B > 8:
        w = w.replace(B=8)
    _say(f"[qk paged] {w.name} P={P}")
    q, K = make_qk_random(w.B, w.C, w.Hq, w.Hkv, w.D, w.v_dtype, seed=5)
    pages, bt = _paged_k(K, P, seed=1)
    g = torch.Generator().manual_seed(2)
    lens = torch.randint(w.C // 2, w.C + 1, (w.B,), generator=g, dtype=torch.int32)
    lens[0] = w.C
    scale = w.D ** -0.5
    ref = oracle_lib.qk_paged(q, pages, bt, lens, w.v_dtype, scale, C=w.C)
    out = _run_paged(q, pages, bt, lens, w.C, scale)
    _check_paged(out, ref, lens, w.v_dtype, w.D, f"qk paged {w.name}")
