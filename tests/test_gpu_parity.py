"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Every test here needs an MI355X and the built libgqa_av.so; all are marked
``gpu``. Inputs are seeded and synthetic (workloads.py). The comparison is the
acceptance gate of tests/parity.py (max-abs for fp32 V, relative L2 for
bf16/fp16 V) plus the fp32-accumulation bound.
"""
from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest
import torch

import gqa_reuse_attn_amd as ga
from tests.parity import assert_parity, gate, rel_l2
from workloads import WORKLOADS, Workload, make_inputs, make_random

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


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
    ga.release()


def _run(attn, V, mode="auto", plan=None, out=None):
    a = attn.to(DEV)
    v = V.to(DEV)
    o = ga.gqa_av_decode(a, v, out=out, mode=mode, plan=plan)
    torch.cuda.synchronize()
    return o.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("wname", list(WORKLOADS))
@pytest.mark.parametrize("mode", ["auto", "per_head"])
def test_workload_full_size(wname, mode, oracle_lib):
    """Full-size decode workloads, in the plan the bench times (auto) and per-head."""
    w = WORKLOADS[wname]
    _say(f"[parity] {wname} mode={mode}")
    attn, V = make_inputs(w, seed=0)
    ref = oracle_lib.full(attn, V, w.v_dtype)
    plan = ga.make_plan(w.B, w.C, w.Hq, w.Hkv, w.D, w.v_dtype, mode,
                        cu_count=torch.cuda.get_device_properties(0).multi_processor_count)
    out = _run(attn, V, mode)
    assert_parity(out, ref, w.v_dtype, w.C, f"{wname}/{mode} plan={plan.as_dict()}")
    _say(f"[parity] {wname} mode={mode} relL2={rel_l2(out, ref):.2e} nsplit={plan.nsplit}")


def _sweep_cases():
    Gs = [1, 2, 3, 4, 5, 7, 8, 9, 12, 16, 17, 32]
    Ds = [64, 96, 128, 256]
    Cs = [1, 2, 63, 64, 65, 1000]
    dts = ["bf16", "f16", "f32"]
    cases = []
    k = 0
    for G in Gs:
        for C in Cs:
            D = Ds[k % len(Ds)]
            dt = dts[k % len(dts)]
            Hkv = 1 + (k % 3)
            ns = [1, 2, 7, 0, 10 ** 6][k % 5]      # 0 = automatic, 10**6 = one row per split
            cases.append((2, C, G * Hkv, Hkv, D, dt, ns))
            k += 1
    return cases


def _plans(B, C, Hq, Hkv, D, dt, ns):
    """The automatic plan, per-head, each reuse engine that can take the shape,
    and both ways of cutting a split context (interleaved blocks, contiguous)."""
    plans = [("auto", ga.make_plan(B, C, Hq, Hkv, D, dt, "auto", nsplit=ns))]
    if Hq // Hkv >= 2:
        plans.append(("per_head", ga.make_plan(B, C, Hq, Hkv, D, dt, "per_head", nsplit=ns)))
        for eng in ("valu", "mfma", "mfma_bf16"):
            try:
                plans.append((eng, ga.make_plan(B, C, Hq, Hkv, D, dt, "reuse", engine=eng, nsplit=ns)))
            except ga.GqaAvError as e:
                assert e.name == "UNSUPPORTED"
    if Hq // Hkv >= 2 and Hkv > 1:
        for eng in ("valu", "mfma_bf16"):
            for ht in sorted({2, Hkv}):
                if Hkv % ht == 0:
                    try:
                        plans.append((f"kv_tile={ht}/{eng}", ga.make_plan(B, C, Hq, Hkv, D, dt, "reuse", engine=eng,
                                                                          nsplit=ns, kv_tile=ht)))
                    except ga.GqaAvError as e:
                        assert e.name == "UNSUPPORTED"
    # the other way of cutting a split context: contiguous ranges (the
    # automatic plans interleave blocks of one step)
    for name, p in list(plans):
        if p.nsplit > 1 and p.interleave:
            mode = "per_head" if p.mode == 0 else "reuse"
            eng = {1: "valu", 2: "mfma", 3: "mfma_bf16"}[p.engine]
            plans.append((f"{name}/contiguous", ga.make_plan(B, C, Hq, Hkv, D, dt, mode, engine=eng, nsplit=ns,
                                                             kv_tile=p.kv_heads_per_tile, split_order="contiguous")))
    return plans


@pytest.mark.parametrize("B,C,Hq,Hkv,D,dt,ns", _sweep_cases())
def test_sweep_small(B, C, Hq, Hkv, D, dt, ns, oracle_lib):
    """Small shapes: G from 1 to 32, ragged C, several D, dtypes, forced splits, both engines."""
    attn, V = make_random(B, C, Hq, Hkv, D, dt, seed=B * 1000 + C + Hq, attn_kind="signed")
    ref = oracle_lib.full(attn, V, dt)
    scale = np.abs(attn.double().numpy()).sum(1).max() * np.abs(V.double().numpy()).max()
    for name, plan in _plans(B, C, Hq, Hkv, D, dt, ns):
        out = _run(attn, V, plan=plan)
        ok, msg = gate(out, ref, dt)
        assert ok, f"{(B, C, Hq, Hkv, D, dt, name)} plan={plan.as_dict()}: {msg}"
        # signed weights cancel; hold the elementwise error to fp32 accumulation
        assert np.abs(out - ref).max() <= 4 * C * 2.0 ** -24 * scale + 1e-30, \
            f"{(B, C, Hq, Hkv, D, dt, name)} plan={plan.as_dict()}"


@pytest.mark.parametrize("wname", list(WORKLOADS))
def test_workload_contiguous_splits(wname, oracle_lib):
    """Full-size workloads with the split context cut into contiguous ranges
    (the automatic plan interleaves blocks of one pipeline step)."""
    w = WORKLOADS[wname]
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    auto = ga.make_plan(w.B, w.C, w.Hq, w.Hkv, w.D, w.v_dtype, cu_count=cu)
    if auto.nsplit == 1:
        pytest.skip("automatic plan does not split the context")
    assert auto.interleave == 1
    _say(f"[parity] {wname} contiguous splits")
    attn, V = make_inputs(w, seed=0)
    ref = oracle_lib.full(attn, V, w.v_dtype)
    plan = ga.make_plan(w.B, w.C, w.Hq, w.Hkv, w.D, w.v_dtype, cu_count=cu, split_order="contiguous")
    assert plan.interleave == 0 and plan.nsplit == auto.nsplit
    out = _run(attn, V, plan=plan)
    assert_parity(out, ref, w.v_dtype, w.C, f"{wname}/contiguous plan={plan.as_dict()}")


@pytest.mark.parametrize("wname,engine", [
    ("llama3-8b-b1-c4096-hq32-hkv8-d128-bf16", "mfma"),
    ("llama3-8b-b1-c4096-hq32-hkv8-d128-bf16", "mfma_bf16"),
    ("g2-b4-c32768-hq16-hkv8-d128-bf16", "mfma"),
    ("g2-b4-c32768-hq16-hkv8-d128-bf16", "mfma_bf16"),
    ("mqa16-b4-c32768-hq16-hkv1-d128-bf16", "valu"),
    ("mqa16-b4-c32768-hq16-hkv1-d128-bf16", "mfma"),
    ("batch64-b64-c8192-hq64-hkv8-d128-bf16", "valu"),
    ("batch64-b64-c8192-hq64-hkv8-d128-bf16", "mfma"),
])
def test_workload_other_engine(wname, engine, oracle_lib):
    """Full-size workloads on the engine the automatic plan does not pick."""
    w = WORKLOADS[wname]
    _say(f"[parity] {wname} engine={engine}")
    attn, V = make_inputs(w, seed=0)
    ref = oracle_lib.full(attn, V, w.v_dtype)
    plan = ga.make_plan(w.B, w.C, w.Hq, w.Hkv, w.D, w.v_dtype, "reuse", engine=engine,
                        cu_count=torch.cuda.get_device_properties(0).multi_processor_count)
    out = _run(attn, V, plan=plan)
    assert_parity(out, ref, w.v_dtype, w.C, f"{wname}/{engine} plan={plan.as_dict()}")


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_one_hot_is_exact(dt):
    """One-hot weights return the selected V row bit for bit, through splits too."""
    B, C, Hq, Hkv, D = 2, 777, 12, 3, 128
    _, V = make_random(B, C, Hq, Hkv, D, dt, seed=5)
    attn = torch.zeros(B, C, Hq)
    G = Hq // Hkv
    sel = {}
    for b in range(B):
        for q in range(Hq):
            c = (97 * b + 31 * q + 13) % C
            attn[b, c, q] = 1.0
            sel[b, q] = c
    Vd = V.to(torch.float32).numpy()
    for mode, ns, eng, comb in (("auto", 0, "auto", "auto"), ("auto", 5, "auto", "kernel"),
                                ("per_head", 3, "auto", "kernel"), ("auto", 1, "auto", "auto"),
                                ("reuse", 0, "mfma", "kernel"), ("reuse", 4, "mfma", "kernel"),
                                ("reuse", 1, "mfma", "auto")):
        plan = ga.make_plan(B, C, Hq, Hkv, D, dt, mode, nsplit=ns, engine=eng, combine=comb)
        out = _run(attn, V, plan=plan).astype(np.float32)
        for (b, q), c in sel.items():
            assert np.array_equal(out[b, q], Vd[b, c, q // G]), (mode, ns, b, q)
    if dt == "bf16":
        for ns, comb in ((0, "kernel"), (4, "kernel"), (1, "auto")):
            plan = ga.make_plan(B, C, Hq, Hkv, D, dt, "reuse", nsplit=ns, engine="mfma_bf16", combine=comb)
            out = _run(attn, V, plan=plan).astype(np.float32)
            for (b, q), c in sel.items():
                assert np.array_equal(out[b, q], Vd[b, c, q // G]), ("mfma_bf16", ns, b, q)


def test_bf16_engine_splits_weights_exactly():
    """The bf16 matrix engine splits each fp32 weight into three bf16 terms.
    With a single nonzero weight per head and V a power of two, the output is
    weight * V exactly: any lost weight bit shows up."""
    B, C, Hq, Hkv, D = 2, 301, 32, 2, 128
    G = Hq // Hkv
    gen = torch.Generator().manual_seed(11)
    mant = torch.rand(B, Hq, generator=gen) + 1.0                 # full 24-bit significands
    # products of every split term stay normal fp32: |w| >= 2^-60, |V| >= 2^-20
    expo = torch.randint(-60, 3, (B, Hq), generator=gen).float()
    w = (mant * torch.pow(2.0, expo)).to(torch.float32)
    w[0, :4] = torch.tensor([1.0 - 2.0 ** -24, 2.0 ** -50 * (1.0 + 2.0 ** -23), -3.75, 65504.0 + 1.0 / 3.0])
    attn = torch.zeros(B, C, Hq)
    sel = {}
    for b in range(B):
        for q in range(Hq):
            c = (53 * b + 17 * q + 5) % C
            attn[b, c, q] = w[b, q]
            sel[b, q] = c
    V = torch.zeros(B, C, Hkv, D, dtype=torch.bfloat16)
    pw = torch.pow(2.0, torch.randint(-20, 20, (B, C, Hkv, D), generator=gen).float())
    V.copy_(pw.to(torch.bfloat16))
    Vd = V.to(torch.float64).numpy()
    for ns, comb, ht in ((1, "auto", 1), (3, "kernel", 1), (5, "kernel", 1), (1, "auto", 2), (4, "kernel", 2)):
        plan = ga.make_plan(B, C, Hq, Hkv, D, "bf16", "reuse", nsplit=ns, engine="mfma_bf16", combine=comb,
                            kv_tile=ht)
        out = _run(attn, V, plan=plan)
        for (b, q), c in sel.items():
            want = (w[b, q].double().item() * Vd[b, c, q // G]).astype(np.float32)
            assert np.array_equal(out[b, q].astype(np.float32), want), (ns, b, q, w[b, q].item())


def test_deterministic_run_to_run():
    w = WORKLOADS["mqa16-b4-c32768-hq16-hkv1-d128-bf16"]
    attn, V = make_inputs(w, seed=1)
    a, v = attn.to(DEV), V.to(DEV)
    plan = ga.make_plan(w.B, w.C, w.Hq, w.Hkv, w.D, w.v_dtype, nsplit=64)
    outs = [ga.gqa_av_decode(a, v, plan=plan).cpu() for _ in range(3)]
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])


def test_zero_context_writes_zeros():
    B, Hq, Hkv, D = 3, 8, 2, 128
    attn = torch.zeros(B, 0, Hq, device=DEV)
    V = torch.zeros(B, 0, Hkv, D, dtype=torch.bfloat16, device=DEV)
    out = torch.full((B, Hq, D), float("nan"), device=DEV)
    ga.gqa_av_decode(attn, V, out=out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


def test_zero_batch_is_noop():
    attn = torch.zeros(0, 16, 8, device=DEV)
    V = torch.zeros(0, 16, 2, 64, dtype=torch.float16, device=DEV)
    out = ga.gqa_av_decode(attn, V)
    torch.cuda.synchronize()
    assert out.shape == (0, 8, 64)


@pytest.mark.parametrize("B,C,Hq,Hkv,D,dt", [
    (1, 300, 4, 2, 127, "bf16"),     # odd D: 2-byte loads
    (2, 129, 6, 3, 1, "f16"),        # D = 1
    (1, 200, 1, 1, 64, "f32"),       # Hq = Hkv = 1
    (2, 150, 64, 1, 64, "bf16"),     # G = 64: four sub-groups of 16
    (1, 90, 4, 2, 2048, "f32"),      # D-row of 8 KB: two D-tiles
    (3, 257, 10, 5, 80, "f16"),      # D = 80
])
def test_edge_shapes(B, C, Hq, Hkv, D, dt, oracle_lib):
    attn, V = make_random(B, C, Hq, Hkv, D, dt, seed=C + D, attn_kind="softmax")
    ref = oracle_lib.full(attn, V, dt)
    for mode in (["auto", "per_head"] if Hq // Hkv >= 2 else ["auto"]):
        out = _run(attn, V, mode)
        assert_parity(out, ref, dt, C, f"{(B, C, Hq, Hkv, D, dt, mode)}")


@pytest.mark.parametrize("B,C,Hq,Hkv,D,dt,ns", [
    (64, 70, 64, 8, 128, "bf16", 2),     # one thread per quad, two splits
    (64, 1000, 64, 8, 128, "bf16", 7),   # two split groups of at most four
    (455, 40, 9, 3, 129, "f32", 3),      # an output of 528255 floats: not whole quads
])
def test_combine_on_large_outputs(B, C, Hq, Hkv, D, dt, ns, oracle_lib):
    """Outputs of at least 2^19 floats take the combine with one thread per
    quad (or a few split groups), scalar when the output is not whole quads;
    and the same with `out` 4 bytes past a 16-byte boundary (scalar stores)."""
    attn, V = make_random(B, C, Hq, Hkv, D, dt, seed=B + C + ns, attn_kind="signed")
    ref = oracle_lib.full(attn, V, dt)
    assert B * Hq * D >= 2 ** 19
    plan = ga.make_plan(B, C, Hq, Hkv, D, dt, nsplit=ns)
    assert plan.nsplit == ns
    a, v = attn.to(DEV), V.to(DEV)
    out = ga.gqa_av_decode(a, v, plan=plan)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert_parity(got, ref, dt, C, f"{(B, C, Hq, Hkv, D, dt, ns)}")
    lib = ga.load()
    buf = torch.full((B * Hq * D + 1,), float("nan"), device=DEV)
    rc = lib.gqa_av_decode_plan(a.data_ptr(), v.data_ptr(), buf.data_ptr() + 4, B, C, Hq, Hkv, D, ga.DTYPES[dt],
                                ctypes.byref(plan), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0, lib.gqa_av_last_error()
    assert torch.equal(buf[1:].view(B, Hq, D), out), "misaligned out gives the same bits"


def test_misaligned_v_narrows_loads(oracle_lib):
    """V starting 2 bytes past a 16-byte boundary still works (auto plan uses 2-byte loads)."""
    B, C, Hq, Hkv, D = 2, 333, 8, 2, 128
    attn, V = make_random(B, C, Hq, Hkv, D, "bf16", seed=9)
    ref = oracle_lib.full(attn, V, "bf16")
    buf = torch.empty(V.numel() + 8, dtype=torch.bfloat16, device=DEV)
    v_off = buf[1:1 + V.numel()].view(B, C, Hkv, D)
    v_off.copy_(V.to(DEV))
    assert v_off.data_ptr() % 16 == 2
    out = ga.gqa_av_decode(attn.to(DEV), v_off)
    torch.cuda.synchronize()
    assert_parity(out.cpu().numpy().astype(np.float64), ref, "bf16", C, "misaligned V")
    # a forced 16-byte plan on that pointer is refused, not run
    plan = ga.make_plan(B, C, Hq, Hkv, D, "bf16")
    with pytest.raises(ga.GqaAvError) as ei:
        ga.gqa_av_decode(attn.to(DEV), v_off, plan=plan)
    assert ei.value.name == "UNSUPPORTED"


def test_side_stream_and_reuse_of_out(oracle_lib):
    w = WORKLOADS["llama3-8b-b1-c4096-hq32-hkv8-d128-bf16"]
    attn, V = make_inputs(w, seed=3)
    ref = oracle_lib.full(attn, V, w.v_dtype)
    s = torch.cuda.Stream()
    a, v = attn.to(DEV), V.to(DEV)
    out = torch.full((w.B, w.Hq, w.D), 7.0, device=DEV)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        for _ in range(3):
            ga.gqa_av_decode(a, v, out=out)
    s.synchronize()
    assert_parity(out.cpu().numpy().astype(np.float64), ref, w.v_dtype, w.C, "side stream")


def test_bf16_rounded_weights_would_fail_accumulation_bound(oracle_lib):
    """The extra fp32-accumulation check catches what the 2e-3 gate lets through."""
    w = WORKLOADS["g2-b4-c32768-hq16-hkv8-d128-bf16"]
    attn, V = make_inputs(w.replace(B=1), seed=0)
    ref = oracle_lib.full(attn, V, w.v_dtype)
    rounded = attn.to(torch.bfloat16).to(torch.float32)
    out = _run(rounded, V)
    ok, _ = gate(out, ref, w.v_dtype)
    assert ok                                  # the official gate passes it ...
    with pytest.raises(AssertionError):
        assert_parity(out, ref, w.v_dtype, w.C)  # ... the accumulation bound does not


def test_workspace_reuse_across_plans(oracle_lib):
    """Plans of different layouts share one cached workspace: each must add only
    its own split partials, whatever the previous plans wrote there."""
    shapes = [(4, 3000, 64, 8, 128, "bf16", "auto"),     # large workspace first
              (1, 3000, 8, 2, 128, "bf16", "per_head"),  # few tiles, many partials
              (2, 3000, 24, 8, 96, "f16", "per_head"),   # more tiles than the previous call
              (1, 3000, 32, 2, 128, "bf16", "auto"),
              (3, 3000, 12, 4, 64, "f32", "per_head")]
    cases = []
    for k, (B, C, Hq, Hkv, D, dt, mode) in enumerate(shapes):
        attn, V = make_random(B, C, Hq, Hkv, D, dt, seed=300 + k)
        cases.append((attn, V, dt, C, mode, oracle_lib.full(attn, V, dt)))
    for rnd in range(4):
        for attn, V, dt, C, mode, ref in cases:
            plan = ga.make_plan(*attn.shape[:2], attn.shape[2], V.shape[2], V.shape[3], dt, mode,
                                nsplit=9 if rnd % 2 == 0 else 4)
            out = _run(attn, V, plan=plan)
            assert_parity(out, ref, dt, C, f"round {rnd} {tuple(V.shape)} {mode} plan={plan.as_dict()}")


def test_bound_call_matches_decode(oracle_lib):
    w = WORKLOADS["llama3-8b-b1-c4096-hq32-hkv8-d128-bf16"]
    attn, V = make_inputs(w, seed=4)
    ref = oracle_lib.full(attn, V, w.v_dtype)
    a, v = attn.to(DEV), V.to(DEV)
    call = ga.bind(a, v)
    for _ in range(3):
        out = call()
    torch.cuda.synchronize()
    assert_parity(out.cpu().numpy().astype(np.float64), ref, w.v_dtype, w.C, "bound call")
    assert torch.equal(out, ga.gqa_av_decode(a, v))


@pytest.mark.parametrize("G", [5, 6, 7])
@pytest.mark.parametrize("ns", [1, 6])
def test_valu_groups_of_5_to_7(G, ns, oracle_lib):
    """VALU tiles of 5-7 heads with 8 elements per lane: 40-56 accumulators, a
    number that is not a multiple of the 32-slot reduction chunk."""
    B, C, Hkv, D = 2, 700, 2, 256
    attn, V = make_random(B, C, G * Hkv, Hkv, D, "bf16", seed=G)
    ref = oracle_lib.full(attn, V, "bf16")
    plan = ga.make_plan(B, C, G * Hkv, Hkv, D, "bf16", "reuse", engine="valu", nsplit=ns)
    assert plan.heads_per_tile == G
    out = _run(attn, V, plan=plan)
    assert_parity(out, ref, "bf16", C, f"G={G} nsplit={ns}")


@pytest.mark.parametrize("wname", ["g2-b4-c32768-hq16-hkv8-d128-bf16", "mqa16-b4-c32768-hq16-hkv1-d128-bf16",
                                   "tiny-f32-b1-c256-hq8-hkv2-d64"])
def test_split_entry_points_equal_decode(wname):
    """gqa_av_decode_pass1 then gqa_av_decode_combine is exactly gqa_av_decode_plan."""
    w = WORKLOADS[wname]
    attn, V = make_inputs(w, seed=6)
    a, v = attn.to(DEV), V.to(DEV)
    call = ga.bind(a, v)
    whole = call().clone()
    call.out.fill_(float("nan"))
    call.pass1()
    out = call.combine()
    torch.cuda.synchronize()
    assert torch.equal(out, whole)



@pytest.mark.parametrize("wname,ht,engine", [
    ("g2-b4-c32768-hq16-hkv8-d128-bf16", 8, "valu"), ("g2-b4-c32768-hq16-hkv8-d128-bf16", 2, "valu"),
    ("g3-b8-c16384-hq24-hkv8-d96-f16", 4, "valu"), ("llama3-8b-b1-c4096-hq32-hkv8-d128-bf16", 8, "valu"),
    ("g2-b4-c32768-hq16-hkv8-d128-bf16", 4, "mfma_bf16"), ("llama3-8b-b1-c4096-hq32-hkv8-d128-bf16", 2, "mfma_bf16"),
    ("batch64-b64-c8192-hq64-hkv8-d128-bf16", 2, "mfma_bf16"),
])
def test_workload_kv_tiles(wname, ht, engine, oracle_lib):
    """Full-size workloads with several adjacent KV heads per workgroup."""
    w = WORKLOADS[wname]
    attn, V = make_inputs(w, seed=0)
    ref = oracle_lib.full(attn, V, w.v_dtype)
    plan = ga.make_plan(w.B, w.C, w.Hq, w.Hkv, w.D, w.v_dtype, "reuse", engine=engine, kv_tile=ht,
                        cu_count=torch.cuda.get_device_properties(0).multi_processor_count)
    out = _run(attn, V, plan=plan)
    assert_parity(out, ref, w.v_dtype, w.C, f"{wname} kv_tile={ht} plan={plan.as_dict()}")


@pytest.mark.parametrize("B,C,G,Hkv,D", [(2, 1000, 8, 4, 128), (1, 777, 16, 8, 64), (3, 301, 5, 4, 256),
                                         (2, 515, 32, 4, 128), (1, 64, 12, 8, 128), (2, 333, 8, 16, 128)])
@pytest.mark.parametrize("waves", [4, 8])
def test_bf16_engine_kv_tiles_small(B, C, G, Hkv, D, waves, oracle_lib):
    """bf16 matrix engine with 1, 2, 4 and (eight waves) 8 KV heads per
    workgroup, four or eight waves per workgroup, ragged splits, one and
    several splits; 32-head sets at G = 32."""
    Hq = G * Hkv
    attn, V = make_random(B, C, Hq, Hkv, D, "bf16", seed=C + G, attn_kind="softmax")
    ref = oracle_lib.full(attn, V, "bf16")
    for ht in (1, 2, 4) + ((8,) if Hkv % 8 == 0 and waves == 8 else ()):
        for ns, comb in ((1, "auto"), (3, "kernel"), (7, "kernel")):
            plan = ga.make_plan(B, C, Hq, Hkv, D, "bf16", "reuse", engine="mfma_bf16", kv_tile=ht, nsplit=ns,
                                combine=comb, waves=waves)
            assert plan.kv_heads_per_tile == ht and plan.threads == 64 * waves
            out = _run(attn, V, plan=plan)
            assert_parity(out, ref, "bf16", C, f"{(B, C, G, Hkv, D)} kv_tile={ht} ns={ns} waves={waves}")


@pytest.mark.parametrize("wname,ht,ns", [
    ("mqa16-b4-c32768-hq16-hkv1-d128-bf16", 1, 0), ("mqa16-b4-c32768-hq16-hkv1-d128-bf16", 1, 32),
    ("batch64-b64-c8192-hq64-hkv8-d128-bf16", 2, 1), ("batch64-b64-c8192-hq64-hkv8-d128-bf16", 4, 2),
    ("batch64-b64-c8192-hq64-hkv8-d128-bf16", 8, 2), ("batch64-b64-c8192-hq64-hkv8-d128-bf16", 8, 0),
])
def test_workload_eight_waves(wname, ht, ns, oracle_lib):
    """Full-size workloads on the bf16 matrix engine with eight waves per workgroup."""
    w = WORKLOADS[wname]
    _say(f"[parity] {wname} waves=8 kv_tile={ht} nsplit={ns}")
    attn, V = make_inputs(w, seed=0)
    ref = oracle_lib.full(attn, V, w.v_dtype)
    plan = ga.make_plan(w.B, w.C, w.Hq, w.Hkv, w.D, w.v_dtype, "reuse", engine="mfma_bf16", kv_tile=ht, nsplit=ns,
                        waves=8, cu_count=torch.cuda.get_device_properties(0).multi_processor_count)
    assert plan.threads == 512
    out = _run(attn, V, plan=plan)
    assert_parity(out, ref, w.v_dtype, w.C, f"{wname} waves=8 plan={plan.as_dict()}")
