"""HIP graph capture of the bound calls (torch.cuda.CUDAGraph on a side
stream): every entry point enqueues only kernel launches once its split
workspace exists, so a decode loop can capture it. Each graph is replayed
several times with new inputs written in place by eager work between the
replays, and every replay must equal an eager call on the same inputs bit for
bit (same plan, same kernels, fixed summation order). All tests need an
MI355X and are marked ``gpu``.
"""
from __future__ import annotations

import sys

import pytest
import torch

import gqa_reuse_attn_amd as ga
from workloads import make_qk_random, make_scores_random

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REPLAYS = 4


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


def _graph_matches_eager(label, bind, x, fresh):
    """bind(stream) -> a bound call reading x; fresh(k) -> new contents of x."""
    _say(f"[graph] {label}")
    s = torch.cuda.Stream()
    call = bind(s)
    call()                                           # eager: allocates the stream's split workspace
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    torch.cuda.synchronize()
    prev = None
    for k in range(REPLAYS):
        x.copy_(fresh(k))                            # eager work on the default stream
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _out(call).clone()
        call()                                       # the eager call on the same inputs
        s.synchronize()
        assert torch.equal(got, _out(call)), f"{label}: replay {k} differs from the eager call"
        assert torch.isfinite(got).all(), f"{label}: replay {k} not finite"
        if prev is not None:
            assert not torch.equal(got, prev), f"{label}: replay {k} did not see the new inputs"
        prev = got
    del g


def _out(call):
    return call.scores if isinstance(call, ga.BoundQk) else call.out


def _weights(B, C, Hq, Hkv, D, dt, seed, softmax):
    s, V = make_scores_random(B, C, Hq, Hkv, D, dt, seed=seed, score_std=2.0)
    x = s if softmax else torch.softmax(s.double(), dim=1).float()
    return x.contiguous().to(DEV), V.to(DEV)


def _fresh(x, seed):
    g = torch.Generator().manual_seed(seed)

    def f(k):
        return (x.cpu() * (1.0 + 0.25 * torch.rand(x.shape, generator=g))).to(DEV)
    return f


@pytest.mark.parametrize("softmax", [False, True])
@pytest.mark.parametrize("shape,engine,combine,kv_tile", [
    ((2, 3000, 16, 8, 128, "bf16"), "auto", "auto", 0),     # VALU, split kernel combine
    ((2, 3000, 64, 8, 128, "bf16"), "auto", "auto", 0),     # bf16 matrix engine
    ((2, 3000, 64, 8, 128, "bf16"), "mfma_bf16", "auto", 8),  # bf16 matrix engine, eight KV heads, eight waves
    ((2, 3000, 32, 4, 64, "f32"), "mfma", "auto", 0),       # fp32 matrix engine (plain only)
    ((2, 3000, 24, 8, 96, "f16"), "valu", "kernel", 0),     # f16 VALU, G = 3, split kernel combine
    ((1, 100, 8, 2, 64, "bf16"), "auto", "auto", 0),        # one split: a single launch
])
def test_graph_dense(shape, engine, combine, kv_tile, softmax):
    if softmax and engine == "mfma":
        pytest.skip("the fused softmax runs on the VALU or bf16 matrix engine")
    B, C, Hq, Hkv, D, dt = shape
    x, V = _weights(B, C, Hq, Hkv, D, dt, seed=C + Hq, softmax=softmax)
    plan = ga.make_plan(B, C, Hq, Hkv, D, dt, engine=engine, combine=combine, softmax=softmax, kv_tile=kv_tile)
    assert plan.kv_heads_per_tile == kv_tile or kv_tile == 0
    bind = ga.bind_softmax if softmax else ga.bind
    _graph_matches_eager(f"dense {shape} {plan.as_dict()}", lambda s: bind(x, V, plan=plan, stream=s), x,
                         _fresh(x, 1))


@pytest.mark.parametrize("softmax", [False, True])
def test_graph_paged_and_fp8(softmax):
    B, C, Hq, Hkv, D, P = 3, 2048, 64, 8, 128, 16
    x, V = _weights(B, C, Hq, Hkv, D, "bf16", seed=5, softmax=softmax)
    maxp = C // P
    perm = torch.randperm(B * maxp, generator=torch.Generator().manual_seed(2)).to(torch.int32)
    pages = torch.empty((B * maxp, P, Hkv, D), dtype=V.dtype, device=DEV)
    pages[perm.long().to(DEV)] = V.reshape(B * maxp, P, Hkv, D)
    bt = perm.view(B, maxp).contiguous().to(DEV)
    lens = torch.tensor([C, 1500, 7], dtype=torch.int32, device=DEV)
    _graph_matches_eager(f"paged softmax={softmax}",
                         lambda s: ga.bind_paged(x, pages, bt, lens, softmax=softmax, stream=s), x, _fresh(x, 2))
    V8 = (V.float() / V.float().abs().max() * 400.0).to(torch.float8_e4m3fn).contiguous()
    scale = torch.full((Hkv,), 0.5, device=DEV)
    _graph_matches_eager(f"fp8 softmax={softmax}",
                         lambda s: ga.bind_fp8(x, V8, scale, softmax=softmax, stream=s), x, _fresh(x, 3))


@pytest.mark.parametrize("shape", [(2, 3000, 16, 8, 128, "bf16"), (2, 777, 64, 8, 128, "bf16")])
def test_graph_qk(shape):
    B, C, Hq, Hkv, D, dt = shape
    q, K = make_qk_random(B, C, Hq, Hkv, D, dt, seed=4)
    q, K = q.to(DEV), K.to(DEV)
    _graph_matches_eager(f"qk {shape}", lambda s: ga.bind_qk(q, K, scale=D ** -0.5, stream=s), q, _fresh(q, 4))


def test_graph_attention():
    B, C, Hq, Hkv, D = 2, 3000, 64, 8, 128
    q, K = make_qk_random(B, C, Hq, Hkv, D, "bf16", seed=6)
    _, V = make_qk_random(B, C, Hq, Hkv, D, "bf16", seed=7)
    q, K, V = q.to(DEV), K.to(DEV), V.to(DEV)
    _graph_matches_eager("attention", lambda s: ga.BoundAttention(q, K, V, scale=0.125, stream=s), q, _fresh(q, 5))


@pytest.mark.parametrize("fp8", [False, True])
def test_graph_attention_paged(fp8):
    """Paged K and V (16-row pages in shuffled order, ragged lengths), bf16 or
    fp8 with per-KV-head scales, captured and replayed."""
    from tests.test_gpu_attention import _page, _quantize
    B, C, Hq, Hkv, D = 3, 3000, 64, 8, 128
    q, K = make_qk_random(B, C, Hq, Hkv, D, "bf16", seed=8)
    _, V = make_qk_random(B, C, Hq, Hkv, D, "bf16", seed=9)
    ks = vs = None
    if fp8:
        K, ks = _quantize(K)
        V, vs = _quantize(V)
        ks, vs = ks.to(DEV), vs.to(DEV)
    kp, vp, bt = _page(K, V, 16, seed=10)
    lens = torch.tensor([3000, 1234, 17], dtype=torch.int32, device=DEV)
    q, kp, vp, bt = q.to(DEV), kp.to(DEV), vp.to(DEV), bt.to(DEV)
    _graph_matches_eager(f"attention paged fp8={fp8}",
                         lambda s: ga.BoundAttentionPaged(q, kp, vp, bt, lens, scale=0.125, C=C, stream=s,
                                                          k_scale=ks, v_scale=vs), q, _fresh(q, 11))


def test_first_split_call_under_capture_is_refused():
    """A split call whose stream has no workspace yet would have to allocate
    inside the capture: it is refused with UNSUPPORTED, nothing is enqueued,
    and the same call made eagerly afterwards succeeds."""
    B, C, Hq, Hkv, D = 2, 3000, 16, 8, 128
    x, V = _weights(B, C, Hq, Hkv, D, "bf16", seed=17, softmax=False)
    plan = ga.make_plan(B, C, Hq, Hkv, D, "bf16", nsplit=6)
    assert plan.nsplit == 6 and plan.workspace_bytes > 0
    s = torch.cuda.Stream()
    call = ga.bind(x, V, plan=plan, stream=s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        with pytest.raises(ga.GqaAvError) as e:
            call()
    assert e.value.name == "UNSUPPORTED" and "capture" in str(e.value)
    torch.cuda.synchronize()
    call()                                           # eagerly: allocates, then runs
    s.synchronize()
    assert torch.isfinite(call.out).all()
    del g


def test_graph_survives_workspace_growth():
    """A graph captured with a small split plan keeps its workspace address:
    a later, larger plan on the same stream grows the workspace (the old buffer
    is retired, not freed), and replaying the first graph still equals an
    eager call of its plan bit for bit."""
    s = torch.cuda.Stream()
    xs, Vs = _weights(1, 2000, 16, 8, 128, "bf16", seed=21, softmax=False)
    small = ga.bind(xs, Vs, plan=ga.make_plan(1, 2000, 16, 8, 128, "bf16", nsplit=4), stream=s)
    small()
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        small()
    torch.cuda.synchronize()
    xl, Vl = _weights(4, 6000, 64, 8, 128, "bf16", seed=22, softmax=False)
    large = ga.bind(xl, Vl, plan=ga.make_plan(4, 6000, 64, 8, 128, "bf16", nsplit=24), stream=s)
    assert large.plan.workspace_bytes > 4 * small.plan.workspace_bytes
    large()                                          # grows the stream's workspace
    s.synchronize()
    want_large = large.out.clone()
    fresh = _fresh(xs, 3)
    prev = None
    for k in range(REPLAYS):
        xs.copy_(fresh(k))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = small.out.clone()
        small()
        s.synchronize()
        assert torch.equal(got, small.out), f"replay {k} after growth differs from the eager call"
        if prev is not None:
            assert not torch.equal(got, prev)
        prev = got
        large()                                      # interleave the large plan's eager calls
        s.synchronize()
        assert torch.equal(large.out, want_large)
    del g
