"""Concurrent use of the library: host threads calling the C ABI at the same
time, each on its own stream (the ctypes calls release the GIL, so the calls
really overlap). Each stream has its own split workspace and the workspace
cache is shared under a mutex. Every result must equal the same call made
alone, bit for bit. All tests need an MI355X and are marked ``gpu``.
"""
from __future__ import annotations

import sys
import threading

import pytest
import torch

import gqa_reuse_attn_amd as ga
from workloads import make_qk_random, make_scores_random

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CALLS = 40


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


def _problems():
    """Several products with split workspaces of different sizes."""
    out = []
    s, V = make_scores_random(2, 8192, 16, 8, 128, "bf16", seed=1)
    a = torch.softmax(s.double(), dim=1).float().contiguous()
    out.append(("av G=2", lambda st, a=a.to(DEV), V=V.to(DEV): ga.bind(a, V, stream=st)))
    s, V = make_scores_random(3, 6000, 64, 8, 128, "bf16", seed=2)
    out.append(("softmax G=8", lambda st, s=s.to(DEV), V=V.to(DEV): ga.bind_softmax(s, V, stream=st)))
    s, V = make_scores_random(2, 5000, 24, 8, 96, "f16", seed=3)
    out.append(("softmax G=3 f16", lambda st, s=s.to(DEV), V=V.to(DEV): ga.bind_softmax(s, V, stream=st)))
    q, K = make_qk_random(2, 7000, 32, 8, 128, "bf16", seed=4)
    out.append(("qk G=4", lambda st, q=q.to(DEV), K=K.to(DEV): ga.bind_qk(q, K, scale=0.125, stream=st)))
    q, K = make_qk_random(2, 5000, 64, 8, 128, "bf16", seed=5)
    _, V = make_qk_random(2, 5000, 64, 8, 128, "bf16", seed=6)
    out.append(("attention G=8", lambda st, q=q.to(DEV), K=K.to(DEV), V=V.to(DEV):
                ga.BoundAttention(q, K, V, scale=0.125, stream=st)))
    return out


def _result(call):
    return call.scores if isinstance(call, ga.BoundQk) else call.out


def test_threads_on_own_streams_match_single_calls():
    probs = _problems()
    # Each problem alone, on a stream of its own.
    ref = []
    for name, bind in probs:
        st = torch.cuda.Stream()
        call = bind(st)
        call()
        st.synchronize()
        ref.append(_result(call).clone())
    # All at once: one host thread and one stream per problem, CALLS calls each.
    calls = [bind(torch.cuda.Stream()) for _, bind in probs]
    errors = []
    start = threading.Barrier(len(calls))

    def work(i):
        try:
            start.wait()
            for _ in range(CALLS):
                calls[i]()
        except Exception as e:                       # reported after the join
            errors.append((probs[i][0], repr(e)))

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(calls))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for (name, _), call, r in zip(probs, calls, ref):
        _say(f"[concurrency] {name}")
        assert torch.equal(_result(call), r), f"{name}: concurrent result differs from the single call"
