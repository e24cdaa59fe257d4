"""CPU tests of the benchmark's host logic: rotation sets come from one
allocation with a bounded number of copies, and the read-ceiling and trial
bookkeeping behave. No GPU needed."""
from __future__ import annotations

import torch

import bench
from workloads import WORKLOADS


def test_every_workload_has_a_bounded_number_of_sets():
    for name, w in WORKLOADS.items():
        n = bench.set_count(w.algorithmic_bytes(), bench.ROTATE_BYTES)
        assert 1 <= n <= bench.MAX_SETS, name
        # past the Infinity Cache unless the cap leaves a small workload resident
        assert n * w.algorithmic_bytes() >= bench.ROTATE_BYTES or n == bench.MAX_SETS, name
    for name in bench.SUITE:
        assert name in WORKLOADS
    assert bench.SUITE[-1] == bench.HEADLINE


def test_set_layout_is_aligned_and_disjoint():
    offs, stride = bench.set_layout([100, 3000, 5, 1])
    assert offs == [0, 256, 3328, 3584]
    assert all(o % 256 == 0 for o in offs) and stride % 4096 == 0 and stride >= offs[-1] + 1


def test_device_sets_are_views_of_one_allocation():
    a = torch.arange(12, dtype=torch.float32).view(3, 4)
    v = torch.arange(30, dtype=torch.int16).to(torch.bfloat16).view(5, 6)
    s = bench.DeviceSets([v, a], [((2, 2), torch.float32)], 5, torch.device("cpu"))
    assert s.nrot == 5 and len(s.sets) == 5
    base = s.buf.untyped_storage().data_ptr()
    for i, (vv, aa, oo) in enumerate(s.sets):
        # every tensor lives inside set i's slice of the one buffer
        for t in (vv, aa, oo):
            assert t.untyped_storage().data_ptr() == base
            off = t.data_ptr() - base
            assert i * s.stride <= off < (i + 1) * s.stride
            assert off % 256 == 0
        assert torch.equal(vv, v) and torch.equal(aa, a)
        assert oo.shape == (2, 2) and oo.dtype == torch.float32
    assert s.base(3).numel() == s.stride


def test_stream_read_rejects_bad_arguments_before_launch():
    import gqa_reuse_attn_amd as ga
    lib = ga.load()
    # NULL source, unaligned sizes, bad load counts: INVALID_ARG, nothing launched
    assert lib.gqa_bench_stream_read(None, 1024, 8, 4, 0, None, None) == 1
    assert lib.gqa_bench_stream_read(16, 1000, 8, 4, 0, 16, None) == 1
    assert lib.gqa_bench_stream_read(16, 1024, 0, 4, 0, 16, None) == 1
    assert lib.gqa_bench_stream_read(16, 1024, 8, 3, 0, 16, None) == 1
    assert lib.gqa_bench_stream_read(16, 1024, 8, 4, 2, 16, None) == 1    # unknown pattern
    assert lib.gqa_bench_stream_read(16, 1 << 40, 1, 4, 0, 16, None) == 1   # slice past 2^31
    assert b"2^31" in lib.gqa_av_last_error()


def test_parse_defaults_run_the_suite():
    a = bench.parse([])
    assert a.workload is None and a.ramp_seconds >= 0.25 and a.gpus == 1
    a = bench.parse(["--gpus", "1", "--steps", "20", "--warmup", "5"])
    assert (a.steps, a.warmup) == (20, 5)


def test_dominant_kernel_patterns_pick_the_right_kernel():
    """The traffic summaries key each operation's dominant kernel by a name
    pattern; a fused-attention bench also runs the unfused pair (score step,
    then the fused softmax kernel), so the attention pattern must take only
    the kernel whose QK template argument (the eighth) is true, whatever
    follows it."""
    import re
    attn = bench.OPS["attn"][1]
    fused = "void gqa_av::av_pass1_mfma_bf16<16, 1, 1, 4, true, 2, false, true, 4>(gqa_av::Pass1Args)"
    fused_paged_fp8 = "void gqa_av::av_pass1_mfma_bf16<16, 1, 1, 2, true, 3, true, true, 4>(gqa_av::Pass1Args)"
    softmax_only = "void gqa_av::av_pass1_mfma_bf16<16, 1, 1, 4, true, 2, false, false, 4>(gqa_av::Pass1Args)"
    scores = "void gqa_av::qk_scores<2, 4, 1, 4, true>(gqa_av::QkArgs)"
    assert re.search(attn, fused) and re.search(attn, fused_paged_fp8)
    assert not re.search(attn, softmax_only) and not re.search(attn, scores)
    assert re.search(bench.OPS["qk"][1], scores) and not re.search(bench.OPS["qk"][1], fused)
    for op in ("av", "softmax"):
        assert re.search(bench.OPS[op][1], softmax_only)
        assert re.search(bench.OPS[op][1], "void gqa_av::av_pass1_valu<2, 16, 2, 4, false, false>(gqa_av::Pass1Args)")
