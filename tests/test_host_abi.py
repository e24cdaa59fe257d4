"""CPU tests of the C ABI: the library loads, exports what the header declares,
and its host-only logic (mode resolution, planning, argument checks) behaves.
No kernel is launched here.
"""
from __future__ import annotations

import ctypes
import glob
import os
import re
import threading

import pytest

import gqa_reuse_attn_amd as ga
from workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa_av.h")


def declared_functions():
    """Every function declared in include/*.h (comments stripped)."""
    names = set()
    for h in sorted(glob.glob(os.path.join(os.path.dirname(HEADER), "*.h"))):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(gqa_\w+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_function():
    lib = ga.load()
    names = declared_functions()
    assert len(names) >= 10, names
    assert {"gqa_qk_decode", "gqa_qk_decode_plan", "gqa_qk_make_plan"} <= set(names)
    assert {"gqa_softmax_av_decode", "gqa_softmax_av_decode_plan"} <= set(names)
    assert {"gqa_av_paged_decode", "gqa_av_paged_decode_plan"} <= set(names)
    assert {"gqa_av_fp8_decode", "gqa_av_fp8_decode_plan"} <= set(names)
    assert {"gqa_attention_decode", "gqa_attention_paged_decode_plan", "gqa_bench_stream_read"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"


def test_exports_are_c_symbols():
    # extern "C": no mangled gqa_av names in the dynamic symbol table
    out = os.popen(f"nm -D --defined-only {ga.LIB_PATH}").read()
    exported = set(re.findall(r"\s(gqa_\w+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


@pytest.mark.parametrize("Hq,Hkv,mode,expect", [
    (32, 8, "auto", "reuse"),          # Llama-style G=4
    (24, 8, "auto", "reuse"),          # G=3
    (16, 8, "auto", "reuse"),          # G=2
    (16, 1, "auto", "reuse"),          # MQA G=16: the page's cap of 8 is not kept
    (64, 1, "auto", "reuse"),          # G=64
    (8, 1, "auto", "reuse"),           # low-ratio MQA
    (8, 8, "auto", "per_head"),        # MHA
    (1, 1, "auto", "per_head"),
    (32, 8, "per_head", "per_head"),   # forced per-head always runs
    (8, 8, "per_head", "per_head"),
    (32, 8, "reuse", "reuse"),
])
def test_resolve_mode(Hq, Hkv, mode, expect):
    assert ga.resolve_mode(Hq, Hkv, mode) == expect


@pytest.mark.parametrize("Hq,Hkv,mode,status", [
    (8, 8, "reuse", "INELIGIBLE"),     # forced reuse with G = 1
    (1, 1, "reuse", "INELIGIBLE"),
    (12, 8, "auto", "INVALID_ARG"),    # not divisible
    (12, 8, "per_head", "INVALID_ARG"),
    (0, 1, "auto", "INVALID_ARG"),
    (8, 0, "auto", "INVALID_ARG"),
    (8, 2, 5, "INVALID_ARG"),          # unknown mode
    (8, 2, -2, "INVALID_ARG"),
])
def test_resolve_mode_errors(Hq, Hkv, mode, status):
    with pytest.raises(ga.GqaAvError) as ei:
        ga.resolve_mode(Hq, Hkv, mode)
    assert ei.value.name == status
    assert str(ei.value)


def _check_plan(p, B, C, Hq, Hkv, D, v_dtype, mode):
    es = 4 if v_dtype == "f32" else 2
    G = Hq // Hkv
    assert p.threads == 256 or (p.threads == 512 and p.engine == 3)
    if p.engine == 2:                                   # MFMA: 16 lanes x D/16 elements per row
        assert p.mode == 1 and D % 16 == 0
        assert p.vec_bytes == D // 16 * es and p.lanes_per_row == 16 and p.row_slots == 16 and p.d_tiles == 1
        assert p.heads_per_tile in (16, 32)
        tile_out = p.heads_per_tile * D
    elif p.engine == 3:                                 # bf16 MFMA: 16-byte pieces, 32-row chunk per wave
        ht = p.kv_heads_per_tile
        assert p.mode == 1 and v_dtype == "bf16" and D in (64, 128, 256) and ht in (1, 2, 4, 8) and Hkv % ht == 0
        assert p.vec_bytes == 16 and p.lanes_per_row == ht * D // 8 and p.d_tiles == 1
        assert p.row_slots == 32 * (p.threads // 64) // ht
        # automatic: eight waves for the plain product with one KV head per
        # workgroup, and with eight (a wave per KV head)
        assert p.threads == 256 or (ht == 1 and not p.softmax) or ht == 8
        assert ht != 8 or (p.threads == 512 and not p.attention)
        assert p.heads_per_tile in (16, 32) and p.heads_per_tile * D <= 4096
        tile_out = ht * p.heads_per_tile * D
    else:
        assert p.vec_bytes in (16, 8, 4, 2) and (D * es) % p.vec_bytes == 0 and p.vec_bytes >= es
        L = D * es // p.vec_bytes
        ht = p.kv_heads_per_tile
        if ht > 1:
            assert p.lanes_per_row == ht * L <= 256 and p.d_tiles == 1 and Hkv % ht == 0
        else:
            assert p.lanes_per_row == min(L, 256)
            assert p.d_tiles == -(-L // p.lanes_per_row)
        assert p.row_slots == min(256 // p.lanes_per_row, 64)
        tile_out = p.heads_per_tile * (p.vec_bytes // es) * p.lanes_per_row
    if C == 0:
        assert p.nsplit == 1
    else:
        assert p.nsplit >= 1 and p.rows_per_split >= 1
        if p.interleave:                                   # blocks of one step, at least one per split
            assert p.nsplit >= 2 and p.page_size == 0 and p.nsplit <= -(-C // p.rows_per_split)
        else:
            assert -(-C // p.rows_per_split) == p.nsplit   # splits tile [0, C) exactly
    if p.mode == 1:
        assert p.heads_per_tile >= min(G, 8) and (p.engine in (2, 3) or p.heads_per_tile <= Hq)
        assert p.subgroups == -(-G // p.heads_per_tile)
        tiles = B * (Hkv // p.kv_heads_per_tile) * p.subgroups * p.d_tiles
        assert p.v_bytes_read == B * C * Hkv * D * es * p.subgroups
    else:
        assert p.heads_per_tile == 1
        tiles = B * Hq * p.d_tiles
        assert p.v_bytes_read == B * C * Hkv * D * es * G
    assert p.grid == tiles * p.nsplit
    if p.nsplit == 1:
        assert p.combine == 0 and p.workspace_bytes == 0
    else:
        assert p.combine == 1 and p.workspace_bytes == p.nsplit * B * Hq * D * 4


@pytest.mark.parametrize("wname", list(WORKLOADS))
@pytest.mark.parametrize("mode", ["auto", "per_head"])
def test_plan_for_workloads(wname, mode):
    w = WORKLOADS[wname]
    p = ga.make_plan(w.B, w.C, w.Hq, w.Hkv, w.D, w.v_dtype, mode)
    _check_plan(p, w.B, w.C, w.Hq, w.Hkv, w.D, w.v_dtype, mode)
    assert p.vec_bytes == 16                         # every decode workload allows 16-byte loads
    if mode == "auto":
        assert p.mode == 1                           # all six have G >= 2
        assert p.v_bytes_read == w.v_bytes()         # V read once
    else:
        assert p.v_bytes_read == w.G * w.v_bytes()


@pytest.mark.parametrize("B,C,Hq,Hkv,D,dt", [
    (1, 1, 1, 1, 1, "bf16"), (2, 0, 4, 2, 8, "f16"), (0, 10, 4, 2, 8, "f32"), (3, 1000, 40, 2, 96, "bf16"),
    (1, 77, 17, 1, 3, "f16"), (2, 65, 9, 3, 2000, "f32"), (1, 5000, 64, 2, 256, "bf16"), (4, 3, 6, 6, 5, "f32"),
])
def test_plan_edges(B, C, Hq, Hkv, D, dt):
    for mode in ("auto", "per_head"):
        p = ga.make_plan(B, C, Hq, Hkv, D, dt, mode)
        _check_plan(p, B, C, Hq, Hkv, D, dt, mode)


@pytest.mark.parametrize("nsplit", [1, 2, 7, 64, 10 ** 6])
def test_forced_nsplit(nsplit):
    C = 1000
    p = ga.make_plan(2, C, 8, 2, 128, "bf16", "auto", nsplit=nsplit, split_order="contiguous")
    assert p.nsplit <= min(nsplit, C) and p.interleave == 0
    assert -(-C // p.rows_per_split) == p.nsplit
    if nsplit <= 64:
        assert p.nsplit == nsplit or C % nsplit != 0
    q = ga.make_plan(2, C, 8, 2, 128, "bf16", "auto", nsplit=nsplit)     # interleaved blocks of one step (64 rows)
    assert q.interleave == (q.nsplit > 1)
    if q.interleave:
        assert q.rows_per_split == 64 and q.nsplit == min(p.nsplit, -(-C // 64))
    else:
        assert q.nsplit == 1 and q.rows_per_split == C


def test_alignment_narrows_loads():
    assert ga.make_plan(1, 64, 8, 2, 128, "bf16", v_align=16).vec_bytes == 16
    assert ga.make_plan(1, 64, 8, 2, 128, "bf16", v_align=8).vec_bytes == 8
    assert ga.make_plan(1, 64, 8, 2, 128, "bf16", v_align=2).vec_bytes == 2
    assert ga.make_plan(1, 64, 8, 2, 127, "bf16").vec_bytes == 2     # odd D
    assert ga.make_plan(1, 64, 8, 2, 6, "bf16").vec_bytes == 4       # 12-byte rows
    assert ga.make_plan(1, 64, 8, 2, 3, "f32").vec_bytes == 4
    with pytest.raises(ga.GqaAvError) as ei:
        ga.make_plan(1, 64, 8, 2, 64, "f32", v_align=2)
    assert ei.value.name == "UNSUPPORTED"


def test_large_groups_use_subgroups():
    p = ga.make_plan(1, 4096, 40, 1, 128, "bf16", engine="valu")
    assert p.mode == 1 and p.heads_per_tile == 16 and p.subgroups == 3
    p = ga.make_plan(1, 4096, 40, 1, 128, "bf16")
    assert p.mode == 1 and p.engine == 3 and p.heads_per_tile == 32 and p.subgroups == 2
    p = ga.make_plan(1, 4096, 40, 1, 128, "f16")
    assert p.mode == 1 and p.engine == 2 and p.heads_per_tile == 32 and p.subgroups == 2


@pytest.mark.parametrize("args,status", [
    ((-1, 4, 8, 2, 16, "bf16"), "INVALID_ARG"),
    ((1, -4, 8, 2, 16, "bf16"), "INVALID_ARG"),
    ((1, 4, 8, 2, 0, "bf16"), "INVALID_ARG"),
    ((1, 4, 9, 2, 16, "bf16"), "INVALID_ARG"),
])
def test_plan_errors(args, status):
    with pytest.raises(ga.GqaAvError) as ei:
        ga.make_plan(*args)
    assert ei.value.name == status


def test_unknown_dtype_and_engine():
    lib = ga.load()
    p = ga.Plan()
    assert lib.gqa_av_make_plan(1, 4, 8, 2, 16, 7, -1, None, ctypes.byref(p)) == 1
    h = ga.Hint(); h.engine = 9
    assert lib.gqa_av_make_plan(1, 4, 8, 2, 16, 2, -1, ctypes.byref(h), ctypes.byref(p)) == 1


def test_decode_plan_rejects_before_launch():
    """Argument errors are returned before any HIP call (so this runs without a GPU)."""
    lib = ga.load()
    B, C, Hq, Hkv, D = 2, 100, 8, 2, 128
    p = ga.make_plan(B, C, Hq, Hkv, D, "bf16")
    fake = ctypes.c_void_p(1 << 20)
    # a plan for another problem
    assert lib.gqa_av_decode_plan(fake, fake, fake, B, C + 5000, Hq, Hkv, D, 2, ctypes.byref(p), None) == 1
    bad = ga.Plan.from_buffer_copy(p); bad.grid += 1
    assert lib.gqa_av_decode_plan(fake, fake, fake, B, C, Hq, Hkv, D, 2, ctypes.byref(bad), None) == 1
    bad = ga.Plan.from_buffer_copy(p); bad.rows_per_split = 1
    assert lib.gqa_av_decode_plan(fake, fake, fake, B, C, Hq, Hkv, D, 2, ctypes.byref(bad), None) == 1
    # null and misaligned pointers
    assert lib.gqa_av_decode_plan(None, fake, fake, B, C, Hq, Hkv, D, 2, ctypes.byref(p), None) == 1
    assert lib.gqa_av_decode_plan(fake, fake, None, B, C, Hq, Hkv, D, 2, ctypes.byref(p), None) == 1
    odd = ctypes.c_void_p((1 << 20) + 2)
    assert lib.gqa_av_decode_plan(odd, fake, fake, B, C, Hq, Hkv, D, 2, ctypes.byref(p), None) == 1
    assert lib.gqa_av_decode_plan(fake, odd, fake, B, C, Hq, Hkv, D, 2, ctypes.byref(p), None) == 3
    assert "aligned" in ga.load().gqa_av_last_error().decode()
    # B == 0 is a no-op that needs no device
    p0 = ga.make_plan(0, C, Hq, Hkv, D, "bf16")
    assert lib.gqa_av_decode_plan(None, None, None, 0, C, Hq, Hkv, D, 2, ctypes.byref(p0), None) == 0
    assert lib.gqa_av_decode_plan(fake, fake, fake, B, C, Hq, Hkv, D, 2, None, None) == 1


def test_status_strings():
    for s in range(5):
        assert ga.status_string(s)
    assert ga.status_string(99) == "unknown status"


def test_product_path_does_not_touch_the_oracle():
    pkg = os.path.join(ROOT, "gqa_reuse_attn_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, flags=re.M), f
                assert "gqa_av_oracle" not in text, f
    deps = os.popen(f"ldd {ga.LIB_PATH} 2>/dev/null").read()
    assert "oracle" not in deps


@pytest.mark.parametrize("wname,engine", [
    ("tiny-f32-b1-c256-hq8-hkv2-d64", 1), ("llama3-8b-b1-c4096-hq32-hkv8-d128-bf16", 1),
    ("g3-b8-c16384-hq24-hkv8-d96-f16", 1), ("g2-b4-c32768-hq16-hkv8-d128-bf16", 1),
    ("mqa16-b4-c32768-hq16-hkv1-d128-bf16", 3), ("batch64-b64-c8192-hq64-hkv8-d128-bf16", 3),
])
def test_auto_engine(wname, engine):
    """Groups of 5 or more heads take a matrix-core engine (bf16 V: the bf16 one),
    smaller ones the VALU engine."""
    w = WORKLOADS[wname]
    assert ga.make_plan(w.B, w.C, w.Hq, w.Hkv, w.D, w.v_dtype).engine == engine
    assert ga.make_plan(w.B, w.C, w.Hq, w.Hkv, w.D, w.v_dtype, "per_head").engine == 1


def test_forced_engines():
    p = ga.make_plan(1, 300, 4, 2, 128, "bf16", engine="mfma")          # G = 2 on MFMA: allowed
    assert p.engine == 2 and p.heads_per_tile == 16 and p.subgroups == 1
    _check_plan(p, 1, 300, 4, 2, 128, "bf16", "auto")
    p = ga.make_plan(1, 300, 64, 1, 128, "bf16")                        # G = 64: 32-head sets
    assert p.engine == 3 and p.heads_per_tile == 32 and p.subgroups == 2
    p = ga.make_plan(1, 300, 64, 1, 256, "bf16")                        # D = 256: 16-head sets
    assert p.engine == 3 and p.heads_per_tile == 16 and p.subgroups == 4
    p = ga.make_plan(1, 300, 64, 1, 128, "f16")                         # fp16 V: the fp32 matrix engine
    assert p.engine == 2 and p.heads_per_tile == 32 and p.subgroups == 2
    p = ga.make_plan(1, 300, 64, 1, 256, "bf16", engine="mfma")
    assert p.engine == 2 and p.heads_per_tile == 16 and p.subgroups == 4
    p = ga.make_plan(1, 300, 4, 2, 64, "bf16", engine="mfma_bf16")      # G = 2 on the bf16 engine: allowed
    assert p.engine == 3 and p.heads_per_tile == 16 and p.subgroups == 1
    _check_plan(p, 1, 300, 4, 2, 64, "bf16", "auto")
    for args, kw in [((1, 300, 16, 1, 96, "bf16"), {}), ((1, 300, 16, 1, 128, "f16"), {}),
                     ((1, 300, 16, 1, 128, "bf16", "per_head"), {}), ((1, 300, 16, 1, 128, "bf16"), {"v_align": 8}),
                     ((1, 300, 16, 1, 512, "bf16"), {})]:
        with pytest.raises(ga.GqaAvError) as ei:
            ga.make_plan(*args, engine="mfma_bf16", **kw)
        assert ei.value.name == "UNSUPPORTED"
    # shapes the bf16 engine cannot take go to the fp32 matrix engine
    assert ga.make_plan(1, 300, 16, 1, 96, "bf16").engine == 2
    assert ga.make_plan(1, 300, 16, 1, 128, "bf16", engine="valu").engine == 1
    for args, kw in [((1, 300, 16, 1, 127, "bf16"), {}), ((1, 300, 16, 1, 128, "bf16", "per_head"), {}),
                     ((1, 300, 16, 1, 96, "f32"), {}), ((1, 300, 16, 1, 128, "bf16"), {"v_align": 8})]:
        with pytest.raises(ga.GqaAvError) as ei:
            ga.make_plan(*args, engine="mfma", **kw)
        assert ei.value.name == "UNSUPPORTED"
    # without the engine forced, shapes the MFMA engine cannot take fall back to VALU
    assert ga.make_plan(1, 300, 16, 1, 127, "bf16").engine == 1
    assert ga.make_plan(1, 300, 16, 1, 128, "bf16", v_align=8).engine == 1


@pytest.mark.parametrize("combine", ["auto", "kernel"])
def test_forced_combine(combine):
    p = ga.make_plan(2, 5000, 16, 8, 128, "bf16", combine=combine, nsplit=9)
    assert p.nsplit == 9 and p.combine == 1
    _check_plan(p, 2, 5000, 16, 8, 128, "bf16", "auto")
    p1 = ga.make_plan(2, 5000, 16, 8, 128, "bf16", combine=combine, nsplit=1)
    assert p1.nsplit == 1 and p1.combine == 0 and p1.workspace_bytes == 0


def test_removed_last_workgroup_combine_is_refused():
    """The in-kernel (last arriving workgroup) combine measured slower than the
    second kernel on every workload and is gone: its old value 2 is refused."""
    lib = ga.load()
    h, p = ga.Hint(), ga.Plan()
    h.combine, h.nsplit = 2, 9
    assert lib.gqa_av_make_plan(2, 5000, 16, 8, 128, 2, -1, ctypes.byref(h), ctypes.byref(p)) == 1
    assert b"combine" in lib.gqa_av_last_error()


def test_zeroed_hint_means_automatic():
    lib = ga.load()
    h, p, q = ga.Hint(), ga.Plan(), ga.Plan()
    assert lib.gqa_av_make_plan(4, 32768, 16, 1, 128, 2, -1, ctypes.byref(h), ctypes.byref(p)) == 0
    assert lib.gqa_av_make_plan(4, 32768, 16, 1, 128, 2, -1, None, ctypes.byref(q)) == 0
    assert p.as_dict() == q.as_dict() and p.engine == 3
    h.combine = 3
    assert lib.gqa_av_make_plan(4, 32768, 16, 1, 128, 2, -1, ctypes.byref(h), ctypes.byref(p)) == 1


def test_kv_tile():
    p = ga.make_plan(4, 32768, 16, 8, 128, "bf16", kv_tile=8)
    assert p.kv_heads_per_tile == 8 and p.lanes_per_row == 128 and p.row_slots == 2
    _check_plan(p, 4, 32768, 16, 8, 128, "bf16", "auto")
    p = ga.make_plan(8, 16384, 24, 8, 96, "f16", kv_tile=4)
    assert p.kv_heads_per_tile == 4 and p.lanes_per_row == 48 and p.row_slots == 5
    _check_plan(p, 8, 16384, 24, 8, 96, "f16", "auto")
    assert ga.make_plan(4, 100, 16, 8, 128, "bf16").kv_heads_per_tile >= 1
    for kw, status in [(dict(kv_tile=3), "INVALID_ARG"),                      # does not divide Hkv
                       (dict(kv_tile=2, mode="per_head"), "UNSUPPORTED"),
                       (dict(kv_tile=2, engine="mfma"), "UNSUPPORTED"),
                       (dict(kv_tile=8, attention=True), "UNSUPPORTED"),                  # not fused attention
                       (dict(kv_tile=8, engine="valu", softmax=True), "UNSUPPORTED"),     # VALU softmax: up to 4
                       (dict(kv_tile=8, engine="mfma_bf16", waves=4), "UNSUPPORTED")]:     # a wave per KV head
        with pytest.raises(ga.GqaAvError) as ei:
            ga.make_plan(4, 100, 16, 8, 128, "bf16", **kw)
        assert ei.value.name == status
    with pytest.raises(ga.GqaAvError) as ei:                                 # 32 x 16 lanes > 256
        ga.make_plan(1, 100, 64, 32, 128, "bf16", kv_tile=32, engine="valu")
    assert ei.value.name == "UNSUPPORTED"


def test_eight_kv_heads_rule():
    """The bf16 matrix engine takes eight KV heads per workgroup on its own
    only for bf16 V at G = 8 (D <= 128; the fused softmax D = 128) while
    the grid fills with at most 8 splits of at least 1024 rows; otherwise
    four (or fewer)."""
    def ht(B, C, Hq, Hkv, D, dt="bf16", **kw):
        p = ga.make_plan(B, C, Hq, Hkv, D, dt, engine="mfma_bf16", cu_count=256, **kw)
        if not kw.get("softmax"):
            _check_plan(p, B, C, Hq, Hkv, D, "bf16", "auto")
        return p.kv_heads_per_tile, p.threads, p.nsplit
    assert ht(64, 8192, 64, 8, 128) == (8, 512, 4)
    assert ht(64, 8192, 64, 8, 64) == (8, 512, 4)
    assert ht(32, 8192, 128, 16, 128) == (8, 512, 4)
    assert ht(64, 8192, 64, 8, 128, page_size=16) == (8, 512, 4)
    assert ht(64, 8192, 64, 8, 128, softmax=True) == (8, 512, 4)           # fused softmax
    assert ht(64, 8192, 64, 8, 64, softmax=True)[0] == 4                   # fused softmax, D = 64
    assert ht(16, 16384, 64, 8, 128)[0] == 4                               # 16 splits needed
    assert ht(32, 8192, 64, 8, 128) == (8, 512, 8)
    p = ga.make_plan(64, 8192, 64, 8, 128, "bf16", attention=True, cu_count=256)
    assert p.kv_heads_per_tile <= 4                                        # fused attention
    assert ht(64, 8192, 64, 8, 128, waves=4)[0] == 4                       # four waves asked for
    assert ht(64, 8192, 64, 8, 256)[0] == 4                                # D = 256
    assert ht(4, 32768, 64, 8, 128)[0] == 4                                # splits would be 512 rows
    for Hq in (32, 40, 48, 128):                                           # G = 4, 5, 6, 16
        assert ht(64, 8192, Hq, 8, 128)[0] == 4
    p = ga.make_plan(64, 8192, 64, 8, 128, "fp8", engine="mfma_bf16", cu_count=256)
    assert p.kv_heads_per_tile < 8                                         # fp8 V


def test_bf16_engine_keeps_split_spans_small():
    """The bf16 matrix engine reads a split through 32-bit buffer offsets: a split's
    rows of V stay under 1 GB, with more splits than asked for if need be."""
    p = ga.make_plan(1, 10_000_000, 16, 1, 128, "bf16", engine="mfma_bf16", nsplit=1)
    assert p.engine == 3 and p.nsplit == 3 and p.rows_per_split * 256 <= 2 ** 30
    _check_plan(p, 1, 10_000_000, 16, 1, 128, "bf16", "auto")
    # rows of V beyond 1 MB are not taken by this engine
    assert ga.make_plan(1, 100, 16 * 8192, 8192, 128, "bf16").engine != 3


def test_qk_plans():
    """Score-step planning: engine by K dtype, tiles per head group, row blocks."""
    p = ga.qk_make_plan(4, 32768, 16, 8, 128, "bf16")
    assert p.mode == 1 and p.engine == 3 and p.heads_per_tile == 16 and p.subgroups == 1
    assert p.kv_heads_per_tile == 4                                   # widest tile that still fills the GPU
    assert p.rows_per_block % 64 == 0 and p.grid == 4 * 2 * -(-32768 // p.rows_per_block)
    assert ga.qk_make_plan(4, 32768, 16, 1, 128, "bf16").kv_heads_per_tile == 1
    assert ga.qk_make_plan(4, 32768, 16, 8, 128, "bf16", kv_tile=2).kv_heads_per_tile == 2
    for kw in (dict(kv_tile=3), dict(kv_tile=8), dict(kv_tile=2, mode="per_head")):
        with pytest.raises(ga.GqaAvError):
            ga.qk_make_plan(4, 32768, 16, 8, 128, "bf16", **kw)
    assert p.k_bytes_read == 4 * 32768 * 8 * 128 * 2
    p = ga.qk_make_plan(4, 32768, 16, 8, 128, "bf16", "per_head")
    assert p.mode == 0 and p.heads_per_tile == 1 and p.k_bytes_read == 2 * 4 * 32768 * 8 * 128 * 2
    assert p.kv_heads_per_tile == 1
    assert ga.qk_make_plan(8, 16384, 24, 8, 96, "f16").engine == 3                # 16-bit matrix path
    assert ga.qk_make_plan(1, 256, 8, 2, 64, "f32").engine == 2
    p = ga.qk_make_plan(1, 300, 40, 1, 128, "bf16")                 # G = 40: 32-head sets
    assert p.heads_per_tile == 32 and p.subgroups == 2
    p = ga.qk_make_plan(1, 300, 40, 1, 256, "bf16")                 # D = 256: 16-head sets
    assert p.heads_per_tile == 16 and p.subgroups == 3
    assert ga.qk_make_plan(2, 1000, 8, 2, 64, "bf16", rows_per_block=100).rows_per_block == 128
    for args in [(1, 10, 8, 2, 48, "bf16"), (1, 10, 8, 2, 288, "bf16")]:
        with pytest.raises(ga.GqaAvError) as ei:
            ga.qk_make_plan(*args)
        assert ei.value.name == "UNSUPPORTED"
    with pytest.raises(ga.GqaAvError) as ei:
        ga.qk_make_plan(1, 10, 9, 2, 64, "bf16")
    assert ei.value.name == "INVALID_ARG"
    with pytest.raises(ga.GqaAvError) as ei:
        ga.qk_make_plan(1, 10, 4, 4, 64, "bf16", "reuse")
    assert ei.value.name == "INELIGIBLE"


def test_qk_decode_plan_rejects_before_launch():
    lib = ga.load()
    p = ga.qk_make_plan(2, 100, 8, 2, 64, "bf16")
    fake = ctypes.c_void_p(1 << 20)
    assert lib.gqa_qk_decode_plan(fake, fake, fake, 2, 5000, 8, 2, 64, 2, ctypes.c_float(1.0), ctypes.byref(p), None) == 1
    assert lib.gqa_qk_decode_plan(None, fake, fake, 2, 100, 8, 2, 64, 2, ctypes.c_float(1.0), ctypes.byref(p), None) == 1
    odd = ctypes.c_void_p((1 << 20) + 2)
    assert lib.gqa_qk_decode_plan(fake, odd, fake, 2, 100, 8, 2, 64, 2, ctypes.c_float(1.0), ctypes.byref(p), None) == 3
    assert lib.gqa_qk_decode_plan(odd, fake, fake, 2, 100, 8, 2, 64, 2, ctypes.c_float(1.0), ctypes.byref(p), None) == 1
    p0 = ga.qk_make_plan(0, 100, 8, 2, 64, "bf16")
    assert lib.gqa_qk_decode_plan(None, None, None, 0, 100, 8, 2, 64, 2, ctypes.c_float(1.0), ctypes.byref(p0), None) == 0


@pytest.mark.parametrize("wname", list(WORKLOADS))
def test_softmax_plans(wname):
    """Fused softmax plans: the VALU or bf16 matrix engine, the kernel combine,
    and a workspace with one (maximum, weight sum) pair per split and (b, q_h)."""
    w = WORKLOADS[wname]
    for mode in ("auto", "per_head"):
        p = ga.make_plan(w.B, w.C, w.Hq, w.Hkv, w.D, w.v_dtype, mode, softmax=True)
        q = ga.make_plan(w.B, w.C, w.Hq, w.Hkv, w.D, w.v_dtype, mode)
        assert p.softmax == 1 and q.softmax == 0
        assert p.engine in (1, 3)
        if p.nsplit > 1:
            assert p.combine == 1
            planes = -(-p.nsplit * w.B * w.Hq * w.D // 4) * 4
            assert p.workspace_bytes == planes * 4 + p.nsplit * w.B * w.Hq * 8
        else:
            assert p.workspace_bytes == 0


def test_softmax_plan_refusals():
    with pytest.raises(ga.GqaAvError) as e:
        ga.make_plan(2, 1000, 16, 2, 128, "f16", "reuse", engine="mfma", softmax=True)
    assert e.value.name == "UNSUPPORTED"
    with pytest.raises(ga.GqaAvError) as e:
        ga.make_plan(1, 1000, 16, 8, 32, "bf16", "reuse", engine="valu", kv_tile=8, softmax=True)
    assert e.value.name == "UNSUPPORTED"
    # f16 / f32 V with a large group: the automatic engine is VALU, not the fp32 matrix engine
    assert ga.make_plan(2, 4096, 32, 2, 128, "f16", "reuse", softmax=True).engine == 1
    assert ga.make_plan(2, 4096, 32, 2, 128, "f16", "reuse").engine == 2
    h = ga.Hint()
    h.softmax = 2
    p = ga.Plan()
    assert ga.load().gqa_av_make_plan(1, 10, 4, 2, 64, 2, -1, ctypes.byref(h), ctypes.byref(p)) == 1


def test_softmax_and_plain_plans_do_not_mix():
    """Each entry point refuses the other's plans before touching the GPU."""
    lib = ga.load()
    fake = ctypes.c_void_p(1 << 20)
    sm = ga.make_plan(2, 100, 8, 2, 64, "bf16", softmax=True)
    pl = ga.make_plan(2, 100, 8, 2, 64, "bf16")
    for fn in ("gqa_av_decode_plan", "gqa_av_decode_pass1", "gqa_av_decode_combine"):
        assert getattr(lib, fn)(fake, fake, fake, 2, 100, 8, 2, 64, 2, ctypes.byref(sm), None) == 1
    for fn in ("gqa_softmax_av_decode_plan", "gqa_softmax_av_decode_pass1", "gqa_softmax_av_decode_combine"):
        assert getattr(lib, fn)(fake, fake, fake, 2, 100, 8, 2, 64, 2, ctypes.byref(pl), None) == 1
    # and the usual checks: wrong sizes, NULL scores, B = 0
    assert lib.gqa_softmax_av_decode_plan(fake, fake, fake, 2, 5000, 8, 2, 64, 2, ctypes.byref(sm), None) == 1
    assert lib.gqa_softmax_av_decode_plan(None, fake, fake, 2, 100, 8, 2, 64, 2, ctypes.byref(sm), None) == 1
    assert "scores" in ga.load().gqa_av_last_error().decode()
    sm0 = ga.make_plan(0, 100, 8, 2, 64, "bf16", softmax=True)
    assert lib.gqa_softmax_av_decode_plan(None, None, None, 0, 100, 8, 2, 64, 2, ctypes.byref(sm0), None) == 0


@pytest.mark.parametrize("wname", list(WORKLOADS))
def test_paged_plans(wname):
    """Paged plans: the VALU engine with 16-byte loads, or the bf16 matrix
    engine for bf16 V in reuse mode at G >= 5 with D of 64, 128 or 256 (as for
    dense V), the kernel combine, and splits whose page lists fit the kernels'
    LDS list (1024 pages)."""
    w = WORKLOADS[wname]
    for P in (1, 16, 256):
        for sm in (False, True):
            for mode in ("auto", "per_head"):
                try:
                    p = ga.make_plan(w.B, w.C, w.Hq, w.Hkv, w.D, w.v_dtype, mode, page_size=P, softmax=sm)
                except ga.GqaAvError as e:
                    assert e.name == "UNSUPPORTED" and (w.D * (4 if w.v_dtype == "f32" else 2)) % 16
                    continue
                bf16_engine = (w.v_dtype == "bf16" and w.D in (64, 128, 256) and w.Hq // w.Hkv >= 5
                               and mode == "auto")
                assert p.engine == (3 if bf16_engine else 1) and p.vec_bytes == 16, (wname, P, sm, mode)
                assert p.page_size == P and p.softmax == int(sm)
                assert -(-p.rows_per_split // P) + 1 <= 1024
                assert p.nsplit == 1 or p.combine == 1


def test_paged_refusals():
    for kw, name in ((dict(page_size=12), "INVALID_ARG"), (dict(page_size=16, engine="mfma"), "UNSUPPORTED"),
                     (dict(page_size=16, engine="mfma_bf16", mode="per_head"), "UNSUPPORTED"),
                     (dict(page_size=1, nsplit=1), "UNSUPPORTED")):          # 4000 rows on 1-row pages: 4000 pages
        with pytest.raises(ga.GqaAvError) as e:
            ga.make_plan(4, 4000, 16, 8, 128, "bf16", **kw)
        assert e.value.name == name, kw
    with pytest.raises(ga.GqaAvError) as e:
        ga.make_plan(4, 1000, 16, 8, 100, "bf16", page_size=16)
    assert e.value.name == "UNSUPPORTED"


def test_paged_calls_reject_before_launch():
    lib = ga.load()
    fake = ctypes.c_void_p(1 << 20)
    pg = ga.make_plan(2, 100, 8, 2, 64, "bf16", page_size=16)
    dense = ga.make_plan(2, 100, 8, 2, 64, "bf16")

    def call(plan, C=100, P=16, maxp=8, npg=16, bt=fake, ln=fake):
        return lib.gqa_av_paged_decode_plan(fake, fake, bt, ln, fake, 2, C, 8, 2, 64, P, maxp, npg, 2,
                                            ctypes.byref(plan), None)
    assert call(dense) == 1                                   # not a paged plan
    assert lib.gqa_av_decode_plan(fake, fake, fake, 2, 100, 8, 2, 64, 2, ctypes.byref(pg), None) == 1
    assert call(pg, P=32) == 1                                # page size differs from the plan's
    assert call(pg, maxp=6) == 1                              # capacity 100 > 6 * 16
    assert call(pg, npg=0) == 1
    assert call(pg, bt=None) == 1 and call(pg, ln=None) == 1
    assert "block_table" in ga.load().gqa_av_last_error().decode()
    odd = ctypes.c_void_p((1 << 20) + 8)                      # pages not 16-byte aligned
    assert lib.gqa_av_paged_decode_plan(fake, odd, fake, fake, fake, 2, 100, 8, 2, 64, 16, 8, 16, 2,
                                        ctypes.byref(pg), None) == 3
    pg0 = ga.make_plan(0, 100, 8, 2, 64, "bf16", page_size=16)
    assert lib.gqa_av_paged_decode_plan(None, None, None, None, None, 0, 100, 8, 2, 64, 16, 8, 16, 2,
                                        ctypes.byref(pg0), None) == 0


def test_fp8_plans():
    """fp8 V: the VALU engine with lane loads of at most 8 bytes (8 values) for
    tiles of more than 4 heads, 16 for smaller ones; V counted at one byte per value."""
    for wname, w in WORKLOADS.items():
        for sm in (False, True):
            p = ga.make_plan(w.B, w.C, w.Hq, w.Hkv, w.D, "fp8", softmax=sm)
            assert p.softmax == int(sm), wname
            G = w.Hq // w.Hkv
            if G >= 5 and w.D in (64, 128, 256):
                assert p.engine == 3 and p.vec_bytes == 8, wname      # bf16 matrix engine, 8-value pieces
            else:
                assert p.engine == 1 and p.vec_bytes <= (16 if p.heads_per_tile <= 4 else 8), wname
            assert p.v_bytes_read == w.B * w.C * w.Hkv * w.D * p.subgroups
    assert ga.make_plan(1, 100, 8, 2, 6, "fp8").vec_bytes == 2
    assert ga.make_plan(1, 100, 8, 2, 6, "fp8", v_align=2).vec_bytes == 2
    assert ga.make_plan(2, 1000, 16, 2, 128, "fp8", "reuse", engine="mfma_bf16").engine == 3
    for kw in (dict(engine="mfma"), dict(page_size=16, engine="valu")):     # paged VALU: 16-byte loads only
        with pytest.raises(ga.GqaAvError) as e:
            ga.make_plan(2, 1000, 16, 2, 128, "fp8", "reuse", **kw)
        assert e.value.name == "UNSUPPORTED", kw
    pf = ga.make_plan(2, 1000, 16, 2, 128, "fp8", "reuse", page_size=16)   # paged fp8 at G = 8: bf16 matrix engine
    assert pf.engine == 3 and pf.vec_bytes == 8 and pf.page_size == 16
    pv = ga.make_plan(2, 1000, 8, 2, 128, "fp8", "reuse", page_size=16)    # paged fp8 at G = 4: VALU, 16 values a lane
    assert pv.engine == 1 and pv.vec_bytes == 16 and pv.page_size == 16
    with pytest.raises(ga.GqaAvError) as e:
        ga.make_plan(2, 1000, 16, 2, 127, "fp8")            # odd D: no 2-byte lane load fits
    assert e.value.name == "UNSUPPORTED"
    pk = ga.qk_make_plan(2, 1000, 16, 2, 128, "fp8")           # fp8 K in the score step: the 16-bit matrix path
    assert pk.engine == 3 and pk.k_bytes_read == 2 * 1000 * 2 * 128
    with pytest.raises(ga.GqaAvError) as e:
        ga.qk_make_plan(2, 1000, 16, 2, 96, "fp8")            # fp8 K needs D % 64 == 0
    assert e.value.name == "UNSUPPORTED"


def test_fp8_calls_reject_before_launch():
    lib = ga.load()
    fake = ctypes.c_void_p(1 << 20)
    p = ga.make_plan(2, 100, 8, 2, 64, "fp8")
    bad_scale = ctypes.c_void_p((1 << 20) + 2)
    assert lib.gqa_av_fp8_decode_plan(fake, fake, bad_scale, fake, 2, 100, 8, 2, 64, ctypes.byref(p), None) == 1
    assert lib.gqa_av_fp8_decode_plan(fake, fake, None, fake, 2, 5000, 8, 2, 64, ctypes.byref(p), None) == 1
    pb = ga.make_plan(2, 100, 8, 2, 64, "bf16")             # a bf16 plan for an fp8 call
    assert lib.gqa_av_fp8_decode_plan(fake, fake, None, fake, 2, 100, 8, 2, 64, ctypes.byref(pb), None) == 1


def test_error_detail_is_per_thread():
    """A failing call in one thread leaves another thread's error detail alone."""
    lib = ga.load()
    seen = {}
    gate = threading.Barrier(2)

    def bad():
        rc = lib.gqa_av_decode(None, None, None, 2, 100, 8, 3, 64, 2, -1, None)   # Hq % Hkv != 0
        gate.wait()
        gate.wait()
        seen["bad"] = (rc, lib.gqa_av_last_error().decode())

    def good():
        gate.wait()
        rc = lib.gqa_av_resolve_mode(16, 8, -1)
        seen["good"] = (rc, lib.gqa_av_last_error().decode())
        gate.wait()

    ts = [threading.Thread(target=bad), threading.Thread(target=good)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert seen["bad"][0] != 0 and seen["bad"][1], seen
    assert seen["good"][0] == 1 and seen["good"][1] == "", seen


def test_qk_paged_plans_and_refusals():
    """Paged score plans: page_size recorded, rows per block capped so a block's
    page list fits in LDS (<= 1023 pages), bad sizes refused before any
    launch, dense and paged plans not interchangeable."""
    for P in (1, 16, 256):
        p = ga.qk_make_plan(4, 32768, 16, 8, 128, "bf16", page_size=P)
        assert p.page_size == P and p.rows_per_block % 64 == 0 and -(-p.rows_per_block // P) + 1 <= 1024
    for kw, name in ((dict(page_size=12), "INVALID_ARG"), (dict(page_size=-4), "INVALID_ARG")):
        with pytest.raises(ga.GqaAvError) as e:
            ga.qk_make_plan(4, 1000, 16, 8, 128, "bf16", **kw)
        assert e.value.name == name, kw
    lib = ga.load()
    fake = ctypes.c_void_p(1 << 20)
    pg = ga.qk_make_plan(2, 100, 8, 2, 64, "bf16", page_size=16)
    dense = ga.qk_make_plan(2, 100, 8, 2, 64, "bf16")

    def call(plan, C=100, P=16, maxp=8, npg=16, bt=fake, ln=fake, ks=None, dt=2):
        return lib.gqa_qk_paged_decode_plan(fake, fake, bt, ln, ks, fake, 2, C, 8, 2, 64, P, maxp, npg, dt,
                                            ctypes.c_float(1.0), ctypes.byref(plan), None)
    assert call(dense) == 1                                   # not a paged plan
    assert lib.gqa_qk_decode_plan(fake, fake, fake, 2, 100, 8, 2, 64, 2, ctypes.c_float(1.0), ctypes.byref(pg),
                                  None) == 1                  # a paged plan on the dense entry point
    assert call(pg, P=32) == 1                                # page size differs from the plan's
    assert call(pg, maxp=6) == 1                              # capacity 100 > 6 * 16
    assert call(pg, npg=0) == 1
    assert call(pg, bt=None) == 1 and call(pg, ln=None) == 1
    assert call(pg, ks=fake) == 1                             # k_scale is for fp8 K
    assert "k_scale" in ga.load().gqa_av_last_error().decode()


@pytest.mark.parametrize("kvdt", ["bf16", "fp8"])
def test_attention_plans(kvdt):
    """Fused attention plans: the bf16 matrix engine with the fused softmax,
    dense or paged, D of 64/128/256; splits tile C; refusals."""
    for B, C, Hq, Hkv, D, P in [(64, 8192, 64, 8, 128, 0), (4, 32768, 16, 8, 128, 16), (1, 4096, 32, 8, 128, 0),
                                (4, 32768, 16, 1, 128, 64), (2, 700, 40, 2, 256, 8), (3, 1, 8, 4, 64, 1)]:
        p = ga.make_plan(B, C, Hq, Hkv, D, kvdt, attention=True, page_size=P, cu_count=256)
        assert p.attention == 1 and p.softmax == 1 and p.engine == 3 and p.page_size == P
        assert p.nsplit == -(-C // p.rows_per_split)
        if P:
            assert p.rows_per_split <= (1024 - 1) * P             # a split's pages fit the LDS list
    for bad in (dict(v_dtype="f16"), dict(D=96), dict(engine="valu"), dict(mode="per_head")):
        kw = dict(B=2, C=100, Hq=8, Hkv=2, D=128, v_dtype=kvdt)
        kw.update(bad)
        with pytest.raises(ga.GqaAvError):
            ga.make_plan(kw.pop("B"), kw.pop("C"), kw.pop("Hq"), kw.pop("Hkv"), kw.pop("D"), kw.pop("v_dtype"),
                         attention=True, **kw)


def test_attention_calls_reject_before_launch():
    lib = ga.load()
    fake = ctypes.c_void_p(1 << 20)
    f = ctypes.c_float(1.0)
    dense = ga.make_plan(2, 100, 8, 2, 128, "bf16", attention=True)
    pg = ga.make_plan(2, 100, 8, 2, 128, "bf16", attention=True, page_size=16)
    plain = ga.make_plan(2, 100, 8, 2, 128, "bf16", softmax=True)

    def paged(plan, ks=None, P=16, maxp=8, dt=2, kp=fake):
        return lib.gqa_attention_paged_decode_plan(fake, kp, fake, fake, fake, ks, None, fake, 2, 100, 8, 2, 128,
                                                   P, maxp, 16, dt, f, ctypes.byref(plan), None)
    assert paged(dense) == 1                                  # not a paged plan
    assert paged(plain) == 1                                  # not an attention plan
    assert lib.gqa_attention_decode_plan(fake, fake, fake, fake, 2, 100, 8, 2, 128, 2, f, ctypes.byref(pg), None) == 1
    assert paged(pg, ks=fake) == 1                            # scales are for fp8
    assert "k_scale" in lib.gqa_av_last_error().decode()
    assert paged(pg, P=32) == 1 and paged(pg, maxp=6) == 1    # page size, capacity
    assert paged(pg, dt=1) == 3                               # f16 K and V
    assert paged(pg, kp=ctypes.c_void_p((1 << 20) + 8)) == 3  # K pages not 16-byte aligned
    pg8 = ga.make_plan(2, 100, 8, 2, 128, "fp8", attention=True, page_size=16)
    assert paged(pg8, dt=3, ks=ctypes.c_void_p((1 << 20) + 2)) == 1   # misaligned k_scale


def test_tuned_plan_choices():
    """The automatic plans the measurements chose (256 CUs): two workgroups per
    CU for the fp8 fused softmax and fused attention, one for the plain fp8
    product and for bf16; attention splits down to 128 rows on a grid smaller
    than the chip; splits of at least 512 rows otherwise."""
    def plan(*shape, dt, **kw):
        return ga.make_plan(*shape, dt, cu_count=256, **kw)
    big = (64, 8192, 64, 8, 128)
    assert plan(*big, dt="fp8", softmax=True).grid == 512
    assert plan(*big, dt="fp8", attention=True).grid == 512
    assert plan(*big, dt="fp8").grid == 256
    assert plan(*big, dt="bf16", attention=True).grid == 256
    assert plan(*big, dt="bf16", softmax=True).grid == 256
    small = (1, 4096, 32, 8, 128)                     # 8 tiles: 32 splits of 128 rows
    for dt in ("bf16", "fp8"):
        p = plan(*small, dt=dt, attention=True)
        assert (p.nsplit, p.rows_per_split, p.grid) == (32, 128, 256)
    mqa = (4, 32768, 16, 1, 128)                      # 64 splits of 512 rows in every variant
    for dt in ("bf16", "fp8"):
        for kw in (dict(attention=True), dict(softmax=True), {}):
            p = plan(*mqa, dt=dt, **kw)
            # the plain product runs eight waves and cuts its splits into
            # interleaved blocks of one step (eight waves of 32 rows), the
            # fused ones four waves and contiguous ranges
            want = (64, 256, 256, 1, 512) if not kw else (64, 512, 256, 0, 256)
            assert (p.nsplit, p.rows_per_split, p.grid, p.interleave, p.threads) == want, (dt, kw)
