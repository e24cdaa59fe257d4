"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each pin is a plain function taking an ``oracle.Oracle`` and raising
AssertionError when the oracle disagrees. ``test_oracle_pins.py`` runs them on
the real oracle and on deliberately broken copies of its source, which must
each fail at least one pin.

What pins what:
  * decode_table      IEEE-754 binary16 / bfloat16 bit patterns with closed-form
                      values, and every 16-bit pattern against torch's own
                      conversion (an independent library routine).
  * brute_force       tiny shapes, all dtypes, against the correctly rounded
                      exact sum (oracle/brute.py), within the oracle's a-priori
                      bound gamma_{C-1} * sum|a*v| + one rounding.
  * mha_einsum        G = 1 equals numpy's einsum 'bch,bchd->bhd' in fp64.
  * repeat_mha        GQA equals MHA over V repeated G times along the head
                      axis: pins kv_h = floor(q_h / G).
  * constant_v        V constant along c gives u * sum_c attn; with softmax
                      weights (columns summing to 1) that is u itself.
  * one_hot           one-hot weights return that V row exactly.
  * linearity, permutation, batch independence: algebraic properties.
  * points            the sampled entry point equals brute force.
  * edges             C = 0 gives zeros; B = 0 gives an empty result;
                      Hq % Hkv != 0 is rejected.

The score step (scores = scale * q . K over d, in the attn layout):
  * qk_brute_force    tiny shapes, all dtypes, against the correctly rounded
                      exact dot products (oracle/brute.py).
  * qk_mha_einsum     G = 1 equals numpy's einsum 'bhd,bchd->bch' in fp64.
  * qk_repeat_mha     GQA equals MHA over K repeated G times (bitwise).
  * qk_one_hot        q = e_j returns scale * K[..., j] exactly.
  * qk_scale_linear   scale by a power of two is exact; linearity in q.
  * qk_composition    softmax over c of the scores, then the AV oracle, equals
                      decode attention written as one numpy fp64 expression:
                      pins that the scores come out in the attn layout.
  * qk_edges          C = 0 and B = 0 give empty results; Hq % Hkv != 0 is
                      rejected; D = 1.

The fused softmax product (out = softmax over c of the scores, times V):
  * sav_library       scipy's softmax over c in fp64, then numpy's einsum with
                      V repeated along the heads: an independent route.
  * sav_shift         adding a constant to every score of a row changes
                      nothing (dyadic scores, so the shifted scores are exact).
  * sav_large         scores near 8192 (where exp without the max overflows)
                      equal the same scores shifted down by 8192.
  * sav_one_hot       one score 800 above the rest returns that V row exactly.
  * sav_uniform       equal scores give the mean of the V rows over c.
  * sav_two_rows      C = 2: the logistic closed form.
  * sav_mask          -inf scores drop their rows: the result equals the
                      oracle over the remaining rows, bit for bit.
  * sav_repeat_mha    GQA equals MHA over V repeated G times (bitwise).
  * sav_edges         C = 0 gives zeros; a row of all -inf gives NaN; B = 0
                      gives an empty result.

Paged V (rows of sequence b in pages block_table[b][c // P], lengths seq_lens):
  * paged_gather      gather each sequence's rows with numpy into a dense
                      cache and run the dense oracles on its first len rows:
                      equal bit for bit (plain and fused softmax).
  * paged_identity    one page per sequence of P = C rows and full lengths is
                      the dense layout: equal to the dense oracles bit for bit.
  * paged_ignores_tail  weights, scores and V rows at or past a sequence's
                      length, and unused pages, change nothing; length 0 gives
                      zeros.
  * paged_rejects     block-table entries outside the cache, lengths outside
                      [0, C] and C above max_pages * P are rejected.

fp8 V (OCP FP8 E4M3 bytes times a float32 scale per KV head):
  * fp8_decode        all 256 bit patterns against torch's float8_e4m3fn, and
                      values the OCP format fixes (448 the largest, 2^-6 the
                      smallest normal, 2^-9 the smallest subnormal, 1.0, -0, NaN).
  * fp8_as_bf16       every E4M3 value is a bfloat16 value: with unit scales the
                      fp8 oracle equals the bf16 oracles on the widened V, bit
                      for bit (plain and fused softmax).
  * fp8_scales        a power-of-two scale per KV head scales exactly that head's
                      group of outputs; one head's scale leaves the others alone.

Paged K in the score step (the paged-V layout and tables):
  * qk_paged_gather   the scores of rows below each length equal the dense
                      score oracle on the sequence's gathered rows (all K
                      types, fp8 with scales), bit for bit; rows past the
                      length are NaN (no score).
  * qk_paged_identity one page per sequence holding the dense K is the dense
                      score oracle, bit for bit.
  * qk_paged_tail     K rows at or past the length and unused pages change
                      nothing.
  * qk_paged_rejects  bad block-table entries, lengths and capacities are
                      rejected.

Fused decode attention (softmax of the scaled scores, times V, in one pass):
  * attn_composition  with dyadic q and small-integer K every score is exact in
                      fp32, and the oracle equals the score oracle followed by
                      the fused softmax-V oracle bit for bit.
  * attn_numpy        numpy's einsum and scipy's softmax in fp64 (an independent
                      route) agree to 1e-12, also for scores near 700.
  * attn_zero_q       q = 0 gives the mean of V over the context.
  * attn_repeat_mha   GQA equals MHA over K and V repeated G times (bitwise).
  * attn_edges        C = 0 gives zeros; B = 0 gives an empty result.

Fused attention over fp8 K and V (E4M3 bytes, per-KV-head scales):
  * attn_fp8_as_bf16  with unit scales it equals the bf16 attention oracle on K
                      and V widened by torch's float8 -> bfloat16 conversion,
                      bit for bit.
  * attn_fp8_scales   a power-of-two v_scale scales exactly its head group's
                      outputs; a power-of-two k_scale equals the bf16
                      attention oracle with scale * k_scale, bit for bit.

Fused attention over a paged K and V cache (two page pools, one block table):
  * attn_paged_gather with shuffled pages of 1, 2, 4, 8 and 16 rows, every
                      dtype and fp8 with distinct K and V scales, it equals
                      dense attention on each sequence's first len rows
                      gathered through the table, bit for bit; length 0 gives
                      zeros.
  * attn_paged_tail   NaN in rows past a length and in unused pages changes
                      nothing.
  * attn_paged_rejects bad block-table entries, lengths and capacities are
                      rejected.

fp8 K in the score step (same bytes and per-KV-head scales):
  * qk_fp8_as_bf16    with unit scales the fp8 score oracle equals the bf16
                      score oracle on K widened by torch's float8 -> bfloat16
                      conversion, bit for bit.
  * qk_fp8_brute      tiny shapes against Python's exact rational arithmetic
                      (fractions) on torch's decoded K, correctly rounded.
  * qk_fp8_scales     a power-of-two k_scale per KV head scales exactly that
                      head's group of score columns; others are left alone.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from oracle.brute import abs_sum, abs_sum_qk, brute_force, brute_force_qk
from workloads import make_qk_random, make_random, make_scores_random

U64 = 2.0 ** -53


def gamma(n: int) -> float:
    nu = n * U64
    return nu / (1.0 - nu)


def _within_bound(o: np.ndarray, exact: np.ndarray, scale: np.ndarray, C: int, what: str):
    bound = gamma(max(C - 1, 0)) * scale + U64 * np.abs(exact) + 1e-300
    err = np.abs(o - exact)
    bad = err > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} elements outside the bound, worst {float((err - bound).max()):.3e}"


def _tiny_cases():
    return [
        # B, C, Hq, Hkv, D, dtype, attn kind
        (1, 1, 1, 1, 1, "f32", "signed"),
        (2, 17, 6, 2, 5, "f32", "signed"),
        (2, 13, 5, 1, 8, "bf16", "signed"),
        (1, 9, 6, 3, 7, "f16", "signed"),
        (2, 11, 4, 4, 3, "bf16", "softmax"),
        (1, 16, 10, 2, 4, "f16", "softmax"),
    ]


def pin_decode_table(orc):
    f16_known = {
        0x0000: 0.0, 0x3C00: 1.0, 0xC000: -2.0, 0x7BFF: 65504.0, 0x0400: 2.0 ** -14,
        0x0001: 2.0 ** -24, 0x03FF: 1023 * 2.0 ** -24, 0x3555: (1 + 0x155 / 1024) * 0.25,
        0x8001: -(2.0 ** -24), 0x7C00: math.inf, 0xFC00: -math.inf,
    }
    bf16_known = {
        0x0000: 0.0, 0x3F80: 1.0, 0xC000: -2.0, 0x0080: 2.0 ** -126, 0x0001: 2.0 ** -133,
        0x3EAB: (1 + 0x2B / 128) * 0.25, 0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127,
        0x8080: -(2.0 ** -126), 0x7F80: math.inf, 0xFF80: -math.inf,
    }
    for dt, known in (("f16", f16_known), ("bf16", bf16_known)):
        bits = np.array(list(known.keys()), dtype=np.uint16)
        got = orc.decode(bits, dt)
        for b, g in zip(bits.tolist(), got.tolist()):
            assert g == known[b], f"{dt} 0x{b:04x}: {g!r} != {known[b]!r}"
    nan_f16 = orc.decode(np.array([0x7E00, 0xFE01], np.uint16), "f16")
    nan_bf16 = orc.decode(np.array([0x7FC0, 0xFF81], np.uint16), "bf16")
    assert np.isnan(nan_f16).all() and np.isnan(nan_bf16).all()
    # every 16-bit pattern against torch's conversion
    allbits = np.arange(65536, dtype=np.uint16)
    t = torch.from_numpy(allbits.view(np.int16).copy())
    for dt, tdt in (("f16", torch.float16), ("bf16", torch.bfloat16)):
        ref = t.view(tdt).to(torch.float64).numpy()
        got = orc.decode(allbits, dt)
        same = (got == ref) | (np.isnan(got) & np.isnan(ref))
        assert same.all(), f"{dt}: {int((~same).sum())} patterns decode differently from torch"
        # signed zero
        assert np.array_equal(np.signbit(got[~np.isnan(got)]), np.signbit(ref[~np.isnan(ref)]))
    f = np.array([1.5, -0.0, 3.4e38, 1e-45, -7.25], dtype=np.float32)
    assert np.array_equal(orc.decode(f, "f32"), f.astype(np.float64))


def pin_brute_force(orc):
    for i, (B, C, Hq, Hkv, D, dt, kind) in enumerate(_tiny_cases()):
        attn, V = make_random(B, C, Hq, Hkv, D, dt, seed=100 + i, attn_kind=kind)
        exact = brute_force(attn, V)
        o = orc.full(attn, V, dt)
        _within_bound(o, exact, abs_sum(attn, V), C, f"brute {B,C,Hq,Hkv,D,dt}")


def pin_mha_einsum(orc):
    for dt in ("f32", "bf16", "f16"):
        attn, V = make_random(2, 37, 3, 3, 6, dt, seed=7, attn_kind="signed")
        ref = np.einsum("bch,bchd->bhd", attn.double().numpy(), V.double().numpy())
        o = orc.full(attn, V, dt)
        _within_bound(o, ref, abs_sum(attn, V), 2 * 37, f"einsum {dt}")


def pin_repeat_mha(orc):
    for dt, (Hq, Hkv) in (("bf16", (8, 2)), ("f16", (6, 3)), ("f32", (5, 1))):
        attn, V = make_random(2, 23, Hq, Hkv, 4, dt, seed=11, attn_kind="signed")
        G = Hq // Hkv
        Vrep = V.repeat_interleave(G, dim=2).contiguous()
        a = orc.full(attn, V, dt)
        b = orc.full(attn, Vrep, dt)
        assert np.array_equal(a, b), f"GQA != MHA over repeated V ({dt}, G={G})"
        # and the repeated form agrees with the textbook einsum
        ref = np.einsum("bch,bchd->bhd", attn.double().numpy(), Vrep.double().numpy())
        _within_bound(a, ref, abs_sum(attn, V), 2 * 23, f"repeat-einsum {dt}")


def pin_constant_v(orc):
    B, C, Hq, Hkv, D = 2, 300, 6, 2, 5
    g = torch.Generator().manual_seed(5)
    u = torch.randn(B, 1, Hkv, D, generator=g).to(torch.bfloat16)
    V = u.expand(B, C, Hkv, D).contiguous()
    logits = torch.randn(B, C, Hq, generator=g, dtype=torch.float64)
    attn = torch.softmax(logits, dim=1).to(torch.float32)
    o = orc.full(attn, V, "bf16")
    G = Hq // Hkv
    ud = u.double().numpy()[:, 0]                             # [B, Hkv, D]
    colsum = np.array([[math.fsum(attn[b, :, q].double().tolist()) for q in range(Hq)] for b in range(B)])
    expect = colsum[:, :, None] * np.repeat(ud, G, axis=1)
    _within_bound(o, expect, np.abs(expect), C, "constant V")
    # columns sum to one up to fp32 rounding of the weights: out ~ u
    assert np.allclose(o, np.repeat(ud, G, axis=1), rtol=C * 2.0 ** -23, atol=0.0), "constant V, unit columns"


def pin_one_hot(orc):
    B, C, Hq, Hkv, D = 3, 41, 8, 4, 6
    for dt in ("f32", "f16", "bf16"):
        _, V = make_random(B, C, Hq, Hkv, D, dt, seed=3)
        attn = torch.zeros(B, C, Hq)
        G = Hq // Hkv
        picks = {}
        for b in range(B):
            for q in range(Hq):
                c = (7 * b + 5 * q + 1) % C
                attn[b, c, q] = 1.0
                picks[b, q] = c
        o = orc.full(attn, V, dt)
        Vd = V.double().numpy()
        for (b, q), c in picks.items():
            assert np.array_equal(o[b, q], Vd[b, c, q // G]), f"one-hot {dt} b={b} q={q}"


def pin_linearity(orc):
    B, C, Hq, Hkv, D = 2, 40, 6, 3, 4
    attn, V = make_random(B, C, Hq, Hkv, D, "bf16", seed=21, attn_kind="signed")
    a1 = attn.clone(); a1[:, C // 2:] = 0
    a2 = attn.clone(); a2[:, :C // 2] = 0
    o = orc.full(attn, V, "bf16")
    o12 = orc.full(a1, V, "bf16") + orc.full(a2, V, "bf16")
    _within_bound(o, o12, 2 * abs_sum(attn, V), C, "linearity")
    o2 = orc.full(attn * 2.0, V, "bf16")
    assert np.array_equal(o2, 2.0 * o), "scaling by 2"


def pin_permutation(orc):
    B, C, Hq, Hkv, D = 2, 33, 4, 2, 5
    attn, V = make_random(B, C, Hq, Hkv, D, "f16", seed=31, attn_kind="signed")
    perm = torch.randperm(C, generator=torch.Generator().manual_seed(1))
    o = orc.full(attn, V, "f16")
    op = orc.full(attn[:, perm].contiguous(), V[:, perm].contiguous(), "f16")
    _within_bound(op, o, 2 * abs_sum(attn, V), C, "permutation")


def pin_batch_independence(orc):
    B, C, Hq, Hkv, D = 3, 19, 6, 2, 4
    attn, V = make_random(B, C, Hq, Hkv, D, "bf16", seed=41, attn_kind="signed")
    o = orc.full(attn, V, "bf16")
    for b in range(B):
        ob = orc.full(attn[b:b + 1].contiguous(), V[b:b + 1].contiguous(), "bf16")
        assert np.array_equal(o[b:b + 1], ob), f"batch {b} depends on other batches"


def pin_points(orc):
    B, C, Hq, Hkv, D = 2, 21, 6, 3, 5
    for dt in ("f32", "f16", "bf16"):
        attn, V = make_random(B, C, Hq, Hkv, D, dt, seed=51, attn_kind="signed")
        exact = brute_force(attn, V)
        rng = np.random.default_rng(0)
        idx = np.stack([rng.integers(0, B, 40), rng.integers(0, Hq, 40), rng.integers(0, D, 40)], 1)
        p = orc.points(attn, V, dt, idx)
        e = exact[idx[:, 0], idx[:, 1], idx[:, 2]]
        s = abs_sum(attn, V)[idx[:, 0], idx[:, 1], idx[:, 2]]
        _within_bound(p, e, s, C, f"points {dt}")


def pin_edges(orc):
    attn = torch.zeros(2, 0, 4)
    V = torch.zeros(2, 0, 2, 3, dtype=torch.bfloat16)
    o = orc.full(attn, V, "bf16")
    assert o.shape == (2, 4, 3) and not o.any(), "C = 0 must give zeros"
    o = orc.full(torch.zeros(0, 5, 4), torch.zeros(0, 5, 2, 3), "f32")
    assert o.shape == (0, 4, 3)
    try:
        orc.full(torch.zeros(1, 2, 5), torch.zeros(1, 2, 2, 3), "f32")
    except ValueError:
        pass
    else:
        raise AssertionError("Hq % Hkv != 0 must be rejected")


def _qk_cases():
    return [
        # B, C, Hq, Hkv, D, dtype
        (1, 1, 1, 1, 1, "f32"),
        (2, 7, 6, 2, 13, "f32"),
        (2, 5, 4, 1, 16, "bf16"),
        (1, 6, 6, 3, 9, "f16"),
        (2, 4, 8, 8, 5, "bf16"),
    ]


def pin_qk_brute_force(orc):
    for i, (B, C, Hq, Hkv, D, dt) in enumerate(_qk_cases()):
        q, K = make_qk_random(B, C, Hq, Hkv, D, dt, seed=500 + i)
        for scale in (1.0, 0.125, 0.3):
            exact = brute_force_qk(q, K, scale)
            o = orc.qk(q, K, dt, scale)
            # a-priori bound: gamma_{D-1} on the sum, one rounding for the scale
            bound = (gamma(max(D - 1, 0)) * abs_sum_qk(q, K) * abs(scale) + 2 * U64 * np.abs(exact)) + 1e-300
            err = np.abs(o - exact)
            assert (err <= bound).all(), f"qk brute {B, C, Hq, Hkv, D, dt} scale {scale}: worst {float((err - bound).max()):.3e}"


def pin_qk_mha_einsum(orc):
    for dt in ("f32", "bf16", "f16"):
        q, K = make_qk_random(2, 9, 3, 3, 24, dt, seed=41)
        ref = np.einsum("bhd,bchd->bch", q.double().numpy(), K.double().numpy()) * 0.25
        o = orc.qk(q, K, dt, 0.25)
        bound = gamma(2 * 24) * abs_sum_qk(q, K) * 0.25 + 1e-300
        assert (np.abs(o - ref) <= bound).all(), f"qk einsum {dt}"


def pin_qk_repeat_mha(orc):
    for dt, (Hq, Hkv) in (("bf16", (8, 2)), ("f16", (6, 3)), ("f32", (5, 1))):
        q, K = make_qk_random(2, 11, Hq, Hkv, 10, dt, seed=43)
        G = Hq // Hkv
        Krep = K.repeat_interleave(G, dim=2).contiguous()
        a = orc.qk(q, K, dt, 0.5)
        b = orc.qk(q, Krep, dt, 0.5)
        assert np.array_equal(a, b), f"qk: GQA != MHA over repeated K ({dt}, G={G})"
        ref = np.einsum("bhd,bchd->bch", q.double().numpy(), Krep.double().numpy()) * 0.5
        bound = gamma(2 * 10) * abs_sum_qk(q, K) * 0.5 + 1e-300
        assert (np.abs(a - ref) <= bound).all(), f"qk repeat-einsum {dt}"


def pin_qk_one_hot(orc):
    for dt in ("f32", "bf16", "f16"):
        B, C, Hq, Hkv, D = 2, 13, 6, 2, 11
        _, K = make_qk_random(B, C, Hq, Hkv, D, dt, seed=47)
        G = Hq // Hkv
        q = torch.zeros(B, Hq, D)
        pick = {}
        for b in range(B):
            for h in range(Hq):
                j = (5 * b + 3 * h + 1) % D
                q[b, h, j] = 1.0
                pick[b, h] = j
        o = orc.qk(q, K, dt, 0.5)
        Kd = K.double().numpy()
        for (b, h), j in pick.items():
            assert np.array_equal(o[b, :, h], 0.5 * Kd[b, :, h // G, j]), f"qk one-hot {dt} b={b} h={h}"


def pin_qk_scale_linear(orc):
    q1, K = make_qk_random(2, 8, 4, 2, 12, "bf16", seed=53)
    q2, _ = make_qk_random(2, 8, 4, 2, 12, "bf16", seed=54)
    base = orc.qk(q1, K, "bf16", 1.0)
    assert np.array_equal(orc.qk(q1, K, "bf16", 0.25), 0.25 * base), "qk: a power-of-two scale must be exact"
    assert np.array_equal(orc.qk(q1, K, "bf16", -1.0), -base), "qk: scale -1 must negate"
    # dyadic q with few significant bits, so 3 q1 - 0.5 q2 is exact in fp32
    q1 = torch.round(q1 * 64) / 64
    q2 = torch.round(q2 * 64) / 64
    base = orc.qk(q1, K, "bf16", 1.0)
    mix = orc.qk(3.0 * q1 - 0.5 * q2, K, "bf16", 1.0)
    ref = 3.0 * base - 0.5 * orc.qk(q2, K, "bf16", 1.0)
    scale = abs_sum_qk(3.0 * q1, K) + abs_sum_qk(0.5 * q2, K)
    assert (np.abs(mix - ref) <= 64 * U64 * scale + 1e-300).all(), "qk linearity in q"


def pin_qk_composition(orc):
    B, C, Hq, Hkv, D = 2, 40, 8, 2, 16
    for dt in ("bf16", "f32"):
        q, K = make_qk_random(B, C, Hq, Hkv, D, dt, seed=59)
        _, V = make_qk_random(B, C, Hq, Hkv, D, dt, seed=61)
        s = orc.qk(q, K, dt, D ** -0.5)                       # [B, C, Hq]
        e = np.exp(s - s.max(axis=1, keepdims=True))
        attn = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
        out = orc.full(torch.from_numpy(attn), V, dt)          # [B, Hq, D]
        G = Hq // Hkv
        Kr = np.repeat(K.double().numpy(), G, axis=2)          # [B, C, Hq, D]
        Vr = np.repeat(V.double().numpy(), G, axis=2)
        logits = np.einsum("bhd,bchd->bhc", q.double().numpy(), Kr) * D ** -0.5
        p = np.exp(logits - logits.max(axis=2, keepdims=True))
        p /= p.sum(axis=2, keepdims=True)
        ref = np.einsum("bhc,bchd->bhd", p, Vr)
        rel = np.abs(out - ref).max() / np.abs(ref).max()
        assert rel < 1e-6, f"qk composition {dt}: {rel:.2e}"      # attn is rounded to fp32 in between


def pin_qk_edges(orc):
    q = torch.zeros(2, 4, 3)
    o = orc.qk(q, torch.zeros(2, 0, 2, 3, dtype=torch.bfloat16), "bf16")
    assert o.shape == (2, 0, 4)
    o = orc.qk(torch.zeros(0, 4, 3), torch.zeros(0, 5, 2, 3), "f32")
    assert o.shape == (0, 5, 4)
    try:
        orc.qk(torch.zeros(1, 5, 3), torch.zeros(1, 2, 2, 3), "f32")
    except ValueError:
        pass
    else:
        raise AssertionError("qk: Hq % Hkv != 0 must be rejected")
    q, K = make_qk_random(1, 3, 2, 1, 1, "f16", seed=67)
    o = orc.qk(q, K, "f16", 2.0)
    assert np.array_equal(o[0, :, 1], 2.0 * q[0, 1, 0].item() * K[0, :, 0, 0].double().numpy()), "qk D = 1"


def _repeat_ref(p: np.ndarray, V: torch.Tensor, Hq: int) -> np.ndarray:
    """sum_c p[b, c, h] * V[b, c, h // G, :] in numpy fp64 (V repeated along heads)."""
    Hkv = V.shape[2]
    Vr = np.repeat(V.double().numpy(), Hq // Hkv, axis=2)      # [B, C, Hq, D]
    return np.einsum("bch,bchd->bhd", p, Vr)


def _dyadic(x: torch.Tensor, bits: int = 8) -> torch.Tensor:
    return torch.round(x * 2 ** bits) / 2 ** bits


def pin_sav_library(orc):
    from scipy.special import softmax
    for i, (B, C, Hq, Hkv, D, dt, std) in enumerate([(2, 37, 6, 2, 5, "f32", 1.0), (1, 64, 8, 1, 16, "bf16", 3.0),
                                                     (2, 19, 9, 3, 7, "f16", 0.5), (1, 1, 2, 2, 3, "f32", 1.0)]):
        s, V = make_scores_random(B, C, Hq, Hkv, D, dt, seed=700 + i, score_std=std)
        p = softmax(s.double().numpy(), axis=1)
        ref = _repeat_ref(p, V, Hq)
        o = orc.softmax_av(s, V, dt)
        scale = _repeat_ref(p, V.abs() if dt == "f32" else V.float().abs(), Hq)
        assert (np.abs(o - ref) <= 64 * C * U64 * (scale + np.abs(ref)) + 1e-300).all(), f"sav library {B, C, Hq, Hkv, D, dt}"


def pin_sav_shift(orc):
    s, V = make_scores_random(2, 45, 4, 2, 6, "bf16", seed=711, score_std=2.0)
    s = _dyadic(s)
    a = orc.softmax_av(s, V, "bf16")
    b = orc.softmax_av(s + 64.0, V, "bf16")
    c = orc.softmax_av(s - 40.0, V, "bf16")
    ref = np.abs(a).max()
    assert np.abs(a - b).max() <= 1e-13 * ref and np.abs(a - c).max() <= 1e-13 * ref, "sav: not shift invariant"


def pin_sav_large(orc):
    s, V = make_scores_random(1, 50, 6, 3, 4, "f32", seed=713, score_std=3.0)
    s = _dyadic(s)
    a = orc.softmax_av(s, V, "f32")
    b = orc.softmax_av(s + 8192.0, V, "f32")
    assert np.isfinite(b).all(), "sav: large scores overflow"
    assert np.abs(a - b).max() <= 1e-13 * np.abs(a).max(), "sav: large scores differ from shifted ones"


def pin_sav_one_hot(orc):
    for dt in ("f32", "bf16", "f16"):
        B, C, Hq, Hkv, D = 2, 17, 6, 2, 5
        s, V = make_scores_random(B, C, Hq, Hkv, D, dt, seed=717)
        G = Hq // Hkv
        pick = {}
        for b in range(B):
            for h in range(Hq):
                c = (3 * b + 5 * h + 2) % C
                s[b, c, h] = 800.0
                pick[b, h] = c
        o = orc.softmax_av(s, V, dt)
        Vd = V.double().numpy()
        for (b, h), c in pick.items():
            assert np.array_equal(o[b, h], Vd[b, c, h // G]), f"sav one-hot {dt} b={b} h={h}"


def pin_sav_uniform(orc):
    for dt in ("f32", "f16"):
        B, C, Hq, Hkv, D = 2, 23, 4, 2, 3
        _, V = make_scores_random(B, C, Hq, Hkv, D, dt, seed=719)
        s = torch.full((B, C, Hq), 1.5)
        o = orc.softmax_av(s, V, dt)
        Vd = V.double().numpy()
        for b in range(B):
            for h in range(Hq):
                for d in range(D):
                    mean = math.fsum(Vd[b, :, h // (Hq // Hkv), d]) / C
                    assert abs(o[b, h, d] - mean) <= 1e-14 * max(1.0, abs(mean)), f"sav uniform {dt}"


def pin_sav_two_rows(orc):
    s, V = make_scores_random(3, 2, 4, 1, 5, "bf16", seed=723, score_std=2.0)
    o = orc.softmax_av(s, V, "bf16")
    Vd, sd = V.double().numpy(), s.double().numpy()
    for b in range(3):
        for h in range(4):
            x = sd[b, 0, h] - sd[b, 1, h]
            w0 = 1.0 / (1.0 + math.exp(-x))
            w1 = 1.0 / (1.0 + math.exp(x))
            ref = w0 * Vd[b, 0, 0] + w1 * Vd[b, 1, 0]
            assert np.abs(o[b, h] - ref).max() <= 1e-14 * max(1.0, np.abs(ref).max()), "sav two rows"


def pin_sav_mask(orc):
    B, C, Hq, Hkv, D = 1, 30, 4, 2, 6
    s, V = make_scores_random(B, C, Hq, Hkv, D, "f32", seed=727)
    keep = [c for c in range(C) if c % 3 != 1]
    for h in range(Hq):
        sm = s.clone()
        sm[:, [c for c in range(C) if c % 3 == 1], :] = float("-inf")
        a = orc.softmax_av(sm, V, "f32")
        b = orc.softmax_av(s[:, keep].contiguous(), V[:, keep].contiguous(), "f32")
        assert np.array_equal(a, b), "sav: -inf scores must drop their rows"


def pin_sav_repeat_mha(orc):
    for dt, (Hq, Hkv) in (("bf16", (8, 2)), ("f16", (6, 3)), ("f32", (5, 1))):
        s, V = make_scores_random(2, 13, Hq, Hkv, 7, dt, seed=729)
        Vrep = V.repeat_interleave(Hq // Hkv, dim=2).contiguous()
        assert np.array_equal(orc.softmax_av(s, V, dt), orc.softmax_av(s, Vrep, dt)), f"sav: GQA != MHA ({dt})"


def pin_sav_edges(orc):
    o = orc.softmax_av(torch.zeros(2, 0, 4), torch.zeros(2, 0, 2, 3, dtype=torch.bfloat16), "bf16")
    assert o.shape == (2, 4, 3) and (o == 0).all(), "sav: C = 0 must give zeros"
    o = orc.softmax_av(torch.zeros(0, 5, 4), torch.zeros(0, 5, 2, 3), "f32")
    assert o.shape == (0, 4, 3)
    s, V = make_scores_random(1, 6, 2, 1, 3, "f32", seed=731)
    s[0, :, 1] = float("-inf")
    o = orc.softmax_av(s, V, "f32")
    assert np.isnan(o[0, 1]).all() and np.isfinite(o[0, 0]).all(), "sav: a row of all -inf gives NaN"


def _paged_case(B, C, Hq, Hkv, D, P, dt, seed, lens=None):
    """Random weights, a shuffled page pool with spare pages, a block table and lengths."""
    g = torch.Generator().manual_seed(seed)
    max_pages = -(-C // P)
    num_pages = B * max_pages + 3
    s, _ = make_scores_random(B, C, Hq, Hkv, D, "f32", seed=seed)
    pages = torch.randn(num_pages, P, Hkv, D, generator=g).to({"f32": torch.float32, "f16": torch.float16,
                                                               "bf16": torch.bfloat16}[dt])
    perm = torch.randperm(num_pages, generator=g)[:B * max_pages].to(torch.int32)
    bt = perm.view(B, max_pages).contiguous()
    if lens is None:
        lens = torch.randint(0, C + 1, (B,), generator=g, dtype=torch.int32)
    return s, pages, bt, torch.as_tensor(lens, dtype=torch.int32)


def _gather(pages, bt, b, n):
    P = pages.shape[1]
    rows = [pages[int(bt[b, c // P]), c % P] for c in range(n)]
    return torch.stack(rows, 0) if rows else pages[:0, 0]


def pin_paged_gather(orc):
    for i, (B, C, Hq, Hkv, D, P, dt) in enumerate([(3, 50, 4, 2, 8, 16, "f32"), (2, 33, 6, 3, 5, 4, "bf16"),
                                                   (2, 64, 8, 1, 16, 8, "f16"), (1, 7, 2, 2, 3, 1, "f32")]):
        s, pages, bt, lens = _paged_case(B, C, Hq, Hkv, D, P, dt, seed=800 + i)
        lens[0] = C
        w = torch.softmax(s.double(), dim=1).float()
        for sm, x in ((False, w), (True, s)):
            o = orc.paged(x, pages, bt, lens, dt, softmax=sm)
            for b in range(B):
                n = int(lens[b])
                Vb = _gather(pages, bt, b, n).unsqueeze(0).contiguous()
                xb = x[b:b + 1, :n].contiguous()
                ref = orc.softmax_av(xb, Vb, dt) if sm else orc.full(xb, Vb, dt)
                assert np.array_equal(o[b], ref[0]), f"paged gather {dt} softmax={sm} b={b}"


def pin_paged_identity(orc):
    for dt in ("f32", "bf16"):
        B, C, Hq, Hkv, D = 3, 21, 6, 2, 7
        s, V = make_scores_random(B, C, Hq, Hkv, D, dt, seed=811)
        bt = torch.arange(B, dtype=torch.int32).view(B, 1)
        lens = torch.full((B,), C, dtype=torch.int32)
        w = torch.softmax(s.double(), dim=1).float()
        assert np.array_equal(orc.paged(w, V, bt, lens, dt), orc.full(w, V, dt)), f"paged identity {dt}"
        assert np.array_equal(orc.paged(s, V, bt, lens, dt, softmax=True), orc.softmax_av(s, V, dt)), \
            f"paged identity softmax {dt}"


def pin_paged_ignores_tail(orc):
    B, C, Hq, Hkv, D, P = 3, 40, 4, 2, 6, 8
    s, pages, bt, lens = _paged_case(B, C, Hq, Hkv, D, P, "f32", seed=821, lens=[17, 0, 40])
    for sm in (False, True):
        a = orc.paged(s, pages, bt, lens, "f32", softmax=sm)
        s2, p2 = s.clone(), pages.clone()
        s2[0, 17:] = 99.0
        s2[1] = -5.0
        used = {int(bt[b, c // P]) for b in range(B) for c in range(int(lens[b]))}
        for pg in range(pages.shape[0]):
            if pg not in used:
                p2[pg] = 1e30
        p2[int(bt[0, 17 // P]), 17 % P:] = -7.0            # rows 17.. of sequence 0's third page
        b2 = orc.paged(s2, p2, bt, lens, "f32", softmax=sm)
        assert np.array_equal(a, b2), f"paged: rows past a length must not count (softmax={sm})"
        assert (a[1] == 0).all(), "paged: a sequence of length 0 gives zeros"


def pin_paged_rejects(orc):
    B, C, Hq, Hkv, D, P = 2, 20, 4, 2, 4, 8
    s, pages, bt, lens = _paged_case(B, C, Hq, Hkv, D, P, "f32", seed=831, lens=[20, 9])
    for bad in ("page", "len", "neg", "capacity"):
        bt2, ln2, s2 = bt.clone(), lens.clone(), s
        if bad == "page":
            bt2[1, 1] = pages.shape[0]
        elif bad == "len":
            ln2[0] = C + 1
        elif bad == "neg":
            ln2[1] = -1
        else:
            s2 = torch.zeros(B, bt.shape[1] * P + 1, Hq)
        try:
            orc.paged(s2, pages, bt2, ln2, "f32")
        except ValueError:
            continue
        raise AssertionError(f"paged oracle accepted a bad {bad}")


def _fp8_case(B, C, Hq, Hkv, D, seed):
    g = torch.Generator().manual_seed(seed)
    raw = torch.randint(0, 256, (B, C, Hkv, D), generator=g, dtype=torch.uint8)
    raw[(raw & 0x7F) == 0x7F] = 0x3C                    # no NaN payloads in V
    s, _ = make_scores_random(B, C, Hq, Hkv, D, "f32", seed=seed)
    return s, raw


def pin_fp8_decode(orc):
    bits = torch.arange(256, dtype=torch.uint8)
    d = orc.decode_fp8(bits)
    ref = bits.view(torch.float8_e4m3fn).double().numpy()
    same = (d == ref) | (np.isnan(d) & np.isnan(ref))
    assert same.all(), f"fp8 decode differs from torch at {np.nonzero(~same)[0][:8]}"
    fixed = {0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x38: 1.0, 0x07: 7 * 2.0 ** -9, 0xC0: -2.0,
             0x77: 240.0}
    for k, v in fixed.items():
        assert d[k] == v, f"fp8 0x{k:02x}: {d[k]} != {v}"
    assert d[0x80] == 0.0 and math.copysign(1.0, d[0x80]) < 0, "fp8 0x80 is -0"
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF]), "fp8 S.1111.111 is NaN"


def pin_fp8_as_bf16(orc):
    for i, (B, C, Hq, Hkv, D) in enumerate([(2, 30, 6, 2, 8), (1, 17, 4, 4, 5), (2, 9, 8, 1, 3)]):
        s, raw = _fp8_case(B, C, Hq, Hkv, D, seed=900 + i)
        v16 = raw.view(torch.float8_e4m3fn).to(torch.bfloat16)
        w = torch.softmax(s.double(), dim=1).float()
        assert np.array_equal(orc.fp8(w, raw), orc.full(w, v16, "bf16")), "fp8 plain != bf16 oracle"
        assert np.array_equal(orc.fp8(s, raw, softmax=True), orc.softmax_av(s, v16, "bf16")), "fp8 softmax != bf16"


def pin_fp8_scales(orc):
    B, C, Hq, Hkv, D = 2, 21, 8, 4, 6
    s, raw = _fp8_case(B, C, Hq, Hkv, D, seed=911)
    G = Hq // Hkv
    base = orc.fp8(s, raw, softmax=True)
    sc = torch.tensor([0.25, 1.0, 8.0, 2.0 ** -10])
    o = orc.fp8(s, raw, sc, softmax=True)
    for q in range(Hq):
        assert np.array_equal(o[:, q], base[:, q] * float(sc[q // G])), f"fp8 scale of head {q}"
    sc2 = torch.ones(Hkv)
    sc2[2] = 3.0
    o2 = orc.fp8(s, raw, sc2)
    b2 = orc.fp8(s, raw)
    for q in range(Hq):
        if q // G != 2:
            assert np.array_equal(o2[:, q], b2[:, q]), "fp8: one head's scale leaked into another head"
    assert not np.array_equal(o2, b2)


def pin_qk_fp8_as_bf16(orc):
    for i, (B, C, Hq, Hkv, D) in enumerate([(2, 13, 6, 2, 16), (1, 7, 4, 4, 9), (2, 5, 8, 1, 32)]):
        q, _ = make_qk_random(B, C, Hq, Hkv, D, "f32", seed=930 + i)
        _, raw = _fp8_case(B, C, Hq, Hkv, D, seed=940 + i)
        k16 = raw.view(torch.float8_e4m3fn).to(torch.bfloat16)
        for scale in (1.0, 0.125, 0.3):
            a = orc.qk_fp8(q, raw, None, scale)
            b = orc.qk(q, k16, "bf16", scale)
            assert np.array_equal(a, b), f"fp8 scores != bf16 scores on the widened K (scale {scale})"


def pin_qk_fp8_brute(orc):
    from fractions import Fraction
    for i, (B, C, Hq, Hkv, D) in enumerate([(1, 3, 4, 2, 5), (2, 2, 3, 1, 4)]):
        q, _ = make_qk_random(B, C, Hq, Hkv, D, "f32", seed=950 + i)
        _, raw = _fp8_case(B, C, Hq, Hkv, D, seed=960 + i)
        kd = raw.view(torch.float8_e4m3fn).double()
        ks = torch.tensor([0.5, 3.0][:Hkv])
        out = orc.qk_fp8(q, raw, ks, 1.0)
        G = Hq // Hkv
        for b in range(B):
            for c in range(C):
                for h in range(Hq):
                    kv = h // G
                    terms = [Fraction(float(q[b, h, d])) * Fraction(float(kd[b, c, kv, d])) * Fraction(float(ks[kv]))
                             for d in range(D)]
                    exact, mag = sum(terms), sum(abs(t) for t in terms)
                    # D - 1 double additions in increasing d: |err| <= gamma_{D-1} * sum |terms|
                    assert abs(Fraction(out[b, c, h]) - exact) <= Fraction(gamma(D - 1)) * mag, \
                        f"fp8 score ({b}, {c}, {h}) not the exact sum"


def pin_qk_fp8_scales(orc):
    B, C, Hq, Hkv, D = 2, 11, 8, 4, 12
    q, _ = make_qk_random(B, C, Hq, Hkv, D, "f32", seed=971)
    _, raw = _fp8_case(B, C, Hq, Hkv, D, seed=972)
    G = Hq // Hkv
    base = orc.qk_fp8(q, raw, None, 0.25)
    sc = torch.tensor([0.25, 1.0, 8.0, 2.0 ** -10])
    o = orc.qk_fp8(q, raw, sc, 0.25)
    for h in range(Hq):
        assert np.array_equal(o[:, :, h], base[:, :, h] * float(sc[h // G])), f"fp8 k_scale of head {h}"
    sc2 = torch.ones(Hkv)
    sc2[1] = 3.0
    o2 = orc.qk_fp8(q, raw, sc2, 0.25)
    for h in range(Hq):
        if h // G != 1:
            assert np.array_equal(o2[:, :, h], base[:, :, h]), "fp8 k_scale leaked into another head"
    assert not np.array_equal(o2, base)


def _qk_paged_case(B, C, Hq, Hkv, D, P, dt, seed, lens):
    """Dense K scattered into shuffled pages (spare pages filled with 7.0),
    with the block table and lengths."""
    q, K = make_qk_random(B, C, Hq, Hkv, D, "f32" if dt == "fp8" else dt, seed=seed)
    if dt == "fp8":
        g = torch.Generator().manual_seed(seed + 1)
        K = torch.randint(0, 256, (B, C, Hkv, D), generator=g, dtype=torch.uint8)
        K[(K & 0x7F) == 0x7F] = 0x3C
    maxp = -(-C // P)
    npg = B * maxp + 3
    g = torch.Generator().manual_seed(seed + 2)
    perm = torch.randperm(npg, generator=g)[:B * maxp].to(torch.int32).view(B, maxp).contiguous()
    pages = torch.full((npg, P, Hkv, D), 7.0).to(K.dtype) if dt != "fp8" else \
        torch.full((npg, P, Hkv, D), 0x48, dtype=torch.uint8)
    for b in range(B):
        for k in range(maxp):
            rows = K[b, k * P:(k + 1) * P]
            pages[int(perm[b, k]), :rows.shape[0]] = rows
    return q, K, pages, perm, torch.tensor(lens, dtype=torch.int32)


def pin_qk_paged_gather(orc):
    for i, (dt, P) in enumerate([("bf16", 4), ("f16", 1), ("f32", 8), ("fp8", 2), ("bf16", 16)]):
        B, C, Hq, Hkv, D = 3, 13, 6, 2, 16
        lens = [13, 6, 0]
        q, K, pages, bt, ln = _qk_paged_case(B, C, Hq, Hkv, D, P, dt, seed=1000 + i, lens=lens)
        ks = torch.tensor([0.5, 4.0]) if dt == "fp8" else None
        out = orc.qk_paged(q, pages, bt, ln, dt, 0.25, ks, C=C)
        for b in range(B):
            n = lens[b]
            if n:
                dense = orc.qk_fp8(q[b:b + 1], K[b:b + 1, :n], ks, 0.25) if dt == "fp8" else \
                    orc.qk(q[b:b + 1], K[b:b + 1, :n], dt, 0.25)
                assert np.array_equal(out[b:b + 1, :n], dense), f"paged scores != dense ({dt}, P={P}, b={b})"
            assert np.isnan(out[b, n:]).all(), f"rows past the length must have no score ({dt}, b={b})"


def pin_qk_paged_identity(orc):
    for dt in ("bf16", "f32"):
        q, K = make_qk_random(2, 9, 4, 2, 12, dt, seed=1010)
        bt = torch.arange(2, dtype=torch.int32).view(2, 1)
        out = orc.qk_paged(q, K, bt, torch.tensor([9, 9], dtype=torch.int32), dt, 0.5)
        assert np.array_equal(out, orc.qk(q, K, dt, 0.5)), f"identity paging != dense ({dt})"


def pin_qk_paged_tail(orc):
    B, C, Hq, Hkv, D, P = 2, 11, 4, 2, 8, 4
    lens = [7, 11]
    q, K, pages, bt, ln = _qk_paged_case(B, C, Hq, Hkv, D, P, "bf16", seed=1020, lens=lens)
    base = orc.qk_paged(q, pages, bt, ln, "bf16", 1.0, C=C)
    p2 = pages.clone()
    used = {int(bt[b, c // P]) for b in range(B) for c in range(lens[b])}
    for pg in range(p2.shape[0]):
        if pg not in used:
            p2[pg] = -3.0
    p2[int(bt[0, 7 // P]), 7 % P:] = 99.0                  # sequence 0's rows 7.. (past its length)
    out = orc.qk_paged(q, p2, bt, ln, "bf16", 1.0, C=C)
    same = (out == base) | (np.isnan(out) & np.isnan(base))
    assert same.all(), "K past the length or in unused pages changed a score"


def pin_qk_paged_rejects(orc):
    q, K, pages, bt, ln = _qk_paged_case(2, 8, 4, 2, 8, 4, "bf16", seed=1030, lens=[8, 5])
    npg = pages.shape[0]
    for bad, args in (("page index", (bt.clone().fill_(npg), ln)), ("negative page", (bt.clone().fill_(-1), ln)),
                      ("length", (bt, torch.tensor([9, 5], dtype=torch.int32))),
                      ("negative length", (bt, torch.tensor([-1, 5], dtype=torch.int32)))):
        try:
            orc.qk_paged(q, pages, args[0], args[1], "bf16", 1.0, C=8)
        except ValueError:
            continue
        raise AssertionError(f"paged score oracle accepted a bad {bad}")
    try:
        orc.qk_paged(q, pages, bt, ln, "bf16", 1.0, C=9)       # capacity above max_pages * P
    except ValueError:
        return
    raise AssertionError("paged score oracle accepted C > max_pages * P")


def pin_attn_composition(orc):
    g = torch.Generator().manual_seed(1100)
    for dt in ("bf16", "f16", "f32"):
        B, C, Hq, Hkv, D = 2, 37, 6, 2, 16
        q = torch.randint(-8, 9, (B, Hq, D), generator=g).float() / 4.0
        K = torch.randint(-4, 5, (B, C, Hkv, D), generator=g).float().to({"bf16": torch.bfloat16,
                                                                           "f16": torch.float16,
                                                                           "f32": torch.float32}[dt])
        _, V = make_qk_random(B, C, Hq, Hkv, D, dt, seed=1101)
        scores = orc.qk(q, K, dt, 0.5)
        s32 = torch.from_numpy(scores).float()
        assert np.array_equal(s32.double().numpy(), scores), "dyadic scores must be exact in fp32"
        assert np.array_equal(orc.attention(q, K, V, dt, 0.5), orc.softmax_av(s32, V, dt)), f"attention != composition ({dt})"


def pin_attn_numpy(orc):
    from scipy.special import softmax
    for i, (B, C, Hq, Hkv, D, sc) in enumerate([(2, 29, 8, 2, 16, 0.25), (1, 40, 4, 4, 8, 1.0), (2, 9, 6, 3, 32, 40.0)]):
        q, K = make_qk_random(B, C, Hq, Hkv, D, "bf16", seed=1110 + i)
        _, V = make_qk_random(B, C, Hq, Hkv, D, "bf16", seed=1120 + i)
        G = Hq // Hkv
        qd, kd, vd = q.double().numpy(), K.double().numpy(), V.double().numpy()
        kq, vq = np.repeat(kd, G, axis=2), np.repeat(vd, G, axis=2)
        s_ = sc * np.einsum("bhd,bchd->bch", qd, kq)
        p_ = softmax(s_, axis=1)
        ref = np.einsum("bch,bchd->bhd", p_, vq)
        out = orc.attention(q, K, V, "bf16", sc)
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-12 * np.abs(vd).max()), f"attention vs numpy (case {i})"
        assert np.abs(s_).max() < 2000.0


def pin_attn_zero_q(orc):
    B, C, Hq, Hkv, D = 2, 50, 4, 2, 8
    _, K = make_qk_random(B, C, Hq, Hkv, D, "f32", seed=1130)
    _, V = make_qk_random(B, C, Hq, Hkv, D, "f32", seed=1131)
    out = orc.attention(torch.zeros(B, Hq, D), K, V, "f32", 1.0)
    mean = V.double().numpy().mean(axis=1)                       # [B, Hkv, D]
    ref = np.repeat(mean, Hq // Hkv, axis=1)
    assert np.allclose(out, ref, rtol=1e-14, atol=1e-15), "q = 0 must average V"


def pin_attn_repeat_mha(orc):
    B, C, Hq, Hkv, D = 2, 21, 6, 2, 12
    q, K = make_qk_random(B, C, Hq, Hkv, D, "bf16", seed=1140)
    _, V = make_qk_random(B, C, Hq, Hkv, D, "bf16", seed=1141)
    G = Hq // Hkv
    Kr = K.repeat_interleave(G, dim=2).contiguous()
    Vr = V.repeat_interleave(G, dim=2).contiguous()
    assert np.array_equal(orc.attention(q, K, V, "bf16", 0.3), orc.attention(q, Kr, Vr, "bf16", 0.3)), "GQA != MHA"


def pin_attn_edges(orc):
    q, K = make_qk_random(2, 0, 4, 2, 8, "bf16", seed=1150)
    V = K.clone()
    assert (orc.attention(q, K, V, "bf16", 1.0) == 0).all(), "C = 0 gives zeros"
    q0, K0 = make_qk_random(0, 5, 4, 2, 8, "bf16", seed=1151)
    assert orc.attention(q0, K0, K0.clone(), "bf16", 1.0).size == 0


def pin_attn_fp8_as_bf16(orc):
    for i, (B, C, Hq, Hkv, D) in enumerate([(2, 23, 6, 2, 16), (1, 40, 8, 1, 8)]):
        q, _ = make_qk_random(B, C, Hq, Hkv, D, "f32", seed=1200 + i)
        _, k8 = _fp8_case(B, C, Hq, Hkv, D, seed=1210 + i)
        _, v8 = _fp8_case(B, C, Hq, Hkv, D, seed=1220 + i)
        k16 = k8.view(torch.float8_e4m3fn).to(torch.bfloat16)
        v16 = v8.view(torch.float8_e4m3fn).to(torch.bfloat16)
        a = orc.attention_fp8(q, k8, v8, None, None, 0.05)
        assert np.array_equal(a, orc.attention(q, k16, v16, "bf16", 0.05)), f"fp8 attention != bf16 (case {i})"


def pin_attn_fp8_scales(orc):
    B, C, Hq, Hkv, D = 2, 19, 8, 4, 8
    q, _ = make_qk_random(B, C, Hq, Hkv, D, "f32", seed=1230)
    _, k8 = _fp8_case(B, C, Hq, Hkv, D, seed=1231)
    _, v8 = _fp8_case(B, C, Hq, Hkv, D, seed=1232)
    G = Hq // Hkv
    base = orc.attention_fp8(q, k8, v8, None, None, 0.02)
    vs = torch.tensor([0.25, 1.0, 8.0, 2.0 ** -10])
    o = orc.attention_fp8(q, k8, v8, None, vs, 0.02)
    for h in range(Hq):
        assert np.array_equal(o[:, h], base[:, h] * float(vs[h // G])), f"fp8 attention v_scale of head {h}"
    k16 = k8.view(torch.float8_e4m3fn).to(torch.bfloat16)
    v16 = v8.view(torch.float8_e4m3fn).to(torch.bfloat16)
    for ks in (0.5, 4.0):
        o2 = orc.attention_fp8(q, k8, v8, torch.full((Hkv,), ks), None, 0.02)
        assert np.array_equal(o2, orc.attention(q, k16, v16, "bf16", 0.02 * ks)), f"fp8 attention k_scale {ks}"


def _attn_paged_case(B, C, Hq, Hkv, D, P, dt, seed, lens):
    """q, two shuffled page pools (K and V, with spare pages) sharing one block
    table, the lengths, and the dense K and V the table describes."""
    g = torch.Generator().manual_seed(seed)
    max_pages = -(-C // P)
    num_pages = B * max_pages + 2
    q, _ = make_qk_random(B, C, Hq, Hkv, D, "f32", seed=seed)
    pools = []
    for _ in range(2):
        if dt == "fp8":
            raw = torch.randint(0, 256, (num_pages, P, Hkv, D), generator=g, dtype=torch.uint8)
            raw[(raw & 0x7F) == 0x7F] = 0x3C                # no NaN payloads
            pools.append(raw)
        else:
            pools.append(torch.randn(num_pages, P, Hkv, D, generator=g).to(
                {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dt]))
    perm = torch.randperm(num_pages, generator=g)[:B * max_pages].to(torch.int32)
    bt = perm.view(B, max_pages).contiguous()
    K = torch.stack([_gather(pools[0], bt, b, C) for b in range(B)], 0)
    V = torch.stack([_gather(pools[1], bt, b, C) for b in range(B)], 0)
    return q, pools[0], pools[1], bt, torch.as_tensor(lens, dtype=torch.int32), K, V


def pin_attn_paged_gather(orc):
    """Paged attention equals dense attention on each sequence's first len rows
    gathered through the table, bit for bit; length 0 gives zeros."""
    for i, (dt, P) in enumerate([("bf16", 4), ("f16", 1), ("f32", 8), ("fp8", 2), ("bf16", 16)]):
        B, C, Hq, Hkv, D = 3, 13, 6, 2, 16
        lens = [13, 6, 0]
        q, kp, vp, bt, ln, K, V = _attn_paged_case(B, C, Hq, Hkv, D, P, dt, seed=1300 + i, lens=lens)
        ks, vs = (torch.tensor([0.5, 0.01]), torch.tensor([4.0, 0.25])) if dt == "fp8" else (None, None)
        sc = 0.003 if dt == "fp8" else 0.25
        out = orc.attention_paged(q, kp, vp, bt, ln, dt, sc, ks, vs, C=C)
        for b in range(B):
            n = lens[b]
            if n:
                dense = orc.attention_fp8(q[b:b + 1], K[b:b + 1, :n], V[b:b + 1, :n], ks, vs, sc) if dt == "fp8" \
                    else orc.attention(q[b:b + 1], K[b:b + 1, :n], V[b:b + 1, :n], dt, sc)
                assert np.array_equal(out[b:b + 1], dense), f"paged attention != dense ({dt}, P={P}, b={b})"
            else:
                assert (out[b] == 0).all(), f"length 0 gives zeros ({dt})"


def pin_attn_paged_tail(orc):
    """K and V rows past a length, and pages no table entry uses, take no part:
    NaN there leaves every output as it was."""
    B, C, Hq, Hkv, D, P = 2, 11, 4, 2, 8, 4
    lens = [7, 11]
    q, kp, vp, bt, ln, _, _ = _attn_paged_case(B, C, Hq, Hkv, D, P, "bf16", seed=1320, lens=lens)
    base = orc.attention_paged(q, kp, vp, bt, ln, "bf16", 0.5, C=C)
    used = {int(bt[b, c // P]) for b in range(B) for c in range(lens[b])}
    k2, v2 = kp.clone(), vp.clone()
    for t in (k2, v2):
        for pg in range(t.shape[0]):
            if pg not in used:
                t[pg] = float("nan")
        t[int(bt[0, 7 // P]), 7 % P:] = float("nan")        # sequence 0's rows 7.. (past its length)
    out = orc.attention_paged(q, k2, v2, bt, ln, "bf16", 0.5, C=C)
    assert np.array_equal(out, base), "K or V past the length or in unused pages changed an output"


def pin_attn_paged_rejects(orc):
    q, kp, vp, bt, ln, _, _ = _attn_paged_case(2, 8, 4, 2, 8, 4, "bf16", seed=1330, lens=[8, 5])
    npg = kp.shape[0]
    for bad, args in (("page index", (bt.clone().fill_(npg), ln)), ("negative page", (bt.clone().fill_(-1), ln)),
                      ("length", (bt, torch.tensor([9, 5], dtype=torch.int32))),
                      ("negative length", (bt, torch.tensor([-1, 5], dtype=torch.int32)))):
        try:
            orc.attention_paged(q, kp, vp, args[0], args[1], "bf16", 1.0, C=8)
        except ValueError:
            continue
        raise AssertionError(f"paged attention oracle accepted a bad {bad}")
    try:
        orc.attention_paged(q, kp, vp, bt, ln, "bf16", 1.0, C=9)
    except ValueError:
        return
    raise AssertionError("paged attention oracle accepted a capacity above max_pages * P")


ALL_PINS = [pin_decode_table, pin_brute_force, pin_mha_einsum, pin_repeat_mha, pin_constant_v,
            pin_one_hot, pin_linearity, pin_permutation, pin_batch_independence, pin_points,
            pin_edges, pin_qk_brute_force, pin_qk_mha_einsum, pin_qk_repeat_mha, pin_qk_one_hot,
            pin_qk_scale_linear, pin_qk_composition, pin_qk_edges, pin_sav_library, pin_sav_shift,
            pin_sav_large, pin_sav_one_hot, pin_sav_uniform, pin_sav_two_rows, pin_sav_mask,
            pin_sav_repeat_mha, pin_sav_edges, pin_paged_gather, pin_paged_identity, pin_paged_ignores_tail,
            pin_paged_rejects, pin_fp8_decode, pin_fp8_as_bf16, pin_fp8_scales, pin_qk_fp8_as_bf16,
            pin_qk_fp8_brute, pin_qk_fp8_scales, pin_qk_paged_gather, pin_qk_paged_identity, pin_qk_paged_tail,
            pin_qk_paged_rejects, pin_attn_composition, pin_attn_numpy, pin_attn_zero_q, pin_attn_repeat_mha,
            pin_attn_edges, pin_attn_fp8_as_bf16, pin_attn_fp8_scales, pin_attn_paged_gather, pin_attn_paged_tail,
            pin_attn_paged_rejects]
