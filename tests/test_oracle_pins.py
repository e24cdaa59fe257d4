"""CPU tests: the oracle against its pins, and planted mistakes that the pins catch.

A planted mistake is a textual edit of the oracle's C source, compiled into a
temporary library. Each one is a plausible slip (wrong head mapping, a dropped
row, a wrong decoder constant, a sign, a transposed or batch-less index) and
must fail at least one pin; the pins are useless otherwise.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
from tests import oracle_pins
from tests.parity import gate
from workloads import WORKLOADS, make_inputs


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, oracle_lib):
    pin(oracle_lib)


# (name, original text, planted text) -- every original must occur in the source.
PLANTS = [
    ("kv_mod_mapping", "const int64_t kv = q / G;", "const int64_t kv = q % Hkv;"),
    ("drop_last_row", "for (int64_t c = 0; c < C; ++c) {", "for (int64_t c = 0; c < C - 1; ++c) {"),
    ("bf16_shift", "uint32_t u = (uint32_t)h << 16;", "uint32_t u = (uint32_t)h << 15;"),
    ("f16_subnormal_scale", "v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);"),
    ("f16_bias", "v = ldexp((double)(m + 1024), e - 25);", "v = ldexp((double)(m + 1024), e - 24);"),
    ("f16_no_sign", "return sign ? -v : v;", "return v;"),
    ("sign_flip", "acc[d] += a * orc_bf16(r[d]);", "acc[d] -= a * orc_bf16(r[d]);"),
    ("attn_transposed", "const double a = (double)attn[(b * C + c) * Hq + q];",
     "const double a = (double)attn[(b * Hq + q) * C + c];"),
    ("v_ignores_batch", "const int64_t row = ((b * C + c) * Hkv + kv) * D;",
     "const int64_t row = ((0 * C + c) * Hkv + kv) * D;"),
    ("f32_as_float_sum", "for (int64_t d = 0; d < D; ++d) acc[d] += a * orc_f32(r + d);",
     "for (int64_t d = 0; d < D; ++d) acc[d] += (float)(a * orc_f32(r + d));"),
    ("points_wrong_head", "const int64_t kv = q / G;\n        double acc = 0.0;",
     "const int64_t kv = q / G + (q % G == 1);\n        double acc = 0.0;"),
    ("qk_kv_mod_mapping", "const int64_t kvh = h / G;", "const int64_t kvh = h % Hkv;"),
    ("qk_drop_last_d", "for (int64_t d = 0; d < D; ++d) dot +=", "for (int64_t d = 0; d < D - 1; ++d) dot +="),
    ("qk_no_scale", "out[h] = dot * scale;", "out[h] = dot;"),
    ("qk_q_of_head_zero", "const float *qrow = q + (b * Hq + h) * D;", "const float *qrow = q + (b * Hq + 0) * D;"),
    ("qk_out_transposed", "orc_qk_row(q, K, dtype, C, Hq, Hkv, D, i / C, i % C, scale, out + i * Hq);",
     "orc_qk_row(q, K, dtype, C, Hq, Hkv, D, i % B, i / B, scale, out + i * Hq);"),
    ("qk_k_ignores_batch", "const int64_t krow = ((b * C + c) * Hkv + kvh) * D;",
     "const int64_t krow = ((0 * C + c) * Hkv + kvh) * D;"),
    ("sav_no_max", "const double e = exp((double)scores[(b * C + c) * Hq + q] - m);",
     "const double e = exp((double)scores[(b * C + c) * Hq + q]);"),
    ("sav_normalise_by_C", "for (int64_t d = 0; d < D; ++d) acc[d] /= l;",
     "for (int64_t d = 0; d < D; ++d) acc[d] /= (double)C;"),
    ("sav_scores_transposed", "const double e = exp((double)scores[(b * C + c) * Hq + q] - m);",
     "const double e = exp((double)scores[(b * Hq + q) * C + c] - m);"),
    ("sav_kv_mod", "const int64_t kv = q / G;\n    for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;\n    if (C == 0) return;",
     "const int64_t kv = q % Hkv;\n    for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;\n    if (C == 0) return;"),
    ("sav_drop_last_row", "for (int64_t c = 0; c < C; ++c) {\n        const double e",
     "for (int64_t c = 0; c < C - 1; ++c) {\n        const double e"),
    ("sav_weight_sum_squared", "l += e;", "l += e * e;"),
    ("sav_max_is_first", "if (s > m) m = s;", "if (c == 0) m = s;"),
    # (paged plants keep every access inside the arrays: a mutant runs in this process)
    ("paged_bt_no_row_stride", "const int64_t page = bt[b * max_pages + c / P];",
     "const int64_t page = bt[b + c / P];"),
    ("paged_reversed_in_page", "const int64_t row = ((page * P + c % P) * Hkv + kv) * D;",
     "const int64_t row = ((page * P + (P - 1 - c % P)) * Hkv + kv) * D;"),
    ("paged_ignores_len", "for (int64_t c = 0; c < len; ++c) {\n        const double x",
     "for (int64_t c = 0; c < C; ++c) {\n        const double x"),
    ("fp8_bias_8", "else v = ldexp((double)(8 + m), e - 10);", "else v = ldexp((double)(8 + m), e - 11);"),
    ("fp8_subnormal_scale", "if (e == 0) v = ldexp((double)m, -9);", "if (e == 0) v = ldexp((double)m, -10);"),
    ("fp8_no_sign", "    return sign ? -v : v;\n}\n\n/* Widen n fp8", "    return v;\n}\n\n/* Widen n fp8"),
    ("fp8_scale_of_query_head", "const double sc = v_scale ? (double)v_scale[kv] : 1.0;",
     "const double sc = v_scale ? (double)v_scale[q % Hkv] : 1.0;"),
    ("fp8_scale_ignored", "acc[d] += a * (orc_e4m3(r[d]) * sc);", "acc[d] += a * orc_e4m3(r[d]);"),
    ("qk_fp8_scale_ignored", "dot += (double)qrow[d] * (orc_e4m3(krow[d]) * ks);",
     "dot += (double)qrow[d] * orc_e4m3(krow[d]);"),
    ("qk_fp8_scale_of_query_head", "const double ks = k_scale ? (double)k_scale[kvh] : 1.0;",
     "const double ks = k_scale ? (double)k_scale[h % Hkv] : 1.0;"),
    ("qk_fp8_no_outer_scale", "out[h] = dot * scale;\n    }\n}\n\nint gqa_qk_fp8_oracle",
     "out[h] = dot;\n    }\n}\n\nint gqa_qk_fp8_oracle"),
    ("qk_fp8_wrong_kv_head", "const uint8_t *krow = K + ((b * C + c) * Hkv + kvh) * D;",
     "const uint8_t *krow = K + ((b * C + c) * Hkv + (Hkv - 1 - kvh)) * D;"),
    ("qk_paged_no_row_stride", "const int64_t page = block_table[b * max_pages + c / P];\n        for (int64_t h",
     "const int64_t page = block_table[b + c / P];\n        for (int64_t h"),
    ("qk_paged_reversed_in_page", "const int64_t row = ((page * P + c % P) * Hkv + kvh) * D;",
     "const int64_t row = ((page * P + (P - 1 - c % P)) * Hkv + kvh) * D;"),
    ("qk_paged_ignores_len", "if (c >= seq_lens[b]) {", "if (c >= C) {"),
    ("qk_paged_fp8_no_scale", "dot += (double)qrow[d] * (orc_e4m3(kr[d]) * ks);", "dot += (double)qrow[d] * orc_e4m3(kr[d]);"),
    ("attn_max_unscaled", "const double sc = dot * scale;\n            if (sc > m) m = sc;",
     "const double sc = dot;\n            if (sc > m) m = sc;"),
    ("attn_exp_unscaled", "const double e = exp(dot * scale - m);", "const double e = exp(dot - m);"),
    ("attn_no_max", "const double e = exp(dot * scale - m);", "const double e = exp(dot * scale);"),
    ("attn_v_from_k", "o[d] += e * orc_load(V, dtype, krow + d);", "o[d] += e * orc_load(K, dtype, krow + d);"),
    ("attn_kv_of_query", "const int64_t b = i / Hq, h = i % Hq, kv = h / G;", "const int64_t b = i / Hq, h = i % Hq, kv = h % Hkv;"),
    ("attn_fp8_v_scale_of_k", "const double vs = v_scale ? (double)v_scale[kv] : 1.0;",
     "const double vs = k_scale ? (double)k_scale[kv] : 1.0;"),
    ("attn_fp8_k_unscaled", "for (int64_t d = 0; d < D; ++d) dot += (double)qrow[d] * (orc_e4m3(kr[d]) * ks);\n            const double e",
     "for (int64_t d = 0; d < D; ++d) dot += (double)qrow[d] * orc_e4m3(kr[d]);\n            const double e"),
    ("paged_bt_ignores_batch", "const int64_t page = bt[b * max_pages + c / P];",
     "const int64_t page = bt[0 * max_pages + c / P];"),
    ("attn_paged_v_from_k_pool", "o[d] += e * orc_kv_elem(v_pages, dtype, v_scale, kv, row + d);",
     "o[d] += e * orc_kv_elem(k_pages, dtype, v_scale, kv, row + d);"),
    ("attn_paged_v_scale_of_k", "o[d] += e * orc_kv_elem(v_pages, dtype, v_scale, kv, row + d);",
     "o[d] += e * orc_kv_elem(v_pages, dtype, k_scale, kv, row + d);"),
    ("attn_paged_sum_past_len", "double l = 0.0;\n        for (int64_t c = 0; c < len; ++c) {",
     "double l = 0.0;\n        for (int64_t c = 0; c < C; ++c) {"),
    ("attn_paged_bt_no_row_stride",
     "const int64_t page = block_table[b * max_pages + c / P];\n            const int64_t row = ((page * P + c % P) * Hkv"
     " + kv) * D;\n            double dot = 0.0;\n            for (int64_t d = 0; d < D; ++d) dot += (double)qrow[d] * "
     "orc_kv_elem(k_pages, dtype, k_scale, kv, row + d);\n            const double e",
     "const int64_t page = block_table[b + c / P];\n            const int64_t row = ((page * P + c % P) * Hkv"
     " + kv) * D;\n            double dot = 0.0;\n            for (int64_t d = 0; d < D; ++d) dot += (double)qrow[d] * "
     "orc_kv_elem(k_pages, dtype, k_scale, kv, row + d);\n            const double e"),
    ("attn_paged_elem_unscaled", "return orc_e4m3(((const uint8_t *)pages)[i]) * (sc ? (double)sc[kv] : 1.0);",
     "return orc_e4m3(((const uint8_t *)pages)[i]);"),
]


@pytest.mark.parametrize("name,orig,planted", PLANTS, ids=[p[0] for p in PLANTS])
def test_planted_mistake_is_caught(name, orig, planted, tmp_path):
    src = open(oracle.SRC).read()
    assert orig in src, f"plant {name}: pattern no longer in the oracle source"
    # kv_mod_mapping touches both places the mapping is written
    mutated = src.replace(orig, planted) if name == "kv_mod_mapping" else src.replace(orig, planted, 1)
    if name == "points_wrong_head":
        assert mutated != src
    p_src = tmp_path / f"{name}.c"
    p_src.write_text(mutated)
    lib = oracle.build(str(p_src), str(tmp_path / f"lib{name}.so"))
    mutant = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name} passed every pin"


def _drop_one_row_per_split(attn: torch.Tensor, nsplit: int) -> torch.Tensor:
    """Zero the last context row of each of nsplit equal C-splits."""
    a = attn.clone()
    C = a.shape[1]
    step = max(1, -(-C // nsplit))
    last = [min(s + step, C) - 1 for s in range(0, C, step)]
    a[:, last, :] = 0.0
    return a


@pytest.mark.slow
@pytest.mark.parametrize("wname", list(WORKLOADS))
def test_gate_bites_on_dropped_row(wname, oracle_lib):
    """A result missing one context row per split must fail the acceptance gate.

    Planted in the oracle's input on the CPU. The large-batch workload is cut to
    8 sequences: the relative error of a dropped row depends on C, not on B.
    """
    w = WORKLOADS[wname]
    if w.B > 8:
        w = w.replace(B=8)
    attn, V = make_inputs(w, seed=0)
    ref = oracle_lib.full(attn, V, w.v_dtype)
    bad = oracle_lib.full(_drop_one_row_per_split(attn, 1), V, w.v_dtype)
    ok, msg = gate(bad.astype(np.float32), ref, w.v_dtype)
    assert not ok, f"{wname}: dropping one row passed the gate ({msg})"
    ok, msg = gate(ref.astype(np.float32), ref, w.v_dtype)
    assert ok, f"{wname}: the exact result rounded to fp32 fails the gate ({msg})"


def test_oracle_header_declares_test_infrastructure():
    head = open(oracle.SRC).read(600)
    assert "TEST INFRASTRUCTURE" in head
    assert "TEST INFRASTRUCTURE" in open(os.path.join(os.path.dirname(oracle.SRC), "__init__.py")).read() or \
        "test infrastructure" in open(os.path.join(os.path.dirname(oracle.SRC), "__init__.py")).read()
