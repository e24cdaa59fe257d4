"""Acceptance gates comparing a GPU fp32 output with the fp64 oracle.

Gate (the tolerance the contraction is held to):
  * fp32 V:       max |out - ref| <= 1e-5 * max |ref| + 1e-6
  * bf16/fp16 V:  ||out - ref||_2 / ||ref||_2 <= 2e-3
Both sides read the same rounded inputs, so the only difference should be fp32
accumulation order. That is checked too, with a bound derived from the
arithmetic: a sum of C fp32 terms in any order has relative error of order
sqrt(C) * 2^-24 for random-sign rounding; ``accum_bound`` allows 8x that.
A kernel that rounded the fp32 weights to bf16 (relative error ~1e-3) passes
the 2e-3 gate but fails this one.
"""
from __future__ import annotations

import math

import numpy as np

U32 = 2.0 ** -24


def rel_l2(out: np.ndarray, ref: np.ndarray) -> float:
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.linalg.norm(ref.ravel()))
    num = float(np.linalg.norm((out - ref).ravel()))
    if den == 0.0:
        return 0.0 if num == 0.0 else math.inf
    return num / den


def max_abs(out: np.ndarray, ref: np.ndarray) -> float:
    d = np.abs(np.asarray(out, np.float64) - np.asarray(ref, np.float64))
    return float(d.max()) if d.size else 0.0


def accum_bound(C: int) -> float:
    return 8.0 * math.sqrt(max(C, 1)) * U32 + 1e-7


def gate(out: np.ndarray, ref: np.ndarray, v_dtype: str) -> tuple[bool, str]:
    """The official acceptance test. Returns (passed, description)."""
    if out.shape != ref.shape:
        return False, f"shape {out.shape} != {ref.shape}"
    if not np.all(np.isfinite(out)):
        return False, "non-finite output"
    if v_dtype == "f32":
        m = max_abs(out, ref)
        bound = 1e-5 * (float(np.abs(ref).max()) if ref.size else 0.0) + 1e-6
        return m <= bound, f"max|err|={m:.3e} bound={bound:.3e}"
    r = rel_l2(out, ref)
    return r <= 2e-3, f"relL2={r:.3e} bound=2e-3"


def assert_parity(out: np.ndarray, ref: np.ndarray, v_dtype: str, C: int, label: str = ""):
    ok, msg = gate(out, ref, v_dtype)
    assert ok, f"{label}: gate failed: {msg}"
    r = rel_l2(out, ref)
    assert r <= accum_bound(C), f"{label}: relL2={r:.3e} above fp32-accumulation bound {accum_bound(C):.3e}"
