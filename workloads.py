"""Seeded synthetic inputs for the GQA decode attention-times-V contraction.

This module only draws inputs. It holds none of the contraction's arithmetic, so
both the CPU oracle (``oracle/``) and the HIP path can take their inputs from it
without sharing any part of the computation under test.

Shapes follow the decode setting of ExecuTorch PR #21063 (GQA-reuse AV coop
GEMV), introduction: ``Hq = G * Hkv`` query heads share each KV head, with the
Llama (G=4), Phi (G=3) and Qwen (G=2) ratios it names, plus the low-ratio and
high-ratio MQA cases its dispatch bullet discusses.

Layouts (dense, row-major):
  attn [B, C, Hq]      float32, softmax over c of Gaussian logits
                       (make_scores hands over the logits themselves, the
                       input of the fused softmax product)
  V    [B, C, Hkv, D]  float32 / float16 / bfloat16 (drawn in fp32, rounded RNE)

Draw order on one CPU ``torch.Generator`` seeded with ``seed``: V values, then
logits, then the outlier row permutation (only when ``outlier_frac > 0``).
The softmax that turns logits into weights is computed in float64 and rounded
to float32; it is input preparation, not part of the contraction.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Tuple

import torch

_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    C: int
    Hq: int
    Hkv: int
    D: int
    v_dtype: str            # "f32" | "f16" | "bf16"
    v_dist: str             # "uniform" (U(-1,1)) | "normal"
    v_std: float = 1.0      # std for "normal"
    logit_std: float = 1.0
    ramp: float = 0.0       # additive logit ramp: 0 at c=0 up to `ramp` at c=C-1
    outlier_frac: float = 0.0   # fraction of (b, c, kv_h) rows scaled by outlier_scale
    outlier_scale: float = 1.0
    description: str = ""

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def v_torch_dtype(self) -> torch.dtype:
        return _DTYPES[self.v_dtype]

    @property
    def v_elem_bytes(self) -> int:
        return 4 if self.v_dtype == "f32" else 2

    def v_bytes(self) -> int:
        return self.B * self.C * self.Hkv * self.D * self.v_elem_bytes

    def attn_bytes(self) -> int:
        return self.B * self.C * self.Hq * 4

    def out_bytes(self) -> int:
        return self.B * self.Hq * self.D * 4

    def algorithmic_bytes(self) -> int:
        """V, attn and out each moved once: the reuse path's minimum traffic."""
        return self.v_bytes() + self.attn_bytes() + self.out_bytes()

    def per_head_bytes(self) -> int:
        """Traffic when every query head re-reads its KV head's V rows."""
        return self.G * self.v_bytes() + self.attn_bytes() + self.out_bytes()

    def flops(self) -> int:
        return 2 * self.B * self.C * self.Hq * self.D

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The six decode workloads, named by what they are and their sizes.
WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    Workload("tiny-f32-b1-c256-hq8-hkv2-d64", B=1, C=256, Hq=8, Hkv=2, D=64,
             v_dtype="f32", v_dist="uniform", logit_std=1.0,
             description="tiny GQA decode, fp32 V ~ U(-1,1), N(0,1) logits"),
    Workload("llama3-8b-b1-c4096-hq32-hkv8-d128-bf16", B=1, C=4096, Hq=32, Hkv=8, D=128,
             v_dtype="bf16", v_dist="normal", v_std=1.0, logit_std=2.0,
             description="Llama-3-8B-shaped decode step, bf16 V ~ N(0,1), N(0,2^2) logits"),
    Workload("g3-b8-c16384-hq24-hkv8-d96-f16", B=8, C=16384, Hq=24, Hkv=8, D=96,
             v_dtype="f16", v_dist="normal", v_std=0.5, logit_std=1.0, ramp=3.0,
             description="G=3 grouping, 8 sequences, fp16 V ~ N(0,0.5^2), N(0,1) logits + linear ramp to +3"),
    Workload("g2-b4-c32768-hq16-hkv8-d128-bf16", B=4, C=32768, Hq=16, Hkv=8, D=128,
             v_dtype="bf16", v_dist="normal", v_std=1.0, logit_std=1.0,
             description="G=2 long context, bf16 V ~ N(0,1), N(0,1) logits"),
    Workload("mqa16-b4-c32768-hq16-hkv1-d128-bf16", B=4, C=32768, Hq=16, Hkv=1, D=128,
             v_dtype="bf16", v_dist="normal", v_std=1.0, logit_std=1.0,
             description="MQA (G=16) long context, bf16 V ~ N(0,1), N(0,1) logits"),
    Workload("batch64-b64-c8192-hq64-hkv8-d128-bf16", B=64, C=8192, Hq=64, Hkv=8, D=128,
             v_dtype="bf16", v_dist="normal", v_std=1.0, logit_std=3.0,
             outlier_frac=0.01, outlier_scale=10.0,
             description="large-batch decode G=8, bf16 V ~ N(0,1) with 1% of rows x10, N(0,3^2) logits"),
]}

TINY = "tiny-f32-b1-c256-hq8-hkv2-d64"
LLAMA = "llama3-8b-b1-c4096-hq32-hkv8-d128-bf16"
G3 = "g3-b8-c16384-hq24-hkv8-d96-f16"
G2_LONG = "g2-b4-c32768-hq16-hkv8-d128-bf16"
MQA_LONG = "mqa16-b4-c32768-hq16-hkv1-d128-bf16"
BATCH64 = "batch64-b64-c8192-hq64-hkv8-d128-bf16"


def _softmax_over_c(logits: torch.Tensor) -> torch.Tensor:
    """Normalise [B, C, Hq] logits over c (dim 1) in float64, round to float32."""
    x = logits.to(torch.float64)
    x = x - x.amax(dim=1, keepdim=True)
    e = torch.exp(x)
    return (e / e.sum(dim=1, keepdim=True)).to(torch.float32)


def _draw(w: Workload, seed: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """(logits [B, C, Hq] fp32, V) for workload ``w`` in the fixed draw order."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    nv = w.B * w.C * w.Hkv * w.D
    if w.v_dist == "uniform":
        v = torch.rand(nv, generator=g, dtype=torch.float32) * 2.0 - 1.0
    elif w.v_dist == "normal":
        v = torch.randn(nv, generator=g, dtype=torch.float32) * w.v_std
    else:
        raise ValueError(f"unknown v_dist {w.v_dist!r}")
    logits = torch.randn(w.B, w.C, w.Hq, generator=g, dtype=torch.float32) * w.logit_std
    if w.ramp != 0.0 and w.C > 1:
        r = torch.arange(w.C, dtype=torch.float32) * (w.ramp / (w.C - 1))
        logits = logits + r.view(1, w.C, 1)
    if w.outlier_frac > 0.0:
        nrows = w.B * w.C * w.Hkv
        k = int(round(w.outlier_frac * nrows))
        rows = torch.randperm(nrows, generator=g)[:k]
        v.view(nrows, w.D)[rows] *= w.outlier_scale
    V = v.view(w.B, w.C, w.Hkv, w.D).to(w.v_torch_dtype)
    return logits.contiguous(), V.contiguous()


def make_inputs(w: Workload, seed: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """Draw (attn, V) on the CPU for workload ``w`` with a fixed draw order."""
    logits, V = _draw(w, seed)
    attn = _softmax_over_c(logits) if w.C > 0 else logits
    return attn.contiguous(), V


def make_scores(w: Workload, seed: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """(scores, V) for the fused softmax product: the same draws as make_inputs,
    with the logits handed over as they are (no softmax)."""
    return _draw(w, seed)


def make_scores_random(B: int, C: int, Hq: int, Hkv: int, D: int, v_dtype: str, seed: int = 0,
                       score_std: float = 1.0) -> Tuple[torch.Tensor, torch.Tensor]:
    """Small ad-hoc shapes for the fused product: V ~ N(0,1), scores ~ N(0, score_std^2)."""
    w = Workload(f"adhoc-b{B}-c{C}-hq{Hq}-hkv{Hkv}-d{D}-{v_dtype}", B=B, C=C, Hq=Hq, Hkv=Hkv, D=D,
                 v_dtype=v_dtype, v_dist="normal", logit_std=score_std)
    return _draw(w, seed)


def make_random(B: int, C: int, Hq: int, Hkv: int, D: int, v_dtype: str,
                seed: int = 0, attn_kind: str = "softmax") -> Tuple[torch.Tensor, torch.Tensor]:
    """Small ad-hoc shapes for sweeps: V ~ N(0,1), attn softmax of N(0,1) or raw N(0,1)."""
    w = Workload(f"adhoc-b{B}-c{C}-hq{Hq}-hkv{Hkv}-d{D}-{v_dtype}", B=B, C=C, Hq=Hq, Hkv=Hkv, D=D,
                 v_dtype=v_dtype, v_dist="normal")
    attn, V = make_inputs(w, seed)
    if attn_kind == "signed":
        g = torch.Generator(device="cpu").manual_seed(seed + 7919)
        attn = torch.randn(B, C, Hq, generator=g, dtype=torch.float32)
    return attn, V


def make_qk_random(B: int, C: int, Hq: int, Hkv: int, D: int, k_dtype: str,
                   seed: int = 0, q_std: float = 1.0) -> Tuple[torch.Tensor, torch.Tensor]:
    """Inputs of the decode score step: q [B, Hq, D] fp32 ~ N(0, q_std^2) and the
    K cache [B, C, Hkv, D] ~ N(0, 1) rounded to k_dtype. Drawn in this order on
    one CPU generator; no arithmetic of the method."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    K = torch.randn(B, C, Hkv, D, generator=g, dtype=torch.float32)
    q = torch.randn(B, Hq, D, generator=g, dtype=torch.float32) * q_std
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[k_dtype]
    return q.contiguous(), K.to(dt).contiguous()
