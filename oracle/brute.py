"""Correctly rounded brute force for tiny shapes (test infrastructure).

Follows the definition of ExecuTorch PR #21063, "...GEMV", introduction
(out[q_h, d] as a sum over c of attn[c, q_h] * V[c, kv_h, d], groups of
G = Hq / Hkv query heads per KV head) with a batch index in front.

Independent of ``gqa_av_oracle.c`` by construction:
  * V is widened by torch's own dtype conversion, not by the C decoders;
  * every product of two values with at most 24 significand bits is exact in
    a Python float (53 bits), and ``math.fsum`` returns the correctly rounded
    sum of its inputs, so each element is the exact result rounded once.
Pure Python loops: only for shapes with a few thousand products per element.
"""
from __future__ import annotations

import math

import numpy as np
import torch


def brute_force(attn: torch.Tensor, V: torch.Tensor) -> np.ndarray:
    """out[B, Hq, D] as float64, correctly rounded from the exact sum."""
    a = attn.detach().cpu().to(torch.float64).tolist()   # [B][C][Hq]
    v = V.detach().cpu().to(torch.float64).tolist()      # [B][C][Hkv][D]
    B, C, Hq = attn.shape
    Hkv, D = V.shape[2], V.shape[3]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        for q in range(Hq):
            kv = q // G
            for d in range(D):
                out[b, q, d] = math.fsum(a[b][c][q] * v[b][c][kv][d] for c in range(C))
    return out


def abs_sum(attn: torch.Tensor, V: torch.Tensor) -> np.ndarray:
    """sum_c |attn * V| per output element (scale for the oracle's error bound)."""
    a = attn.detach().cpu().to(torch.float64).numpy()
    v = V.detach().cpu().to(torch.float64).numpy()
    G = a.shape[2] // v.shape[2]
    vq = np.repeat(v, G, axis=2)                       # [B, C, Hq, D]
    return np.einsum("bch,bchd->bhd", np.abs(a), np.abs(vq))


def brute_force_qk(q: torch.Tensor, K: torch.Tensor, scale: float) -> np.ndarray:
    """scores[B, C, Hq] as float64: the exact sum over d rounded once, times scale."""
    qa = q.detach().cpu().to(torch.float64).tolist()     # [B][Hq][D]
    k = K.detach().cpu().to(torch.float64).tolist()      # [B][C][Hkv][D]
    B, Hq, D = q.shape
    C, Hkv = K.shape[1], K.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, C, Hq), dtype=np.float64)
    for b in range(B):
        for c in range(C):
            for h in range(Hq):
                kv = h // G
                out[b, c, h] = math.fsum(qa[b][h][d] * k[b][c][kv][d] for d in range(D)) * scale
    return out


def abs_sum_qk(q: torch.Tensor, K: torch.Tensor) -> np.ndarray:
    """sum_d |q * K| per score (scale for the oracle's error bound)."""
    qa = q.detach().cpu().to(torch.float64).numpy()
    k = K.detach().cpu().to(torch.float64).numpy()
    G = qa.shape[1] // k.shape[2]
    kq = np.repeat(k, G, axis=2)                       # [B, C, Hq, D]
    return np.einsum("bhd,bchd->bch", np.abs(qa), np.abs(kq))
