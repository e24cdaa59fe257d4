"""CPU oracle for the GQA decode attention-times-V contraction (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product package
``gqa_reuse_attn_amd`` never imports it, and the two share no code.

``gqa_av_oracle.c`` holds the definition (ExecuTorch PR #21063, "...GEMV",
introduction, with a batch index added): fp64 sums over context positions c of
exact fp32 x V products, kv_h = floor(q_h / G). It also holds the decode score
step that precedes it (not on the page: scale * sum over d of q * K with the
same head grouping, output in the attn layout) and the fused product that
takes the scores and applies the softmax over c itself (the page's attn is
that softmax), and both over a paged V cache with per-sequence lengths. ``brute.py`` holds
pure-Python correctly rounded versions of both for tiny shapes. Every function here is
pinned by ``tests/test_oracle_pins.py``; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "gqa_av_oracle.c")
LIB = os.path.join(_HERE, "libgqa_av_oracle.so")

DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}

# Plain, portable flags: no -march (the library may run on another host),
# no contraction or reassociation of the fp64 sum.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra"]


def build(src: str = SRC, out: str = LIB, extra_flags: Optional[list] = None) -> str:
    """Compile the oracle with gcc into a shared library; returns its path."""
    cmd = ["gcc", *CFLAGS, *(extra_flags or []), "-o", out, src, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    return out


class Oracle:
    """ctypes view of one compiled oracle library (the real one or a test mutant)."""

    def __init__(self, path: str = LIB):
        if not os.path.exists(path):
            raise FileNotFoundError(f"oracle library {path} is not built; call oracle.build()")
        self.path = path
        lib = ctypes.CDLL(path)
        i64, vp, ip = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.gqa_av_oracle.argtypes = [vp, vp, ip, i64, i64, i64, i64, i64, vp, ip]
        lib.gqa_av_oracle.restype = ip
        lib.gqa_av_oracle_points.argtypes = [vp, vp, ip, i64, i64, i64, i64, i64, vp, i64, vp, ip]
        lib.gqa_av_oracle_points.restype = ip
        lib.gqa_av_oracle_decode.argtypes = [vp, ip, i64, vp]
        lib.gqa_av_oracle_decode.restype = ip
        lib.gqa_qk_oracle.argtypes = [vp, vp, ip, i64, i64, i64, i64, i64, ctypes.c_double, vp, ip]
        lib.gqa_qk_oracle.restype = ip
        lib.gqa_softmax_av_oracle.argtypes = [vp, vp, ip, i64, i64, i64, i64, i64, vp, ip]
        lib.gqa_softmax_av_oracle.restype = ip
        lib.gqa_av_paged_oracle.argtypes = [vp, vp, vp, vp, ip, ip, i64, i64, i64, i64, i64, i64, i64, i64, vp, ip]
        lib.gqa_av_paged_oracle.restype = ip
        lib.gqa_fp8_oracle_decode.argtypes = [vp, i64, vp]
        lib.gqa_fp8_oracle_decode.restype = ip
        lib.gqa_fp8_oracle.argtypes = [vp, vp, vp, ip, i64, i64, i64, i64, i64, vp, ip]
        lib.gqa_fp8_oracle.restype = ip
        lib.gqa_qk_fp8_oracle.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_double, vp, ip]
        lib.gqa_qk_fp8_oracle.restype = ip
        lib.gqa_qk_paged_oracle.argtypes = [vp, vp, vp, vp, ip, vp, i64, i64, i64, i64, i64, i64, i64, i64,
                                            ctypes.c_double, vp, ip]
        lib.gqa_qk_paged_oracle.restype = ip
        lib.gqa_attention_oracle.argtypes = [vp, vp, vp, ip, i64, i64, i64, i64, i64, ctypes.c_double, vp, ip]
        lib.gqa_attention_oracle.restype = ip
        lib.gqa_attention_fp8_oracle.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_double, vp, ip]
        lib.gqa_attention_paged_oracle.argtypes = [vp, vp, vp, vp, vp, ip, vp, vp, i64, i64, i64, i64, i64, i64, i64,
                                                   i64, ctypes.c_double, vp, ip]
        lib.gqa_attention_paged_oracle.restype = ip
        lib.gqa_attention_fp8_oracle.restype = ip
        self.lib = lib

    @staticmethod
    def _np_inputs(attn, V, v_dtype: str):
        a = _as_numpy(attn, np.float32)
        if v_dtype == "f32":
            v = _as_numpy(V, np.float32)
        else:
            v = _as_numpy(V, np.uint16)
        return np.ascontiguousarray(a), np.ascontiguousarray(v)

    def full(self, attn, V, v_dtype: str, nthreads: int = 0) -> np.ndarray:
        """out[B, Hq, D] (float64) for attn [B,C,Hq] fp32 and V [B,C,Hkv,D]."""
        a, v = self._np_inputs(attn, V, v_dtype)
        B, C, Hq = a.shape
        _, C2, Hkv, D = v.shape
        assert C2 == C and v.shape[0] == B
        out = np.empty((B, Hq, D), dtype=np.float64)
        rc = self.lib.gqa_av_oracle(a.ctypes.data, v.ctypes.data, DTYPE_CODE[v_dtype],
                                    B, C, Hq, Hkv, D, out.ctypes.data, nthreads)
        if rc != 0:
            raise ValueError(f"oracle rejected the arguments (status {rc})")
        return out

    def qk(self, q, K, k_dtype: str, scale: float = 1.0, nthreads: int = 0) -> np.ndarray:
        """scores[B, C, Hq] (float64) for q [B,Hq,D] fp32 and K [B,C,Hkv,D]."""
        qa, k = self._np_inputs(q, K, k_dtype)
        B, Hq, D = qa.shape
        B2, C, Hkv, D2 = k.shape
        assert B2 == B and D2 == D
        out = np.empty((B, C, Hq), dtype=np.float64)
        rc = self.lib.gqa_qk_oracle(qa.ctypes.data, k.ctypes.data, DTYPE_CODE[k_dtype],
                                    B, C, Hq, Hkv, D, float(scale), out.ctypes.data, nthreads)
        if rc != 0:
            raise ValueError(f"oracle rejected the arguments (status {rc})")
        return out

    def qk_fp8(self, q, K8, k_scale=None, scale: float = 1.0, nthreads: int = 0) -> np.ndarray:
        """scores[B, C, Hq] (float64) for q [B,Hq,D] fp32, K8 [B,C,Hkv,D] OCP FP8
        E4M3 bytes (uint8 or torch.float8_e4m3fn) and k_scale [Hkv] fp32 or None."""
        qa = np.ascontiguousarray(_as_numpy(q, np.float32))
        k = np.ascontiguousarray(_fp8_bytes(K8))
        B, Hq, D = qa.shape
        B2, C, Hkv, D2 = k.shape
        assert B2 == B and D2 == D
        ks = None if k_scale is None else np.ascontiguousarray(_as_numpy(k_scale, np.float32))
        out = np.empty((B, C, Hq), dtype=np.float64)
        rc = self.lib.gqa_qk_fp8_oracle(qa.ctypes.data, k.ctypes.data, None if ks is None else ks.ctypes.data,
                                        B, C, Hq, Hkv, D, float(scale), out.ctypes.data, nthreads)
        if rc != 0:
            raise ValueError(f"oracle rejected the arguments (status {rc})")
        return out

    def qk_paged(self, q, pages, block_table, seq_lens, k_dtype: str, scale: float = 1.0, k_scale=None,
                 C: Optional[int] = None, nthreads: int = 0) -> np.ndarray:
        """scores[B, C, Hq] (float64) for q [B,Hq,D] fp32 over paged K: pages
        [num_pages,P,Hkv,D] of k_dtype ("fp8": E4M3 bytes with k_scale [Hkv] or
        None), block_table [B,max_pages] int32, seq_lens [B] int32; C is the
        capacity (default max_pages * P). Rows at or past a sequence's length
        are NaN."""
        qa = np.ascontiguousarray(_as_numpy(q, np.float32))
        if k_dtype == "fp8":
            k, code = np.ascontiguousarray(_fp8_bytes(pages)), 3
        else:
            _, k = self._np_inputs(qa, pages, k_dtype)
            code = DTYPE_CODE[k_dtype]
        bt = np.ascontiguousarray(_as_numpy(block_table, np.int32), dtype=np.int32)
        ln = np.ascontiguousarray(_as_numpy(seq_lens, np.int32), dtype=np.int32)
        B, Hq, D = qa.shape
        num_pages, P, Hkv, D2 = k.shape
        assert D2 == D and bt.shape[0] == B and ln.shape == (B,)
        max_pages = bt.shape[1]
        C = max_pages * P if C is None else C
        ks = None if k_scale is None else np.ascontiguousarray(_as_numpy(k_scale, np.float32))
        out = np.empty((B, C, Hq), dtype=np.float64)
        rc = self.lib.gqa_qk_paged_oracle(qa.ctypes.data, k.ctypes.data, bt.ctypes.data, ln.ctypes.data, code,
                                          None if ks is None else ks.ctypes.data, B, C, Hq, Hkv, D, P, max_pages,
                                          num_pages, float(scale), out.ctypes.data, nthreads)
        if rc != 0:
            raise ValueError(f"oracle rejected the arguments (status {rc})")
        return out

    def attention(self, q, K, V, kv_dtype: str, scale: float = 1.0, nthreads: int = 0) -> np.ndarray:
        """out[B, Hq, D] (float64): softmax over c of scale * q . K, times V;
        q [B,Hq,D] fp32, K and V [B,C,Hkv,D] of kv_dtype."""
        qa, k = self._np_inputs(q, K, kv_dtype)
        _, v = self._np_inputs(q, V, kv_dtype)
        B, Hq, D = qa.shape
        B2, C, Hkv, D2 = k.shape
        assert B2 == B and D2 == D and v.shape == k.shape
        out = np.empty((B, Hq, D), dtype=np.float64)
        rc = self.lib.gqa_attention_oracle(qa.ctypes.data, k.ctypes.data, v.ctypes.data, DTYPE_CODE[kv_dtype],
                                           B, C, Hq, Hkv, D, float(scale), out.ctypes.data, nthreads)
        if rc != 0:
            raise ValueError(f"oracle rejected the arguments (status {rc})")
        return out

    def attention_fp8(self, q, K8, V8, k_scale=None, v_scale=None, scale: float = 1.0, nthreads: int = 0) -> np.ndarray:
        """out[B, Hq, D] (float64): fused attention over fp8 K and V (E4M3 bytes,
        uint8 or torch.float8_e4m3fn) with per-KV-head scales ([Hkv] fp32 or None)."""
        qa = np.ascontiguousarray(_as_numpy(q, np.float32))
        k, v = np.ascontiguousarray(_fp8_bytes(K8)), np.ascontiguousarray(_fp8_bytes(V8))
        B, Hq, D = qa.shape
        B2, C, Hkv, D2 = k.shape
        assert B2 == B and D2 == D and v.shape == k.shape
        ks = None if k_scale is None else np.ascontiguousarray(_as_numpy(k_scale, np.float32))
        vs = None if v_scale is None else np.ascontiguousarray(_as_numpy(v_scale, np.float32))
        out = np.empty((B, Hq, D), dtype=np.float64)
        rc = self.lib.gqa_attention_fp8_oracle(qa.ctypes.data, k.ctypes.data, None if ks is None else ks.ctypes.data,
                                               v.ctypes.data, None if vs is None else vs.ctypes.data,
                                               B, C, Hq, Hkv, D, float(scale), out.ctypes.data, nthreads)
        if rc != 0:
            raise ValueError(f"oracle rejected the arguments (status {rc})")
        return out

    def attention_paged(self, q, k_pages, v_pages, block_table, seq_lens, kv_dtype: str, scale: float = 1.0,
                        k_scale=None, v_scale=None, C: Optional[int] = None, nthreads: int = 0) -> np.ndarray:
        """out[B, Hq, D] (float64): fused attention over a paged K and V cache,
        two page pools [num_pages,P,Hkv,D] of kv_dtype ("fp8": E4M3 bytes with
        k_scale and v_scale [Hkv] or None) sharing block_table [B,max_pages]
        int32; only rows c < seq_lens[b] count; C is the capacity (default
        max_pages * P)."""
        qa = np.ascontiguousarray(_as_numpy(q, np.float32))
        if kv_dtype == "fp8":
            k, v, code = np.ascontiguousarray(_fp8_bytes(k_pages)), np.ascontiguousarray(_fp8_bytes(v_pages)), 3
        else:
            _, k = self._np_inputs(qa, k_pages, kv_dtype)
            _, v = self._np_inputs(qa, v_pages, kv_dtype)
            code = DTYPE_CODE[kv_dtype]
            if k_scale is not None or v_scale is not None:
                raise ValueError("k_scale and v_scale are for fp8 pages")
        bt = np.ascontiguousarray(_as_numpy(block_table, np.int32), dtype=np.int32)
        ln = np.ascontiguousarray(_as_numpy(seq_lens, np.int32), dtype=np.int32)
        B, Hq, D = qa.shape
        num_pages, P, Hkv, D2 = k.shape
        assert D2 == D and v.shape == k.shape and bt.shape[0] == B and ln.shape == (B,)
        max_pages = bt.shape[1]
        C = max_pages * P if C is None else C
        ks = None if k_scale is None else np.ascontiguousarray(_as_numpy(k_scale, np.float32))
        vs = None if v_scale is None else np.ascontiguousarray(_as_numpy(v_scale, np.float32))
        out = np.empty((B, Hq, D), dtype=np.float64)
        rc = self.lib.gqa_attention_paged_oracle(qa.ctypes.data, k.ctypes.data, v.ctypes.data, bt.ctypes.data,
                                                 ln.ctypes.data, code, None if ks is None else ks.ctypes.data,
                                                 None if vs is None else vs.ctypes.data, B, C, Hq, Hkv, D, P,
                                                 max_pages, num_pages, float(scale), out.ctypes.data, nthreads)
        if rc != 0:
            raise ValueError(f"oracle rejected the arguments (status {rc})")
        return out

    def softmax_av(self, scores, V, v_dtype: str, nthreads: int = 0) -> np.ndarray:
        """out[B, Hq, D] (float64): softmax over c of scores [B,C,Hq] fp32, times V."""
        a, v = self._np_inputs(scores, V, v_dtype)
        B, C, Hq = a.shape
        _, C2, Hkv, D = v.shape
        assert C2 == C and v.shape[0] == B
        out = np.empty((B, Hq, D), dtype=np.float64)
        rc = self.lib.gqa_softmax_av_oracle(a.ctypes.data, v.ctypes.data, DTYPE_CODE[v_dtype],
                                            B, C, Hq, Hkv, D, out.ctypes.data, nthreads)
        if rc != 0:
            raise ValueError(f"oracle rejected the arguments (status {rc})")
        return out

    def paged(self, w, pages, block_table, seq_lens, v_dtype: str, softmax: bool = False,
              nthreads: int = 0) -> np.ndarray:
        """out[B, Hq, D] (float64) for weights (or scores) [B,C,Hq] fp32, pages
        [num_pages, P, Hkv, D], block_table [B, max_pages] int32, seq_lens [B] int32."""
        a, v = self._np_inputs(w, pages, v_dtype)
        bt = np.ascontiguousarray(_as_numpy(block_table, np.int32), dtype=np.int32)
        ln = np.ascontiguousarray(_as_numpy(seq_lens, np.int32), dtype=np.int32)
        B, C, Hq = a.shape
        num_pages, P, Hkv, D = v.shape
        max_pages = bt.shape[1]
        assert bt.shape[0] == B and ln.shape == (B,)
        out = np.empty((B, Hq, D), dtype=np.float64)
        rc = self.lib.gqa_av_paged_oracle(a.ctypes.data, v.ctypes.data, bt.ctypes.data, ln.ctypes.data,
                                          DTYPE_CODE[v_dtype], int(bool(softmax)), B, C, Hq, Hkv, D, P, max_pages,
                                          num_pages, out.ctypes.data, nthreads)
        if rc != 0:
            raise ValueError(f"oracle rejected the arguments (status {rc})")
        return out

    def fp8(self, w, V8, v_scale=None, softmax: bool = False, nthreads: int = 0) -> np.ndarray:
        """out[B, Hq, D] (float64) for weights (or scores) [B,C,Hq] fp32, V8 [B,C,Hkv,D]
        OCP FP8 E4M3 bytes (uint8 or torch.float8_e4m3fn) and v_scale [Hkv] fp32 or None."""
        a = np.ascontiguousarray(_as_numpy(w, np.float32))
        v = np.ascontiguousarray(_fp8_bytes(V8))
        B, C, Hq = a.shape
        B2, C2, Hkv, D = v.shape
        assert (B2, C2) == (B, C)
        sc = None if v_scale is None else np.ascontiguousarray(_as_numpy(v_scale, np.float32))
        out = np.empty((B, Hq, D), dtype=np.float64)
        rc = self.lib.gqa_fp8_oracle(a.ctypes.data, v.ctypes.data, None if sc is None else sc.ctypes.data,
                                     int(bool(softmax)), B, C, Hq, Hkv, D, out.ctypes.data, nthreads)
        if rc != 0:
            raise ValueError(f"oracle rejected the arguments (status {rc})")
        return out

    def decode_fp8(self, raw) -> np.ndarray:
        """Widen OCP FP8 E4M3 bytes to float64."""
        v = np.ascontiguousarray(_fp8_bytes(raw))
        out = np.empty(v.size, dtype=np.float64)
        self.lib.gqa_fp8_oracle_decode(v.ctypes.data, v.size, out.ctypes.data)
        return out.reshape(v.shape)

    def points(self, attn, V, v_dtype: str, idx: np.ndarray, nthreads: int = 0) -> np.ndarray:
        """Selected elements out[b, q, d] for idx rows (b, q, d)."""
        a, v = self._np_inputs(attn, V, v_dtype)
        B, C, Hq = a.shape
        _, _, Hkv, D = v.shape
        idx = np.ascontiguousarray(idx, dtype=np.int64)
        out = np.empty(idx.shape[0], dtype=np.float64)
        rc = self.lib.gqa_av_oracle_points(a.ctypes.data, v.ctypes.data, DTYPE_CODE[v_dtype],
                                           B, C, Hq, Hkv, D, idx.ctypes.data, idx.shape[0],
                                           out.ctypes.data, nthreads)
        if rc != 0:
            raise ValueError(f"oracle rejected the arguments (status {rc})")
        return out

    def decode(self, raw: np.ndarray, v_dtype: str) -> np.ndarray:
        """Widen raw V elements (uint16 bits or float32) to float64."""
        raw = np.ascontiguousarray(raw)
        out = np.empty(raw.size, dtype=np.float64)
        rc = self.lib.gqa_av_oracle_decode(raw.ctypes.data, DTYPE_CODE[v_dtype], raw.size,
                                           out.ctypes.data)
        if rc != 0:
            raise ValueError("bad dtype")
        return out.reshape(raw.shape)


def _as_numpy(x, np_dtype):
    """torch CPU tensor or numpy array -> numpy array of the given bit type."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if np_dtype == np.uint16 and x.dtype in (torch.float16, torch.bfloat16):
                return x.view(torch.int16).numpy().view(np.uint16)
            if np_dtype == np.float32:
                assert x.dtype == torch.float32, x.dtype
            return x.numpy()
    except ImportError:  # pragma: no cover
        pass
    x = np.asarray(x)
    if np_dtype == np.uint16 and x.dtype == np.float16:
        return x.view(np.uint16)
    return x


def _fp8_bytes(x) -> np.ndarray:
    """The raw bytes of an fp8 tensor (torch float8 or uint8) or array."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype != torch.uint8:
                x = x.view(torch.uint8)
            return x.numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.uint8)


_DEFAULT: Optional[Oracle] = None


def get(build_if_missing: bool = True) -> Oracle:
    """The compiled oracle (built on first use when missing or older than its source)."""
    global _DEFAULT
    if _DEFAULT is None:
        stale = (not os.path.exists(LIB)) or os.path.getmtime(LIB) < os.path.getmtime(SRC)
        if stale:
            if not build_if_missing:
                raise FileNotFoundError(LIB)
            build()
        _DEFAULT = Oracle(LIB)
    return _DEFAULT
