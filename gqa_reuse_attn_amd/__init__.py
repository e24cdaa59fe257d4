"""Python binding of libgqa_av.so: GQA decode attention-times-V on MI355X.

    out[b, q_h, d] = sum_c attn[b, c, q_h] * V[b, c, q_h // G, d],   G = Hq // Hkv

(ExecuTorch PR #21063, "...GEMV", introduction; batch index added.) The same
library holds the decode score step before it (not on that page; the same
head grouping, output in the attn layout):

    scores[b, c, q_h] = scale * sum_d q[b, q_h, d] * K[b, c, q_h // G, d]

and the fused product that takes those scores and applies the softmax over c
itself (the page's attn is that softmax):

    out[b, q_h, d] = sum_c softmax_c(scores[b, :, q_h])[c] * V[b, c, q_h // G, d]

Every step runs in the HIP library; this module only checks tensors and marshals
pointers, sizes and the stream through ctypes. PyTorch provides device memory
and streams. There is no CPU fallback: if the library is missing, calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Union

__all__ = [
    "LIB_PATH", "GqaAvError", "Hint", "Plan", "load", "resolve_mode", "make_plan",
    "gqa_av_decode", "gqa_av_decode_plan", "bind", "BoundCall", "release", "status_string", "MODES", "DTYPES",
    "QkHint", "QkPlan", "qk_make_plan", "gqa_qk_decode", "bind_qk", "gqa_softmax_av_decode", "bind_softmax",
    "gqa_av_paged_decode", "bind_paged", "gqa_av_fp8_decode", "bind_fp8", "stream_read", "gqa_av_decode_strided",
]

# GQA_AV_LIBRARY may name another build of the same library (tuning variants).
LIB_PATH = os.environ.get("GQA_AV_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgqa_av.so")

MODES = {"auto": -1, "per_head": 0, "reuse": 1}
ENGINES = {"auto": 0, "valu": 1, "mfma": 2, "mfma_bf16": 3}
COMBINES = {"auto": 0, "kernel": 1}
SPLIT_ORDERS = {"auto": 0, "contiguous": 1, "interleaved": 2}
DTYPES = {"f32": 0, "f16": 1, "bf16": 2, "fp8": 3}   # fp8: OCP FP8 E4M3 (V only)
STATUS = {0: "OK", 1: "INVALID_ARG", 2: "INELIGIBLE", 3: "UNSUPPORTED", 4: "HIP"}


class GqaAvError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"gqa_av: {self.name}: {detail}")


class Hint(ctypes.Structure):
    _fields_ = [("engine", ctypes.c_int32), ("nsplit", ctypes.c_int32), ("cu_count", ctypes.c_int32),
                ("v_align", ctypes.c_int32), ("combine", ctypes.c_int32), ("kv_tile", ctypes.c_int32),
                ("softmax", ctypes.c_int32), ("page_size", ctypes.c_int32), ("attention", ctypes.c_int32),
                ("waves", ctypes.c_int32), ("split_order", ctypes.c_int32), ("reserved", ctypes.c_int32 * 2)]


class Plan(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("engine", ctypes.c_int32), ("heads_per_tile", ctypes.c_int32),
                ("subgroups", ctypes.c_int32), ("vec_bytes", ctypes.c_int32), ("lanes_per_row", ctypes.c_int32),
                ("row_slots", ctypes.c_int32), ("d_tiles", ctypes.c_int32), ("nsplit", ctypes.c_int32),
                ("threads", ctypes.c_int32), ("rows_per_split", ctypes.c_int64), ("grid", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_int64), ("v_bytes_read", ctypes.c_int64),
                ("combine", ctypes.c_int32), ("kv_heads_per_tile", ctypes.c_int32), ("softmax", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("attention", ctypes.c_int32), ("interleave", ctypes.c_int32)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_ if name != "reserved"}

    def __repr__(self) -> str:
        return f"Plan({self.as_dict()})"


class QkHint(ctypes.Structure):
    _fields_ = [("rows_per_block", ctypes.c_int64), ("cu_count", ctypes.c_int32), ("kv_tile", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("reserved", ctypes.c_int32 * 3)]


class QkPlan(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("engine", ctypes.c_int32), ("heads_per_tile", ctypes.c_int32),
                ("subgroups", ctypes.c_int32), ("rows_per_block", ctypes.c_int64), ("grid", ctypes.c_int64),
                ("k_bytes_read", ctypes.c_int64), ("kv_heads_per_tile", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("attention", ctypes.c_int32), ("reserved", ctypes.c_int32 * 1)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_ if name != "reserved"}

    def __repr__(self) -> str:
        return f"QkPlan({self.as_dict()})"


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m gqa_reuse_attn_amd.build` "
                           "(or __graft_entry__.build()); there is no CPU fallback")
    lib = ctypes.CDLL(path)
    i64, i32, vp, ip = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int
    lib.gqa_av_resolve_mode.argtypes = [i64, i64, ip]
    lib.gqa_av_resolve_mode.restype = ip
    lib.gqa_av_make_plan.argtypes = [i64, i64, i64, i64, i64, ip, ip, ctypes.POINTER(Hint), ctypes.POINTER(Plan)]
    lib.gqa_av_make_plan.restype = ip
    lib.gqa_av_decode.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, ip, ip, vp]
    lib.gqa_av_decode.restype = ip
    for fn in ("gqa_av_decode_plan", "gqa_av_decode_pass1", "gqa_av_decode_combine"):
        getattr(lib, fn).argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, ip, ctypes.POINTER(Plan), vp]
        getattr(lib, fn).restype = ip
    lib.gqa_av_decode_strided.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, ip, ip, vp]
    lib.gqa_av_decode_strided.restype = ip
    lib.gqa_av_decode_strided_plan.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, ip, ctypes.POINTER(Plan),
                                               vp]
    lib.gqa_av_decode_strided_plan.restype = ip
    lib.gqa_av_decode_noalloc.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, ip, ip, vp]
    lib.gqa_av_decode_noalloc.restype = ip
    lib.gqa_softmax_av_decode.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, ip, ip, vp]
    lib.gqa_softmax_av_decode.restype = ip
    for fn in ("gqa_softmax_av_decode_plan", "gqa_softmax_av_decode_pass1", "gqa_softmax_av_decode_combine"):
        getattr(lib, fn).argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, ip, ctypes.POINTER(Plan), vp]
        getattr(lib, fn).restype = ip
    lib.gqa_av_paged_decode.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64, ip, ip, ip, vp]
    lib.gqa_av_paged_decode.restype = ip
    for fn in ("gqa_av_paged_decode_plan", "gqa_av_paged_decode_pass1", "gqa_av_paged_decode_combine"):
        getattr(lib, fn).argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64, ip,
                                     ctypes.POINTER(Plan), vp]
        getattr(lib, fn).restype = ip
    lib.gqa_av_fp8_decode.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, ip, ip, vp]
    lib.gqa_av_fp8_decode.restype = ip
    lib.gqa_attention_decode.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, ip, ctypes.c_float, ip, vp]
    lib.gqa_attention_decode.restype = ip
    lib.gqa_attention_fp8_decode.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float, ip, vp]
    lib.gqa_attention_fp8_decode.restype = ip
    for fn in ("gqa_attention_fp8_decode_plan", "gqa_attention_fp8_decode_pass1", "gqa_attention_fp8_decode_combine"):
        getattr(lib, fn).argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float,
                                     ctypes.POINTER(Plan), vp]
        getattr(lib, fn).restype = ip
    lib.gqa_attention_paged_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64,
                                               i64, ip, ctypes.c_float, ip, vp]
    lib.gqa_attention_paged_decode.restype = ip
    for fn in ("gqa_attention_paged_decode_plan", "gqa_attention_paged_decode_pass1",
               "gqa_attention_paged_decode_combine"):
        getattr(lib, fn).argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64, ip,
                                     ctypes.c_float, ctypes.POINTER(Plan), vp]
        getattr(lib, fn).restype = ip
    for fn in ("gqa_attention_decode_plan", "gqa_attention_decode_pass1", "gqa_attention_decode_combine"):
        getattr(lib, fn).argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, ip, ctypes.c_float,
                                     ctypes.POINTER(Plan), vp]
        getattr(lib, fn).restype = ip
    for fn in ("gqa_av_fp8_decode_plan", "gqa_av_fp8_decode_pass1", "gqa_av_fp8_decode_combine"):
        getattr(lib, fn).argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.POINTER(Plan), vp]
        getattr(lib, fn).restype = ip
    lib.gqa_av_status_string.argtypes = [ip]
    lib.gqa_av_status_string.restype = ctypes.c_char_p
    lib.gqa_av_last_error.argtypes = []
    lib.gqa_av_last_error.restype = ctypes.c_char_p
    lib.gqa_av_release.argtypes = []
    lib.gqa_av_release.restype = ip
    lib.gqa_qk_make_plan.argtypes = [i64, i64, i64, i64, i64, ip, ip, ctypes.POINTER(QkHint), ctypes.POINTER(QkPlan)]
    lib.gqa_qk_make_plan.restype = ip
    lib.gqa_qk_decode.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, ip, ctypes.c_float, ip, vp]
    lib.gqa_qk_decode.restype = ip
    lib.gqa_qk_fp8_decode.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float, ip, vp]
    lib.gqa_qk_fp8_decode.restype = ip
    lib.gqa_qk_fp8_decode_plan.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float,
                                           ctypes.POINTER(QkPlan), vp]
    lib.gqa_qk_fp8_decode_plan.restype = ip
    lib.gqa_qk_paged_decode.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64, ip,
                                        ctypes.c_float, ip, vp]
    lib.gqa_qk_paged_decode.restype = ip
    lib.gqa_qk_paged_decode_plan.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64, ip,
                                             ctypes.c_float, ctypes.POINTER(QkPlan), vp]
    lib.gqa_qk_paged_decode_plan.restype = ip
    lib.gqa_qk_decode_plan.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, ip, ctypes.c_float,
                                       ctypes.POINTER(QkPlan), vp]
    lib.gqa_qk_decode_plan.restype = ip
    lib.gqa_bench_stream_read.argtypes = [vp, i64, i32, i32, i32, vp, vp]
    lib.gqa_bench_stream_read.restype = ip
    _lib = lib
    return lib


def stream_read(buf, nbytes: int, workgroups: int, loads_in_flight: int, sink, stream=None,
                pattern: int = 0) -> None:
    """Enqueue the plain streaming read of gqa_bench.h over the first nbytes of
    the GPU tensor `buf` (a measurement aid: the bandwidth ceiling, no part of
    the product). sink: a GPU uint32/int32 tensor of at least 256 elements;
    pattern 0: a contiguous slice per workgroup, 1: grid-stride batches."""
    torch = _torch()
    if not (buf.is_cuda and sink.is_cuda) or nbytes > buf.numel() * buf.element_size() or sink.numel() < 256 \
            or sink.element_size() != 4:
        raise ValueError("buf must be a GPU tensor of at least nbytes bytes and sink 256 32-bit GPU words")
    if stream is None:
        stream = torch.cuda.current_stream(buf.device)
    rc = load().gqa_bench_stream_read(buf.data_ptr(), int(nbytes), int(workgroups), int(loads_in_flight),
                                      int(pattern), sink.data_ptr(), stream.cuda_stream)
    if rc != 0:
        _raise(rc)


def status_string(status: int) -> str:
    return load().gqa_av_status_string(status).decode()


def _raise(status: int):
    detail = load().gqa_av_last_error().decode()
    raise GqaAvError(status, detail or status_string(status))


def _mode(mode: Union[str, int]) -> int:
    if isinstance(mode, str):
        if mode not in MODES:
            raise ValueError(f"mode must be one of {sorted(MODES)}, got {mode!r}")
        return MODES[mode]
    return int(mode)


def resolve_mode(Hq: int, Hkv: int, mode: Union[str, int] = "auto") -> str:
    """'reuse' or 'per_head' for this head shape (host only, no GPU needed)."""
    r = load().gqa_av_resolve_mode(Hq, Hkv, _mode(mode))
    if r < 0:
        _raise(-r)
    return "reuse" if r == 1 else "per_head"


def make_plan(B: int, C: int, Hq: int, Hkv: int, D: int, v_dtype: str, mode: Union[str, int] = "auto",
              engine: Union[str, int] = "auto", nsplit: int = 0, cu_count: int = 0, v_align: int = 0,
              combine: Union[str, int] = "auto", kv_tile: int = 0, softmax: bool = False,
              page_size: int = 0, attention: bool = False, waves: int = 0,
              split_order: Union[str, int] = "auto") -> Plan:
    """Host-only planning (no GPU needed). nsplit/cu_count/v_align/kv_tile <= 0 mean automatic.

    engine: "auto" | "valu" | "mfma" | "mfma_bf16"; combine: "auto" | "kernel";
    kv_tile: adjacent KV heads per workgroup; softmax: plan the fused softmax product;
    page_size > 0: plan for a paged V cache with that many rows per page;
    attention: plan the fused decode attention (scores from q and K; bf16);
    waves: waves per workgroup (4, or 8 on the bf16 matrix engine for the plain product or
    eight KV heads per workgroup);
    split_order: "auto" | "contiguous" | "interleaved" (how a split context is cut).
    """
    h = Hint()
    h.engine = ENGINES[engine] if isinstance(engine, str) else int(engine)
    h.combine = COMBINES[combine] if isinstance(combine, str) else int(combine)
    h.nsplit, h.cu_count, h.v_align, h.kv_tile = int(nsplit), int(cu_count), int(v_align), int(kv_tile)
    h.softmax = 1 if softmax else 0
    h.page_size = int(page_size)
    h.attention = 1 if attention else 0
    h.waves = int(waves)
    h.split_order = SPLIT_ORDERS[split_order] if isinstance(split_order, str) else int(split_order)
    p = Plan()
    rc = load().gqa_av_make_plan(B, C, Hq, Hkv, D, DTYPES[v_dtype], _mode(mode), ctypes.byref(h), ctypes.byref(p))
    if rc != 0:
        _raise(rc)
    return p


def _torch():
    import torch
    return torch


def _check(attn, V, out):
    torch = _torch()
    vmap = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16", torch.float8_e4m3fn: "fp8"}
    if attn.dim() != 3 or V.dim() != 4:
        raise ValueError(f"attn must be [B,C,Hq] and V [B,C,Hkv,D]; got {tuple(attn.shape)} and {tuple(V.shape)}")
    B, C, Hq = attn.shape
    if V.shape[0] != B or V.shape[1] != C:
        raise ValueError(f"V {tuple(V.shape)} does not match attn {tuple(attn.shape)} in B or C")
    Hkv, D = V.shape[2], V.shape[3]
    if attn.dtype != torch.float32:
        raise TypeError(f"attn must be float32, got {attn.dtype}")
    if V.dtype not in vmap:
        raise TypeError(f"V must be float32, float16, bfloat16 or float8_e4m3fn, got {V.dtype}")
    if not (attn.is_cuda and V.is_cuda):
        raise ValueError("attn and V must be GPU tensors")
    if attn.device != V.device:
        raise ValueError("attn and V must be on the same device")
    if not (attn.is_contiguous() and V.is_contiguous()):
        raise ValueError("attn and V must be contiguous")
    if out is not None:
        if out.dtype != torch.float32 or tuple(out.shape) != (B, Hq, D) or not out.is_contiguous() \
                or out.device != attn.device:
            raise ValueError(f"out must be a contiguous float32 [{B},{Hq},{D}] tensor on {attn.device}")
    return B, C, Hq, Hkv, D, vmap[V.dtype]


def gqa_av_decode(attn, V, out=None, mode: Union[str, int] = "auto", stream=None, plan: Optional[Plan] = None):
    """out[b,q_h,d] = sum_c attn[b,c,q_h] * V[b,c,q_h//G,d] on the GPU; returns out.

    attn: float32 [B,C,Hq]; V: float32/float16/bfloat16 [B,C,Hkv,D]; both
    contiguous on one GPU. mode: "auto" | "per_head" | "reuse" (or -1/0/1).
    stream: a torch.cuda.Stream (default: the current stream). plan: an
    explicit Plan from make_plan for the same problem (tests, sweeps).
    """
    torch = _torch()
    B, C, Hq, Hkv, D, vdt = _check(attn, V, out)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=attn.device)
    if stream is None:
        stream = torch.cuda.current_stream(attn.device)
    lib = load()
    with torch.cuda.device(attn.device):
        if plan is None:
            rc = lib.gqa_av_decode(attn.data_ptr(), V.data_ptr(), out.data_ptr(), B, C, Hq, Hkv, D,
                                   DTYPES[vdt], _mode(mode), stream.cuda_stream)
        else:
            rc = lib.gqa_av_decode_plan(attn.data_ptr(), V.data_ptr(), out.data_ptr(), B, C, Hq, Hkv, D,
                                        DTYPES[vdt], ctypes.byref(plan), stream.cuda_stream)
    if rc != 0:
        _raise(rc)
    return out


def gqa_av_decode_strided(attn, V, C: int, out=None, mode: Union[str, int] = "auto", stream=None,
                          plan: Optional[Plan] = None):
    """The product over a capacity-strided V cache: V [B, C_max, Hkv, D] (any
    C_max >= C, contiguous), rows c < C of each sequence; attn [B, C, Hq]
    float32; returns out [B, Hq, D] float32."""
    torch = _torch()
    vmap = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16", torch.float8_e4m3fn: "fp8"}
    if attn.dim() != 3 or V.dim() != 4 or attn.shape[1] != C or V.shape[1] < C or V.shape[0] != attn.shape[0]:
        raise ValueError(f"attn must be [B,{C},Hq] and V [B,C_max>={C},Hkv,D]; got {tuple(attn.shape)} and "
                         f"{tuple(V.shape)}")
    if attn.dtype != torch.float32 or V.dtype not in vmap:
        raise TypeError("attn must be float32 and V float32, float16, bfloat16 or float8_e4m3fn")
    if not (attn.is_cuda and V.is_cuda and attn.device == V.device and attn.is_contiguous() and V.is_contiguous()):
        raise ValueError("attn and V must be contiguous tensors on one GPU")
    B, _, Hq = attn.shape
    C_max, Hkv, D = V.shape[1], V.shape[2], V.shape[3]
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=attn.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (B, Hq, D) or not out.is_contiguous() \
            or out.device != attn.device:
        raise ValueError(f"out must be a contiguous float32 [{B},{Hq},{D}] tensor on {attn.device}")
    if stream is None:
        stream = torch.cuda.current_stream(attn.device)
    lib = load()
    with torch.cuda.device(attn.device):
        if plan is None:
            rc = lib.gqa_av_decode_strided(attn.data_ptr(), V.data_ptr(), out.data_ptr(), B, C, C_max, Hq, Hkv, D,
                                           DTYPES[vmap[V.dtype]], _mode(mode), stream.cuda_stream)
        else:
            rc = lib.gqa_av_decode_strided_plan(attn.data_ptr(), V.data_ptr(), out.data_ptr(), B, C, C_max, Hq, Hkv,
                                                D, DTYPES[vmap[V.dtype]], ctypes.byref(plan), stream.cuda_stream)
    if rc != 0:
        _raise(rc)
    return out


def gqa_av_decode_plan(attn, V, plan: Plan, out=None, stream=None):
    """gqa_av_decode with an explicit plan."""
    return gqa_av_decode(attn, V, out=out, stream=stream, plan=plan)


class BoundCall:
    """One problem's arguments, checked once, for repeated calls (decode loops, benchmarks).

    Calling the object enqueues the kernels on the bound stream through the C
    ABI with no per-call Python checks. The bound tensors are referenced here
    and must not be resized or freed while the object is used.
    """

    def __init__(self, attn, V, out=None, plan: Optional[Plan] = None, mode: Union[str, int] = "auto",
                 stream=None, softmax: bool = False):
        torch = _torch()
        B, C, Hq, Hkv, D, vdt = _check(attn, V, out)
        if out is None:
            out = torch.empty((B, Hq, D), dtype=torch.float32, device=attn.device)
        if stream is None:
            stream = torch.cuda.current_stream(attn.device)
        if plan is None:
            props = torch.cuda.get_device_properties(attn.device)
            addr = V.data_ptr()
            align = 16 if addr % 16 == 0 else (addr & -addr)
            plan = make_plan(B, C, Hq, Hkv, D, vdt, mode, cu_count=props.multi_processor_count, v_align=align,
                             softmax=softmax)
        self.attn, self.V, self.out, self.plan, self.stream = attn, V, out, plan, stream
        lib = load()
        pre = "gqa_softmax_av_decode" if plan.softmax else "gqa_av_decode"
        self._fn = getattr(lib, pre + "_plan")
        self._pass1 = getattr(lib, pre + "_pass1")
        self._combine = getattr(lib, pre + "_combine")
        self._args = (attn.data_ptr(), V.data_ptr(), out.data_ptr(), B, C, Hq, Hkv, D, DTYPES[vdt],
                      ctypes.byref(plan), stream.cuda_stream)

    def __call__(self):
        rc = self._fn(*self._args)
        if rc != 0:
            _raise(rc)
        return self.out

    def pass1(self):
        """Only the V-streaming launch (see gqa_av_decode_pass1); combine() must follow."""
        rc = self._pass1(*self._args)
        if rc != 0:
            _raise(rc)

    def combine(self):
        """The split combine launch (see gqa_av_decode_combine); completes `out`."""
        rc = self._combine(*self._args)
        if rc != 0:
            _raise(rc)
        return self.out


def bind(attn, V, out=None, plan: Optional[Plan] = None, mode: Union[str, int] = "auto", stream=None) -> BoundCall:
    """A BoundCall for (attn, V, out): see BoundCall."""
    return BoundCall(attn, V, out=out, plan=plan, mode=mode, stream=stream)


def gqa_softmax_av_decode(scores, V, out=None, mode: Union[str, int] = "auto", stream=None,
                          plan: Optional[Plan] = None):
    """out[b,q_h,d] = sum_c softmax_c(scores[b,:,q_h])[c] * V[b,c,q_h//G,d] on the GPU; returns out.

    scores: float32 [B,C,Hq] (the attn layout); V and the rest as gqa_av_decode.
    plan: a make_plan(..., softmax=True) plan for the same problem.
    """
    torch = _torch()
    B, C, Hq, Hkv, D, vdt = _check(scores, V, out)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=scores.device)
    if stream is None:
        stream = torch.cuda.current_stream(scores.device)
    lib = load()
    with torch.cuda.device(scores.device):
        if plan is None:
            rc = lib.gqa_softmax_av_decode(scores.data_ptr(), V.data_ptr(), out.data_ptr(), B, C, Hq, Hkv, D,
                                           DTYPES[vdt], _mode(mode), stream.cuda_stream)
        else:
            rc = lib.gqa_softmax_av_decode_plan(scores.data_ptr(), V.data_ptr(), out.data_ptr(), B, C, Hq, Hkv, D,
                                                DTYPES[vdt], ctypes.byref(plan), stream.cuda_stream)
    if rc != 0:
        _raise(rc)
    return out


def bind_softmax(scores, V, out=None, plan: Optional[Plan] = None, mode: Union[str, int] = "auto",
                 stream=None) -> BoundCall:
    """A BoundCall of the fused softmax product for (scores, V, out)."""
    return BoundCall(scores, V, out=out, plan=plan, mode=mode, stream=stream, softmax=True)


def _check_scale(v_scale, Hkv, device):
    if v_scale is None:
        return None
    torch = _torch()
    if v_scale.dtype != torch.float32 or tuple(v_scale.shape) != (Hkv,) or not v_scale.is_contiguous() \
            or v_scale.device != device:
        raise ValueError(f"v_scale must be a contiguous float32 [{Hkv}] tensor on {device}")
    return v_scale


def gqa_av_fp8_decode(w, V, v_scale=None, out=None, softmax: bool = False, mode: Union[str, int] = "auto",
                      stream=None, plan: Optional[Plan] = None):
    """The AV product (or, softmax=True, the fused softmax product on scores w)
    with V in OCP FP8 E4M3 (torch.float8_e4m3fn [B,C,Hkv,D]) and a float32 scale
    per KV head (v_scale [Hkv], None = 1)."""
    torch = _torch()
    B, C, Hq, Hkv, D, vdt = _check(w, V, out)
    if vdt != "fp8":
        raise TypeError("V must be torch.float8_e4m3fn")
    sc = _check_scale(v_scale, Hkv, w.device)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=w.device)
    if stream is None:
        stream = torch.cuda.current_stream(w.device)
    lib = load()
    sp = sc.data_ptr() if sc is not None else None
    with torch.cuda.device(w.device):
        if plan is None:
            rc = lib.gqa_av_fp8_decode(w.data_ptr(), V.data_ptr(), sp, out.data_ptr(), B, C, Hq, Hkv, D,
                                       1 if softmax else 0, _mode(mode), stream.cuda_stream)
        else:
            rc = lib.gqa_av_fp8_decode_plan(w.data_ptr(), V.data_ptr(), sp, out.data_ptr(), B, C, Hq, Hkv, D,
                                            ctypes.byref(plan), stream.cuda_stream)
    if rc != 0:
        _raise(rc)
    return out


class BoundFp8:
    """An fp8 call with checked, bound arguments for loops (see BoundCall)."""

    def __init__(self, w, V, v_scale=None, out=None, plan: Optional[Plan] = None, softmax: bool = False,
                 mode: Union[str, int] = "auto", stream=None):
        torch = _torch()
        B, C, Hq, Hkv, D, vdt = _check(w, V, out)
        if vdt != "fp8":
            raise TypeError("V must be torch.float8_e4m3fn")
        sc = _check_scale(v_scale, Hkv, w.device)
        if out is None:
            out = torch.empty((B, Hq, D), dtype=torch.float32, device=w.device)
        if stream is None:
            stream = torch.cuda.current_stream(w.device)
        if plan is None:
            cu = torch.cuda.get_device_properties(w.device).multi_processor_count
            addr = V.data_ptr()
            plan = make_plan(B, C, Hq, Hkv, D, "fp8", mode, cu_count=cu, softmax=softmax,
                             v_align=16 if addr % 16 == 0 else (addr & -addr))
        self.tensors, self.out, self.plan = (w, V, sc), out, plan
        lib = load()
        self._fn, self._pass1, self._combine = (lib.gqa_av_fp8_decode_plan, lib.gqa_av_fp8_decode_pass1,
                                                lib.gqa_av_fp8_decode_combine)
        self._args = (w.data_ptr(), V.data_ptr(), sc.data_ptr() if sc is not None else None, out.data_ptr(),
                      B, C, Hq, Hkv, D, ctypes.byref(plan), stream.cuda_stream)

    def __call__(self):
        rc = self._fn(*self._args)
        if rc != 0:
            _raise(rc)
        return self.out

    def pass1(self):
        """Only the V-streaming launch (see gqa_av_fp8_decode_pass1); combine() must follow."""
        rc = self._pass1(*self._args)
        if rc != 0:
            _raise(rc)

    def combine(self):
        """The split combine launch; completes `out`."""
        rc = self._combine(*self._args)
        if rc != 0:
            _raise(rc)
        return self.out


def bind_fp8(w, V, v_scale=None, out=None, plan: Optional[Plan] = None, softmax: bool = False,
             mode: Union[str, int] = "auto", stream=None) -> BoundFp8:
    return BoundFp8(w, V, v_scale=v_scale, out=out, plan=plan, softmax=softmax, mode=mode, stream=stream)


def _check_paged(w, pages, block_table, seq_lens, out):
    torch = _torch()
    vmap = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16", torch.float8_e4m3fn: "fp8"}
    if w.dim() != 3 or pages.dim() != 4 or block_table.dim() != 2 or seq_lens.dim() != 1:
        raise ValueError("w [B,C,Hq], pages [num_pages,page_size,Hkv,D], block_table [B,max_pages], seq_lens [B]")
    B, C, Hq = w.shape
    num_pages, P, Hkv, D = pages.shape
    if block_table.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("block_table and seq_lens must have B rows")
    if w.dtype != torch.float32 or pages.dtype not in vmap:
        raise TypeError("w must be float32 and pages float32/float16/bfloat16/float8_e4m3fn")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_table and seq_lens must be int32")
    ts = (w, pages, block_table, seq_lens)
    if not all(t.is_cuda and t.device == w.device and t.is_contiguous() for t in ts):
        raise ValueError("all tensors must be contiguous and on the same GPU")
    if out is not None and (out.dtype != torch.float32 or tuple(out.shape) != (B, Hq, D) or not out.is_contiguous()
                            or out.device != w.device):
        raise ValueError(f"out must be a contiguous float32 [{B},{Hq},{D}] tensor on {w.device}")
    return B, C, Hq, Hkv, D, P, block_table.shape[1], num_pages, vmap[pages.dtype]


def gqa_av_paged_decode(w, pages, block_table, seq_lens, out=None, softmax: bool = False,
                        mode: Union[str, int] = "auto", stream=None, plan: Optional[Plan] = None):
    """The AV product (or, softmax=True, the fused softmax product on scores w)
    over a paged V cache: row c of sequence b is pages[block_table[b, c // P], c % P];
    only rows c < seq_lens[b] count. w: float32 [B,C,Hq] (C the capacity);
    pages: [num_pages,P,Hkv,D]; block_table: int32 [B,max_pages]; seq_lens: int32 [B]."""
    torch = _torch()
    B, C, Hq, Hkv, D, P, maxp, npg, vdt = _check_paged(w, pages, block_table, seq_lens, out)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=w.device)
    if stream is None:
        stream = torch.cuda.current_stream(w.device)
    lib = load()
    args = (w.data_ptr(), pages.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(), out.data_ptr(),
            B, C, Hq, Hkv, D, P, maxp, npg, DTYPES[vdt])
    with torch.cuda.device(w.device):
        if plan is None:
            rc = lib.gqa_av_paged_decode(*args, 1 if softmax else 0, _mode(mode), stream.cuda_stream)
        else:
            rc = lib.gqa_av_paged_decode_plan(*args, ctypes.byref(plan), stream.cuda_stream)
    if rc != 0:
        _raise(rc)
    return out


class BoundPaged:
    """A paged call with checked, bound arguments for loops (see BoundCall)."""

    def __init__(self, w, pages, block_table, seq_lens, out=None, plan: Optional[Plan] = None, softmax: bool = False,
                 mode: Union[str, int] = "auto", stream=None):
        torch = _torch()
        B, C, Hq, Hkv, D, P, maxp, npg, vdt = _check_paged(w, pages, block_table, seq_lens, out)
        if out is None:
            out = torch.empty((B, Hq, D), dtype=torch.float32, device=w.device)
        if stream is None:
            stream = torch.cuda.current_stream(w.device)
        if plan is None:
            cu = torch.cuda.get_device_properties(w.device).multi_processor_count
            plan = make_plan(B, C, Hq, Hkv, D, vdt, mode, cu_count=cu, softmax=softmax, page_size=P)
        self.tensors, self.out, self.plan = (w, pages, block_table, seq_lens), out, plan
        lib = load()
        self._fn, self._pass1, self._combine = (lib.gqa_av_paged_decode_plan, lib.gqa_av_paged_decode_pass1,
                                                lib.gqa_av_paged_decode_combine)
        self._args = (w.data_ptr(), pages.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(), out.data_ptr(),
                      B, C, Hq, Hkv, D, P, maxp, npg, DTYPES[vdt], ctypes.byref(plan), stream.cuda_stream)

    def __call__(self):
        rc = self._fn(*self._args)
        if rc != 0:
            _raise(rc)
        return self.out

    def pass1(self):
        """Only the V-streaming launch (see gqa_av_paged_decode_pass1); combine() must follow."""
        rc = self._pass1(*self._args)
        if rc != 0:
            _raise(rc)

    def combine(self):
        """The split combine launch; completes `out`."""
        rc = self._combine(*self._args)
        if rc != 0:
            _raise(rc)
        return self.out


def bind_paged(w, pages, block_table, seq_lens, out=None, plan: Optional[Plan] = None, softmax: bool = False,
               mode: Union[str, int] = "auto", stream=None) -> BoundPaged:
    return BoundPaged(w, pages, block_table, seq_lens, out=out, plan=plan, softmax=softmax, mode=mode, stream=stream)


def release() -> None:
    """Free the library's cached split-C workspaces."""
    rc = load().gqa_av_release()
    if rc != 0:
        _raise(rc)


# ---- decode score step ----------------------------------------------------------

def qk_make_plan(B: int, C: int, Hq: int, Hkv: int, D: int, k_dtype: str, mode: Union[str, int] = "auto",
                 rows_per_block: int = 0, cu_count: int = 0, kv_tile: int = 0, page_size: int = 0) -> QkPlan:
    """Host-only planning of the score step (no GPU needed); 0 means automatic
    (page_size: 0 for dense K, else paged K with that many rows per page)."""
    h = QkHint()
    h.rows_per_block, h.cu_count, h.kv_tile = int(rows_per_block), int(cu_count), int(kv_tile)
    h.page_size = int(page_size)
    p = QkPlan()
    rc = load().gqa_qk_make_plan(B, C, Hq, Hkv, D, DTYPES[k_dtype], _mode(mode), ctypes.byref(h), ctypes.byref(p))
    if rc != 0:
        _raise(rc)
    return p


def _check_qk(q, K, scores):
    torch = _torch()
    kmap = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16", torch.float8_e4m3fn: "fp8"}
    if q.dim() != 3 or K.dim() != 4:
        raise ValueError(f"q must be [B,Hq,D] and K [B,C,Hkv,D]; got {tuple(q.shape)} and {tuple(K.shape)}")
    B, Hq, D = q.shape
    if K.shape[0] != B or K.shape[3] != D:
        raise ValueError(f"K {tuple(K.shape)} does not match q {tuple(q.shape)} in B or D")
    C, Hkv = K.shape[1], K.shape[2]
    if q.dtype != torch.float32:
        raise TypeError(f"q must be float32, got {q.dtype}")
    if K.dtype not in kmap:
        raise TypeError(f"K must be float32, float16, bfloat16 or float8_e4m3fn, got {K.dtype}")
    if not (q.is_cuda and K.is_cuda) or q.device != K.device:
        raise ValueError("q and K must be GPU tensors on one device")
    if not (q.is_contiguous() and K.is_contiguous()):
        raise ValueError("q and K must be contiguous")
    if scores is not None:
        if scores.dtype != torch.float32 or tuple(scores.shape) != (B, C, Hq) or not scores.is_contiguous() \
                or scores.device != q.device:
            raise ValueError(f"scores must be a contiguous float32 [{B},{C},{Hq}] tensor on {q.device}")
    return B, C, Hq, Hkv, D, kmap[K.dtype]


def gqa_qk_decode(q, K, scores=None, scale: float = 1.0, mode: Union[str, int] = "auto", stream=None,
                  plan: Optional[QkPlan] = None, k_scale=None):
    """scores[b,c,q_h] = scale * sum_d q[b,q_h,d] * K[b,c,q_h//G,d] on the GPU; returns scores.

    q: float32 [B,Hq,D]; K: float32/float16/bfloat16 [B,C,Hkv,D], or
    float8_e4m3fn with k_scale (float32 [Hkv], None = 1) multiplying each KV
    head's K; both contiguous on one GPU. The result has the attn layout
    [B,C,Hq] of gqa_av_decode.
    """
    torch = _torch()
    B, C, Hq, Hkv, D, kdt = _check_qk(q, K, scores)
    ks = _qk_scale(k_scale, kdt, Hkv, q.device)
    if scores is None:
        scores = torch.empty((B, C, Hq), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    lib = load()
    with torch.cuda.device(q.device):
        if kdt == "fp8":
            kp = ks.data_ptr() if ks is not None else None
            if plan is None:
                rc = lib.gqa_qk_fp8_decode(q.data_ptr(), K.data_ptr(), kp, scores.data_ptr(), B, C, Hq, Hkv, D,
                                           float(scale), _mode(mode), stream.cuda_stream)
            else:
                rc = lib.gqa_qk_fp8_decode_plan(q.data_ptr(), K.data_ptr(), kp, scores.data_ptr(), B, C, Hq, Hkv, D,
                                                float(scale), ctypes.byref(plan), stream.cuda_stream)
        elif plan is None:
            rc = lib.gqa_qk_decode(q.data_ptr(), K.data_ptr(), scores.data_ptr(), B, C, Hq, Hkv, D, DTYPES[kdt],
                                   float(scale), _mode(mode), stream.cuda_stream)
        else:
            rc = lib.gqa_qk_decode_plan(q.data_ptr(), K.data_ptr(), scores.data_ptr(), B, C, Hq, Hkv, D,
                                        DTYPES[kdt], float(scale), ctypes.byref(plan), stream.cuda_stream)
    if rc != 0:
        _raise(rc)
    return scores


def _qk_scale(k_scale, kdt, Hkv, device):
    if k_scale is not None and kdt != "fp8":
        raise ValueError("k_scale is for fp8 K (torch.float8_e4m3fn)")
    if k_scale is None:
        return None
    torch = _torch()
    if k_scale.dtype != torch.float32 or tuple(k_scale.shape) != (Hkv,) or not k_scale.is_contiguous() \
            or k_scale.device != device:
        raise ValueError(f"k_scale must be a contiguous float32 [{Hkv}] tensor on {device}")
    return k_scale


class BoundQk:
    """Pre-checked score-step call for loops (see BoundCall)."""

    def __init__(self, q, K, scores=None, scale: float = 1.0, plan: Optional[QkPlan] = None,
                 mode: Union[str, int] = "auto", stream=None, k_scale=None):
        torch = _torch()
        B, C, Hq, Hkv, D, kdt = _check_qk(q, K, scores)
        ks = _qk_scale(k_scale, kdt, Hkv, q.device)
        if scores is None:
            scores = torch.empty((B, C, Hq), dtype=torch.float32, device=q.device)
        if plan is None:
            cu = torch.cuda.get_device_properties(q.device).multi_processor_count
            plan = qk_make_plan(B, C, Hq, Hkv, D, kdt, mode, cu_count=cu)
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        self.q, self.K, self.scores, self.plan, self.k_scale = q, K, scores, plan, ks
        if kdt == "fp8":
            self._fn = load().gqa_qk_fp8_decode_plan
            self._args = (q.data_ptr(), K.data_ptr(), ks.data_ptr() if ks is not None else None, scores.data_ptr(),
                          B, C, Hq, Hkv, D, ctypes.c_float(scale), ctypes.byref(plan), stream.cuda_stream)
        else:
            self._fn = load().gqa_qk_decode_plan
            self._args = (q.data_ptr(), K.data_ptr(), scores.data_ptr(), B, C, Hq, Hkv, D, DTYPES[kdt],
                          ctypes.c_float(scale), ctypes.byref(plan), stream.cuda_stream)

    def __call__(self):
        rc = self._fn(*self._args)
        if rc != 0:
            _raise(rc)
        return self.scores


def bind_qk(q, K, scores=None, scale: float = 1.0, plan: Optional[QkPlan] = None, mode: Union[str, int] = "auto",
            stream=None, k_scale=None) -> BoundQk:
    return BoundQk(q, K, scores=scores, scale=scale, plan=plan, mode=mode, stream=stream, k_scale=k_scale)


def _check_qk_paged(q, pages, block_table, seq_lens, scores, C):
    """Shapes, dtypes and devices of a paged score call; returns (B, C, Hq, Hkv, D, P, max_pages, num_pages, kdt)."""
    torch = _torch()
    kmap = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16", torch.float8_e4m3fn: "fp8"}
    if q.dim() != 3 or pages.dim() != 4 or block_table.dim() != 2 or seq_lens.dim() != 1:
        raise ValueError("q [B,Hq,D], pages [num_pages,P,Hkv,D], block_table [B,max_pages], seq_lens [B]")
    B, Hq, D = q.shape
    num_pages, P, Hkv, D2 = pages.shape
    if D2 != D:
        raise ValueError(f"q's D={D} does not match the pages' D={D2}")
    if q.dtype != torch.float32 or pages.dtype not in kmap:
        raise TypeError("q must be float32 and pages float32, float16, bfloat16 or float8_e4m3fn")
    if block_table.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("block_table and seq_lens must have B rows")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_table and seq_lens must be int32")
    for t in (q, pages, block_table, seq_lens):
        if not t.is_cuda or t.device != q.device or not t.is_contiguous():
            raise ValueError("q, pages, block_table and seq_lens must be contiguous GPU tensors on one device")
    max_pages = block_table.shape[1]
    if C is None:
        C = scores.shape[1] if scores is not None else max_pages * P
    if scores is not None and (scores.dtype != torch.float32 or tuple(scores.shape) != (B, C, Hq)
                               or not scores.is_contiguous() or scores.device != q.device):
        raise ValueError(f"scores must be a contiguous float32 [{B},{C},{Hq}] tensor on {q.device}")
    return B, C, Hq, Hkv, D, P, max_pages, num_pages, kmap[pages.dtype]


def gqa_qk_paged_decode(q, pages, block_table, seq_lens, scores=None, C: Optional[int] = None, scale: float = 1.0,
                        mode: Union[str, int] = "auto", stream=None, plan: Optional[QkPlan] = None, k_scale=None):
    """The score step over a paged K cache: row c of sequence b is
    pages[block_table[b, c // P], c % P]; the scores of rows c < seq_lens[b]
    are written, the rest of scores [B, C, Hq] (C the capacity, default
    max_pages * P; a new scores tensor starts as zeros) is left as it was."""
    torch = _torch()
    B, C, Hq, Hkv, D, P, maxp, npg, kdt = _check_qk_paged(q, pages, block_table, seq_lens, scores, C)
    ks = _qk_scale(k_scale, kdt, Hkv, q.device)
    if scores is None:
        scores = torch.zeros((B, C, Hq), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    lib = load()
    args = (q.data_ptr(), pages.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(),
            ks.data_ptr() if ks is not None else None, scores.data_ptr(), B, C, Hq, Hkv, D, P, maxp, npg, DTYPES[kdt],
            float(scale))
    with torch.cuda.device(q.device):
        if plan is None:
            rc = lib.gqa_qk_paged_decode(*args, _mode(mode), stream.cuda_stream)
        else:
            rc = lib.gqa_qk_paged_decode_plan(*args, ctypes.byref(plan), stream.cuda_stream)
    if rc != 0:
        _raise(rc)
    return scores


class BoundQkPaged:
    """A paged score call with checked, bound arguments for loops (see BoundCall)."""

    def __init__(self, q, pages, block_table, seq_lens, scores=None, C: Optional[int] = None, scale: float = 1.0,
                 plan: Optional[QkPlan] = None, mode: Union[str, int] = "auto", stream=None, k_scale=None):
        torch = _torch()
        B, C, Hq, Hkv, D, P, maxp, npg, kdt = _check_qk_paged(q, pages, block_table, seq_lens, scores, C)
        ks = _qk_scale(k_scale, kdt, Hkv, q.device)
        if scores is None:
            scores = torch.zeros((B, C, Hq), dtype=torch.float32, device=q.device)
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        if plan is None:
            cu = torch.cuda.get_device_properties(q.device).multi_processor_count
            plan = qk_make_plan(B, C, Hq, Hkv, D, kdt, mode, cu_count=cu, page_size=P)
        self.tensors, self.scores, self.plan, self.k_scale = (q, pages, block_table, seq_lens), scores, plan, ks
        self._fn = load().gqa_qk_paged_decode_plan
        self._args = (q.data_ptr(), pages.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(),
                      ks.data_ptr() if ks is not None else None, scores.data_ptr(), B, C, Hq, Hkv, D, P, maxp, npg,
                      DTYPES[kdt], ctypes.c_float(scale), ctypes.byref(plan), stream.cuda_stream)

    def __call__(self):
        rc = self._fn(*self._args)
        if rc != 0:
            _raise(rc)
        return self.scores


# ---- fused decode attention ----------------------------------------------------

def _check_attention(q, K, V, out):
    torch = _torch()
    if q.dim() != 3 or K.dim() != 4 or tuple(V.shape) != tuple(K.shape):
        raise ValueError("q [B,Hq,D], K and V [B,C,Hkv,D] of one shape")
    B, Hq, D = q.shape
    _, C, Hkv, D2 = K.shape
    if K.shape[0] != B or D2 != D:
        raise ValueError(f"K {tuple(K.shape)} does not match q {tuple(q.shape)} in B or D")
    if q.dtype != torch.float32 or K.dtype != V.dtype or K.dtype not in (torch.bfloat16, torch.float8_e4m3fn):
        raise TypeError("q must be float32, K and V both bfloat16 or both float8_e4m3fn")
    for t in (q, K, V):
        if not t.is_cuda or t.device != q.device or not t.is_contiguous():
            raise ValueError("q, K and V must be contiguous GPU tensors on one device")
    if out is not None and (out.dtype != torch.float32 or tuple(out.shape) != (B, Hq, D) or not out.is_contiguous()
                            or out.device != q.device):
        raise ValueError(f"out must be a contiguous float32 [{B},{Hq},{D}] tensor on {q.device}")
    return B, C, Hq, Hkv, D, ("fp8" if K.dtype == torch.float8_e4m3fn else "bf16")


def _attention_args(q, K, V, out, B, C, Hq, Hkv, D, kvdt, scale, k_scale, v_scale):
    """The C arguments (before mode/plan and stream) of the bf16 or fp8 entry points."""
    if kvdt != "fp8":
        if k_scale is not None or v_scale is not None:
            raise ValueError("k_scale and v_scale are for fp8 K and V")
        return (q.data_ptr(), K.data_ptr(), V.data_ptr(), out.data_ptr(), B, C, Hq, Hkv, D, DTYPES["bf16"],
                ctypes.c_float(scale))
    ks = _check_scale(k_scale, Hkv, q.device)
    vs = _check_scale(v_scale, Hkv, q.device)
    return (q.data_ptr(), K.data_ptr(), ks.data_ptr() if ks is not None else None, V.data_ptr(),
            vs.data_ptr() if vs is not None else None, out.data_ptr(), B, C, Hq, Hkv, D, ctypes.c_float(scale))


def gqa_attention_decode(q, K, V, out=None, scale: float = 1.0, mode: Union[str, int] = "auto", stream=None,
                         plan: Optional[Plan] = None, k_scale=None, v_scale=None):
    """Fused decode attention on the GPU: out[b,q_h] = softmax_c(scale * q[b,q_h] . K[b,c,q_h//G]) @ V[b,:,q_h//G];
    q float32 [B,Hq,D], K and V bfloat16 [B,C,Hkv,D] (D of 64, 128 or 256), or both float8_e4m3fn with
    per-KV-head scales k_scale and v_scale (float32 [Hkv], None = 1); returns out [B,Hq,D] float32."""
    torch = _torch()
    B, C, Hq, Hkv, D, kvdt = _check_attention(q, K, V, out)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    lib = load()
    args = _attention_args(q, K, V, out, B, C, Hq, Hkv, D, kvdt, scale, k_scale, v_scale)
    fp8 = kvdt == "fp8"
    with torch.cuda.device(q.device):
        if plan is None:
            fn = lib.gqa_attention_fp8_decode if fp8 else lib.gqa_attention_decode
            rc = fn(*args, _mode(mode), stream.cuda_stream)
        else:
            fn = lib.gqa_attention_fp8_decode_plan if fp8 else lib.gqa_attention_decode_plan
            rc = fn(*args, ctypes.byref(plan), stream.cuda_stream)
    if rc != 0:
        _raise(rc)
    return out


class BoundAttention:
    """A fused attention call with checked, bound arguments for loops (see BoundCall)."""

    def __init__(self, q, K, V, out=None, scale: float = 1.0, plan: Optional[Plan] = None,
                 mode: Union[str, int] = "auto", stream=None, k_scale=None, v_scale=None):
        torch = _torch()
        B, C, Hq, Hkv, D, kvdt = _check_attention(q, K, V, out)
        if out is None:
            out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        if plan is None:
            cu = torch.cuda.get_device_properties(q.device).multi_processor_count
            plan = make_plan(B, C, Hq, Hkv, D, kvdt, mode, cu_count=cu, attention=True)
        self.tensors, self.out, self.plan = (q, K, V, k_scale, v_scale), out, plan
        lib = load()
        if kvdt == "fp8":
            self._fn, self._pass1, self._combine = (lib.gqa_attention_fp8_decode_plan,
                                                    lib.gqa_attention_fp8_decode_pass1,
                                                    lib.gqa_attention_fp8_decode_combine)
        else:
            self._fn, self._pass1, self._combine = (lib.gqa_attention_decode_plan, lib.gqa_attention_decode_pass1,
                                                    lib.gqa_attention_decode_combine)
        self._args = _attention_args(q, K, V, out, B, C, Hq, Hkv, D, kvdt, scale, k_scale, v_scale) + \
            (ctypes.byref(plan), stream.cuda_stream)

    def __call__(self):
        rc = self._fn(*self._args)
        if rc != 0:
            _raise(rc)
        return self.out

    def pass1(self):
        rc = self._pass1(*self._args)
        if rc != 0:
            _raise(rc)

    def combine(self):
        rc = self._combine(*self._args)
        if rc != 0:
            _raise(rc)
        return self.out


def _check_attention_paged(q, k_pages, v_pages, block_table, seq_lens, out, C):
    torch = _torch()
    if q.dim() != 3 or k_pages.dim() != 4 or tuple(v_pages.shape) != tuple(k_pages.shape) or \
            block_table.dim() != 2 or seq_lens.dim() != 1:
        raise ValueError("q [B,Hq,D], k_pages and v_pages [num_pages,page_size,Hkv,D] of one shape, "
                         "block_table [B,max_pages], seq_lens [B]")
    B, Hq, D = q.shape
    num_pages, P, Hkv, D2 = k_pages.shape
    if D2 != D or block_table.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("pages, block_table and seq_lens do not match q")
    if q.dtype != torch.float32 or k_pages.dtype != v_pages.dtype or \
            k_pages.dtype not in (torch.bfloat16, torch.float8_e4m3fn):
        raise TypeError("q must be float32, k_pages and v_pages both bfloat16 or both float8_e4m3fn")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_table and seq_lens must be int32")
    for t in (q, k_pages, v_pages, block_table, seq_lens):
        if not t.is_cuda or t.device != q.device or not t.is_contiguous():
            raise ValueError("all tensors must be contiguous and on the same GPU")
    if out is not None and (out.dtype != torch.float32 or tuple(out.shape) != (B, Hq, D) or not out.is_contiguous()
                            or out.device != q.device):
        raise ValueError(f"out must be a contiguous float32 [{B},{Hq},{D}] tensor on {q.device}")
    maxp = block_table.shape[1]
    C = maxp * P if C is None else int(C)
    return B, C, Hq, Hkv, D, P, maxp, num_pages, ("fp8" if k_pages.dtype == torch.float8_e4m3fn else "bf16")


def _attention_paged_args(q, k_pages, v_pages, block_table, seq_lens, out, B, C, Hq, Hkv, D, P, maxp, npg, kvdt,
                          scale, k_scale, v_scale):
    if kvdt != "fp8" and (k_scale is not None or v_scale is not None):
        raise ValueError("k_scale and v_scale are for fp8 K and V")
    ks = _check_scale(k_scale, Hkv, q.device)
    vs = _check_scale(v_scale, Hkv, q.device)
    return (q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(),
            ks.data_ptr() if ks is not None else None, vs.data_ptr() if vs is not None else None, out.data_ptr(),
            B, C, Hq, Hkv, D, P, maxp, npg, DTYPES[kvdt], ctypes.c_float(scale))


def gqa_attention_paged_decode(q, k_pages, v_pages, block_table, seq_lens, out=None, scale: float = 1.0,
                               C: Optional[int] = None, mode: Union[str, int] = "auto", stream=None,
                               plan: Optional[Plan] = None, k_scale=None, v_scale=None):
    """Fused decode attention over a paged K and V cache: k_pages and v_pages
    [num_pages,P,Hkv,D] (bfloat16, or float8_e4m3fn with per-KV-head scales)
    share block_table int32 [B,max_pages]; row c of sequence b is row c % P of
    page block_table[b, c // P]; only rows c < seq_lens[b] count. C is the
    capacity (default max_pages * P). Returns out [B,Hq,D] float32."""
    torch = _torch()
    B, C, Hq, Hkv, D, P, maxp, npg, kvdt = _check_attention_paged(q, k_pages, v_pages, block_table, seq_lens, out, C)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    lib = load()
    args = _attention_paged_args(q, k_pages, v_pages, block_table, seq_lens, out, B, C, Hq, Hkv, D, P, maxp, npg,
                                 kvdt, scale, k_scale, v_scale)
    with torch.cuda.device(q.device):
        if plan is None:
            rc = lib.gqa_attention_paged_decode(*args, _mode(mode), stream.cuda_stream)
        else:
            rc = lib.gqa_attention_paged_decode_plan(*args, ctypes.byref(plan), stream.cuda_stream)
    if rc != 0:
        _raise(rc)
    return out


class BoundAttentionPaged:
    """A paged fused attention call with checked, bound arguments for loops (see BoundCall)."""

    def __init__(self, q, k_pages, v_pages, block_table, seq_lens, out=None, scale: float = 1.0,
                 C: Optional[int] = None, plan: Optional[Plan] = None, mode: Union[str, int] = "auto", stream=None,
                 k_scale=None, v_scale=None):
        torch = _torch()
        B, C, Hq, Hkv, D, P, maxp, npg, kvdt = _check_attention_paged(q, k_pages, v_pages, block_table, seq_lens,
                                                                      out, C)
        if out is None:
            out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        if plan is None:
            cu = torch.cuda.get_device_properties(q.device).multi_processor_count
            plan = make_plan(B, C, Hq, Hkv, D, kvdt, mode, cu_count=cu, attention=True, page_size=P)
        self.tensors = (q, k_pages, v_pages, block_table, seq_lens, k_scale, v_scale)
        self.out, self.plan = out, plan
        lib = load()
        self._fn, self._pass1, self._combine = (lib.gqa_attention_paged_decode_plan,
                                                lib.gqa_attention_paged_decode_pass1,
                                                lib.gqa_attention_paged_decode_combine)
        self._args = _attention_paged_args(q, k_pages, v_pages, block_table, seq_lens, out, B, C, Hq, Hkv, D, P,
                                           maxp, npg, kvdt, scale, k_scale, v_scale) + \
            (ctypes.byref(plan), stream.cuda_stream)

    def __call__(self):
        rc = self._fn(*self._args)
        if rc != 0:
            _raise(rc)
        return self.out

    def pass1(self):
        rc = self._pass1(*self._args)
        if rc != 0:
            _raise(rc)

    def combine(self):
        rc = self._combine(*self._args)
        if rc != 0:
            _raise(rc)
        return self.out
