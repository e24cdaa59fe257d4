"""Benchmark of the GQA decode attention-times-V path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--mode auto|per_head|reuse]

A step is one call of the whole path (pass 1, and the split combine when the
context is split) over one batch of synthetic decode input already resident in
HBM. Several copies of the inputs are rotated so that the total exceeds twice
the 256 MB Infinity Cache and every step reads V and attn from HBM.

Prints ONE JSON line: µs per call and achieved GB/s over the algorithmic bytes
(V + attn + out, each once); a roofline for the dominant kernel (pass 1, timed
alone: K back-to-back launches between HIP events on the launch stream) against
8 TB/s HBM; and the CPU oracle timed on this host as a baseline.

Other modes (measurement plumbing, no JSON line):
    --copy-calibration MB   device-to-device copy of MB MiB three times, to scale
                            the FETCH_SIZE / WRITE_SIZE counters
    --summarize-trace DIR   write a kernel-trace summary from rocprofv3 CSV output
    --summarize-pmc ...     write a traffic summary from four rocprofv3 --pmc runs
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GQA decode AV: µs/call and achieved HBM GB/s (% of MI355X peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
ROTATE_BYTES = 512 * 2 ** 20   # 2 x the 256 MB Infinity Cache
DEFAULT_WORKLOAD = "g2-b4-c32768-hq16-hkv8-d128-bf16"
PROFILES = os.path.join(ROOT, "profiles")
_CSRC = os.path.join(ROOT, "gqa_reuse_attn_amd", "csrc")
# The sources each operation's kernels are built from (a profile records their hash).
KERNEL_SOURCES = {
    "av": [os.path.join(_CSRC, f) for f in ("av_kernels.hpp", "combine_kernels.hpp", "dispatch.hpp",
                                             "valu_launch.hpp", "mfma_bf16_launch.hpp", "gqa_av.hip")]
          + sorted(glob.glob(os.path.join(_CSRC, "launch_valu_*.hip")))
          + sorted(glob.glob(os.path.join(_CSRC, "launch_mfma*.hip"))),
    "qk": [os.path.join(_CSRC, f) for f in ("av_kernels.hpp", "qk_kernels.hpp", "qk_host.hpp", "qk_launch.hpp",
                                             "dispatch.hpp")]
          + sorted(glob.glob(os.path.join(_CSRC, "launch_qk_*.hip"))),
}
KERNEL_SOURCES["softmax"] = KERNEL_SOURCES["av"]
KERNEL_SOURCES["attn"] = KERNEL_SOURCES["av"]
# Profile file prefix and the dominant kernel's name fragment, per operation.
# op: (profile prefix, regular expression for the dominant kernel's name)
OPS = {"av": ("pass1", "pass1"), "qk": ("qk", "qk_scores"), "softmax": ("softmax_pass1", "pass1"),
       "attn": ("attn_pass1", r"av_pass1_mfma_bf16<[^>]*, true>")}   # scores from q and K (dense or paged)
SOFTMAX_METRIC = "GQA decode fused softmax x V: µs/call and achieved HBM GB/s (% of MI355X peak)"


def source_hash(op: str = "av") -> str:
    """SHA-256 over the kernel sources: identifies the kernels a profile was taken on."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[op]:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[1])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--op", default="av", choices=["av", "qk", "softmax", "attn"],
                   help="av: attention-times-V (the headline); qk: the decode score step before it; "
                        "softmax: the fused softmax x V product on the scores; attn: fused decode attention "
                        "(scores, softmax and product in one pass over bf16 K and V)")
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=-1,
                   help="untimed warmup steps; -1 (default): at least 20 and about 0.25 s of GPU work, "
                        "which MI355X needs to reach steady clocks")
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--mode", default="auto", choices=["auto", "per_head", "reuse"])
    p.add_argument("--nsplit", type=int, default=0, help="force the number of context splits (0 = plan)")
    p.add_argument("--engine", default="auto", choices=["auto", "valu", "mfma", "mfma_bf16"])
    p.add_argument("--combine", default="auto", choices=["auto", "kernel", "last"],
                   help="how split partials are added (plan default: auto)")
    p.add_argument("--kv-tile", type=int, default=0, help="adjacent KV heads per VALU workgroup (0 = plan)")
    p.add_argument("--v-fp8", action="store_true",
                   help="av / softmax with V quantized to OCP FP8 E4M3 with a scale per KV head (half the V bytes)")
    p.add_argument("--k-fp8", action="store_true",
                   help="qk with K quantized to OCP FP8 E4M3 with a scale per KV head (half the K bytes)")
    p.add_argument("--page-size", type=int, default=0,
                   help="av / softmax over a paged V cache (qk: a paged K cache) with this many rows per page "
                        "(shuffled pages, full lengths); 0 = dense")
    p.add_argument("--graph", action="store_true",
                   help="dense av / softmax: time the K whole calls as one captured HIP graph (no host launch "
                        "cost between calls) instead of K stream launches")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU oracle time budget")
    p.add_argument("--rotate-mb", type=float, default=ROTATE_BYTES / 2 ** 20)
    p.add_argument("--copy-calibration", type=float, default=0.0, metavar="MB")
    p.add_argument("--summarize-trace", metavar="DIR")
    p.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"))
    p.add_argument("--copy-bytes", type=float, default=1024.0, help="MiB per copy in the calibration runs")
    p.add_argument("--out", help="summary file to write (with --summarize-*)")
    p.add_argument("--command", default="", help="the command line the summarized data came from")
    return p.parse_args()


# ---- measurement plumbing ------------------------------------------------------

def _rows(d: str, suffix: str):
    files = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    with open(files[0]) as fh:
        return list(csv.DictReader(fh))


def summarize_trace(d: str, out: str, command: str, op: str = "av"):
    rows = _rows(d, "kernel_stats.csv")
    lines = ["# rocprofv3 kernel trace summary", f"command: {command}", f"kernel_sources_sha256: {source_hash(op)}", "",
             "| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| {r['Name'][:90]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                     f"{float(r['MinNs']) / 1e3:.3f} | {float(r['MaxNs']) / 1e3:.3f} | {float(r['Percentage']):.1f} |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter_medians(d: str):
    vals = {}
    for r in _rows(d, "counter_collection.csv"):
        vals.setdefault((r["Kernel_Name"], r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    return {k: statistics.median(v) for k, v in vals.items()}


def summarize_pmc(dirs, copy_mib: float, out: str, command: str, op: str = "av"):
    fetch, write, cfetch, cwrite = (_counter_medians(d) for d in dirs)
    copy_bytes = copy_mib * 2 ** 20

    def copy_factor(m, counter):
        vals = [v for (k, c), v in m.items() if c == counter and "copyBuffer" in k]
        return copy_bytes / (max(vals) * 1024.0)
    ff, wf = copy_factor(cfetch, "FETCH_SIZE"), copy_factor(cwrite, "WRITE_SIZE")
    lines = ["# rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE summary", f"command: {command}",
             f"kernel_sources_sha256: {source_hash(op)}",
             f"copy_calibration: {copy_mib:.0f} MiB device-to-device copy (__amd_rocclr_copyBuffer)",
             f"fetch_scale: {ff:.4f}", f"write_scale: {wf:.4f}", "",
             "| kernel | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | scaled HBM bytes/dispatch |",
             "|---|---|---|---|"]
    extra = []
    for (k, c), v in sorted(fetch.items()):
        if "gqa_av" not in k:
            continue
        w = write.get((k, "WRITE_SIZE"), 0.0)
        traffic = v * 1024 * ff + w * 1024 * wf
        lines.append(f"| {k[:90]} | {v:.1f} | {w:.1f} | {traffic:.0f} |")
        prefix, fragment = OPS[op]
        if re.search(fragment, k):
            extra.append(f"{prefix}_traffic_bytes: {traffic:.0f}")
    lines += [""] + extra
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def recorded_traffic(workload: str, mode: str, op: str = "av", variant: str = ""):
    """The dominant kernel's HBM bytes per launch from the committed PMC summary
    (variant: "" for dense V, "_fp8" or "_paged<P>"), if it was taken on the
    current kernel sources (else None)."""
    prefix = OPS[op][0]
    f = os.path.join(PROFILES, f"{prefix}{variant}_{workload}_{mode}_traffic.md")
    if not os.path.exists(f):
        return None
    kv = {}
    for line in open(f):
        if ":" in line and not line.startswith("|"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    key = f"{prefix}_traffic_bytes"
    if kv.get("kernel_sources_sha256") != source_hash(op) or key not in kv:
        return None
    return float(kv[key])


def copy_calibration(mib: float):
    import torch
    n = int(mib * 2 ** 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {n} bytes x3", flush=True)


# ---- CPU baseline ---------------------------------------------------------------

def cpu_baseline(w, attn, V, budget_s: float, softmax: bool = False):
    """The CPU oracle (fp64, OpenMP) on the same workload, repeated for ~budget_s."""
    import oracle
    orc = oracle.get()
    threads = int(os.environ.get("OMP_NUM_THREADS") or 0) or len(os.sched_getaffinity(0))
    fn = orc.softmax_av if softmax else orc.full
    reps = 0
    t0 = time.perf_counter()
    while True:
        fn(attn, V, w.v_dtype, nthreads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 1000:
            break
    per_call = el / reps
    return {
        "value": round(w.algorithmic_bytes() / per_call / 1e9, 3),
        "unit": "GB/s",
        "us_per_call": round(per_call * 1e6, 1),
        "cores": threads,
        "kind": "oracle",
        "sample": f"full workload {w.name}{' (fused softmax)' if softmax else ''}, {reps} calls in {el:.1f} s "
                  "(fp64 C oracle, OpenMP)",
    }


def _oracle_rate(fn, alg_bytes: int, budget_s: float, what: str):
    """Time fn(nthreads) (an oracle call) repeatedly for ~budget_s on all host threads."""
    threads = int(os.environ.get("OMP_NUM_THREADS") or 0) or len(os.sched_getaffinity(0))
    reps, t0 = 0, time.perf_counter()
    while True:
        fn(threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 1000:
            break
    per = el / reps
    return {"value": round(alg_bytes / per / 1e9, 3), "unit": "GB/s", "us_per_call": round(per * 1e6, 1),
            "cores": threads, "kind": "oracle",
            "sample": f"full {what}, {reps} calls in {el:.1f} s (fp64 C oracle, OpenMP)"}


# ---- benchmark --------------------------------------------------------------------

def _warm(args, calls, nrot):
    """Untimed warmup: W calls, or (W < 0) at least 20 and about 0.25 s of GPU work."""
    import torch
    warmup = args.warmup
    if warmup < 0:
        t0 = time.perf_counter()
        for i in range(20):
            calls[i % nrot]()
        torch.cuda.synchronize()
        per_call = (time.perf_counter() - t0) / 20
        warmup = 20 + int(0.25 / max(per_call, 1e-6))
        for i in range(20, warmup):
            calls[i % nrot]()
    else:
        for i in range(warmup):
            calls[i % nrot]()
    torch.cuda.synchronize()
    args.warmup = warmup


def _timed(calls, nrot, steps, stream):
    """ms per call over `steps` back-to-back calls, HIP events on the launch stream."""
    import torch
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        calls[i % nrot]()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def _timed_pass1(calls, nrot, steps, stream):
    """ms per pass-1 launch over `steps` back-to-back pass-1 launches on the
    rotating inputs, HIP events on the launch stream. (Events around each
    single launch would add its dispatch latency, about 3 us.)"""
    import torch
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record(stream)
    for i in range(steps):
        calls[i % nrot].pass1()
    p1.record(stream)
    torch.cuda.synchronize()
    return p0.elapsed_time(p1) / steps


def _pass1_roofline(alg: int, p1_ms: float, traffic):
    gbs = alg / (p1_ms / 1e3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": "pass 1 (V streaming)",
            "us_per_launch": round(p1_ms * 1e3, 3),
            "timing": "HIP events around K back-to-back pass-1 launches on the launch stream"}


QK_METRIC = "GQA decode QK scores: µs/call and achieved HBM GB/s (% of MI355X peak)"
FP8_METRIC = "GQA decode AV with fp8 V: µs/call and achieved HBM GB/s (% of MI355X peak)"


def bench_fp8(args, w, dev, props):
    """The AV product (or the fused softmax product) with the workload's V
    quantized to OCP FP8 E4M3 with a float32 scale per KV head (max |V| / 448).
    Algorithmic bytes: V at one byte per value, the weights, the output."""
    import torch

    import gqa_reuse_attn_amd as ga
    from workloads import make_inputs, make_scores

    softmax = args.op == "softmax"
    x_h, V_h = (make_scores if softmax else make_inputs)(w, seed=0)
    Vf = V_h.float()
    scale_h = (Vf.abs().amax(dim=(0, 1, 3)).clamp_min(1e-30) / 448.0).contiguous()
    q_h = (Vf / scale_h.view(1, 1, -1, 1)).to(torch.float8_e4m3fn).contiguous()
    del Vf
    alg = w.B * w.C * w.Hkv * w.D + w.attn_bytes() + w.out_bytes()
    plan = ga.make_plan(w.B, w.C, w.Hq, w.Hkv, w.D, "fp8", args.mode, engine=args.engine, nsplit=args.nsplit,
                        cu_count=props.multi_processor_count, kv_tile=args.kv_tile, softmax=softmax)
    nrot = max(1, math.ceil(args.rotate_mb * 2 ** 20 / alg))
    x0, q0, sc = x_h.to(dev), q_h.to(dev), scale_h.to(dev)
    calls = []
    for i in range(nrot):
        x, q = (x0, q0) if i == 0 else (x0.clone(), q0.clone())
        calls.append(ga.bind_fp8(x, q, sc, plan=plan))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    _warm(args, calls, nrot)
    ms = _timed(calls, nrot, args.steps, stream)
    gbs = alg / (ms / 1e3) / 1e9
    p1_ms = _timed_pass1(calls, nrot, args.steps, stream)
    print(f"[bench] fp8 {'softmax ' if softmax else ''}{ms * 1e3:.2f} us/call, {gbs:.1f} GB/s "
          f"({100 * gbs / HBM_PEAK_GBS:.1f}% of peak); pass 1 {p1_ms * 1e3:.2f} us; {nrot} rotation sets, "
          f"plan {plan.as_dict()}", file=sys.stderr, flush=True)
    default_plan = args.nsplit == 0 and args.engine == "auto" and args.kv_tile == 0
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.get()
        cpu = _oracle_rate(lambda n: orc.fp8(x_h, q_h, scale_h, softmax=softmax, nthreads=n), alg,
                           args.cpu_seconds, f"fp8 {w.name}")
    line = {
        "metric": FP8_METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "us_per_call": round(ms * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"fp8{'-softmax' if softmax else ''}:{w.name}", "B": w.B, "C": w.C, "Hq": w.Hq,
                   "Hkv": w.Hkv, "G": w.G, "D": w.D, "v_dtype": "fp8_e4m3", "mode": args.mode,
                   "algorithmic_bytes": alg, "rotation_sets": nrot, "plan": plan.as_dict()},
        "roofline": _pass1_roofline(alg, p1_ms, recorded_traffic(w.name, args.mode, args.op, "_fp8")
                                    if default_plan else None),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


PAGED_METRIC = "GQA decode AV over a paged V cache: µs/call and achieved HBM GB/s (% of MI355X peak)"


def bench_paged(args, w, dev, props):
    """The AV product (or the fused softmax product) with V as a paged cache:
    the workload's V cut into pages of --page-size rows, stored in a shuffled
    order, every sequence at full length. Same algorithmic bytes as the dense
    call (plus the block table and lengths, which are negligible)."""
    import torch

    import gqa_reuse_attn_amd as ga
    from workloads import make_inputs, make_scores

    softmax = args.op == "softmax"
    P = args.page_size
    if w.C % P:
        raise SystemExit(f"--page-size {P} must divide C={w.C}")
    x_h, V_h = (make_scores if softmax else make_inputs)(w, seed=0)
    maxp = w.C // P
    npg = w.B * maxp
    g = torch.Generator().manual_seed(0)
    perm = torch.randperm(npg, generator=g)
    chunks = V_h.reshape(npg, P, w.Hkv, w.D)
    pages_h = torch.empty_like(chunks)
    pages_h[perm] = chunks                           # chunk i (sequence i // maxp) lives in page perm[i]
    bt = perm.to(torch.int32).view(w.B, maxp).contiguous().to(dev)
    lens = torch.full((w.B,), w.C, dtype=torch.int32, device=dev)
    plan = ga.make_plan(w.B, w.C, w.Hq, w.Hkv, w.D, w.v_dtype, args.mode, engine=args.engine, nsplit=args.nsplit,
                        cu_count=props.multi_processor_count, kv_tile=args.kv_tile, softmax=softmax, page_size=P)
    per_set = w.algorithmic_bytes()
    nrot = max(1, math.ceil(args.rotate_mb * 2 ** 20 / per_set))
    x0, p0 = x_h.to(dev), pages_h.to(dev)
    calls = []
    for i in range(nrot):
        x, pg = (x0, p0) if i == 0 else (x0.clone(), p0.clone())
        calls.append(ga.bind_paged(x, pg, bt, lens, plan=plan))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    _warm(args, calls, nrot)
    ms = _timed(calls, nrot, args.steps, stream)
    gbs = w.algorithmic_bytes() / (ms / 1e3) / 1e9
    p1_ms = _timed_pass1(calls, nrot, args.steps, stream)
    print(f"[bench] paged P={P} {'softmax ' if softmax else ''}{ms * 1e3:.2f} us/call, {gbs:.1f} GB/s "
          f"({100 * gbs / HBM_PEAK_GBS:.1f}% of peak); pass 1 {p1_ms * 1e3:.2f} us; {nrot} rotation sets, "
          f"plan {plan.as_dict()}", file=sys.stderr, flush=True)
    default_plan = args.nsplit == 0 and args.engine == "auto" and args.kv_tile == 0
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.get()
        bt_h, lens_h = bt.cpu(), lens.cpu()
        cpu = _oracle_rate(lambda n: orc.paged(x_h, pages_h, bt_h, lens_h, w.v_dtype, softmax=softmax, nthreads=n),
                           w.algorithmic_bytes(), args.cpu_seconds, f"paged P={P} {w.name}")
    line = {
        "metric": PAGED_METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "us_per_call": round(ms * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"paged{P}{'-softmax' if softmax else ''}:{w.name}", "B": w.B, "C": w.C, "Hq": w.Hq,
                   "Hkv": w.Hkv, "G": w.G, "D": w.D, "v_dtype": w.v_dtype, "mode": args.mode, "page_size": P,
                   "algorithmic_bytes": w.algorithmic_bytes(), "rotation_sets": nrot, "plan": plan.as_dict()},
        "roofline": _pass1_roofline(w.algorithmic_bytes(), p1_ms,
                                    recorded_traffic(w.name, args.mode, args.op, f"_paged{P}") if default_plan else None),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def bench_qk(args, w, dev, props):
    """The decode score step on the workload's shape: K (the workload's V dtype)
    once + q once + scores once per call. One kernel per call, so it is also
    the roofline kernel."""
    import torch

    import gqa_reuse_attn_amd as ga
    from workloads import make_qk_random

    q_h, K_h = make_qk_random(w.B, w.C, w.Hq, w.Hkv, w.D, w.v_dtype, seed=0)
    kdt, ks_h = w.v_dtype, None
    if args.k_fp8:
        # per-KV-head scale max|K| / 448 and the E4M3 bytes of K / scale
        Kf = K_h.float()
        ks_h = (Kf.abs().amax(dim=(0, 1, 3)).clamp_min(1e-30) / 448.0).contiguous()
        K_h = (Kf / ks_h.view(1, 1, -1, 1)).to(torch.float8_e4m3fn).contiguous()
        kdt = "fp8"
        del Kf
    es = {"f32": 4, "fp8": 1}.get(kdt, 2)
    alg = w.B * w.C * w.Hkv * w.D * es + 4 * w.B * w.Hq * w.D + 4 * w.B * w.C * w.Hq
    P = args.page_size
    plan = ga.qk_make_plan(w.B, w.C, w.Hq, w.Hkv, w.D, kdt, args.mode, cu_count=props.multi_processor_count,
                           page_size=P)
    nrot = max(1, math.ceil(args.rotate_mb * 2 ** 20 / alg))
    q0, k0 = q_h.to(dev), K_h.to(dev)
    ks = ks_h.to(dev) if ks_h is not None else None
    calls = []
    if P > 0:
        # paged K: the workload's K cut into pages of P rows in a shuffled order, full lengths
        if w.C % P:
            raise SystemExit(f"--page-size {P} must divide C={w.C}")
        maxp = w.C // P
        perm = torch.randperm(w.B * maxp, generator=torch.Generator().manual_seed(0))
        pages_h = torch.empty((w.B * maxp, P, w.Hkv, w.D), dtype=K_h.dtype)
        pages_h.view(torch.uint8 if kdt == "fp8" else K_h.dtype)[perm] = \
            K_h.view(torch.uint8 if kdt == "fp8" else K_h.dtype).reshape(w.B * maxp, P, w.Hkv, w.D)
        bt = perm.to(torch.int32).view(w.B, maxp).contiguous().to(dev)
        lens = torch.full((w.B,), w.C, dtype=torch.int32, device=dev)
        p0 = pages_h.to(dev)
        for i in range(nrot):
            calls.append(ga.BoundQkPaged(q0 if i == 0 else q0.clone(), p0 if i == 0 else p0.clone(), bt, lens,
                                         C=w.C, scale=w.D ** -0.5, plan=plan, k_scale=ks))
    else:
        for i in range(nrot):
            calls.append(ga.bind_qk(q0 if i == 0 else q0.clone(), k0 if i == 0 else k0.clone(), scale=w.D ** -0.5,
                                    plan=plan, k_scale=ks))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    _warm(args, calls, nrot)
    ms = _timed(calls, nrot, args.steps, stream)
    gbs = alg / (ms / 1e3) / 1e9
    print(f"[bench] qk {ms * 1e3:.2f} us/call, {gbs:.1f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of peak); "
          f"{nrot} rotation sets, plan {plan.as_dict()}", file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.get()
        threads = int(os.environ.get("OMP_NUM_THREADS") or 0) or len(os.sched_getaffinity(0))
        reps, t0 = 0, time.perf_counter()
        while True:
            if args.k_fp8:
                orc.qk_fp8(q_h, K_h, ks_h, w.D ** -0.5, nthreads=threads)
            else:
                orc.qk(q_h, K_h, w.v_dtype, w.D ** -0.5, nthreads=threads)
            reps += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds or reps >= 1000:
                break
        cpu = {"value": round(alg / (el / reps) / 1e9, 3), "unit": "GB/s", "us_per_call": round(el / reps * 1e6, 1),
               "cores": threads, "kind": "oracle",
               "sample": f"full score step of {w.name}{' (fp8 K)' if args.k_fp8 else ''}, {reps} calls in {el:.1f} s "
                         "(fp64 C oracle, OpenMP)"}
    line = {
        "metric": QK_METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "us_per_call": round(ms * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"qk{'-fp8' if args.k_fp8 else ''}{f'-paged{P}' if P else ''}:{w.name}", "B": w.B,
                   "C": w.C, "Hq": w.Hq, "page_size": P,
                   "Hkv": w.Hkv, "G": w.G, "D": w.D, "k_dtype": "fp8_e4m3" if args.k_fp8 else w.v_dtype, "mode": args.mode, "algorithmic_bytes": alg, "rotation_sets": nrot,
                   "kernels_per_call": 1, "plan": plan.as_dict()},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(w.name, args.mode, "qk", ("_fp8" if args.k_fp8 else "") +
                                                 (f"_paged{P}" if P else "")),
                     "kernel": "qk_scores", "us_per_launch": round(ms * 1e3, 3),
                     "timing": "HIP events around K back-to-back launches on the launch stream"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


ATTN_METRIC = "GQA fused decode attention (q.K, softmax, x V in one pass): µs/call and achieved HBM GB/s (% of MI355X peak)"


def bench_attn(args, w, dev, props):
    """Fused decode attention on the workload's shape (bf16 K and V, D of 64,
    128 or 256): K and V once + q + out per call. The score step followed by
    the fused softmax product on the same inputs is timed beside it."""
    import torch

    import gqa_reuse_attn_amd as ga
    from workloads import make_inputs, make_qk_random

    if w.v_dtype != "bf16" or w.D not in (64, 128, 256):
        raise SystemExit("--op attn takes the bf16 workloads with D of 64, 128 or 256")
    q_h, K_h = make_qk_random(w.B, w.C, w.Hq, w.Hkv, w.D, "bf16", seed=0)
    _, V_h = make_inputs(w, seed=0)
    scale = w.D ** -0.5
    kvdt, ks_h, vs_h = "bf16", None, None
    if args.v_fp8:
        # fp8 K and V: per-KV-head scale max|x| / 448 and the E4M3 bytes of x / scale
        def quant(X):
            Xf = X.float()
            sc = (Xf.abs().amax(dim=(0, 1, 3)).clamp_min(1e-30) / 448.0).contiguous()
            return (Xf / sc.view(1, 1, -1, 1)).to(torch.float8_e4m3fn).contiguous(), sc
        (K_h, ks_h), (V_h, vs_h) = quant(K_h), quant(V_h)
        kvdt = "fp8"
    kv_bytes = w.v_bytes() // (2 if args.v_fp8 else 1)
    alg = 2 * kv_bytes + 4 * w.B * w.Hq * w.D + w.out_bytes()
    P = args.page_size
    plan = ga.make_plan(w.B, w.C, w.Hq, w.Hkv, w.D, kvdt, args.mode, nsplit=args.nsplit, kv_tile=args.kv_tile,
                        cu_count=props.multi_processor_count, attention=True, page_size=P)
    nrot = max(1, math.ceil(args.rotate_mb * 2 ** 20 / alg))
    if P:
        # A paged cache: K and V cut into pages of P rows, both pools in one
        # shuffled order (one block table), every sequence at full length.
        if w.C % P:
            raise SystemExit(f"--page-size {P} must divide C={w.C}")
        maxp = w.C // P
        perm = torch.randperm(w.B * maxp, generator=torch.Generator().manual_seed(0))
        K_d, V_d = K_h, V_h
        K_h, V_h = torch.empty_like(K_d).view(-1, P, w.Hkv, w.D), torch.empty_like(V_d).view(-1, P, w.Hkv, w.D)
        K_h[perm] = K_d.reshape(-1, P, w.Hkv, w.D)
        V_h[perm] = V_d.reshape(-1, P, w.Hkv, w.D)
        bt_h = perm.to(torch.int32).view(w.B, maxp).contiguous()
        lens_h = torch.full((w.B,), w.C, dtype=torch.int32)
        bt, lens = bt_h.to(dev), lens_h.to(dev)
    q0, k0, v0 = q_h.to(dev), K_h.to(dev), V_h.to(dev)
    ks = ks_h.to(dev) if ks_h is not None else None
    vs = vs_h.to(dev) if vs_h is not None else None
    sets = [(q0, k0, v0) if i == 0 else (q0.clone(), k0.clone(), v0.clone()) for i in range(nrot)]
    if P:
        calls = [ga.BoundAttentionPaged(q, k, v, bt, lens, scale=scale, plan=plan, k_scale=ks, v_scale=vs)
                 for q, k, v in sets]
    else:
        calls = [ga.BoundAttention(q, k, v, scale=scale, plan=plan, k_scale=ks, v_scale=vs) for q, k, v in sets]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    _warm(args, calls, nrot)
    ms = _timed(calls, nrot, args.steps, stream)
    gbs = alg / (ms / 1e3) / 1e9
    p1_ms = _timed_pass1(calls, nrot, args.steps, stream)
    # the unfused pair on the same inputs: score step, then the fused softmax product
    scores = [torch.empty((w.B, w.C, w.Hq), device=dev) for _ in range(nrot)]
    if P:
        # (the paged product takes no V scale: the same work with unit scales)
        qk = [ga.BoundQkPaged(q, k, bt, lens, scores=sc, scale=scale, k_scale=ks) for (q, k, _), sc in zip(sets, scores)]
        sav = [ga.bind_paged(sc, v, bt, lens, softmax=True) for (_, _, v), sc in zip(sets, scores)]
    else:
        qk = [ga.bind_qk(q, k, scores=sc, scale=scale, k_scale=ks) for (q, k, _), sc in zip(sets, scores)]
        sav = [(ga.BoundFp8(sc, v, vs, softmax=True) if args.v_fp8 else ga.bind_softmax(sc, v))
               for (_, _, v), sc in zip(sets, scores)]
    pair = [lambda i=i: (qk[i](), sav[i]()) for i in range(nrot)]
    _warm(args, pair, nrot)
    pair_ms = _timed(pair, nrot, args.steps, stream)
    print(f"[bench] attn {ms * 1e3:.2f} us/call, {gbs:.1f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of peak); pass 1 "
          f"{p1_ms * 1e3:.2f} us; score step + fused softmax {pair_ms * 1e3:.2f} us; {nrot} rotation sets, "
          f"plan {plan.as_dict()}", file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.get()
        nb = max(1, min(w.B, int(2e8 // max(1, w.C * w.Hq * w.D * 4))))    # a bounded sample of sequences
        part = alg * nb // w.B
        if P:
            fn = lambda n: orc.attention_paged(q_h[:nb], K_h, V_h, bt_h[:nb], lens_h[:nb], kvdt, scale, ks_h,  # noqa: E731
                                               vs_h, C=w.C, nthreads=n)
        elif args.v_fp8:
            fn = lambda n: orc.attention_fp8(q_h[:nb], K_h[:nb], V_h[:nb], ks_h, vs_h, scale, nthreads=n)  # noqa: E731
        else:
            fn = lambda n: orc.attention(q_h[:nb], K_h[:nb], V_h[:nb], "bf16", scale, nthreads=n)  # noqa: E731
        cpu = _oracle_rate(fn, part, args.cpu_seconds, f"attention of {nb} of the {w.B} sequences of {w.name}")
    line = {
        "metric": ATTN_METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "us_per_call": round(ms * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"attn{'-fp8' if args.v_fp8 else ''}{f'-paged{P}' if P else ''}:{w.name}", "B": w.B,
                   "C": w.C, "Hq": w.Hq, "page_size": P,
                   "Hkv": w.Hkv, "G": w.G, "D": w.D, "kv_dtype": "fp8_e4m3" if args.v_fp8 else "bf16", "mode": args.mode, "algorithmic_bytes": alg, "rotation_sets": nrot,
                   "unfused_us_per_call": round(pair_ms * 1e3, 3), "plan": plan.as_dict()},
        "roofline": _pass1_roofline(alg, p1_ms, recorded_traffic(w.name, args.mode, "attn", ("_fp8" if args.v_fp8 else "")
                                                                 + (f"_paged{P}" if P else ""))
                                    if args.nsplit == 0 and args.kv_tile == 0 else None),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.out, args.command, args.op)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc, args.copy_bytes, args.out, args.command, args.op)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): this path has no "
              "multi-GPU code; see DESIGN.md for how it would shard.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import torch

    import gqa_reuse_attn_amd as ga
    from workloads import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ga.load()
    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    print(f"[bench] {args.op} {w.name} mode={args.mode} on {props.name} ({props.multi_processor_count} CUs)",
          file=sys.stderr, flush=True)
    if args.op == "qk":
        bench_qk(args, w, dev, props)
        return
    if args.op == "attn":
        bench_attn(args, w, dev, props)
        return
    if args.page_size > 0:
        bench_paged(args, w, dev, props)
        return
    if args.v_fp8:
        bench_fp8(args, w, dev, props)
        return

    softmax = args.op == "softmax"
    if softmax:
        from workloads import make_scores
        attn_h, V_h = make_scores(w, seed=0)        # the workload's logits, as scores
    else:
        attn_h, V_h = make_inputs(w, seed=0)
    plan = ga.make_plan(w.B, w.C, w.Hq, w.Hkv, w.D, w.v_dtype, args.mode, nsplit=args.nsplit,
                        engine=args.engine, combine=args.combine, kv_tile=args.kv_tile,
                        cu_count=props.multi_processor_count, softmax=softmax)
    per_set = w.v_bytes() + w.attn_bytes() + w.out_bytes()
    nrot = max(1, math.ceil(args.rotate_mb * 2 ** 20 / per_set))
    sets = []
    a0, v0 = attn_h.to(dev), V_h.to(dev)
    for i in range(nrot):
        a = a0 if i == 0 else a0.clone()
        v = v0 if i == 0 else v0.clone()
        sets.append((a, v, torch.empty(w.B, w.Hq, w.D, device=dev)))
    torch.cuda.synchronize()
    # --graph: the calls are bound to a side stream, which graph capture needs.
    stream = torch.cuda.Stream(dev) if args.graph else torch.cuda.current_stream(dev)
    calls = [(ga.bind_softmax if softmax else ga.bind)(a, v, o, plan=plan, stream=stream) for a, v, o in sets]

    _warm(args, calls, nrot)

    # Whole calls: the metric.
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(args.steps):
                calls[i % nrot]()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            graph.replay()                           # warm replay
            g0.record(stream)
            graph.replay()
            g1.record(stream)
        torch.cuda.synchronize()
        ms = g0.elapsed_time(g1) / args.steps
    else:
        ms = _timed(calls, nrot, args.steps, stream)
    gbs = w.algorithmic_bytes() / (ms / 1e3) / 1e9

    # The dominant kernel alone: K back-to-back pass-1 launches over the same
    # rotating inputs, bracketed by events on the launch stream.
    p1_ms = _timed_pass1(calls, nrot, args.steps, stream)
    p1_gbs = w.algorithmic_bytes() / (p1_ms / 1e3) / 1e9
    print(f"[bench] {ms * 1e3:.2f} us/call, {gbs:.1f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of peak); "
          f"pass 1 {p1_ms * 1e3:.2f} us = {p1_gbs:.1f} GB/s; {nrot} rotation sets, plan {plan.as_dict()}",
          file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, attn_h, V_h, args.cpu_seconds, softmax=softmax)

    split_kernel = plan.nsplit > 1 and plan.combine == 1
    traffic = recorded_traffic(w.name, args.mode, args.op) if (args.nsplit == 0 and args.engine == "auto"
                                                             and args.combine == "auto" and args.kv_tile == 0) else None
    line = {
        "metric": SOFTMAX_METRIC if softmax else METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "us_per_call": round(ms * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": ("softmax:" if softmax else "") + w.name, "B": w.B, "C": w.C, "Hq": w.Hq, "Hkv": w.Hkv,
            "G": w.G, "D": w.D,
            "v_dtype": w.v_dtype, "mode": args.mode, "algorithmic_bytes": w.algorithmic_bytes(),
            "rotation_sets": nrot, "kernels_per_call": 2 if split_kernel else 1, "plan": plan.as_dict(),
            "launch": "one HIP graph of K calls" if args.graph else "K stream launches",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(p1_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(p1_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "pass 1 (V streaming)",
            "us_per_launch": round(p1_ms * 1e3, 3),
            "timing": "HIP events around K back-to-back pass-1 launches on the launch stream",
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
