"""Benchmark of the GQA decode attention-times-V path on one MI355X.

    python bench.py [--steps K] [--warmup W]            # the suite: every decode workload
    python bench.py --workload NAME [--mode auto|per_head|reuse] ...

A step is one call of the whole path (pass 1, and the split combine when the
context is split) over one batch of synthetic decode input already resident in
HBM. Copies of the inputs, carved from one device allocation, are rotated so
that together they exceed twice the 256 MB Infinity Cache and every step reads
V and attn from HBM (inputs smaller than that are capped at 64 copies and
labelled cache-resident).

Procedure for every timed quantity (per workload):
  1. clock ramp: untimed calls for at least --ramp-seconds (0.25 s; MI355X
     needs about that long under load to reach steady clocks);
  2. W untimed warmup calls;
  3. trials: K back-to-back calls between two HIP events on the launch stream,
     bracketed by synchronisations, repeated until the standard error of the
     trial means is at most 0.5 % of their median (at least 5 trials, 100 calls
     and 1 ms in total; at most 30 trials); the median and its SE are reported.

The default run prints ONE JSON line. Its headline is the large-batch workload
(B=64, C=8192, Hq=64, Hkv=8, D=128, bf16; 1.21 GB per call), the largest that
the metric is quoted on: µs per call and GB/s over the algorithmic bytes
(V + attn + out, each once); the roofline of the dominant kernel (pass 1 alone,
K back-to-back launches) against 8 TB/s; the plain-read ceiling of the same
byte count on the same device (gqa_bench.h); the CPU oracle as a baseline; and
under "configs" the same measurements for every other decode workload, with
the reuse / per-head HBM traffic ratio from the committed counter profiles.

Other modes (measurement plumbing, no JSON line):
    --copy-calibration MB   device-to-device copy of MB MiB three times, to scale
                            the FETCH_SIZE / WRITE_SIZE counters
    --summarize-trace DIR   write a kernel-trace summary from rocprofv3 CSV output
    --summarize-pmc ...     write a traffic summary from four rocprofv3 --pmc runs
    --summarize-counters DIR  per-kernel medians of any rocprofv3 --pmc counters
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
MAX_SETS = 64                  # rotation copies at most (small inputs stay cache-resident)
HEADLINE = "batch64-b64-c8192-hq64-hkv8-d128-bf16"
SUITE = ["tiny-f32-b1-c256-hq8-hkv2-d64", "llama3-8b-b1-c4096-hq32-hkv8-d128-bf16",
         "g3-b8-c16384-hq24-hkv8-d96-f16", "g2-b4-c32768-hq16-hkv8-d128-bf16",
         "mqa16-b4-c32768-hq16-hkv1-d128-bf16", HEADLINE]
READ_GRIDS = (256, 512, 1024, 2048)    # plain-read sweep: workgroups ...
READ_LOADS = (4, 8, 16)                # ... x 16-byte loads per lane and batch ...
READ_PATTERNS = (0, 1)                 # ... x contiguous slices / grid-stride batches
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
       "attn": ("attn_pass1", r"av_pass1_mfma_bf16<(?:[^,>]+, ){7}true\b")}   # QK: scores from q and K (dense or paged)
SOFTMAX_METRIC = "GQA decode fused softmax x V: µs/call and achieved HBM GB/s (% of MI355X peak)"
QK_METRIC = "GQA decode QK scores: µs/call and achieved HBM GB/s (% of MI355X peak)"
FP8_METRIC = "GQA decode AV with fp8 V: µs/call and achieved HBM GB/s (% of MI355X peak)"
PAGED_METRIC = "GQA decode AV over a paged V cache: µs/call and achieved HBM GB/s (% of MI355X peak)"
ATTN_METRIC = ("GQA fused decode attention (q.K, softmax, x V in one pass): µs/call and achieved HBM GB/s "
               "(% of MI355X peak)")
TIMING = ("median of trials of K back-to-back launches between HIP events on the launch stream, each trial "
          "bracketed by synchronisations, after a clock ramp and W warmup calls")


def source_hash(op: str = "av") -> str:
    """SHA-256 over the kernel sources: identifies the kernels a profile was taken on."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[op]:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse(argv=None):
    p = argparse.ArgumentParser(description=__doc__.splitlines()[1])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--op", default="av", choices=["av", "qk", "softmax", "attn"],
                   help="av: attention-times-V (the headline); qk: the decode score step before it; "
                        "softmax: the fused softmax x V product on the scores; attn: fused decode attention "
                        "(scores, softmax and product in one pass over bf16 K and V)")
    p.add_argument("--steps", type=int, default=200, help="calls per timed trial (K)")
    p.add_argument("--warmup", type=int, default=20, help="untimed warmup calls after the clock ramp (W)")
    p.add_argument("--ramp-seconds", type=float, default=0.25,
                   help="untimed clock ramp before the warmup (MI355X needs ~0.25 s under load)")
    p.add_argument("--workload", default=None,
                   help="one workload (default: the suite, headline " + HEADLINE + ")")
    p.add_argument("--mode", default="auto", choices=["auto", "per_head", "reuse"])
    p.add_argument("--per-head", action="store_true", help="suite / av: also time every workload in per-head mode")
    p.add_argument("--nsplit", type=int, default=0, help="force the number of context splits (0 = plan)")
    p.add_argument("--engine", default="auto", choices=["auto", "valu", "mfma", "mfma_bf16"])
    p.add_argument("--kv-tile", type=int, default=0, help="adjacent KV heads per workgroup (0 = plan)")
    p.add_argument("--waves", type=int, default=0, help="waves per workgroup (0 = plan; 8: bf16 matrix engine)")
    p.add_argument("--split-order", default="auto", choices=["auto", "contiguous", "interleaved"],
                   help="how a split context is cut (plan default: auto)")
    p.add_argument("--v-fp8", action="store_true",
                   help="av / softmax with V quantized to OCP FP8 E4M3 with a scale per KV head (half the V bytes)")
    p.add_argument("--k-fp8", action="store_true",
                   help="qk with K quantized to OCP FP8 E4M3 with a scale per KV head (half the K bytes)")
    p.add_argument("--page-size", type=int, default=0,
                   help="av / softmax over a paged V cache (qk: a paged K cache) with this many rows per page "
                        "(shuffled pages, full lengths); 0 = dense")
    p.add_argument("--graph", action="store_true",
                   help="dense av / softmax: time the K whole calls of a trial as one captured HIP graph")
    p.add_argument("--no-read-ceiling", action="store_true", help="skip the plain-read ceiling")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU oracle time budget")
    p.add_argument("--rotate-mb", type=float, default=ROTATE_BYTES / 2 ** 20)
    p.add_argument("--copy-calibration", type=float, default=0.0, metavar="MB")
    p.add_argument("--summarize-trace", metavar="DIR")
    p.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"))
    p.add_argument("--summarize-counters", metavar="DIR", help="per-kernel medians of any --pmc counters")
    p.add_argument("--copy-bytes", type=float, default=1024.0, help="MiB per copy in the calibration runs")
    p.add_argument("--out", help="summary file to write (with --summarize-*)")
    p.add_argument("--command", default="", help="the command line the summarized data came from")
    return p.parse_args(argv)


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


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


def summarize_counters(d: str, out: str, command: str, op: str = "av"):
    """Per-kernel medians over dispatches of whatever counters a rocprofv3
    --pmc run collected (derived ones included), one column per counter."""
    vals = _counter_medians(d)
    kernels = sorted({k for k, _ in vals if "gqa_av" in k})
    counters = sorted({c for _, c in vals})
    lines = ["# rocprofv3 --pmc counter summary (median over dispatches)", f"command: {command}",
             f"kernel_sources_sha256: {source_hash(op)}", "",
             "| kernel | " + " | ".join(counters) + " |", "|---|" + "---|" * len(counters)]
    for k in kernels:
        lines.append(f"| {k[:90]} | " + " | ".join(f"{vals.get((k, c), float('nan')):.2f}" for c in counters) + " |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _profile_kv(path: str):
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("|"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    return kv


def recorded_traffic(workload: str, mode: str, op: str = "av", variant: str = "", require_current: bool = True):
    """The dominant kernel's HBM bytes per launch from the committed PMC summary
    (variant: "" for dense V, "_fp8" or "_paged<P>"). None if there is none, or
    (require_current) if it was not taken on the current kernel sources."""
    prefix = OPS[op][0]
    f = os.path.join(PROFILES, f"{prefix}{variant}_{workload}_{mode}_traffic.md")
    if not os.path.exists(f):
        return None
    kv = _profile_kv(f)
    key = f"{prefix}_traffic_bytes"
    if key not in kv or (require_current and kv.get("kernel_sources_sha256") != source_hash(op)):
        return None
    return float(kv[key])


def fetch_ratio(w) -> dict | None:
    """Reuse / per-head HBM bytes of pass 1 from the committed counter profiles
    (the page's claim: reuse cuts V traffic about G-fold)."""
    reuse = recorded_traffic(w.name, "auto", require_current=False)
    per_head = recorded_traffic(w.name, "per_head", require_current=False)
    if reuse is None or per_head is None:
        return None
    current = (recorded_traffic(w.name, "auto") is not None and recorded_traffic(w.name, "per_head") is not None)
    return {"value": round(reuse / per_head, 4), "reuse_bytes": reuse, "per_head_bytes": per_head,
            "algorithmic_ratio": round(w.algorithmic_bytes() / w.per_head_bytes(), 4),
            "profiles_on_current_sources": current}


def copy_calibration(mib: float):
    import torch
    n = int(mib * 2 ** 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {n} bytes x3", flush=True)


# ---- inputs: rotation sets in one allocation --------------------------------------

def _align(n: int, a: int) -> int:
    return (n + a - 1) // a * a


def set_count(per_set: int, rotate_bytes: float) -> int:
    """Rotation copies for inputs of per_set bytes: enough to exceed rotate_bytes, at most MAX_SETS."""
    return max(1, min(MAX_SETS, math.ceil(rotate_bytes / max(1, per_set))))


def set_layout(parts) -> tuple[list[int], int]:
    """Byte offsets of `parts` (byte sizes) inside one rotation set, each 256-byte
    aligned, and the set stride (4 KiB aligned)."""
    offs, o = [], 0
    for n in parts:
        offs.append(o)
        o = _align(o + n, 256)
    return offs, _align(max(o, 1), 4096)


class DeviceSets:
    """nrot copies of a list of tensors in ONE device allocation.

    host: CPU tensors copied into every set; outs: (shape, dtype) of tensors
    left uninitialised in every set. sets[i] lists set i's views, host tensors
    first. Set 0 is filled from the host, the others by device copies of set 0.
    """

    def __init__(self, host, outs, nrot: int, dev):
        import torch
        shapes = [(tuple(t.shape), t.dtype) for t in host] + [(tuple(s), d) for s, d in outs]
        sizes = [math.prod(s) * torch.empty((), dtype=d).element_size() for s, d in shapes]
        self.offsets, self.stride = set_layout(sizes)
        self.nrot = nrot
        self.set_bytes = sum(sizes)
        self.buf = torch.empty(nrot * self.stride, dtype=torch.uint8, device=dev)
        self.sets = []
        for i in range(nrot):
            views = []
            for (shape, dt), off, n in zip(shapes, self.offsets, sizes):
                b = self.buf[i * self.stride + off: i * self.stride + off + n]
                views.append(b.view(dt).view(shape))
            self.sets.append(views)
        for t, v in zip(host, self.sets[0]):
            v.copy_(t.contiguous().view(v.dtype).view(v.shape), non_blocking=False)
        for i in range(1, nrot):
            self.buf[i * self.stride:(i + 1) * self.stride].copy_(self.buf[:self.stride])
        if self.buf.is_cuda:
            torch.cuda.synchronize()

    def base(self, i: int):
        """The bytes of set i (from its first tensor)."""
        return self.buf[i * self.stride:(i + 1) * self.stride]


# ---- timing -------------------------------------------------------------------------

def ramp(fns, seconds: float) -> dict:
    """Untimed calls for at least `seconds` of wall time (clock ramp)."""
    import torch
    t0 = time.perf_counter()
    n, batch = 0, 8
    while True:
        for _ in range(batch):
            fns[n % len(fns)]()
            n += 1
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        if el >= seconds:
            break
        batch = min(4096, batch * 2)
    return {"seconds": round(el, 3), "calls": n}


def prepare(args, fns) -> dict:
    """Clock ramp, then W warmup calls."""
    import torch
    r = ramp(fns, args.ramp_seconds)
    for i in range(args.warmup):
        fns[i % len(fns)]()
    torch.cuda.synchronize()
    return r


def trials(fns, steps: int, stream, min_trials: int = 5, max_trials: int = 30, rel_se: float = 0.005,
           min_calls: int = 100, min_ms: float = 1.0) -> dict:
    """Repeated trials of `steps` back-to-back calls of fns (rotating) between two
    HIP events on `stream`, each bracketed by synchronisations. Stops when the
    standard error of the per-call means is at most rel_se of their median
    (after at least min_trials trials, min_calls calls and min_ms of timed work),
    or after max_trials trials (more if min_calls needs them)."""
    import torch
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per, k = [], 0
    cap = max(max_trials, math.ceil(min_calls / steps))
    while True:
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(steps):
            fns[k % len(fns)]()
            k += 1
        end.record(stream)
        torch.cuda.synchronize()
        per.append(start.elapsed_time(end) / steps)
        n = len(per)
        med = statistics.median(per)
        se = statistics.stdev(per) / math.sqrt(n) if n > 1 else float("inf")
        enough = n >= min_trials and n * steps >= min_calls and sum(per) * steps >= min_ms
        if (enough and se <= rel_se * med) or n >= cap:
            break
    return {"median_us": round(med * 1e3, 3), "se_us": round(se * 1e3, 4), "mean_us": round(statistics.mean(per) * 1e3, 3),
            "trials": n, "steps_per_trial": steps}


def rate(nbytes: int, us: float) -> dict:
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"gbs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


def read_ceiling(args, sets: DeviceSets, nbytes: int, stream) -> dict | None:
    """The plain streaming read (gqa_bench.h) of nbytes from each rotation set in
    turn, best over workgroup counts and loads in flight: the practical HBM
    ceiling for this byte count on this device."""
    import torch

    import gqa_reuse_attn_amd as ga
    nbytes = nbytes // 16 * 16
    if args.no_read_ceiling or nbytes <= 0:
        return None
    sink = torch.zeros(256, dtype=torch.int32, device=stream.device)
    best = None
    for pat in READ_PATTERNS:
        for wg in READ_GRIDS:
            for lif in READ_LOADS:
                if pat == 1 and nbytes < 256 * 16 * lif * wg:
                    continue                       # the grid-stride pattern needs a batch per workgroup
                fns = [lambda i=i, wg=wg, lif=lif, pat=pat: ga.stream_read(sets.base(i), nbytes, wg, lif, sink,
                                                                           stream, pattern=pat)
                       for i in range(sets.nrot)]
                for f in fns[:8]:
                    f()
                t = trials(fns, args.steps, stream, min_trials=3, max_trials=10, rel_se=0.01)
                if best is None or t["median_us"] < best["us"]:
                    best = {"us": t["median_us"], "se_us": t["se_us"], "workgroups": wg, "loads_in_flight": lif,
                            "pattern": "grid-stride batches" if pat else "contiguous slice per workgroup"}
    best.update(rate(nbytes, best["us"]))
    best["bytes"] = nbytes
    best["kernel"] = "gqa_bench_stream_read: 16-byte non-temporal loads, best of both patterns"
    return best


# ---- CPU baseline ---------------------------------------------------------------

def _threads() -> int:
    return int(os.environ.get("OMP_NUM_THREADS") or 0) or len(os.sched_getaffinity(0))


def _oracle_rate(fn, alg_bytes: int, budget_s: float, what: str):
    """Time fn(nthreads) (an oracle call) repeatedly for ~budget_s on all host threads."""
    threads = _threads()
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
            "sample": f"{what}, {reps} calls in {el:.1f} s (fp64 C oracle, OpenMP)"}


def cpu_baseline(w, attn, V, budget_s: float, softmax: bool = False):
    """The CPU oracle (fp64, OpenMP) on the same workload, repeated for ~budget_s."""
    import oracle
    orc = oracle.get()
    fn = orc.softmax_av if softmax else orc.full
    return _oracle_rate(lambda n: fn(attn, V, w.v_dtype, nthreads=n), w.algorithmic_bytes(), budget_s,
                        f"full workload {w.name}{' (fused softmax)' if softmax else ''}")


# ---- the AV product (and the fused softmax product) on dense V ---------------------

def _plan_dict(plan) -> dict:
    keep = ("mode", "engine", "heads_per_tile", "kv_heads_per_tile", "vec_bytes", "lanes_per_row", "row_slots",
            "nsplit", "rows_per_split", "interleave", "grid", "threads", "combine", "workspace_bytes")
    d = plan.as_dict()
    return {k: d[k] for k in keep}


def measure_av(args, w, dev, props, mode: str, softmax: bool = False, host=None) -> dict:
    """Whole calls, pass 1 alone and the read ceiling of one workload (dense V)."""
    import torch

    import gqa_reuse_attn_amd as ga
    from workloads import make_inputs, make_scores

    if host is None:
        host = (make_scores if softmax else make_inputs)(w, seed=0)
    attn_h, V_h = host
    plan = ga.make_plan(w.B, w.C, w.Hq, w.Hkv, w.D, w.v_dtype, mode, nsplit=args.nsplit,
                        engine=args.engine, kv_tile=args.kv_tile, waves=args.waves,
                        split_order=args.split_order, cu_count=props.multi_processor_count, softmax=softmax)
    alg = w.algorithmic_bytes()
    nrot = set_count(alg, args.rotate_mb * 2 ** 20)
    sets = DeviceSets([V_h, attn_h], [((w.B, w.Hq, w.D), torch.float32)], nrot, dev)
    # --graph: the calls are bound to a side stream, which graph capture needs.
    stream = torch.cuda.Stream(dev) if args.graph else torch.cuda.current_stream(dev)
    bind = ga.bind_softmax if softmax else ga.bind
    calls = [bind(a, v, o, plan=plan, stream=stream) for v, a, o in sets.sets]
    r = prepare(args, calls)
    if args.graph:
        # One graph of K calls (rotating through the sets); a trial is one replay.
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for k in range(args.steps):
                calls[k % nrot]()
        torch.cuda.synchronize()

        def replay():
            with torch.cuda.stream(stream):
                graph.replay()
        replay()
        t = trials([replay], 1, stream, min_calls=1, min_ms=0.0)
        for key in ("median_us", "se_us", "mean_us"):
            t[key] = round(t[key] / args.steps, 4)
        t["steps_per_trial"] = args.steps
        t["launch"] = "one HIP graph of K calls per trial"
    else:
        t = trials(calls, args.steps, stream)
    p1 = trials([c.pass1 for c in calls], args.steps, stream)
    # the next stream work must not find split partials of a pass 1 without combine
    torch.cuda.synchronize()
    ceil = read_ceiling(args, sets, alg, stream)
    res = {
        "workload": w.name, "B": w.B, "C": w.C, "Hq": w.Hq, "Hkv": w.Hkv, "G": w.G, "D": w.D,
        "v_dtype": w.v_dtype, "mode": mode, "algorithmic_bytes": alg, "plan": _plan_dict(plan),
        "kernels_per_call": 2 if plan.nsplit > 1 and plan.combine == 1 else 1,
        "rotation_sets": nrot, "cache_resident": nrot * alg < args.rotate_mb * 2 ** 20,
        "clock_ramp": r, "call": t, "call_rate": rate(alg, t["median_us"]),
        "pass1": p1, "pass1_rate": rate(alg, p1["median_us"]), "read_ceiling": ceil,
    }
    if ceil:
        res["call_vs_read_ceiling"] = round(ceil["us"] / t["median_us"], 4)
        res["pass1_vs_read_ceiling"] = round(ceil["us"] / p1["median_us"], 4)
    log(f"{w.name} {mode}{' softmax' if softmax else ''}: call {t['median_us']:.2f} ± {t['se_us']:.3f} us "
        f"({100 * res['call_rate']['frac_of_peak']:.1f}% of peak), pass 1 {p1['median_us']:.2f} us "
        f"({100 * res['pass1_rate']['frac_of_peak']:.1f}%), read ceiling "
        f"{ceil['us'] if ceil else float('nan'):.2f} us; {nrot} sets; plan {_plan_dict(plan)}")
    del calls, sets
    torch.cuda.empty_cache()
    return res


def _line(metric: str, args, res: dict, roofline: dict, cpu, extra_config=None) -> dict:
    t = res["call"]
    cfg = {"workload": res["workload"], "B": res["B"], "C": res["C"], "Hq": res["Hq"], "Hkv": res["Hkv"],
           "G": res["G"], "D": res["D"], "v_dtype": res["v_dtype"], "mode": res["mode"],
           "algorithmic_bytes": res["algorithmic_bytes"], "rotation_sets": res["rotation_sets"],
           "cache_resident": res["cache_resident"], "kernels_per_call": res.get("kernels_per_call"),
           "plan": res["plan"], "launch": t.get("launch", "K stream launches"),
           "clock_ramp_s": res["clock_ramp"]["seconds"], "timing": TIMING}
    cfg.update(extra_config or {})
    return {
        "metric": metric, "value": res["call_rate"]["gbs"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(t["median_us"] / 1e3, 6), "us_per_call": t["median_us"],
        "us_per_call_se": t["se_us"], "trials": t["trials"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic", "config": cfg, "roofline": roofline,
        "whole_call_frac_of_peak": res["call_rate"]["frac_of_peak"], "read_ceiling": res.get("read_ceiling"),
        "cpu_baseline": cpu,
    }


def _pass1_roofline(res: dict, traffic) -> dict:
    p1 = res["pass1"]
    return {"bound": "hbm", "achieved": res["pass1_rate"]["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": res["pass1_rate"]["frac_of_peak"], "traffic": traffic, "kernel": "pass 1 (V streaming)",
            "us_per_launch": p1["median_us"], "us_per_launch_se": p1["se_us"],
            "timing": "pass 1 alone: " + TIMING}


def _summary(res: dict) -> dict:
    """The per-workload entry of the suite's "configs"."""
    keep = ("B", "C", "Hq", "Hkv", "G", "D", "v_dtype", "algorithmic_bytes", "plan", "kernels_per_call",
            "rotation_sets", "cache_resident", "call", "call_rate", "pass1", "pass1_rate", "read_ceiling",
            "call_vs_read_ceiling", "pass1_vs_read_ceiling")
    return {k: res[k] for k in keep if k in res}


def run_suite(args, dev, props):
    """Every decode workload in the automatic mode; the headline line is the large batch."""
    import torch

    from workloads import WORKLOADS, make_inputs
    configs, headline, host5 = {}, None, None
    for name in SUITE:
        w = WORKLOADS[name]
        host = make_inputs(w, seed=0)
        res = measure_av(args, w, dev, props, "auto", host=host)
        entry = _summary(res)
        fr = fetch_ratio(w)
        entry["fetch_ratio_reuse_per_head"] = fr
        if args.per_head:
            ph = measure_av(args, w, dev, props, "per_head", host=host)
            entry["per_head"] = {k: ph[k] for k in ("call", "call_rate", "pass1", "pass1_rate", "plan")}
        configs[name] = entry
        if name == HEADLINE:
            headline, host5 = res, host
        del host
        torch.cuda.empty_cache()
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        w = WORKLOADS[HEADLINE]
        cpu = cpu_baseline(w, host5[0], host5[1], args.cpu_seconds)
    traffic = recorded_traffic(HEADLINE, "auto")
    line = _line(METRIC, args, headline, _pass1_roofline(headline, traffic), cpu,
                 {"suite": "every decode workload under configs (automatic plans); headline: the large batch"})
    line["configs"] = configs
    print(json.dumps(line), flush=True)


def run_one_av(args, w, dev, props):
    softmax = args.op == "softmax"
    res = measure_av(args, w, dev, props, args.mode, softmax=softmax)
    cpu = None
    if not args.no_cpu_baseline:
        from workloads import make_inputs, make_scores
        log("timing the CPU oracle")
        attn_h, V_h = (make_scores if softmax else make_inputs)(w, seed=0)
        cpu = cpu_baseline(w, attn_h, V_h, args.cpu_seconds, softmax=softmax)
    default_plan = (args.nsplit == 0 and args.engine == "auto" and args.kv_tile == 0 and args.waves == 0
                    and args.split_order == "auto")
    traffic = recorded_traffic(w.name, args.mode, args.op) if default_plan else None
    line = _line(SOFTMAX_METRIC if softmax else METRIC, args, res, _pass1_roofline(res, traffic), cpu)
    if softmax:
        line["config"]["workload"] = "softmax:" + w.name
    print(json.dumps(line), flush=True)


# ---- variants: fp8 V, paged V, the score step, fused attention -------------------------

def _variant_line(metric, args, w, workload, alg, nrot, plan_d, r, t, p1, cpu, traffic, extra=None):
    cfg = {"workload": workload, "B": w.B, "C": w.C, "Hq": w.Hq, "Hkv": w.Hkv, "G": w.G, "D": w.D,
           "mode": args.mode, "algorithmic_bytes": alg, "rotation_sets": nrot, "plan": plan_d,
           "clock_ramp_s": r["seconds"], "timing": TIMING}
    cfg.update(extra or {})
    p = p1 or t
    pr = rate(alg, p["median_us"])
    return {
        "metric": metric, "value": rate(alg, t["median_us"])["gbs"], "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t["median_us"] / 1e3, 6),
        "us_per_call": t["median_us"], "us_per_call_se": t["se_us"], "trials": t["trials"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": cfg,
        "roofline": {"bound": "hbm", "achieved": pr["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": pr["frac_of_peak"], "traffic": traffic,
                     "kernel": "pass 1" if p1 else "the one kernel of the call",
                     "us_per_launch": p["median_us"], "us_per_launch_se": p["se_us"], "timing": TIMING},
        "cpu_baseline": cpu,
    }


def _quant_fp8(X):
    """Per-KV-head scale max|x| / 448 and the E4M3 values of x / scale."""
    import torch
    Xf = X.float()
    sc = (Xf.abs().amax(dim=(0, 1, 3)).clamp_min(1e-30) / 448.0).contiguous()
    return (Xf / sc.view(1, 1, -1, 1)).to(torch.float8_e4m3fn).contiguous(), sc


def bench_fp8(args, w, dev, props):
    """The AV product (or the fused softmax product) with the workload's V
    quantized to OCP FP8 E4M3 with a float32 scale per KV head (max |V| / 448).
    Algorithmic bytes: V at one byte per value, the weights, the output."""
    import torch

    import gqa_reuse_attn_amd as ga
    from workloads import make_inputs, make_scores

    softmax = args.op == "softmax"
    x_h, V_h = (make_scores if softmax else make_inputs)(w, seed=0)
    q_h, scale_h = _quant_fp8(V_h)
    alg = w.B * w.C * w.Hkv * w.D + w.attn_bytes() + w.out_bytes()
    plan = ga.make_plan(w.B, w.C, w.Hq, w.Hkv, w.D, "fp8", args.mode, engine=args.engine, nsplit=args.nsplit,
                        cu_count=props.multi_processor_count, kv_tile=args.kv_tile, softmax=softmax,
                        waves=args.waves)
    nrot = set_count(alg, args.rotate_mb * 2 ** 20)
    sets = DeviceSets([q_h, x_h], [((w.B, w.Hq, w.D), torch.float32)], nrot, dev)
    sc = scale_h.to(dev)
    stream = torch.cuda.current_stream(dev)
    calls = [ga.bind_fp8(x, q, sc, out=o, plan=plan) for q, x, o in sets.sets]
    r = prepare(args, calls)
    t = trials(calls, args.steps, stream)
    p1 = trials([c.pass1 for c in calls], args.steps, stream)
    torch.cuda.synchronize()
    log(f"fp8 {'softmax ' if softmax else ''}{t['median_us']:.2f} us/call, pass 1 {p1['median_us']:.2f} us; "
        f"{nrot} sets, plan {_plan_dict(plan)}")
    default_plan = args.nsplit == 0 and args.engine == "auto" and args.kv_tile == 0 and args.waves == 0
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.get()
        cpu = _oracle_rate(lambda n: orc.fp8(x_h, q_h, scale_h, softmax=softmax, nthreads=n), alg,
                           args.cpu_seconds, f"full fp8 workload {w.name}")
    traffic = recorded_traffic(w.name, args.mode, args.op, "_fp8") if default_plan else None
    print(json.dumps(_variant_line(FP8_METRIC, args, w, f"fp8{'-softmax' if softmax else ''}:{w.name}", alg, nrot,
                                   _plan_dict(plan), r, t, p1, cpu, traffic, {"v_dtype": "fp8_e4m3"})), flush=True)


def _shuffled_pages(w, P, X):
    """X [B, C, Hkv, D] cut into pages of P rows stored in a seeded shuffled order."""
    import torch
    if w.C % P:
        raise SystemExit(f"--page-size {P} must divide C={w.C}")
    maxp = w.C // P
    perm = torch.randperm(w.B * maxp, generator=torch.Generator().manual_seed(0))
    flat = X.view(torch.uint8) if X.dtype == torch.float8_e4m3fn else X
    pages = torch.empty((w.B * maxp, P, w.Hkv, w.D), dtype=flat.dtype)
    pages[perm] = flat.reshape(w.B * maxp, P, w.Hkv, w.D)
    if X.dtype == torch.float8_e4m3fn:
        pages = pages.view(torch.float8_e4m3fn)
    bt = perm.to(torch.int32).view(w.B, maxp).contiguous()
    lens = torch.full((w.B,), w.C, dtype=torch.int32)
    return pages, bt, lens


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
    x_h, V_h = (make_scores if softmax else make_inputs)(w, seed=0)
    pages_h, bt_h, lens_h = _shuffled_pages(w, P, V_h)
    bt, lens = bt_h.to(dev), lens_h.to(dev)
    plan = ga.make_plan(w.B, w.C, w.Hq, w.Hkv, w.D, w.v_dtype, args.mode, engine=args.engine, nsplit=args.nsplit,
                        cu_count=props.multi_processor_count, kv_tile=args.kv_tile, softmax=softmax, page_size=P,
                        waves=args.waves)
    alg = w.algorithmic_bytes()
    nrot = set_count(alg, args.rotate_mb * 2 ** 20)
    sets = DeviceSets([pages_h, x_h], [((w.B, w.Hq, w.D), torch.float32)], nrot, dev)
    stream = torch.cuda.current_stream(dev)
    calls = [ga.bind_paged(x, pg, bt, lens, out=o, plan=plan) for pg, x, o in sets.sets]
    r = prepare(args, calls)
    t = trials(calls, args.steps, stream)
    p1 = trials([c.pass1 for c in calls], args.steps, stream)
    torch.cuda.synchronize()
    log(f"paged P={P} {'softmax ' if softmax else ''}{t['median_us']:.2f} us/call, pass 1 {p1['median_us']:.2f} us; "
        f"{nrot} sets, plan {_plan_dict(plan)}")
    default_plan = args.nsplit == 0 and args.engine == "auto" and args.kv_tile == 0 and args.waves == 0
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.get()
        cpu = _oracle_rate(lambda n: orc.paged(x_h, pages_h, bt_h, lens_h, w.v_dtype, softmax=softmax, nthreads=n),
                           alg, args.cpu_seconds, f"full paged P={P} {w.name}")
    traffic = recorded_traffic(w.name, args.mode, args.op, f"_paged{P}") if default_plan else None
    print(json.dumps(_variant_line(PAGED_METRIC, args, w, f"paged{P}{'-softmax' if softmax else ''}:{w.name}", alg,
                                   nrot, _plan_dict(plan), r, t, p1, cpu, traffic,
                                   {"v_dtype": w.v_dtype, "page_size": P})), flush=True)


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
        K_h, ks_h = _quant_fp8(K_h)
        kdt = "fp8"
    es = {"f32": 4, "fp8": 1}.get(kdt, 2)
    alg = w.B * w.C * w.Hkv * w.D * es + 4 * w.B * w.Hq * w.D + 4 * w.B * w.C * w.Hq
    P = args.page_size
    plan = ga.qk_make_plan(w.B, w.C, w.Hq, w.Hkv, w.D, kdt, args.mode, cu_count=props.multi_processor_count,
                           page_size=P)
    nrot = set_count(alg, args.rotate_mb * 2 ** 20)
    ks = ks_h.to(dev) if ks_h is not None else None
    scores_out = [((w.B, w.C, w.Hq), torch.float32)]
    if P > 0:
        pages_h, bt_h, lens_h = _shuffled_pages(w, P, K_h)
        bt, lens = bt_h.to(dev), lens_h.to(dev)
        sets = DeviceSets([pages_h, q_h], scores_out, nrot, dev)
        calls = [ga.BoundQkPaged(q, pg, bt, lens, scores=s, C=w.C, scale=w.D ** -0.5, plan=plan, k_scale=ks)
                 for pg, q, s in sets.sets]
    else:
        sets = DeviceSets([K_h, q_h], scores_out, nrot, dev)
        calls = [ga.bind_qk(q, k, scores=s, scale=w.D ** -0.5, plan=plan, k_scale=ks) for k, q, s in sets.sets]
    stream = torch.cuda.current_stream(dev)
    r = prepare(args, calls)
    t = trials(calls, args.steps, stream)
    log(f"qk {t['median_us']:.2f} us/call; {nrot} sets, plan {plan.as_dict()}")
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.get()
        if args.k_fp8:
            fn = lambda n: orc.qk_fp8(q_h, K_h, ks_h, w.D ** -0.5, nthreads=n)  # noqa: E731
        else:
            fn = lambda n: orc.qk(q_h, K_h, w.v_dtype, w.D ** -0.5, nthreads=n)  # noqa: E731
        cpu = _oracle_rate(fn, alg, args.cpu_seconds,
                           f"full score step of {w.name}{' (fp8 K)' if args.k_fp8 else ''}")
    traffic = recorded_traffic(w.name, args.mode, "qk", ("_fp8" if args.k_fp8 else "") + (f"_paged{P}" if P else ""))
    print(json.dumps(_variant_line(QK_METRIC, args, w, f"qk{'-fp8' if args.k_fp8 else ''}{f'-paged{P}' if P else ''}:"
                                   f"{w.name}", alg, nrot, plan.as_dict(), r, t, None, cpu, traffic,
                                   {"k_dtype": "fp8_e4m3" if args.k_fp8 else w.v_dtype, "page_size": P,
                                    "kernels_per_call": 1})), flush=True)


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
        (K_h, ks_h), (V_h, vs_h) = _quant_fp8(K_h), _quant_fp8(V_h)
        kvdt = "fp8"
    kv_bytes = w.v_bytes() // (2 if args.v_fp8 else 1)
    alg = 2 * kv_bytes + 4 * w.B * w.Hq * w.D + w.out_bytes()
    P = args.page_size
    plan = ga.make_plan(w.B, w.C, w.Hq, w.Hkv, w.D, kvdt, args.mode, nsplit=args.nsplit, kv_tile=args.kv_tile,
                        cu_count=props.multi_processor_count, attention=True, page_size=P)
    nrot = set_count(alg, args.rotate_mb * 2 ** 20)
    if P:
        # A paged cache: K and V cut into pages of P rows, both pools in one
        # shuffled order (one block table), every sequence at full length.
        K_h, bt_h, lens_h = _shuffled_pages(w, P, K_h)
        V_h, _, _ = _shuffled_pages(w, P, V_h)
        bt, lens = bt_h.to(dev), lens_h.to(dev)
    outs = [((w.B, w.Hq, w.D), torch.float32), ((w.B, w.C, w.Hq), torch.float32)]   # out, scores of the pair
    sets = DeviceSets([q_h, K_h, V_h], outs, nrot, dev)
    ks = ks_h.to(dev) if ks_h is not None else None
    vs = vs_h.to(dev) if vs_h is not None else None
    if P:
        calls = [ga.BoundAttentionPaged(q, k, v, bt, lens, out=o, scale=scale, plan=plan, k_scale=ks, v_scale=vs)
                 for q, k, v, o, _ in sets.sets]
    else:
        calls = [ga.BoundAttention(q, k, v, out=o, scale=scale, plan=plan, k_scale=ks, v_scale=vs)
                 for q, k, v, o, _ in sets.sets]
    stream = torch.cuda.current_stream(dev)
    r = prepare(args, calls)
    t = trials(calls, args.steps, stream)
    p1 = trials([c.pass1 for c in calls], args.steps, stream)
    torch.cuda.synchronize()
    # the unfused pair on the same inputs: score step, then the fused softmax product
    if P:
        # (the paged product takes no V scale: the same work with unit scales)
        qk = [ga.BoundQkPaged(q, k, bt, lens, scores=s, scale=scale, k_scale=ks) for q, k, _, _, s in sets.sets]
        sav = [ga.bind_paged(s, v, bt, lens, out=o, softmax=True) for _, _, v, o, s in sets.sets]
    else:
        qk = [ga.bind_qk(q, k, scores=s, scale=scale, k_scale=ks) for q, k, _, _, s in sets.sets]
        sav = [(ga.BoundFp8(s, v, vs, out=o, softmax=True) if args.v_fp8 else ga.bind_softmax(s, v, out=o))
               for _, _, v, o, s in sets.sets]
    pair = [lambda i=i: (qk[i](), sav[i]()) for i in range(nrot)]
    prepare(args, pair)
    tp = trials(pair, args.steps, stream)
    log(f"attn {t['median_us']:.2f} us/call, pass 1 {p1['median_us']:.2f} us; score step + fused softmax "
        f"{tp['median_us']:.2f} us; {nrot} sets, plan {_plan_dict(plan)}")
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
    traffic = (recorded_traffic(w.name, args.mode, "attn", ("_fp8" if args.v_fp8 else "") + (f"_paged{P}" if P else ""))
               if args.nsplit == 0 and args.kv_tile == 0 else None)
    print(json.dumps(_variant_line(ATTN_METRIC, args, w, f"attn{'-fp8' if args.v_fp8 else ''}"
                                   f"{f'-paged{P}' if P else ''}:{w.name}", alg, nrot, _plan_dict(plan), r, t, p1,
                                   cpu, traffic, {"kv_dtype": "fp8_e4m3" if args.v_fp8 else "bf16", "page_size": P,
                                                  "unfused_us_per_call": tp["median_us"]})), flush=True)


def main(argv=None):
    args = parse(argv)
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.out, args.command, args.op)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc, args.copy_bytes, args.out, args.command, args.op)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.out, args.command, args.op)
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
    from workloads import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ga.load()
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    if args.workload is None:
        if args.op != "av" or args.v_fp8 or args.page_size or args.k_fp8:
            raise SystemExit("the suite runs the dense AV product; name a --workload for the other operations")
        log(f"suite of {len(SUITE)} workloads on {props.name} ({props.multi_processor_count} CUs); "
            f"headline {HEADLINE}")
        run_suite(args, dev, props)
        return
    w = WORKLOADS[args.workload]
    log(f"{args.op} {w.name} mode={args.mode} on {props.name} ({props.multi_processor_count} CUs)")
    if args.op == "qk":
        bench_qk(args, w, dev, props)
    elif args.op == "attn":
        bench_attn(args, w, dev, props)
    elif args.page_size > 0:
        bench_paged(args, w, dev, props)
    elif args.v_fp8:
        bench_fp8(args, w, dev, props)
    else:
        run_one_av(args, w, dev, props)


if __name__ == "__main__":
    main()
