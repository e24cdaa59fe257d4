"""Benchmark of the GQA decode attention-times-V path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--mode auto|per_head]

A step is one call of the whole path (pass 1, and pass 2 when the context is
split) over one batch of synthetic decode input already resident in HBM.
Several copies of the inputs are rotated so that the total exceeds twice the
256 MB Infinity Cache and every step reads V and attn from HBM.

Prints ONE JSON line: µs per call and achieved GB/s over the algorithmic bytes
(V + attn + out, each once), the roofline fraction against 8 TB/s HBM, and the
CPU oracle timed on this host as a baseline.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GQA decode AV: µs/call and achieved HBM GB/s (% of MI355X peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
ROTATE_BYTES = 512 * 2 ** 20   # 2 x the 256 MB Infinity Cache
DEFAULT_WORKLOAD = "g2-b4-c32768-hq16-hkv8-d128-bf16"


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[1])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--mode", default="auto", choices=["auto", "per_head", "reuse"])
    p.add_argument("--nsplit", type=int, default=0, help="force the number of context splits (0 = plan)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU oracle time budget")
    p.add_argument("--rotate-mb", type=float, default=ROTATE_BYTES / 2 ** 20)
    return p.parse_args()


def cpu_baseline(w, attn, V, budget_s: float):
    """The CPU oracle (fp64, OpenMP) on the same workload, repeated for ~budget_s."""
    import oracle
    orc = oracle.get()
    threads = int(os.environ.get("OMP_NUM_THREADS") or 0) or len(os.sched_getaffinity(0))
    reps = 0
    t0 = time.perf_counter()
    while True:
        orc.full(attn, V, w.v_dtype, nthreads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 1000:
            break
    per_call = el / reps
    return {
        "value": w.algorithmic_bytes() / per_call / 1e9,
        "unit": "GB/s",
        "us_per_call": per_call * 1e6,
        "cores": threads,
        "kind": "oracle",
        "sample": f"full workload {w.name}, {reps} calls in {el:.1f} s (fp64 C oracle, OpenMP)",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): this path has no "
              "multi-GPU code; see DESIGN.md for how it would shard.", file=sys.stderr)
        sys.exit(2)

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
    print(f"[bench] {w.name} mode={args.mode} on {props.name} ({props.multi_processor_count} CUs)",
          file=sys.stderr, flush=True)

    attn_h, V_h = make_inputs(w, seed=0)
    plan = ga.make_plan(w.B, w.C, w.Hq, w.Hkv, w.D, w.v_dtype, args.mode, nsplit=args.nsplit,
                        cu_count=props.multi_processor_count)
    per_set = w.v_bytes() + w.attn_bytes() + w.out_bytes()
    nrot = max(1, math.ceil(args.rotate_mb * 2 ** 20 / per_set))
    sets = []
    a0, v0 = attn_h.to(dev), V_h.to(dev)
    for i in range(nrot):
        a = a0 if i == 0 else a0.clone()
        v = v0 if i == 0 else v0.clone()
        sets.append((a, v, torch.empty(w.B, w.Hq, w.D, device=dev)))
    torch.cuda.synchronize()

    calls = [ga.bind(a, v, o, plan=plan) for a, v, o in sets]

    def step(i):
        calls[i % nrot]()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    gbs = w.algorithmic_bytes() / (ms / 1e3) / 1e9
    print(f"[bench] {ms * 1e3:.2f} us/call, {gbs:.1f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of peak), "
          f"{nrot} rotation sets, plan {plan.as_dict()}", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, attn_h, V_h, args.cpu_seconds)

    kernels = 1   # pass 1 and the split-C combine are one kernel
    line = {
        "metric": METRIC,
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
            "workload": w.name, "B": w.B, "C": w.C, "Hq": w.Hq, "Hkv": w.Hkv, "G": w.G, "D": w.D,
            "v_dtype": w.v_dtype, "mode": args.mode, "algorithmic_bytes": w.algorithmic_bytes(),
            "rotation_sets": nrot, "kernels_per_call": kernels, "plan": plan.as_dict(),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": None,
            "timing": "HIP events around the timed calls on the launch stream; one kernel per call",
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
