#!/usr/bin/env python3
"""Benchmark of the QMoE layer on one MI355X.

One step = one qmoe_forward call (route, group, fc1 + activation, fc2,
combine) over one batch of synthetic inputs already resident in HBM.  The
default workload is the int2 GeGLU decode layer (T=8, hidden=inter=2048,
E=8, top-2, block 128, fractional zero point 1.5, fp16); ``--workload N``
selects another of the five named workloads.

To keep the weights from being served by the 256 MB Infinity Cache, each step
uses the next of C identical copies of the expert weights (C copies span
>= 1 GiB), so every step streams its weights from HBM.

Prints one JSON line: tokens/s over the timed steps, the dominant kernel's
roofline (fc1: packed-weight bytes of the selected experts per launch for
decode -> GB/s vs 8 TB/s; 2*R*H*2I flops per launch for prefill -> TFLOP/s vs
2.5 PFLOP/s dense fp16/bf16), and the CPU oracle timed on the host cores on a
bounded sample as a baseline.

The timed region runs the steps with nothing else on the stream; the fc1
kernel's average duration comes from a second pass over the same number of
steps with a HIP event pair around each fc1 launch (on the library's stream),
so the event overhead does not enter the step time.

--calibrate-copy adds one elementwise kernel of known traffic (neg of a 256
MiB float32 tensor: 256 MiB read, 256 MiB written) before the timed region,
for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE; --pmc-summary DIR prints the
per-kernel averages of the rocprofv3 CSV files under DIR (no GPU use).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import qmoe_synth as synth  # noqa: E402
import quantized_mixture_experts_route_amd as qm  # noqa: E402

METRIC = "QMoE layer tokens/s; decode HBM GB/s and prefill TFLOP/s vs MI355X peak"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0  # dense fp16 / bf16
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 256 MiB elementwise kernel before the timed region")
    ap.add_argument("--digest", action="store_true",
                    help="print the digest of the kernel sources that traffic counters are tied to")
    ap.add_argument("--pmc-summary", metavar="DIR",
                    help="summarize rocprofv3 CSV files under DIR and exit")
    ap.add_argument("--graph", action="store_true",
                    help="also time the layer replayed from HIP graphs (one per weight copy)")
    ap.add_argument("--stages", action="store_true",
                    help="also time every stage separately after the timed region")
    return ap.parse_args()


def _to_device(inp, spec, dev):
    dt = torch.float16 if spec["dtype"] == 1 else torch.bfloat16

    def bits(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(dt).to(dev)

    projs = {}
    for name in ("fc1", "fc2"):
        zp = inp[name + "_zp"]
        projs[name] = qm.Projection(torch.from_numpy(inp[name + "_codes"]).to(dev),
                                    bits(inp[name + "_scales"]),
                                    None if zp is None else torch.from_numpy(zp).to(dev),
                                    spec[name + "_bits"])
    return bits(inp["hidden"]), torch.from_numpy(inp["logits"]).to(dev), projs


def _proj_bytes(p: qm.Projection) -> int:
    n = p.codes.numel() + p.scales.numel() * 2
    if p.zero_points is not None:
        n += p.zero_points.numel()
    return n


def _copy_proj(p: qm.Projection) -> qm.Projection:
    return qm.Projection(p.codes.clone(), p.scales.clone(),
                         None if p.zero_points is None else p.zero_points.clone(), p.bits)


def _cpu_baseline(inp, spec, min_seconds):
    """The oracle on a bounded token sample, repeated to >= min_seconds."""
    import oracle
    T = spec["T"]
    per_token = 6.0 * spec["k"] * spec["H"] * spec["I"]
    n_tok = int(max(1, min(T, 2.5e9 // per_token)))  # keep one pass to a few seconds
    tokens = np.linspace(0, T - 1, n_tok).astype(np.int64)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(inp, spec, tokens)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    return {"value": round(reps * n_tok / el, 4), "unit": "tokens/s",
            "cores": min(threads, n_tok), "kind": "oracle",
            "sample": f"{n_tok} of {T} tokens, {reps} passes, {el:.1f} s, double precision"}


CALIBRATION_BYTES = 256 << 20


def kernel_source_digest():
    """sha256 over the library's kernel sources: traffic counters recorded for
    another digest belong to other kernels and are not reported."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "quantized_mixture_experts_route_amd", "csrc", "*"))):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(os.path.basename(f).encode())
            with open(f, "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def _pmc_summary(root):
    """Per-kernel averages of rocprofv3 counter and kernel-stats CSV files."""
    import csv
    import glob
    from collections import defaultdict
    def short(name):
        return name.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]

    vals = defaultdict(lambda: defaultdict(list))
    for f in glob.glob(os.path.join(root, "**", "*_counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            vals[short(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    for name, counters in sorted(vals.items()):
        if "rocprim" in name or "fillBuffer" in name:
            continue
        avg = {c: sum(v) / len(v) for c, v in counters.items()}
        print(f"{name}: " + ", ".join(f"{c}={a:.6g} (n={len(counters[c])})" for c, a in avg.items()))
        if "neg" in name:
            for c, a in avg.items():
                if c in ("FETCH_SIZE", "WRITE_SIZE"):
                    print(f"  calibration {c}: {a * 1024 / CALIBRATION_BYTES:.4f} x bytes moved")
    for f in glob.glob(os.path.join(root, "**", "*_kernel_stats.csv"), recursive=True):
        print(f"{f}:")
        print("| kernel | calls | avg us | min us | max us |\n|---|---|---|---|---|")
        for r in csv.DictReader(open(f)):
            if "rocprim" in r["Name"]:
                continue
            print(f"| {short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} "
                  f"| {float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")


def main():
    a = _args()
    if a.digest:
        print(kernel_source_digest())
        return
    if a.pmc_summary:
        _pmc_summary(a.pmc_summary)
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              "(the layer's multi-GPU expert-parallel sharding is a design, not built)",
              file=sys.stderr)
        sys.exit(2)
    spec = synth.workload(a.workload)
    decode = spec["T"] * spec["k"] <= qm.DECODE_MAX_ROUTES
    steps = a.steps if a.steps is not None else (200 if decode else (20 if spec["T"] > 1024 else 100))
    warmup = a.warmup if a.warmup is not None else max(3, steps // 10)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    inp = synth.make_inputs(spec, synth.seed_for(a.workload))
    hidden, logits, projs = _to_device(inp, spec, dev)
    T, H, I, E, k = spec["T"], spec["H"], spec["I"], spec["E"], spec["k"]
    per_copy = _proj_bytes(projs["fc1"]) + _proj_bytes(projs["fc2"])
    copies = int(min(64, max(2, math.ceil((1 << 30) / per_copy))))
    fc1s = [projs["fc1"]] + [_copy_proj(projs["fc1"]) for _ in range(copies - 1)]
    fc2s = [projs["fc2"]] + [_copy_proj(projs["fc2"]) for _ in range(copies - 1)]
    dt = qm.dtype_code(hidden.dtype)
    ws = qm.alloc_workspace(T, H, I, E, k, dt, dev)
    out = torch.empty_like(hidden)

    def step(i):
        qm.forward(hidden, logits, fc1s[i % copies], fc2s[i % copies], top_k=k,
                   block_size=spec["block_size"], normalize=spec["normalize"],
                   activation=spec["act"], zero_point_offset=spec["zpo"], out=out, workspace=ws)

    if a.calibrate_copy:
        src = torch.ones(CALIBRATION_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / steps

    # fc1 kernel duration: HIP events around each fc1 launch over another
    # `steps` steps (same weight rotation)
    qm.timer_start(qm.STAGE_FC1)
    for i in range(steps):
        step(warmup + steps + i)
    fc1_ms, fc1_n = qm.timer_stop()
    fc1_avg_ms = fc1_ms / max(fc1_n, 1)

    # algorithmic work of one fc1 launch
    ids, _ = qm.route(logits, k, spec["normalize"])
    selected = torch.unique(ids).numel()
    fc1 = projs["fc1"]
    if decode:
        per_expert = _proj_bytes(fc1) // E
        work = selected * per_expert
        achieved = work / (fc1_avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        work = 2.0 * T * k * H * (2 * I)
        achieved = work / (fc1_avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_PEAK_TFLOPS, 4)}
    roof["kernel"] = "fc1 (+ gated activation)"
    roof["kernel_avg_ms"] = round(fc1_avg_ms, 5)
    traffic = None
    if os.path.exists(PROFILE_TRAFFIC):
        with open(PROFILE_TRAFFIC) as f:
            traffic = json.load(f).get(spec["name"])
    if isinstance(traffic, dict) and traffic.get("kernel_source_sha256") == kernel_source_digest():
        roof["traffic"] = traffic.get("bytes_per_launch")
    else:
        roof["traffic"] = None

    result = {
        "metric": METRIC, "value": round(T / (ms_per_step * 1e-3), 2), "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16" if spec["dtype"] == 1 else "bf16", "data": "synthetic",
        "config": {"workload": spec["name"], "T": T, "H": H, "I": I, "E": E, "top_k": k,
                   "fc1_bits": spec["fc1_bits"], "fc2_bits": spec["fc2_bits"],
                   "block_size": spec["block_size"], "path": "decode" if decode else "prefill",
                   "selected_experts": selected, "weight_copies": copies,
                   "parallelism": "single GPU"},
        "roofline": roof,
    }

    if a.graph:
        # one captured layer per weight copy, replayed in the same rotation
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(0)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(c)
            graphs.append(g)
        for i in range(warmup):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            graphs[(warmup + i) % copies].replay()
        torch.cuda.synchronize()
        g_ms = (time.perf_counter() - t0) * 1e3 / steps
        result["graph_replay"] = {"ms_per_step": round(g_ms, 5),
                                  "tokens_per_s": round(T / (g_ms * 1e-3), 2)}
        del graphs

    if a.stages:
        stage_ms = {}
        for name, st in (("route", qm.STAGE_ROUTE), ("group", qm.STAGE_GROUP),
                         ("fc1", qm.STAGE_FC1), ("fc2", qm.STAGE_FC2),
                         ("combine", qm.STAGE_COMBINE)):
            qm.timer_start(st)
            for i in range(steps):
                step(i)
            ms, n = qm.timer_stop()
            stage_ms[name] = round(ms / max(n, 1), 5)
        result["stage_avg_ms"] = stage_ms

    if not a.no_cpu_baseline:
        result["cpu_baseline"] = _cpu_baseline(inp, spec, a.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
