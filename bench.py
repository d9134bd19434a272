#!/usr/bin/env python3
"""Benchmark of the QMoE layer on one MI355X.

One step = one qmoe_forward call (route, group, fc1 + activation, fc2,
combine) over one batch of synthetic inputs already resident in HBM.  The
headline line runs the large skewed prefill layer (T=4096, hidden=4096,
inter=14336, E=8, top-2, int4, block 128, bf16), the largest of the five
workloads; ``per_config`` holds the same measurement for every workload
(tiny int4, int2 GeGLU decode, int4 + u8 zero-point prefill, 512-expert
int3/int2 decode, skewed prefill).

Timing protocol, per workload:
- before every call (warm-up and timed), a 1 GiB buffer is read, so the L2
  and the 256 MB Infinity Cache hold none of the layer's weights or inputs;
- a HIP event pair on the call's stream brackets each timed call (the flush
  is outside it); per-call times give mean, median, p10 and p90; the host
  wall clock over the timed loop is reported beside them;
- the fc1 and fc2 kernels' average durations come from event pairs that the
  library records in those kernels' own dispatch packets, over as many
  further calls under the same protocol.

Rooflines: ``roofline`` is the dominant kernel, fc1 (decode: packed-weight
bytes of the selected experts per launch over 8 TB/s; prefill: 4*R*H*I flops
per launch over 2.5 PFLOP/s dense bf16/fp16).  ``gemm_roofline`` is the
layer's two grouped projections together (decode: fc1 + fc2 packed bytes
over the summed durations; prefill: 6*R*H*I flops over the summed
durations).  ``cpu_baseline`` is the double-precision CPU oracle timed on the
host cores on a bounded token sample of the headline workload.

--calibrate-copy adds one elementwise kernel of known traffic (neg of a 256
MiB float32 tensor: 256 MiB read, 256 MiB written) before the timed region,
for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE; --pmc-summary DIR prints the
per-kernel averages of the rocprofv3 CSV files under DIR (no GPU use).
"""
from __future__ import annotations

import argparse
import json
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
HEADLINE = 5
FLUSH_BYTES = 1 << 30
CALIBRATION_BYTES = 256 << 20


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=HEADLINE, choices=[1, 2, 3, 4, 5],
                    help="workload of the headline line")
    ap.add_argument("--no-per-config", action="store_true",
                    help="measure the headline workload only")
    ap.add_argument("--min-steps-per-config", type=int, default=100,
                    help="per_config entries time at least this many calls")
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
                    help="also time the headline layer replayed from a HIP graph")
    ap.add_argument("--stages", action="store_true",
                    help="also time every stage of the headline layer separately")
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


def _cpu_baseline(inp, spec, min_seconds):
    """The oracle on a bounded token sample, repeated to >= min_seconds."""
    import oracle
    T = spec["T"]
    host_cores = len(os.sched_getaffinity(0))
    threads = int(os.environ.get("OMP_NUM_THREADS", host_cores))
    n_tok = min(T, threads)  # one token per thread and pass, every thread busy
    tokens = np.linspace(0, T - 1, n_tok).astype(np.int64)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(inp, spec, tokens)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    return {"value": round(reps * n_tok / el, 4), "unit": "tokens/s",
            "cores": min(threads, n_tok), "host_cores": host_cores, "kind": "oracle",
            "sample": f"{n_tok} of {T} tokens of {spec['name']}, {reps} passes, {el:.1f} s, "
                      f"double precision, OpenMP over tokens"}


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


class Layer:
    """One workload's inputs on the device and a callable layer step."""

    def __init__(self, cfg, dev):
        self.cfg = cfg
        self.spec = spec = synth.workload(cfg)
        self.inp = synth.make_inputs(spec, synth.seed_for(cfg))
        self.hidden, self.logits, self.projs = _to_device(self.inp, spec, dev)
        T, H, I, E, k = spec["T"], spec["H"], spec["I"], spec["E"], spec["k"]
        self.ws = qm.alloc_workspace(T, H, I, E, k, qm.dtype_code(self.hidden.dtype), dev)
        self.out = torch.empty_like(self.hidden)
        self.decode = T * k <= qm.DECODE_MAX_ROUTES

    def __call__(self):
        s = self.spec
        qm.forward(self.hidden, self.logits, self.projs["fc1"], self.projs["fc2"], top_k=s["k"],
                   block_size=s["block_size"], normalize=s["normalize"], activation=s["act"],
                   zero_point_offset=s["zpo"], out=self.out, workspace=self.ws)


class Flush:
    """Reads a 1 GiB buffer: afterwards no cache level holds the layer's data."""

    def __init__(self, dev):
        self.buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
        self.acc = torch.empty((), dtype=torch.float32, device=dev)

    def __call__(self):
        torch.sum(self.buf, dim=0, out=self.acc)


def _time_calls(step, flush, steps, warmup):
    """Per-call HIP event times (ms) of `steps` calls, each after a cache flush."""
    for _ in range(warmup):
        flush()
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        flush()
        starts[i].record()
        step()
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return np.array([s.elapsed_time(e) for s, e in zip(starts, ends)]), wall


def _stage_avg(step, flush, stage, steps):
    """Average duration (ms) of one stage's kernel, from event pairs in its dispatch packets."""
    qm.timer_start(stage)
    for _ in range(steps):
        flush()
        step()
    ms, n = qm.timer_stop()
    return ms / max(n, 1), n


def _traffic(name):
    if not os.path.exists(PROFILE_TRAFFIC):
        return None
    with open(PROFILE_TRAFFIC) as f:
        rec = json.load(f).get(name)
    if isinstance(rec, dict) and rec.get("kernel_source_sha256") == kernel_source_digest():
        return rec.get("bytes_per_launch")
    return None


def measure(layer: Layer, flush, steps, warmup):
    spec = layer.spec
    T, H, I, E, k = spec["T"], spec["H"], spec["I"], spec["E"], spec["k"]
    per_call, wall = _time_calls(layer, flush, steps, warmup)
    fc1_ms, _ = _stage_avg(layer, flush, qm.STAGE_FC1, steps)
    fc2_ms, _ = _stage_avg(layer, flush, qm.STAGE_FC2, steps)
    ids, _ = qm.route(layer.logits, k, spec["normalize"])
    selected = int(torch.unique(ids).numel())
    mean_ms = float(per_call.mean())
    entry = {
        "workload": spec["name"], "T": T, "H": H, "I": I, "E": E, "top_k": k,
        "fc1_bits": spec["fc1_bits"], "fc2_bits": spec["fc2_bits"],
        "block_size": spec["block_size"], "dtype": "f16" if spec["dtype"] == 1 else "bf16",
        "path": "decode" if layer.decode else "prefill", "selected_experts": selected,
        "steps": steps, "warmup": warmup,
        "tokens_per_s": round(T / (mean_ms * 1e-3), 2),
        "layer_ms": {"mean": round(mean_ms, 5), "median": round(float(np.median(per_call)), 5),
                     "p10": round(float(np.percentile(per_call, 10)), 5),
                     "p90": round(float(np.percentile(per_call, 90)), 5),
                     "wall_mean": round(wall * 1e3 / steps, 5)},
        "fc1_ms": round(fc1_ms, 5), "fc2_ms": round(fc2_ms, 5),
    }
    if layer.decode:
        b1 = selected * (_proj_bytes(layer.projs["fc1"]) // E)
        b2 = selected * (_proj_bytes(layer.projs["fc2"]) // E)
        a1 = b1 / (fc1_ms * 1e-3) / 1e9
        ag = (b1 + b2) / ((fc1_ms + fc2_ms) * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(a1, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(a1 / HBM_PEAK_GBS, 4), "kernel": "fc1 (+ gated activation)",
                "kernel_avg_ms": round(fc1_ms, 5), "work_per_launch": b1,
                "work_unit": "packed weight bytes (codes + scales + zero points) of the selected experts"}
        gemm = {"bound": "hbm", "achieved": round(ag, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ag / HBM_PEAK_GBS, 4), "kernels": "fc1 + fc2",
                "ms": round(fc1_ms + fc2_ms, 5), "work": b1 + b2}
    else:
        f1 = 4.0 * T * k * H * I
        fl = 6.0 * T * k * H * I
        a1 = f1 / (fc1_ms * 1e-3) / 1e12
        ag = fl / ((fc1_ms + fc2_ms) * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(a1, 1), "peak": MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(a1 / MFMA_PEAK_TFLOPS, 4),
                "kernel": "fc1 (+ gated activation)", "kernel_avg_ms": round(fc1_ms, 5),
                "work_per_launch": f1, "work_unit": "flops 2*R*H*2I"}
        gemm = {"bound": "mfma", "achieved": round(ag, 1), "peak": MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ag / MFMA_PEAK_TFLOPS, 4),
                "kernels": "fc1 + fc2", "ms": round(fc1_ms + fc2_ms, 5), "work": fl}
    roof["traffic"] = _traffic(spec["name"])
    entry["roofline"] = roof
    entry["gemm_roofline"] = gemm
    return entry


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
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    qm.load_library()
    flush = Flush(dev)

    if a.calibrate_copy:
        src = torch.ones(CALIBRATION_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    head = Layer(a.workload, dev)
    print(f"# {head.spec['name']}: {a.warmup} warm-up + {a.steps} timed calls", file=sys.stderr,
          flush=True)
    h = measure(head, flush, a.steps, a.warmup)
    props = torch.cuda.get_device_properties(dev)
    result = {
        "metric": METRIC, "value": h["tokens_per_s"], "unit": "tokens/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": h["layer_ms"]["mean"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": h["dtype"], "data": "synthetic",
        "config": {"workload": h["workload"], "T": h["T"], "H": h["H"], "I": h["I"],
                   "E": h["E"], "top_k": h["top_k"], "fc1_bits": h["fc1_bits"],
                   "fc2_bits": h["fc2_bits"], "block_size": h["block_size"], "path": h["path"],
                   "selected_experts": h["selected_experts"], "parallelism": "single GPU"},
        "timing": dict(h["layer_ms"], method="HIP event pair per call on the call's stream, "
                       "1 GiB read before every call (outside the pair)"),
        "roofline": h["roofline"],
        "gemm_roofline": h["gemm_roofline"],
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                   "compute_units": props.multi_processor_count},
    }

    if a.graph:
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            head()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            head()
        per_call, _ = _time_calls(graph.replay, flush, a.steps, a.warmup)
        result["graph_replay_ms"] = {"mean": round(float(per_call.mean()), 5),
                                     "median": round(float(np.median(per_call)), 5)}
        del graph

    if a.stages:
        stage_ms = {}
        for name, st in (("route", qm.STAGE_ROUTE), ("group", qm.STAGE_GROUP),
                         ("fc1", qm.STAGE_FC1), ("fc2", qm.STAGE_FC2),
                         ("combine", qm.STAGE_COMBINE)):
            ms, _ = _stage_avg(head, flush, st, a.steps)
            stage_ms[name] = round(ms, 5)
        result["stage_avg_ms"] = stage_ms

    if not a.no_per_config:
        per = {}
        for cfg in (1, 2, 3, 4, 5):
            if cfg == a.workload:
                per[h["workload"]] = h
                continue
            layer = Layer(cfg, dev)
            steps = max(a.steps, a.min_steps_per_config)
            print(f"# {layer.spec['name']}: {steps} timed calls", file=sys.stderr, flush=True)
            e = measure(layer, flush, steps, max(a.warmup, 10))
            per[e["workload"]] = e
            del layer
            torch.cuda.empty_cache()
        result["per_config"] = per

    if not a.no_cpu_baseline:
        print("# CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = _cpu_baseline(head.inp, head.spec, a.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
