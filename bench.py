"""Benchmark of the BitLinear forward pass on one MI355X.

Default workload: decode (M=1) over the seven BitLinear projections of a
d=2048 / ffn=8192 decoder layer -- one grouped forward per step.  The metric
is GB/s of packed (2-bit) weights streamed, as a fraction of HBM bandwidth.
A secondary measurement times the matrix-core prefill path (M=2048 over a
d=2560 / ffn=6912 FFN) in int8 TOPS against the int8 MFMA peak.

Protocol: inputs are seeded synthetic tensors resident in HBM before the
timed region.  To measure HBM rather than the 256 MB Infinity Cache, each
step uses the next of R copies of the layer's packed weights (R copies span
at least 1 GiB).  Steps are replayed from a captured HIP graph (one graph
holds one pass over the R copies), so host launch overhead is not timed.
The timed region is bracketed by torch.cuda.synchronize() and by HIP events
recorded on the stream the kernels run on.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--m M]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "BitLinear decode GB/s of packed weights (% HBM peak); prefill int8 TOPS (% MFMA)"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published
MFMA_I8_PEAK_TOPS = 5000.0  # MI355X dense int8 matrix peak, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=4096)
    ap.add_argument("--warmup", type=int, default=256)
    ap.add_argument("--workload", default="decode_1b_m1")
    ap.add_argument("--m", type=int, default=None)
    ap.add_argument("--rotate-bytes", type=float, default=float(1 << 30))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch steps from Python, no graph")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    return ap.parse_args()


def dev_bf16(torch, bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def prepare(torch, bl, wls, wl, m, copies, dev):
    """Packed weights (packed on the GPU by the library), R rotated copies,
    activations, and one prepared grouped call per copy."""
    xs, packed, scales = [], [], []
    for pi in range(len(wl.projections)):
        w = torch.from_numpy(wls.weights(wl, pi)).to(dev)
        p, s = bl.pack_weights(w)
        del w
        packed.append(p)
        scales.append(s)
        xs.append(dev_bf16(torch, wls.activations(wl, pi, m), dev))
    calls = []
    for c in range(copies):
        ps = packed if c == 0 else [p.clone() for p in packed]
        calls.append(bl.GroupedCall(xs, ps, scales))
    torch.cuda.synchronize()
    return calls


def time_steps(torch, calls, steps, warmup, eager):
    """Run `steps` steps (step i uses copy i % R); returns (host seconds,
    event seconds, steps actually run)."""
    stream = torch.cuda.current_stream()
    r = len(calls)
    if eager:
        for i in range(warmup):
            calls[i % r]()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record(stream)
        for i in range(steps):
            calls[i % r]()
        ev1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return t1 - t0, ev0.elapsed_time(ev1) / 1e3, steps
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for c in calls:  # warm once outside capture
            c()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    reps = max(1, steps // r)
    for _ in range(max(1, warmup // r)):
        g.replay()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(reps):
        g.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return t1 - t0, ev0.elapsed_time(ev1) / 1e3, reps * r


def cpu_baseline(wls, wl, m, budget_s):
    """The oracle as it stands, on host cores, over whole passes of the layer
    (all projections at token count m) until about `budget_s` seconds."""
    import oracle

    try:
        from threadpoolctl import threadpool_info

        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    proj = []
    for pi in range(len(wl.projections)):
        w = wls.weights(wl, pi)
        p, s = oracle.pack_weights(w)
        proj.append((wls.activations(wl, pi, m), p, s))
        del w
    done_bytes, passes = 0, 0
    t0 = time.perf_counter()
    while True:
        for x, p, s in proj:
            oracle.forward(x, p, s)
            done_bytes += p.nbytes
        passes += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {
        "value": done_bytes / dt / 1e9,
        "unit": "GB/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": f"{passes} full pass(es) of the {wl.name} layer at M={m} "
                  f"({len(proj)} projections, {wl.packed_bytes} packed bytes each pass), "
                  f"{dt:.1f} s on host cores (numpy; BLAS threads={blas_threads}, "
                  f"affinity={len(os.sched_getaffinity(0))})",
    }


def prefill_measure(torch, bl, wls, dev, steps):
    wl = wls.WORKLOADS["prefill_2b_m2048"]
    m = wl.ms[0]
    calls = prepare(torch, bl, wls, wl, m, 1, dev)
    host_s, ev_s, n = time_steps(torch, calls, max(8, steps // 64), 4, eager=False)
    tops = wl.ops(m) * n / ev_s / 1e12
    return {
        "workload": wl.name, "m": m, "value": tops, "unit": "TOPS",
        "ms_per_step": ev_s / n * 1e3, "ops_per_step": wl.ops(m), "steps": n,
        "roofline": {"bound": "mfma", "achieved": tops, "peak": MFMA_I8_PEAK_TOPS,
                     "unit": "TFLOP/s", "frac": tops / MFMA_I8_PEAK_TOPS, "traffic": None},
    }


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(see the sharding notes in DESIGN.md); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    from bit_gemm_bitlinear_amd import bitlinear as bl
    from bit_gemm_bitlinear_amd import workloads as wls

    dev = torch.device("cuda:0")
    wl = wls.WORKLOADS[args.workload]
    m = args.m if args.m is not None else wl.ms[0]
    copies = max(1, int(np.ceil(args.rotate_bytes / wl.packed_bytes)))
    calls = prepare(torch, bl, wls, wl, m, copies, dev)
    host_s, ev_s, n = time_steps(torch, calls, args.steps, args.warmup, args.eager)
    per_step = ev_s / n
    gbs = wl.packed_bytes / per_step / 1e9

    out = {
        "metric": METRIC,
        "value": gbs,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": n,
        "warmup": args.warmup,
        "ms_per_step": per_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "m": m,
            "projections": [[p.name, p.n, p.k] for p in wl.projections],
            "packed_bytes_per_step": wl.packed_bytes,
            "rotated_weight_copies": copies,
            "launch": "eager" if args.eager else "hip-graph",
            "host_ms_per_step": host_s / n * 1e3,
        },
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None},
    }
    if not args.no_prefill:
        out["prefill"] = prefill_measure(torch, bl, wls, dev, args.steps)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wls, wl, m, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
