"""Benchmark of the BitLinear forward pass on one MI355X.

Headline: decode (M=1) over the seven BitLinear projections of the 8B-class
layer (d=4096, ffn=14336, GQA k/v 1024) -- one grouped forward per step, one
kernel launch.  The metric is GB/s of packed (2-bit) weights streamed, as a
fraction of HBM bandwidth.  Every other workload is measured in the same run
and reported in the `configs` array: decode configurations in GB/s of packed
weights (HBM roofline), prefill configurations in int8 TOPS (matrix-core
roofline).

Protocol (every configuration):
  * inputs are seeded synthetic tensors, packed and tiled on the GPU by the
    library, resident in HBM before the timed region;
  * to measure HBM rather than the 256 MB Infinity Cache, step i uses copy
    i % R of the configuration's operands (decode: the packed weights;
    prefill: weights, activations and outputs), R copies spanning >= 1 GiB;
  * a "sample" is one replay of a captured HIP graph of exactly --steps
    steps; graphs cover successive ranges of the copy rotation;
  * --warmup steps run untimed first; then samples are replayed back to back
    (at least --min-seconds of GPU time, the headline --headline-seconds),
    each bracketed by HIP events on the stream the graph is launched on,
    with torch.cuda.synchronize() before and after;
  * ms_per_step is the median over samples of (sample time / steps); the
    10th/90th percentiles and the minimum are reported as the spread.

    python bench.py [--steps K] [--warmup W] [--only W:M[,W:M]]

Profiling helpers (the summaries under profiles/ are written by these):

    python bench.py --pmc-probe --workload W --m M   eager steps + a copy kernel of known size
    python bench.py --summarize-stats DIR            text summary of a rocprofv3 --stats run
    python bench.py --summarize-pmc FDIR WDIR --workload W --m M --pmc-kernel decode|prefill
                                                     HBM traffic per dispatch, scaled by the copy kernel
    python bench.py --summarize-counters DIR --workload W --m M --pmc-kernel prefill
                                                     matrix-core counters per dispatch
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "BitLinear decode GB/s of packed weights (% HBM peak); prefill int8 TOPS (% MFMA)"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published
MFMA_I8_PEAK_TOPS = 5000.0  # MI355X dense int8 matrix peak, published (POPS x 1000)

# (workload, M) of every configuration: the headline (the largest single-GPU
# decode configuration) first, the other decode configurations, then the
# matrix-core ones, so that no decode measurement follows the heat of a
# prefill one.
CONFIGS = [("layer_8b", 1), ("single_2048_m8", 8), ("decode_1b_m1", 1), ("decode_3b", 1),
           ("decode_3b", 4), ("decode_3b", 16), ("prefill_2b_m2048", 2048), ("layer_8b", 512)]
HEADLINE = ("layer_8b", 1)

# Per kernel: the name rocprofv3 reports and the sources it is built from (a
# counter figure measured on other sources is stale and is not reported).
PMC_KERNELS = {
    "decode": {"name": "decode_kernel",
               "sources": ["decode.hip", "decode_fused.hip", "decode_kernels.hpp", "abi.hip",
                           "common.hpp", "row_div.hpp", "internal.hpp"]},
    "prefill": {"name": "prefill_kernel",
                "sources": ["prefill.hip", "prefill_plan.hpp", "abi.hip", "common.hpp",
                            "row_div.hpp", "internal.hpp"]},
}
COPY_PROBE_MIB = 512


def traffic_file(kind, workload, m):
    return os.path.join(ROOT, "profiles", f"{PMC_KERNELS[kind]['name']}_{workload}_m{m}_traffic.txt")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100, help="steps per timed sample")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--min-seconds", type=float, default=0.3,
                    help="GPU time of the timed samples per configuration")
    ap.add_argument("--headline-seconds", type=float, default=1.5)
    ap.add_argument("--only", default="", help="comma list of workload:M to measure")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--m", type=int, default=None)
    ap.add_argument("--rotate-bytes", type=float, default=float(1 << 30))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the ceilings, warm-cache, copy, other-layout and bf16 context")
    ap.add_argument("--cpu-seconds", type=float, default=0.5,
                    help="CPU time per oracle measurement (single-threaded and all cores)")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="eager steps of --workload at --m, then a copy kernel of known size")
    ap.add_argument("--summarize-stats", metavar="DIR")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-counters", metavar="DIR")
    ap.add_argument("--pmc-kernel", choices=sorted(PMC_KERNELS), default="decode")
    ap.add_argument("--command", default="", help="command line recorded in a summary")
    ap.add_argument("--layout", choices=["tiled", "rows"], default="tiled",
                    help="weight layout: the 16-row tiled layout, or row-major [N][K/4]")
    ap.add_argument("--lut-eval", action="store_true",
                    help="the lookup-table contraction against the matrix-core decode, M = 1")
    ap.add_argument("--lut-shape", default="", help="N,K: one projection shape for --lut-eval")
    ap.add_argument("--curve", action="store_true",
                    help="decode GB/s against weight bytes for one projection (1 MiB .. 1 GiB)")
    return ap.parse_args()


def sources_sha256(kind: str) -> str:
    h = hashlib.sha256()
    for name in PMC_KERNELS[kind]["sources"]:
        with open(os.path.join(ROOT, "bit_gemm_bitlinear_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def dev_bf16(torch, bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def is_prefill(m):
    return m > 16


def step_bytes(wl, m):
    """Bytes one step's operands occupy: packed weights (+ activations and
    bf16 outputs for prefill, which rotates them too)."""
    b = wl.packed_bytes
    if is_prefill(m):
        b += sum(2 * m * (p.k + p.n) for p in wl.projections)
    return b


_WEIGHTS = {}   # workload -> latent fp32 weights of every projection (host)
_PACKED = {}    # (workload, tiled) -> (packed weights, scales) on the GPU


def latent_weights(wls, wl):
    """The workload's seeded latent weights, drawn once per run."""
    if wl.name not in _WEIGHTS:
        _WEIGHTS[wl.name] = [wls.weights(wl, pi) for pi in range(len(wl.projections))]
    return _WEIGHTS[wl.name]


def packed_weights(torch, bl, wls, wl, dev, tiled):
    """Weights packed on the GPU by the library (and put in the 16-row tiled
    layout), once per workload and layout."""
    key = (wl.name, tiled)
    if key not in _PACKED:
        _PACKED.clear()  # one workload's weights on the GPU at a time
        packed, scales = [], []
        for w in latent_weights(wls, wl):
            p, s = bl.pack_weights(torch.from_numpy(w).to(dev))
            packed.append(bl.tile_weights(p) if tiled else p)
            scales.append(s)
        _PACKED[key] = (packed, scales)
    return _PACKED[key]


def prepare(torch, bl, wls, wl, m, copies, dev, tiled=True):
    """R prepared grouped calls over the workload's packed weights and
    activations at M; copy c > 0 clones the weights (and for prefill the
    activations, with outputs of its own)."""
    packed, scales = packed_weights(torch, bl, wls, wl, dev, tiled)
    xs = [dev_bf16(torch, wls.activations(wl, pi, m), dev) for pi in range(len(wl.projections))]
    calls = []
    for c in range(copies):
        ps = packed if c == 0 else [p.clone() for p in packed]
        cx = xs if (c == 0 or not is_prefill(m)) else [x.clone() for x in xs]
        calls.append(bl.GroupedCall(cx, ps, scales))
    torch.cuda.synchronize()
    return calls


def capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        fn()  # warm once outside capture
    stream.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    return g


def time_config(torch, calls, steps, warmup, min_seconds):
    """Graphs of exactly `steps` steps over successive ranges of the copy
    rotation; warmup, then samples replayed back to back, each between two
    HIP events on the replay stream.  Returns per-step seconds of every
    sample and the sample count."""
    r = len(calls)
    ngraphs = r // math.gcd(r, steps)
    graphs = []
    for gi in range(ngraphs):
        base = gi * steps

        def body(base=base):
            for j in range(steps):
                calls[(base + j) % r]()

        graphs.append(capture(torch, body))
    stream = torch.cuda.current_stream()
    for i in range(max(1, -(-warmup // steps))):
        graphs[i % ngraphs].replay()
    torch.cuda.synchronize()
    # calibrate the sample count from one pass over the graphs
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for g in graphs:
        g.replay()
    ev[1].record(stream)
    torch.cuda.synchronize()
    per_sample = max(ev[0].elapsed_time(ev[1]) / 1e3 / ngraphs, 1e-7)
    samples = int(min(max(5, math.ceil(min_seconds / per_sample)), 20000))
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(samples + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(samples):
        graphs[i % ngraphs].replay()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    secs = np.array([evs[i].elapsed_time(evs[i + 1]) / 1e3 for i in range(samples)])
    return secs / steps, samples


def spread(per_step):
    return {"ms_per_step_p10": float(np.percentile(per_step, 10) * 1e3),
            "ms_per_step_p90": float(np.percentile(per_step, 90) * 1e3),
            "ms_per_step_min": float(per_step.min() * 1e3)}


def measure(torch, bl, wls, name, m, args, dev, min_seconds, tiled=True):
    wl = wls.WORKLOADS[name]
    copies = max(1, int(math.ceil(args.rotate_bytes / step_bytes(wl, m))))
    calls = prepare(torch, bl, wls, wl, m, copies, dev, tiled)
    per_step, samples = time_config(torch, calls, args.steps, args.warmup, min_seconds)
    del calls
    torch.cuda.empty_cache()
    t = float(np.median(per_step))
    shapes = [(p.n, p.k) for p in wl.projections]
    out = {"workload": name, "m": m, "ms_per_step": t * 1e3, **spread(per_step),
           "samples": samples, "steps_per_sample": args.steps, "rotated_copies": copies,
           "kernel_launches_per_step": bl.forward_grouped_launches(m, shapes),
           "weight_layout": "tiled" if tiled else "rows"}
    if is_prefill(m):
        tops = wl.ops(m) / t / 1e12
        out.update(value=tops, unit="TOPS", ops_per_step=wl.ops(m),
                   roofline={"bound": "mfma", "achieved": tops, "peak": MFMA_I8_PEAK_TOPS,
                             "unit": "TOP/s", "frac": tops / MFMA_I8_PEAK_TOPS,
                             "traffic": read_traffic("prefill", name, m),
                             "note": "from the whole step (activation quantization + "
                                     "matrix-core GEMM [+ the K-part sum])"})
    else:
        gbs = wl.packed_bytes / t / 1e9
        out.update(value=gbs, unit="GB/s", packed_bytes_per_step=wl.packed_bytes,
                   roofline={"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                             "traffic": read_traffic("decode", name, m)})
    return out


def copy_bandwidth(torch, dev, mib=1024, reps=10):
    """Context: a plain device copy (torch elementwise kernel), read+write bytes / time."""
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(2):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        torch.neg(a, out=b)
    ev1.record()
    torch.cuda.synchronize()
    s = ev0.elapsed_time(ev1) / 1e3 / reps
    del a, b
    return 2 * mib * (1 << 20) / s / 1e9


def measured_ceilings(torch, dev, reps=10):
    """The GPU's achievable ceilings from the probe kernels
    (include/bitlinear_probes.h): a streaming read of 1 GiB, and the int8
    matrix-core loop with prefill-like operands (random activation bytes and
    weight codes, changing every operation) and with constant operands."""
    from bit_gemm_bitlinear_amd import probes

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(n):
            fn()
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / 1e3 / n

    nbytes = 1 << 30
    buf = torch.randint(-128, 128, (nbytes,), dtype=torch.int8, device=dev)
    sink = torch.zeros(probes.SINK_WORDS, dtype=torch.int32, device=dev)
    read_s = timed(lambda: probes.stream_read(buf, sink), reps)
    del buf
    wgs = torch.cuda.get_device_properties(dev).multi_processor_count * 4
    msink = torch.empty(wgs * 256, dtype=torch.int32, device=dev)
    iters = 2048
    ops = probes.OPS_PER_ROUND_PER_WG * iters * wgs
    rand_s = timed(lambda: probes.mfma_i8(wgs, iters, 1, msink), reps)
    const_s = timed(lambda: probes.mfma_i8(wgs, iters, 0, msink), reps)
    return {
        "stream_read_GBs": nbytes / read_s / 1e9,
        "mfma_i8_loop_TOPS": ops / rand_s / 1e12,
        "mfma_i8_loop_const_TOPS": ops / const_s / 1e12,
        "note": "probe kernels: 16-byte streaming read of 1 GiB; v_mfma_i32_32x32x32_i8 loop "
                "from registers, prefill-like operands (and constant operands)",
    }


def warm_cache(torch, bl, wls, name, m, args, dev):
    """The same decode step with one weight copy (resident in the Infinity Cache)."""
    wl = wls.WORKLOADS[name]
    calls = prepare(torch, bl, wls, wl, m, 1, dev)
    per_step, _ = time_config(torch, calls, args.steps, args.warmup, 0.1)
    del calls
    return wl.packed_bytes / float(np.median(per_step)) / 1e9


def native_bf16(torch, bl, wls, name, m, dev, min_seconds=0.2):
    """Context: the same layer as dense bf16 weights -- the library's
    "universal" export u / w_scale of the packed weights -- through
    torch.matmul (the vendor BLAS), weights rotated like the ternary step;
    the bytes a bf16 model streams per step and the time it takes."""
    wl = wls.WORKLOADS[name]
    wbytes = sum(2 * p.n * p.k for p in wl.projections)
    copies = max(1, int(math.ceil((1 << 30) / wbytes))) if not is_prefill(m) else 1
    g = torch.Generator(device="cpu").manual_seed(3)
    packed, scales = packed_weights(torch, bl, wls, wl, dev, True)
    xs = [torch.randn(m, p.k, generator=g).to(torch.bfloat16).to(dev) for p in wl.projections]
    ys = [torch.empty(m, p.n, dtype=torch.bfloat16, device=dev) for p in wl.projections]
    # both weight orientations the vendor library is given by frameworks:
    # [N, K] as nn.Linear stores it (F.linear), and [K, N] (x @ w); the
    # faster one is reported
    best, times = None, {}
    for orient in ("linear_NK", "matmul_KN"):
        w0 = [bl.export_bf16(p, s, k=pr.k) for p, s, pr in zip(packed, scales, wl.projections)]
        if orient == "matmul_KN":
            w0 = [w.t().contiguous() for w in w0]
        ws = [w0] + [[w.clone() for w in w0] for _ in range(copies - 1)]
        if orient == "linear_NK":  # x @ w.T, as F.linear computes it (2-D: no batched product)
            calls = [lambda c=c: [torch.mm(x, w.t(), out=y) for x, w, y in zip(xs, ws[c], ys)]
                     for c in range(copies)]
        else:
            calls = [lambda c=c: [torch.matmul(x, w, out=y) for x, w, y in zip(xs, ws[c], ys)]
                     for c in range(copies)]
        r = _time_native(torch, calls, copies, min_seconds)
        del ws, w0, calls
        torch.cuda.empty_cache()
        r["orientation"] = orient
        times[orient] = r["ms_per_step"]
        if best is None or r["ms_per_step"] < best["ms_per_step"]:
            best = r
    t = best["ms_per_step"] / 1e3
    del xs, ys
    out = {"workload": name, "m": m, "ms_per_step": t * 1e3, "weight_bytes_per_step": wbytes,
           "rotated_copies": copies, "launch": best["launch"],
           "weight_orientation": best["orientation"], "ms_per_step_by_orientation": times}
    if is_prefill(m):
        out["TFLOPs"] = wl.ops(m) / t / 1e12
    else:
        out["GBs_of_bf16_weights"] = wbytes / t / 1e9
    return out


def _time_native(torch, calls, copies, min_seconds):
    """ms per step of vendor-library calls: replayed graphs, or eager
    launches when the library refuses capture."""
    steps = 20
    launch = "hip-graph"
    try:
        per_step, _ = time_config(torch, calls, steps, steps, min_seconds)
    except Exception:  # the vendor library refused graph capture: eager launches
        launch = "eager"
        torch.cuda.synchronize()
        for i in range(steps):
            calls[i % copies]()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record()
        for i in range(50 * steps):
            calls[i % copies]()
        ev1.record()
        torch.cuda.synchronize()
        per_step = np.array([ev0.elapsed_time(ev1) / 1e3 / (50 * steps)])
    return {"ms_per_step": float(np.median(per_step)) * 1e3, "launch": launch}


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on the host cores


def latent_context(torch, bl, dev, min_seconds=0.1):
    """Context for on-the-fly ternarization: bitlinear_forward_latent (exact
    absmean, ternarization and packing, then the forward) against the
    forward on weights packed once, one projection at M = 1, the fp32
    weights rotated over copies spanning >= 1 GiB."""
    out = []
    g = torch.Generator(device="cpu").manual_seed(5)
    for n, k in ((4096, 4096), (14336, 4096)):
        w0 = (torch.randn(n, k, generator=g) * 0.02).to(dev)
        copies = max(1, int(math.ceil((1 << 30) / (4 * n * k))))
        ws = [w0] + [w0.clone() for _ in range(copies - 1)]
        x = torch.randn(1, k, generator=g).to(torch.bfloat16).to(dev)
        y = torch.empty(1, n, dtype=torch.bfloat16, device=dev)
        packs = [bl.pack_weights(w) for w in ws]
        lat = [lambda w=w: bl.forward_latent(x, w, out=y) for w in ws]
        pk = [lambda p=p: bl.forward(x, p[0], p[1], out=y) for p in packs]
        t_lat = float(np.median(time_config(torch, lat, 20, 20, min_seconds)[0]))
        t_pk = float(np.median(time_config(torch, pk, 20, 20, min_seconds)[0]))
        out.append({"n": n, "k": k, "m": 1, "rotated_copies": copies,
                    "latent_us": t_lat * 1e6, "packed_us": t_pk * 1e6,
                    "latent_GBs_of_fp32_weights": 4 * n * k / t_lat / 1e9})
        del ws, packs, lat, pk
        torch.cuda.empty_cache()
    return out


def _threads_info():
    try:
        from threadpoolctl import threadpool_info

        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def _time_oracle(fn, budget_s):
    """One untimed call, then fn() at least once and until about budget_s;
    returns seconds per call."""
    fn()
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    return (time.perf_counter() - t0) / n, n


def cpu_baseline(wls, budget_s):
    """The oracle (oracle/, NumPy, never tuned) on a bounded sample of every
    configuration, single-threaded and on all cores, plus its weight packing;
    the headline configuration's all-core figure is `value`."""
    import oracle
    from threadpoolctl import threadpool_limits

    all_threads = _threads_info()
    rows = []
    ns_max = 512  # output rows of every projection in the sample
    packed_sample = {}
    for name, m in CONFIGS:
        wl = wls.WORKLOADS[name]
        # the first 512 output rows of every projection (weights of that
        # slice packed by the oracle); decode: every token row, prefill: the
        # first 64
        ms = m if not is_prefill(m) else 64
        if name not in packed_sample:
            packed_sample[name] = [oracle.pack_weights(np.ascontiguousarray(w[:ns_max]))
                                   for w in latent_weights(wls, wl)]
        proj = [(wls.activations(wl, pi, m)[:ms], p, s)
                for pi, (p, s) in enumerate(packed_sample[name])]

        def one_pass():
            for x, p, s in proj:
                oracle.forward(x, p, s)

        nbytes = sum(p.nbytes for _, p, _ in proj)
        ops = sum(2 * ms * p.shape[0] * 4 * p.shape[1] for _, p, _ in proj)
        res = {"workload": name, "m": m, "sample": (
            f"the first {ns_max} output rows of each of the {len(proj)} projections, "
            f"{ms} of {m} token rows ({nbytes} packed bytes, {ops} int8 ops per pass)")}
        for label, threads in (("single_thread", 1), ("all_cores", all_threads)):
            with threadpool_limits(limits=threads):
                sec, n = _time_oracle(one_pass, budget_s)
            if not is_prefill(m):
                res[label] = {"value": nbytes / sec / 1e9, "unit": "GB/s",
                              "threads": threads, "passes": n}
            else:
                res[label] = {"value": ops / sec / 1e12, "unit": "TOPS", "threads": threads,
                              "passes": n}
        rows.append(res)
        del proj
    # weight preparation (absmean, ternarize, pack) on the 2048 x 2048 projection
    w = latent_weights(wls, wls.WORKLOADS["single_2048_m8"])[0]
    sec, n = _time_oracle(lambda: oracle.pack_weights(w), budget_s)
    pack = {"value": w.nbytes / sec / 1e9, "unit": "GB/s of fp32 weights read",
            "sample": "oracle.pack_weights on the 2048x2048 fp32 projection", "passes": n,
            "threads": 1}
    head = next(r for r in rows if (r["workload"], r["m"]) == HEADLINE)
    return {
        "value": head["all_cores"]["value"], "unit": head["all_cores"]["unit"],
        "cores": int(all_threads), "kind": "oracle",
        "sample": f"{head['sample']} of {HEADLINE[0]} (all cores); per configuration below, "
                  f"single-threaded and on all cores, each ~{budget_s:.1f} s "
                  f"(numpy; BLAS threads={all_threads}, affinity={len(os.sched_getaffinity(0))}, "
                  f"os.cpu_count={os.cpu_count()})",
        "per_config": rows, "pack": pack,
    }


# ---------------------------------------------------------------------------
# rocprofv3 output summaries


def _csv_rows(pattern):
    rows = []
    for path in sorted(glob.glob(pattern, recursive=True)):
        with open(path, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def summarize_stats(d, command):
    rows = _csv_rows(os.path.join(d, "**", "*kernel_stats.csv"))
    if not rows:
        sys.exit(f"no kernel_stats.csv under {d}")
    out = ["# rocprofv3 kernel statistics", f"command: {command}", "",
           f"{'calls':>7} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'total_%':>7}  kernel"]
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    for r in rows:
        out.append(f"{int(r['Calls']):7d} {float(r['AverageNs'])/1e3:9.3f} "
                   f"{float(r['MinNs'])/1e3:9.3f} {float(r['MaxNs'])/1e3:9.3f} "
                   f"{float(r['Percentage']):7.2f}  {r['Name'][:140]}")
    print("\n".join(out))


def _per_kernel_counter(d, counter):
    """Counter value per dispatch, by kernel name."""
    rows = _csv_rows(os.path.join(d, "**", "*counter_collection.csv"))
    acc = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        key = (r["Kernel_Name"], r.get("Dispatch_Id", r.get("Correlation_Id")))
        acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    by_name = {}
    for (name, _), v in acc.items():
        by_name.setdefault(name, []).append(v)
    return by_name


def summarize_pmc(fdir, wdir, command, kind, workload, m):
    fetch = _per_kernel_counter(fdir, "FETCH_SIZE")
    write = _per_kernel_counter(wdir, "WRITE_SIZE")
    copy_name = next((n for n in fetch if "neg" in n.lower()), None)
    names = [n for n in fetch if PMC_KERNELS[kind]["name"] in n]
    if copy_name is None or not names:
        sys.exit(f"kernels not found: {list(fetch)[:8]}")
    copy_bytes = COPY_PROBE_MIB * (1 << 20)
    cf = float(np.median(fetch[copy_name]))
    cw = float(np.median(write[copy_name]))
    f_fac, w_fac = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    fl = [v for n in names for v in fetch[n]]
    wr = [v for n in names for v in write.get(n, [])]
    df, dw = float(np.mean(fl)), float(np.mean(wr))
    traffic = df * 1024 * f_fac + dw * 1024 * w_fac
    lines = [
        f"# HBM traffic of the {kind} kernel on {workload} at M={m} "
        "(rocprofv3 PMC, one counter per run)",
        f"command: {command}",
        f"sources_sha256: {sources_sha256(kind)}",
        f"workload: {workload}",
        f"m: {m}",
        "kernel: " + "; ".join(n[:120] for n in names),
        f"dispatches: {len(fl)} (FETCH_SIZE run), {len(wr)} (WRITE_SIZE run)",
        f"FETCH_SIZE_KiB_per_dispatch: {df:.1f}",
        f"WRITE_SIZE_KiB_per_dispatch: {dw:.1f}",
        f"copy_kernel: {copy_name[:140]}",
        f"copy_kernel_bytes_read: {copy_bytes}",
        f"copy_kernel_bytes_written: {copy_bytes}",
        f"copy_FETCH_SIZE_KiB: {cf:.1f}",
        f"copy_WRITE_SIZE_KiB: {cw:.1f}",
        f"fetch_scale: {f_fac:.4f}",
        f"write_scale: {w_fac:.4f}",
        f"traffic_bytes_per_dispatch: {traffic:.0f}",
        f"fetched_bytes_per_dispatch: {df * 1024 * f_fac:.0f}",
        f"written_bytes_per_dispatch: {dw * 1024 * w_fac:.0f}",
    ]
    print("\n".join(lines))


def summarize_counters(d, command, kind, workload, m):
    """Mean per dispatch of every counter in a --pmc run, for the kernel."""
    rows = _csv_rows(os.path.join(d, "**", "*counter_collection.csv"))
    names = sorted({r["Counter_Name"] for r in rows})
    lines = [f"# rocprofv3 counters of the {kind} kernel on {workload} at M={m}",
             f"command: {command}", f"sources_sha256: {sources_sha256(kind)}",
             f"workload: {workload}", f"m: {m}"]
    for c in names:
        per = _per_kernel_counter(d, c)
        for kn, vals in per.items():
            if PMC_KERNELS[kind]["name"] in kn:
                lines.append(f"{c}: {float(np.mean(vals)):.6g}  (dispatches {len(vals)}; {kn[:90]})")
    print("\n".join(lines))


def read_traffic(kind, workload, m):
    """Traffic figure of the committed PMC summary of a kernel on a
    configuration, or None if it is missing or was measured on other sources
    of that kernel."""
    try:
        with open(traffic_file(kind, workload, m)) as f:
            kv = dict(l.split(": ", 1) for l in f.read().splitlines() if ": " in l)
    except OSError:
        return None
    if kv.get("sources_sha256") != sources_sha256(kind):
        return None
    try:
        return float(kv["traffic_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


def pmc_probe(torch, bl, wls, args):
    dev = torch.device("cuda:0")
    wl = wls.WORKLOADS[args.workload or HEADLINE[0]]
    m = args.m if args.m is not None else wl.ms[0]
    copies = max(1, int(math.ceil(args.rotate_bytes / step_bytes(wl, m))))
    calls = prepare(torch, bl, wls, wl, m, copies, dev, args.layout == "tiled")
    for i in range(args.steps):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    del calls
    n = COPY_PROBE_MIB * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    print(f"pmc probe: {args.steps} eager steps of {wl.name} at M={m}, "
          f"3 copies of {COPY_PROBE_MIB} MiB", flush=True)


def bandwidth_curve(torch, bl, dev, layout, args, k=4096, sizes_mib=(1, 4, 16, 64, 256, 1024)):
    """Decode (M=1) on a single N x K projection of random packed bytes (code 3
    included: timing only), cold: rotated over copies spanning >= 1 GiB."""
    rows = []
    g = torch.Generator(device="cpu").manual_seed(1)
    x = torch.randn(1, k, generator=g).to(torch.bfloat16).to(dev)
    ws = torch.ones(1, dtype=torch.float32, device=dev)
    for mib in sizes_mib:
        n = mib * (1 << 20) * 4 // k
        copies = max(1, (1 << 30) // (mib << 20)) if mib < 1024 else 2
        base = torch.randint(0, 256, (n, k // 4), dtype=torch.uint8, device=dev)
        if layout == "tiled":
            base = bl.tile_weights(base)
        calls = [bl.GroupedCall([x], [base if c == 0 else base.clone()], [ws]) for c in range(copies)]
        per_step, _ = time_config(torch, calls, max(2, min(args.steps, 64)), 4, 0.2)
        us = float(np.median(per_step)) * 1e6
        rows.append({"MiB": mib, "n": n, "k": k, "layout": layout, "us": us,
                     "GBs": (mib << 20) / (us * 1e-6) / 1e9})
        del calls, base
        torch.cuda.empty_cache()
    return rows


def lut_eval(torch, bl, dev, args, shapes=((8192, 2048), (2048, 8192), (16384, 4096), (4096, 8192))):
    """The lookup-table contraction (probe library) against the matrix-core
    decode on single projections at M = 1, same tiled weights, rotated over
    copies spanning >= 1 GiB: one launch per step each (the decode path also
    quantizes the bf16 row and dequantizes, the table path takes ready
    codes and returns int32)."""
    from bit_gemm_bitlinear_amd import probes

    rows = []
    g = torch.Generator(device="cpu").manual_seed(5)
    for n, k in shapes:
        nbytes = n * k // 4
        copies = max(1, (1 << 30) // nbytes)
        base = bl.tile_weights(torch.randint(0, 3, (n, k // 4), dtype=torch.uint8, device=dev))
        ws = [base] + [base.clone() for _ in range(copies - 1)]
        x = torch.randn(1, k, generator=g).to(torch.bfloat16).to(dev)
        q = torch.randint(-127, 128, (k,), dtype=torch.int8, device=dev)
        scale = torch.ones(1, dtype=torch.float32, device=dev)
        acc = torch.empty(n, dtype=torch.int32, device=dev)
        mfma = [bl.GroupedCall([x], [w], [scale]) for w in ws]
        lut = [lambda w=w: probes.lut_decode_acc(q, w, acc) for w in ws]
        t_m, _ = time_config(torch, mfma, 20, 5, 0.2)
        t_l, _ = time_config(torch, lut, 20, 5, 0.2)
        um, ul = float(np.median(t_m)) * 1e6, float(np.median(t_l)) * 1e6
        rows.append({"n": n, "k": k, "packed_bytes": nbytes, "mfma_decode_us": um,
                     "lut_us": ul, "mfma_decode_GBs": nbytes / um / 1e3, "lut_GBs": nbytes / ul / 1e3})
        del ws, mfma, lut, base
        torch.cuda.empty_cache()
    return rows


def main():
    args = parse()
    if args.summarize_stats:
        return summarize_stats(args.summarize_stats, args.command)
    if args.summarize_pmc:
        return summarize_pmc(*args.summarize_pmc, args.command, args.pmc_kernel,
                             args.workload, args.m)
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters, args.command, args.pmc_kernel,
                                  args.workload, args.m)
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (how it would "
              "shard is described in the design notes); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        sys.exit("--steps must be >= 1 and --warmup >= 0")
    import torch

    from bit_gemm_bitlinear_amd import bitlinear as bl
    from bit_gemm_bitlinear_amd import workloads as wls

    if args.pmc_probe:
        return pmc_probe(torch, bl, wls, args)
    dev = torch.device("cuda:0")
    if args.curve:
        for r in bandwidth_curve(torch, bl, dev, args.layout, args):
            print(json.dumps(r), flush=True)
        return
    if args.lut_eval:
        shapes = ((tuple(int(v) for v in args.lut_shape.split(",")),) if args.lut_shape else
                  ((8192, 2048), (2048, 8192), (16384, 4096), (4096, 8192)))
        for r in lut_eval(torch, bl, dev, args, shapes):
            print(json.dumps(r), flush=True)
        return

    configs = CONFIGS
    if args.only:
        configs = [(s.split(":")[0], int(s.split(":")[1])) for s in args.only.split(",")]
    head = HEADLINE if HEADLINE in configs else configs[0]
    tiled = args.layout == "tiled"
    rows = []
    for name, m in configs:
        secs = args.headline_seconds if (name, m) == head else args.min_seconds
        r = measure(torch, bl, wls, name, m, args, dev, secs, tiled)
        print(f"# {name} M={m}: {r['ms_per_step'] * 1e3:.2f} us/step, {r['value']:.1f} "
              f"{r['unit']} ({r['roofline']['frac'] * 100:.1f}% of the roofline), "
              f"{r['samples']} samples", file=sys.stderr, flush=True)
        rows.append(r)
    h = next(r for r in rows if (r["workload"], r["m"]) == head)
    wl = wls.WORKLOADS[head[0]]
    out = {
        "metric": METRIC,
        "value": h["value"],
        "unit": h["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": head[0], "m": head[1],
            "projections": [[p.name, p.n, p.k] for p in wl.projections],
            "packed_bytes_per_step": wl.packed_bytes,
            "weight_layout": args.layout,
            "kernel_launches_per_step": h["kernel_launches_per_step"],
            "rotated_weight_copies": h["rotated_copies"],
            "launch": "hip-graph",
            "samples": h["samples"], "steps_per_sample": args.steps,
            "timed_steps": h["samples"] * args.steps,
            "ms_per_step_p10": h["ms_per_step_p10"], "ms_per_step_p90": h["ms_per_step_p90"],
            "ms_per_step_min": h["ms_per_step_min"],
        },
        "roofline": {k: v for k, v in h["roofline"].items() if k != "note"},
        "configs": rows,
    }
    if not args.no_context:
        ctx = {}
        ctx["warm_mall_GBs"] = warm_cache(torch, bl, wls, head[0], head[1], args, dev) \
            if not is_prefill(head[1]) else None
        ctx["warm_mall_note"] = "the headline step with one weight copy (resident in the 256 MB Infinity Cache)"
        ctx["copy_GBs"] = copy_bandwidth(torch, dev)
        ctx["copy_note"] = "plain device copy of 1 GiB (read + write bytes / time), torch elementwise kernel"
        other = measure(torch, bl, wls, head[0], head[1], args, dev, 0.2, not tiled)
        ctx["other_layout"] = other["weight_layout"]
        ctx["other_layout_GBs"] = other["value"]
        ctx["native_bf16"] = []
        for n, m in (("layer_8b", 1), ("decode_1b_m1", 1), ("prefill_2b_m2048", 2048),
                     ("layer_8b", 512)):
            try:
                ctx["native_bf16"].append(native_bf16(torch, bl, wls, n, m, dev))
            except Exception as e:  # context only: never fail the run for it
                ctx["native_bf16"].append({"workload": n, "m": m,
                                           "unavailable": f"{type(e).__name__}: {e}"[:200]})
        ctx["native_bf16_note"] = ("the same layers as dense bf16 weights (the library's bf16 "
                                   "export of the packed weights) through the vendor BLAS "
                                   "(torch.mm, weights [N, K] as nn.Linear stores them and "
                                   "[K, N]; the faster is reported), rotated like the ternary "
                                   "steps; compare ms_per_step with the configs array")
        ctx["latent_forward"] = latent_context(torch, bl, dev)
        ctx["latent_forward_note"] = ("bitlinear_forward_latent (exact absmean, packing, then the "
                                      "forward, from fp32 weights) against the forward on weights "
                                      "packed once; one projection, M = 1")
        # token counts inside the decode path (up to 16 rows)
        ctx["decode_m"] = []
        for n in ("decode_3b", "layer_8b"):
            for mm in (2, 4, 8):
                r = measure(torch, bl, wls, n, mm, args, dev, 0.1)
                wl_n = wls.WORKLOADS[n]
                ctx["decode_m"].append({"workload": n, "m": mm,
                                        "us_per_step": r["ms_per_step"] * 1e3,
                                        "GBs_packed": wl_n.packed_bytes / (r["ms_per_step"] * 1e-3) / 1e9,
                                        "kernel_launches_per_step": r["kernel_launches_per_step"]})
        # token counts between decode and prefill: the mid-M path (tiles of
        # 32 / 64 / 128 rows, chosen by M) on the 3B- and 8B-class layers
        ctx["mid_m"] = []
        for n in ("decode_3b", "layer_8b"):
            for mm in (16, 32, 64, 128, 256):
                r = measure(torch, bl, wls, n, mm, args, dev, 0.1)
                wl_n = wls.WORKLOADS[n]
                ctx["mid_m"].append({"workload": n, "m": mm, "us_per_step": r["ms_per_step"] * 1e3,
                                     "GBs_packed": wl_n.packed_bytes / (r["ms_per_step"] * 1e-3) / 1e9,
                                     "TOPS": wl_n.ops(mm) / (r["ms_per_step"] * 1e-3) / 1e12,
                                     "kernel_launches_per_step": r["kernel_launches_per_step"]})
        peaks = measured_ceilings(torch, dev)
        peaks["headline_frac_of_stream_read"] = h["value"] / peaks["stream_read_GBs"]
        for r in rows:
            r["frac_of_measured_ceiling"] = r["value"] / (
                peaks["mfma_i8_loop_TOPS"] if r["unit"] == "TOPS" else peaks["stream_read_GBs"])
        out["measured_peaks"] = peaks
        out["context"] = ctx
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wls, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
