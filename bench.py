"""Benchmark of the BitLinear forward pass on one MI355X.

Default workload: decode (M=1) over the seven BitLinear projections of a
d=2048 / ffn=8192 decoder layer -- one grouped forward per step, which is one
kernel launch (activation quantization is fused into the decode kernel).  The
metric is GB/s of packed (2-bit) weights streamed, as a fraction of HBM
bandwidth.  A secondary measurement times the matrix-core prefill path (M=2048
over the d=2560 / ffn=6912 FFN) in int8 TOPS against the int8 MFMA peak.

Protocol: inputs are seeded synthetic tensors resident in HBM before the
timed region.  To measure HBM rather than the 256 MB Infinity Cache, each
step uses the next of R copies of the layer's packed weights (R copies span
at least 1 GiB).  Steps are replayed from a captured HIP graph (one graph
holds one pass over the R copies), so host launch overhead is not timed.
The timed region is bracketed by torch.cuda.synchronize() and by HIP events
recorded on the stream the kernels are launched on.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--m M]

Profiling helpers (the summaries under profiles/ are written by these):

    python bench.py --pmc-probe ...            eager steps + a copy kernel of known size
    python bench.py --summarize-stats DIR      text summary of a rocprofv3 --stats run
    python bench.py --summarize-pmc FDIR WDIR [--pmc-kernel decode|prefill]
                                               HBM traffic per dispatch from FETCH_SIZE /
                                               WRITE_SIZE runs, scaled by the copy kernel
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
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

# Per kernel: the name rocprofv3 reports, the sources it is built from (a
# traffic figure measured on other sources is stale and is not reported) and
# the committed summary of its HBM traffic.
PMC_KERNELS = {
    "decode": {
        "name": "decode_kernel",
        "sources": ["decode.hip", "common.hpp", "row_div.hpp", "internal.hpp"],
        "file": os.path.join(ROOT, "profiles", "decode_kernel_decode_1b_m1_traffic.txt"),
    },
    "prefill": {
        "name": "prefill_kernel",
        "sources": ["prefill.hip", "prefill_plan.hpp", "abi.hip", "common.hpp", "row_div.hpp",
                    "internal.hpp"],
        "file": os.path.join(ROOT, "profiles", "prefill_kernel_prefill_2b_m2048_traffic.txt"),
    },
}
COPY_PROBE_MIB = 512


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
    ap.add_argument("--no-context", action="store_true",
                    help="skip the warm-cache and copy-bandwidth context numbers")
    ap.add_argument("--eager", action="store_true", help="launch steps from Python, no graph")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--pmc-probe", action="store_true",
                    help="eager steps of the workload, then a copy kernel of known size")
    ap.add_argument("--summarize-stats", metavar="DIR")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--pmc-kernel", choices=sorted(PMC_KERNELS), default="decode",
                    help="kernel whose traffic --summarize-pmc reports")
    ap.add_argument("--command", default="", help="command line recorded in a summary")
    ap.add_argument("--layout", choices=["tiled", "rows"], default="tiled",
                    help="weight layout: the 16-row tiled layout, or row-major [N][K/4]")
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


def prepare(torch, bl, wls, wl, m, copies, dev, tiled=True):
    """Packed weights (packed on the GPU by the library, then put in the
    16-row tiled layout), R rotated copies, activations, and one prepared
    grouped call per copy."""
    xs, packed, scales = [], [], []
    for pi in range(len(wl.projections)):
        w = torch.from_numpy(wls.weights(wl, pi)).to(dev)
        p, s = bl.pack_weights(w)
        del w
        if tiled:
            p = bl.tile_weights(p)
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
    # graph replays are launched on the current stream: the events go there too
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(reps):
        g.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return t1 - t0, ev0.elapsed_time(ev1) / 1e3, reps * r


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
                  f"affinity={len(os.sched_getaffinity(0))}, os.cpu_count={os.cpu_count()})",
    }


def prefill_measure(torch, bl, wls, dev, steps, tiled=True):
    wl = wls.WORKLOADS["prefill_2b_m2048"]
    m = wl.ms[0]
    # one weight copy (6.5 MB of packed weights stay cached, as in a model
    # whose prefill is compute bound); 8 steps per captured graph so the
    # replay launches do not show between steps
    calls = prepare(torch, bl, wls, wl, m, 1, dev, tiled) * 8
    host_s, ev_s, n = time_steps(torch, calls, max(64, steps // 8), 16, eager=False)
    tops = wl.ops(m) * n / ev_s / 1e12
    return {
        "workload": wl.name, "m": m, "value": tops, "unit": "TOPS",
        "note": "end to end: activation quantization pass + MFMA GEMM, 3 projections",
        "weight_layout": "tiled" if tiled else "rows",
        "library_int8_gemm_TOPS": library_int8_gemm(torch, wl, m, dev),
        "library_int8_gemm_note": "context: torch._int_mm (dense int8 x int8 -> int32, "
                                  "vendor GEMM library) on the same three shapes",
        "ms_per_step": ev_s / n * 1e3, "ops_per_step": wl.ops(m), "steps": n,
        "roofline": {"bound": "mfma", "achieved": tops, "peak": MFMA_I8_PEAK_TOPS,
                     "unit": "TFLOP/s", "frac": tops / MFMA_I8_PEAK_TOPS,
                     "traffic": read_traffic("prefill")},
    }


def library_int8_gemm(torch, wl, m, dev, reps=20):
    """Dense int8 GEMM of the vendor library on the same shapes (context only)."""
    try:
        mats = []
        for p in wl.projections:
            a = torch.randint(-127, 128, (m, p.k), dtype=torch.int8, device=dev)
            b = torch.randint(-1, 2, (p.k, p.n), dtype=torch.int8, device=dev)
            mats.append((a, b))
        for a, b in mats:
            torch._int_mm(a, b)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        for _ in range(reps):
            for a, b in mats:
                torch._int_mm(a, b)
        ev1.record()
        torch.cuda.synchronize()
        return wl.ops(m) * reps / (ev0.elapsed_time(ev1) / 1e3) / 1e12
    except Exception as e:  # pragma: no cover - depends on the installed torch
        return f"unavailable: {type(e).__name__}"


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
    """Mean counter value per dispatch, by kernel name."""
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


def summarize_pmc(fdir, wdir, command, kind):
    fetch = _per_kernel_counter(fdir, "FETCH_SIZE")
    write = _per_kernel_counter(wdir, "WRITE_SIZE")
    copy_name = next((n for n in fetch if "neg" in n.lower()), None)
    dec_name = next((n for n in fetch if PMC_KERNELS[kind]["name"] in n), None)
    if copy_name is None or dec_name is None:
        sys.exit(f"kernels not found: {list(fetch)[:8]}")
    copy_bytes = COPY_PROBE_MIB * (1 << 20)
    cf = float(np.median(fetch[copy_name]))
    cw = float(np.median(write[copy_name]))
    f_fac, w_fac = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    df = float(np.mean(fetch[dec_name]))
    dw = float(np.mean(write[dec_name]))
    traffic = df * 1024 * f_fac + dw * 1024 * w_fac
    lines = [
        f"# HBM traffic of the {kind} kernel (rocprofv3 PMC, one counter per run)",
        f"command: {command}",
        f"sources_sha256: {sources_sha256(kind)}",
        f"kernel: {dec_name[:140]}",
        f"dispatches: {len(fetch[dec_name])} (FETCH_SIZE run), {len(write.get(dec_name, []))} (WRITE_SIZE run)",
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
    ]
    print("\n".join(lines))


def read_traffic(kind):
    """Traffic figure of the committed PMC summary of a kernel, or None if it
    is missing or was measured on other sources of that kernel."""
    try:
        with open(PMC_KERNELS[kind]["file"]) as f:
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
    wl = wls.WORKLOADS[args.workload]
    m = args.m if args.m is not None else wl.ms[0]
    copies = max(1, int(np.ceil(args.rotate_bytes / wl.packed_bytes)))
    tiled = args.layout == "tiled"
    calls = prepare(torch, bl, wls, wl, m, copies, dev, tiled)
    time_steps(torch, calls, args.steps, 0, eager=True)
    del calls
    # the prefill workload, a few eager steps (one weight copy, as timed)
    pwl = wls.WORKLOADS["prefill_2b_m2048"]
    pcalls = prepare(torch, bl, wls, pwl, pwl.ms[0], 1, dev, tiled)
    time_steps(torch, pcalls, 8, 0, eager=True)
    del pcalls
    n = COPY_PROBE_MIB * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    print(f"pmc probe: {args.steps} eager steps of {wl.name}, 8 of prefill_2b_m2048, "
          f"3 copies of {COPY_PROBE_MIB} MiB", flush=True)


def bandwidth_curve(torch, bl, dev, layout, k=4096, sizes_mib=(1, 4, 16, 64, 256, 1024)):
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
        steps = max(64, min(4096, 256 * copies // max(1, mib // 16)))
        _, ev_s, nrun = time_steps(torch, calls, steps, min(64, steps), False)
        us = ev_s / nrun * 1e6
        rows.append({"MiB": mib, "n": n, "k": k, "layout": layout, "us": us,
                     "GBs": (mib << 20) / (us * 1e-6) / 1e9})
        del calls, base
        torch.cuda.empty_cache()
    return rows


def main():
    args = parse()
    if args.summarize_stats:
        return summarize_stats(args.summarize_stats, args.command)
    if args.summarize_pmc:
        return summarize_pmc(*args.summarize_pmc, args.command, args.pmc_kernel)
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    from bit_gemm_bitlinear_amd import bitlinear as bl
    from bit_gemm_bitlinear_amd import workloads as wls

    if args.pmc_probe:
        return pmc_probe(torch, bl, wls, args)
    if args.curve:
        for r in bandwidth_curve(torch, bl, torch.device("cuda:0"), args.layout):
            print(json.dumps(r), flush=True)
        return

    dev = torch.device("cuda:0")
    wl = wls.WORKLOADS[args.workload]
    m = args.m if args.m is not None else wl.ms[0]
    copies = max(1, int(np.ceil(args.rotate_bytes / wl.packed_bytes)))
    tiled = args.layout == "tiled"
    calls = prepare(torch, bl, wls, wl, m, copies, dev, tiled)
    host_s, ev_s, n = time_steps(torch, calls, args.steps, args.warmup, args.eager)
    per_step = ev_s / n
    gbs = wl.packed_bytes / per_step / 1e9
    traffic = (read_traffic("decode") if (args.workload == "decode_1b_m1" and m == 1 and tiled)
               else None)

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
            "weight_layout": args.layout,
            "kernel_launches_per_step": 1,
            "rotated_weight_copies": copies,
            "launch": "eager" if args.eager else "hip-graph",
            "host_ms_per_step": host_s / n * 1e3,
        },
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": traffic},
    }
    if not args.no_context:
        # the same step with one weight copy: resident in the Infinity Cache
        w_calls = calls[:1] * len(calls)  # as many launches per graph, all on copy 0
        _, w_s, w_n = time_steps(torch, w_calls, args.steps, args.warmup, args.eager)
        del calls
        out["context"] = {
            "warm_mall_GBs": wl.packed_bytes / (w_s / w_n) / 1e9,
            "warm_mall_note": "same step, one weight copy (16 MiB stays in the 256 MB Infinity Cache)",
            "copy_GBs": copy_bandwidth(torch, dev),
            "copy_note": "plain device copy of 1 GiB (read + write bytes / time), torch elementwise kernel",
        }
        # the same step on the other weight layout
        o_calls = prepare(torch, bl, wls, wl, m, copies, dev, not tiled)
        _, o_s, o_n = time_steps(torch, o_calls, args.steps, args.warmup, args.eager)
        del o_calls
        out["context"]["other_layout"] = "rows" if tiled else "tiled"
        out["context"]["other_layout_GBs"] = wl.packed_bytes / (o_s / o_n) / 1e9
    else:
        del calls
    if not args.no_prefill:
        out["prefill"] = prefill_measure(torch, bl, wls, dev, args.steps, tiled)
    if not args.no_context:
        peaks = measured_ceilings(torch, dev)
        peaks["decode_frac_of_stream_read"] = gbs / peaks["stream_read_GBs"]
        if "prefill" in out:
            peaks["prefill_frac_of_mfma_loop"] = out["prefill"]["value"] / peaks["mfma_i8_loop_TOPS"]
        out["measured_peaks"] = peaks
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wls, wl, m, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
