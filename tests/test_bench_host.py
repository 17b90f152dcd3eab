"""Host-side logic of bench.py (no GPU): the configuration list, the
one-GPU guard, and the rocprofv3 summaries that the roofline's traffic
figure comes from (the copy-kernel scaling and the sources check)."""

import csv
import io
import os
import subprocess
import sys
from contextlib import redirect_stdout

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from bit_gemm_bitlinear_amd import workloads as wls  # noqa: E402


def test_configs_cover_every_workload_and_headline_is_largest_decode():
    names = {w for w, _ in bench.CONFIGS}
    assert names == set(wls.WORKLOADS), "every workload is measured"
    for w, m in bench.CONFIGS:
        assert m in wls.WORKLOADS[w].ms, (w, m)
    assert bench.HEADLINE in bench.CONFIGS and bench.CONFIGS[0] == bench.HEADLINE
    decode = [(wls.WORKLOADS[w].packed_bytes, (w, m)) for w, m in bench.CONFIGS
              if not bench.is_prefill(m)]
    assert max(decode)[1] == bench.HEADLINE
    # decode configurations run before the matrix-core ones
    kinds = [bench.is_prefill(m) for _, m in bench.CONFIGS]
    assert kinds == sorted(kinds)


def test_step_bytes():
    wl = wls.WORKLOADS["prefill_2b_m2048"]
    assert bench.step_bytes(wl, 1) == wl.packed_bytes
    extra = sum(2 * 2048 * (p.k + p.n) for p in wl.projections)
    assert bench.step_bytes(wl, 2048) == wl.packed_bytes + extra


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_traffic_summary_scales_by_the_copy_kernel(tmp_path):
    """FETCH_SIZE and WRITE_SIZE are scaled by what they read for a copy of
    known size (512 MiB read and written): a copy that reports half its read
    bytes gives a fetch factor of 2.  Counters of one dispatch split over
    rows (several XCDs) are added."""
    mib = bench.COPY_PROBE_MIB
    copy = "vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>"
    kern = "void bl::decode_kernel<0, true, false, false, 1>(bl::DecodeArgs)"
    fd, wd = str(tmp_path / "f"), str(tmp_path / "w")
    _write_counters(fd, [
        {"Dispatch_Id": 1, "Kernel_Name": kern, "Counter_Name": "FETCH_SIZE", "Counter_Value": 6000},
        {"Dispatch_Id": 1, "Kernel_Name": kern, "Counter_Name": "FETCH_SIZE", "Counter_Value": 4000},
        {"Dispatch_Id": 2, "Kernel_Name": kern, "Counter_Name": "FETCH_SIZE", "Counter_Value": 10000},
        {"Dispatch_Id": 3, "Kernel_Name": copy, "Counter_Name": "FETCH_SIZE",
         "Counter_Value": mib * 1024 // 2},
    ])
    _write_counters(wd, [
        {"Dispatch_Id": 1, "Kernel_Name": kern, "Counter_Name": "WRITE_SIZE", "Counter_Value": 50},
        {"Dispatch_Id": 2, "Kernel_Name": kern, "Counter_Name": "WRITE_SIZE", "Counter_Value": 70},
        {"Dispatch_Id": 3, "Kernel_Name": copy, "Counter_Name": "WRITE_SIZE",
         "Counter_Value": mib * 1024},
    ])
    buf = io.StringIO()
    with redirect_stdout(buf):
        bench.summarize_pmc(fd, wd, "cmd", "decode", "layer_8b", 1)
    kv = dict(l.split(": ", 1) for l in buf.getvalue().splitlines() if ": " in l)
    assert float(kv["fetch_scale"]) == pytest.approx(2.0)
    assert float(kv["write_scale"]) == pytest.approx(1.0)
    assert kv["dispatches"].startswith("2 (FETCH_SIZE run), 2 (WRITE_SIZE run)")
    assert int(kv["fetched_bytes_per_dispatch"]) == 10000 * 1024 * 2
    assert int(kv["written_bytes_per_dispatch"]) == 60 * 1024
    assert int(kv["traffic_bytes_per_dispatch"]) == 10000 * 1024 * 2 + 60 * 1024
    assert kv["sources_sha256"] == bench.sources_sha256("decode")


def test_traffic_is_reported_only_for_the_sources_it_was_measured_on(tmp_path, monkeypatch):
    path = tmp_path / "t.txt"
    good = f"sources_sha256: {bench.sources_sha256('prefill')}\ntraffic_bytes_per_dispatch: 123\n"
    monkeypatch.setattr(bench, "traffic_file", lambda kind, w, m: str(path))
    path.write_text(good)
    assert bench.read_traffic("prefill", "x", 1) == 123.0
    path.write_text(good.replace(bench.sources_sha256("prefill")[:8], "00000000"))
    assert bench.read_traffic("prefill", "x", 1) is None
    path.unlink()
    assert bench.read_traffic("prefill", "x", 1) is None


def test_committed_traffic_summaries_match_the_sources():
    """Every configuration's committed traffic summary was measured on the
    kernel sources in the tree (otherwise the bench reports no traffic)."""
    for w, m in bench.CONFIGS:
        kind = "prefill" if bench.is_prefill(m) else "decode"
        assert bench.read_traffic(kind, w, m) is not None, (w, m)


def test_stats_summary_orders_kernels_by_total_time(tmp_path):
    d = tmp_path / "s"
    d.mkdir()
    with open(d / "run_kernel_stats.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs",
                                          "Percentage", "MinNs", "MaxNs"])
        w.writeheader()
        w.writerow({"Name": "small", "Calls": 10, "TotalDurationNs": 1000, "AverageNs": 100,
                    "Percentage": 10, "MinNs": 90, "MaxNs": 110})
        w.writerow({"Name": "big", "Calls": 10, "TotalDurationNs": 9000, "AverageNs": 900,
                    "Percentage": 90, "MinNs": 800, "MaxNs": 1000})
    buf = io.StringIO()
    with redirect_stdout(buf):
        bench.summarize_stats(str(d), "cmd")
    lines = buf.getvalue().splitlines()
    assert lines[1] == "command: cmd"
    assert lines[4].split()[-1] == "big" and lines[5].split()[-1] == "small"
    assert float(lines[4].split()[1]) == pytest.approx(0.9)
