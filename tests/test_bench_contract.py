"""CPU checks of the measurement tooling: the benchmark's one-GPU contract, the kernel-source
hash that keys recorded HBM traffic, and the rocprofv3 summary's counter scaling (fed with
small CSV files in the rocprofv3 layout)."""
import csv
import json
import os
import subprocess
import sys

import pytest

from paged_kv_cache_224_amd import profile_summary as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_source_hash_ignores_comments_only(tmp_path):
    src = tmp_path / "k.hip"
    src.write_text("int f() {  // the answer\n  return 42;\n}\n\n")
    h = P.source_hash(str(src))
    src.write_text("// a header comment\nint f() {  // a different comment\n  return 42;   \n}\n")
    assert P.source_hash(str(src)) == h
    src.write_text("int f() {\n  return 43;\n}\n")
    assert P.source_hash(str(src)) != h


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        w.writerows(rows)


def _counters(path, name, per_kernel):
    hdr = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    rows = []
    for k, vals in per_kernel.items():
        for i, v in enumerate(vals):
            rows.append([i, k, 131072, name, v])
    _write_csv(path, hdr, rows)


@pytest.mark.parametrize("fetch_copy_kib", [524288.0, 1048576.0])
def test_summary_scales_counters_by_the_copy(tmp_path, monkeypatch, fetch_copy_kib):
    """A 1 GiB copy that FETCH_SIZE reports as half its bytes doubles every kernel's FETCH_SIZE;
    the recorded traffic is (scaled fetch + scaled write) KiB x 1024 per dispatch."""
    monkeypatch.setattr(P, "ROOT", str(tmp_path))
    out = tmp_path / "OUT"
    dec = "void (anonymous namespace)::pa_decode_kernel<128, 1, true, 2, 2, false>(DecodeParams)"
    red = "void (anonymous namespace)::pa_reduce_kernel<128, true>(void*)"
    _write_csv(str(out / "kt" / "run_kernel_stats.csv"), ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"],
               [[dec, 4, 95000.0, 94000, 96000], [red, 4, 4500.0, 4000, 5000]])
    _counters(str(out / "fetch" / "run_counter_collection.csv"), "FETCH_SIZE", {dec: [1000.0, 3000.0], red: [10.0]})
    _counters(str(out / "write" / "run_counter_collection.csv"), "WRITE_SIZE", {dec: [50.0, 50.0], red: [1.0]})
    _counters(str(out / "copyf" / "run_counter_collection.csv"), "FETCH_SIZE",
              {"__amd_rocclr_copyBuffer": [fetch_copy_kib]})
    _counters(str(out / "copyw" / "run_counter_collection.csv"), "WRITE_SIZE",
              {"__amd_rocclr_copyBuffer": [1048576.0]})
    bench = {"roofline": {"bytes_per_launch": 4_000_000}, "decode_kernel_ms_mean": 0.098}
    (out / "bench.json").write_text("[bench] noise line\n" + json.dumps(bench) + "\n")
    P.summarize(str(out), "wl", "balanced")
    rec = json.load(open(tmp_path / "profiles" / "pa_decode_wl_traffic.json"))
    scale = 1048576.0 / fetch_copy_kib
    assert rec["fetch_scale"] == pytest.approx(scale)
    assert rec["write_scale"] == pytest.approx(1.0)
    assert rec["decode_read_bytes"] == pytest.approx(2000.0 * scale * 1024)      # mean of the dispatches
    assert rec["decode_write_bytes"] == pytest.approx(50.0 * 1024)
    assert rec["trace_average_ns"] == pytest.approx(95000.0)
    assert rec["kernel_source_sha256_16"] == P.source_hash()
    text = open(tmp_path / "profiles" / "pa_decode_wl.md").read()
    assert "rocprofv3 --kernel-trace --stats" in text and "pa_reduce_kernel" in text
