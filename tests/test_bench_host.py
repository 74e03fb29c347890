"""Host logic of bench.py that needs no GPU: the counter summary that
roofline.traffic comes from, and its invalidation when the kernel changes."""
import csv
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _counter_csv(path, counter, rows):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(cols)
        for i, (name, v) in enumerate(rows):
            w.writerow([i, name, counter, v])


def test_traffic_summary_scales_by_the_copy(tmp_path, monkeypatch):
    gemm = f"void fgmoe::(anonymous namespace)::{bench.GATE_UP_KERNEL}(fgmoe::GemmArgs)"
    f = tmp_path / "f.csv"
    w = tmp_path / "w.csv"
    # FETCH reads half the copy's bytes, WRITE all of them; other kernels are ignored
    _counter_csv(f, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 12.0), ("__amd_rocclr_copyBuffer", 524288.0),
                                  (gemm, 1000.0), (gemm, 1002.0), ("other", 5.0)])
    _counter_csv(w, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 1048576.0), (gemm, 300.0), (gemm, 300.0)])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    bench.traffic_summary(str(f), str(w))
    t = json.loads(out.read_text())
    assert t["fetch_kib"] == 1001.0 and t["write_kib"] == 300.0
    assert t["copy_fetch_kib"] == 524288.0 and t["copy_write_kib"] == 1048576.0
    # bytes per launch: 1001 KiB read x 2 + 300 KiB written x 1
    assert abs(bench.measured_traffic() - (1001 * 2 + 300) * 1024) < 1e-6


def test_traffic_is_null_once_the_kernel_changes(tmp_path, monkeypatch):
    t = dict(fetch_kib=1.0, write_kib=1.0, copy_bytes=1 << 30, copy_fetch_kib=524288.0, copy_write_kib=1048576.0,
             sources=bench.TRAFFIC_SOURCES, sources_sha256="0" * 64)
    out = tmp_path / "traffic.json"
    out.write_text(json.dumps(t))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    assert bench.measured_traffic() is None
    t["sources_sha256"] = bench.kernel_sources_hash(bench.TRAFFIC_SOURCES)
    out.write_text(json.dumps(t))
    assert bench.measured_traffic() is not None



def test_step_time_percentiles():
    """The per-step distribution the benchmark reports: median, p10, p90 and
    the count, from the event-timed step times."""
    import bench
    d = bench.percentiles([float(v) for v in range(1, 102)])     # 1 .. 101
    assert d == dict(median=51.0, p10=11.0, p90=91.0, n=101)
    d = bench.percentiles([5.0] * 7)
    assert d["median"] == d["p10"] == d["p90"] == 5.0 and d["n"] == 7
