"""CPU checks of bench.py's host-only helpers: the rocprofv3 csv summaries,
the traffic ingestion with its copy-kernel calibration, the source digest
that ties a counter run to the kernel sources, and the one-GPU guard."""
import argparse
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

FWD = "void kia_forward_kernel<64, 0, 0, false, false, false>(FwdArgs) [clone .kd]"
ROWS = "void kia_backward_rows_kernel<64, 0, 0, false, 0, true>(BwdArgs)"
COLS = "void kia_backward_cols_kernel<64, false>(BwdArgs)"
GEO = "kia_geometry_kernel(GeoArgs)"
COPY = "void at::native::vectorized_elementwise_kernel<4, copy_kernel>(...)"
OTHER = "void at::native::fill_kernel(...)"


def write_pmc(d, rows):
    """A rocprofv3 --pmc csv: rows of (kernel name, counter, value)."""
    os.makedirs(os.path.join(d, "host", "1234"), exist_ok=True)
    path = os.path.join(d, "host", "1234", "1234_counter_collection.csv")
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (k, c, v) in enumerate(rows):
            w.writerow([i, i, k, c, v])
    return path


def write_stats(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_kernel_stats.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        for r in rows:
            w.writerow(r)


def test_kernel_key_maps_template_names():
    assert bench._kernel_key(FWD) == "forward"
    assert bench._kernel_key(ROWS) == "backward_rows"
    assert bench._kernel_key(COLS) == "backward_cols"
    assert bench._kernel_key(GEO) == "geometry"
    assert bench._kernel_key(COPY) is None


def test_counter_means_average_dispatches(tmp_path):
    write_pmc(str(tmp_path), [(FWD, "FETCH_SIZE", 10), (FWD, "FETCH_SIZE", 30),
                              (FWD, "WRITE_SIZE", 99), (ROWS, "FETCH_SIZE", 5)])
    m = bench._counter_means(str(tmp_path), "FETCH_SIZE")
    assert m == {FWD: 20.0, ROWS: 5.0}


def test_find_csv_missing(tmp_path):
    with pytest.raises(FileNotFoundError):
        bench._find_csv(str(tmp_path), "counter_collection.csv")


def ingest_args(d, **kw):
    a = dict(ingest_pmc=d, copy_calib=256, workload="c2", K=None, calibration=None,
             reconstruction=None, surrogate=None, grad_rule=None)
    a.update(kw)
    return argparse.Namespace(**a)


def test_ingest_scales_by_the_copy_kernel(tmp_path, monkeypatch, capsys):
    d = str(tmp_path / "pmc")
    copy_bytes = 256 << 20
    # the copy kernel's counters read 2x fetch and 1.25x write of its true bytes
    write_pmc(os.path.join(d, "copy_fetch"), [(COPY, "FETCH_SIZE", 2 * copy_bytes / 1024), (OTHER, "FETCH_SIZE", 1)])
    write_pmc(os.path.join(d, "copy_write"), [(COPY, "WRITE_SIZE", 1.25 * copy_bytes / 1024)])
    write_pmc(os.path.join(d, "fetch"), [(FWD, "FETCH_SIZE", 4000), (FWD, "FETCH_SIZE", 6000),
                                         (ROWS, "FETCH_SIZE", 800), (COPY, "FETCH_SIZE", 7)])
    write_pmc(os.path.join(d, "write"), [(FWD, "WRITE_SIZE", 250), (ROWS, "WRITE_SIZE", 500)])
    out_file = str(tmp_path / "profiles" / "traffic.json")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", out_file)
    bench.ingest_pmc(ingest_args(d, grad_rule="p1"))
    tr = json.load(open(out_file))
    assert tr["workload"] == "c2"
    assert tr["variant"] == dict(bench.DEFAULT_VARIANT["c2"], grad_rule="p1")
    assert tr["source_digest"] == bench.source_digest()
    cal = tr["copy_calibration"]
    assert cal["bytes_each_way"] == copy_bytes
    assert cal["fetch_scale"] == 0.5 and cal["write_scale"] == 0.8
    assert set(tr["kernels"]) == {"forward", "backward_rows"}
    f = tr["kernels"]["forward"]
    assert f["kernel_name"] == FWD
    assert f["fetch_bytes"] == int(5000 * 1024 * 0.5)
    assert f["write_bytes"] == int(250 * 1024 * 0.8)
    assert f["hbm_bytes_per_launch"] == int(5000 * 1024 * 0.5 + 250 * 1024 * 0.8)
    r = tr["kernels"]["backward_rows"]
    assert r["hbm_bytes_per_launch"] == int(800 * 1024 * 0.5) + int(500 * 1024 * 0.8)
    assert json.loads(capsys.readouterr().out) == tr


def test_ingest_kernel_without_write_pass(tmp_path, monkeypatch, capsys):
    d = str(tmp_path / "pmc")
    write_pmc(os.path.join(d, "copy_fetch"), [(COPY, "FETCH_SIZE", 1024)])
    write_pmc(os.path.join(d, "copy_write"), [(COPY, "WRITE_SIZE", 1024)])
    write_pmc(os.path.join(d, "fetch"), [(COLS, "FETCH_SIZE", 3)])
    write_pmc(os.path.join(d, "write"), [(FWD, "WRITE_SIZE", 9)])
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "t.json"))
    bench.ingest_pmc(ingest_args(d, copy_calib=1))
    capsys.readouterr()
    tr = json.load(open(tmp_path / "t.json"))
    assert tr["kernels"]["backward_cols"]["write_bytes"] == 0
    assert tr["kernels"]["backward_cols"]["fetch_bytes"] == 3 * 1024


def test_summarize_trace_table(tmp_path):
    write_stats(str(tmp_path), [(ROWS, 200, 38_000_000, 190_000.0, 40.5, 189_000, 191_500, 1.0),
                                (FWD, 200, 20_000_000, 100_000.0, 21.25, 99_000, 101_000, 1.0)])
    lines = bench.summarize_trace(str(tmp_path)).splitlines()
    assert lines[0].startswith("| kernel | calls | avg (us)")
    assert lines[2] == f"| `{ROWS[:90]}` | 200 | 190.0 | 189.0 | 191.5 | 38.000 | 40.5% |"
    assert lines[3] == f"| `{FWD[:90]}` | 200 | 100.0 | 99.0 | 101.0 | 20.000 | 21.2% |"


def test_summarize_pmc_columns_and_gaps(tmp_path):
    a, b = str(tmp_path / "a"), str(tmp_path / "b")
    write_pmc(a, [(FWD, "SQ_WAVES", 100), (FWD, "SQ_WAVES", 300), (ROWS, "SQ_WAVES", 50), (COPY, "SQ_WAVES", 1)])
    write_pmc(b, [(ROWS, "TCC_HIT_sum", 7.5)])
    lines = bench.summarize_pmc([a, b]).splitlines()
    assert lines[0] == "| counter | forward | backward_rows |"
    assert lines[1] == "|---|---|---|"
    assert lines[2] == "| SQ_WAVES | 200 | 50 |"
    assert lines[3] == "| TCC_HIT_sum | — | 7.5 |"


def test_source_digest_follows_every_source(tmp_path, monkeypatch):
    src = tmp_path / "csrc"
    src.mkdir()
    (src / "a.hip").write_text("kernel A\n")
    (src / "b.hpp").write_text("header\n")
    monkeypatch.setattr(bench, "CSRC", str(src))
    d0 = bench.source_digest()
    assert len(d0) == 16 and d0 == bench.source_digest()
    (src / "b.hpp").write_text("header \n")
    d1 = bench.source_digest()
    assert d1 != d0
    (src / "b.hpp").rename(src / "c.hpp")
    assert bench.source_digest() not in (d0, d1)


def test_committed_traffic_file_names_a_measured_variant():
    tr = json.load(open(bench.TRAFFIC_FILE))
    assert tr["variant"] == bench.DEFAULT_VARIANT[tr["workload"]]
    assert set(tr["kernels"]) >= {"forward", "backward_rows", "backward_cols"}
    for k in tr["kernels"].values():
        # each figure is truncated to whole bytes on its own
        assert abs(k["hbm_bytes_per_launch"] - k["fetch_bytes"] - k["write_bytes"]) <= 1
        assert k["fetch_bytes"] > 0 and k["write_bytes"] > 0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
