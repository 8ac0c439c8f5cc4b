"""Host-side parts of the measurement: bench.py's refusal of several GPUs, and the
rocprofv3 summary script on small hand-made CSV files (CPU only)."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from cross_model_attention_causal_amd import rocprof_summary as rs  # noqa: E402


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"] and line["n_gpus"] == 2


def _write(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0].keys()))
        w.writeheader()
        w.writerows(rows)


def _counter_rows(kernel, counter, values):
    """One row per (dispatch, dimension); the dimensions of a dispatch add up."""
    rows = []
    for disp, per_dim in enumerate(values):
        for v in per_dim:
            rows.append({"Dispatch_Id": disp, "Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": v})
    return rows


def test_counter_means_add_dimensions_then_average_dispatches(tmp_path):
    p = str(tmp_path / "run" / "x" / "p_counter_collection.csv")
    _write(p, _counter_rows("cma::k_a(int)", "FETCH_SIZE", [[10, 20], [30, 40]]))
    m = rs.counter_means(str(tmp_path / "run"))
    # dispatch 0: 30, dispatch 1: 70 -> mean 50
    assert m == {"cma::k_a(int)": {"FETCH_SIZE": 50.0}}


def test_traffic_calibrates_on_the_copy_kernel(tmp_path):
    gib_kib = (1 << 30) / 1024
    d = tmp_path
    _write(str(d / "f" / "a_counter_collection.csv"), _counter_rows("void cma::k_mapped_av_bsr(x)", "FETCH_SIZE", [[1000]]))
    _write(str(d / "w" / "a_counter_collection.csv"), _counter_rows("void cma::k_mapped_av_bsr(x)", "WRITE_SIZE", [[100]]))
    # the calibration run also holds a small fill kernel, which must not be taken
    _write(str(d / "cf" / "a_counter_collection.csv"),
           _counter_rows("fill_kernel", "FETCH_SIZE", [[5]]) +
           _counter_rows("__amd_rocclr_copyBuffer", "FETCH_SIZE", [[gib_kib / 2]]))
    _write(str(d / "cw" / "a_counter_collection.csv"),
           _counter_rows("fill_kernel", "WRITE_SIZE", [[5]]) +
           _counter_rows("__amd_rocclr_copyBuffer", "WRITE_SIZE", [[gib_kib]]))
    out_md, out_js = str(d / "t.md"), str(d / "t.json")
    rs.main(["traffic", str(d / "f"), str(d / "w"), str(d / "cf"), str(d / "cw"), out_md, out_js,
             "--workload", "w", "--cmd", "c", "--cal-cmd", "cc"])
    js = json.load(open(out_js))["k_mapped_av_bsr"]
    # the copy's FETCH_SIZE reads half of the 1 GiB it moves: factor 2; WRITE_SIZE factor 1
    assert js["fetch_factor"] == pytest.approx(2.0)
    assert js["write_factor"] == pytest.approx(1.0)
    assert js["bytes_per_launch"] == int(1000 * 1024 * 2.0 + 100 * 1024 * 1.0)
    assert len(js["sha256"]) == 64 and js["source"] == "mapped_av.hip"


def test_counters_derive_unit_shares(tmp_path):
    k = "void cma::k_block_stats<128, 2>(cma::CompressArgs)"
    cyc = 1000.0
    rows = (_counter_rows(k, "GRBM_GUI_ACTIVE", [[8 * cyc]]) +
            _counter_rows(k, "SQ_VALU_MFMA_BUSY_CYCLES", [[0.5 * 1024 * cyc]]) +
            _counter_rows(k, "SQ_BUSY_CU_CYCLES", [[0.9 * 256 * cyc]]) +
            _counter_rows(k, "TA_BUSY_avr", [[0.25 * cyc]]))
    _write(str(tmp_path / "r" / "p_counter_collection.csv"), rows)
    out = str(tmp_path / "c.md")
    rs.main(["counters", out, str(tmp_path / "r"), "--title", "t", "--cmd", "c"])
    text = open(out).read()
    assert "| MFMA busy | 0.500 |" in text
    assert "| CU busy | 0.900 |" in text
    assert "| address unit busy | 0.250 |" in text


def test_kernel_time_table(tmp_path):
    _write(str(tmp_path / "k" / "p_kernel_stats.csv"),
           [{"Name": "cma::k_x(int)", "Calls": 3, "TotalDurationNs": 3000, "AverageNs": 1000, "Percentage": 100.0,
             "MinNs": 900, "MaxNs": 1100}])
    out = str(tmp_path / "kt.md")
    rs.main(["kernel-time", str(tmp_path / "k"), out, "--title", "t", "--cmd", "c"])
    assert "| `cma::k_x(int)` | 3 | 1.0 | 0.9 | 1.1 | 100.00 % |" in open(out).read()
