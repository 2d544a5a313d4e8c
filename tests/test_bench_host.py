"""Host logic of bench.py (no GPU): the profile summaries it writes under
profiles/ and the roofline bound.  The rocprofv3 outputs are small synthetic
CSV files with the columns rocprofv3 writes."""
import csv
import io
import json
import os
import sys
from contextlib import redirect_stdout

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import bench  # noqa: E402

GEMM = ("void moe::(anonymous namespace)::grouped_gemm_split<256, 256, 2, 4, 64, 3, 0, 4>"
        "(moe::(anonymous namespace)::GemmArgs)")
TOPK = "void moe::(anonymous namespace)::topk_kernel<4>(long, int, int, int, float*)"
TORCH = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<long> >(int)"


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def _run(fn, *a, **k):
    buf = io.StringIO()
    with redirect_stdout(buf):
        fn(*a, **k)
    return buf.getvalue()


def test_short_names_and_library_filter():
    assert bench._short(GEMM) == "grouped_gemm_split<256, 256, 2, 4, 64, 3, 0, 4>"
    assert bench._short(TOPK) == "topk_kernel<4>"
    assert bench._is_libmoe(bench._short(GEMM)) and bench._is_libmoe("combine_token_kernel")
    assert not bench._is_libmoe(bench._short(TORCH))


def test_trace_summary_takes_the_timed_steps_only(tmp_path):
    """2 steps before, 3 timed, 4 after; the GEMM launches once per step
    with duration 100 + step, top-K twice per step; a torch kernel outside
    the pattern is left out."""
    rows, t = [], 0
    for step in range(9):
        for name, n, dur in ((GEMM, 1, 100 + step), (TOPK, 2, 5)):
            for _ in range(n):
                rows.append([name, t, t + dur * 1000])
                t += 10 ** 6
    rows.append([TORCH, t, t + 1000])
    _write(str(tmp_path / "run" / "run_kernel_trace.csv"),
           ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    out = _run(bench.trace_summary, str(tmp_path), 2, 3, 4)
    line = [l for l in out.splitlines() if "grouped_gemm_split" in l][0]
    cells = [c.strip() for c in line.strip("|").split("|")]
    assert cells[1] == "3" and cells[2] == "103.0" and cells[3] == "102.0" and cells[4] == "104.0"
    topk = [l for l in out.splitlines() if "topk_kernel" in l][0]
    assert topk.split("|")[2].strip() == "6"       # two launches in each of 3 steps
    assert "FillFunctor" not in out


def test_counter_summary_averages_and_derives(tmp_path):
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    _write(str(tmp_path / "a" / "run_counter_collection.csv"), hdr,
           [[GEMM, "SQ_WAVE_CYCLES", 1000], [GEMM, "SQ_WAVE_CYCLES", 3000],
            [GEMM, "SQ_WAIT_ANY", 500], [GEMM, "SQ_WAIT_ANY", 500],
            [TORCH, "SQ_WAVE_CYCLES", 7]])
    _write(str(tmp_path / "b" / "run_counter_collection.csv"), hdr,
           [[GEMM, "TA_TA_BUSY_sum", 256 * 50], [GEMM, "GRBM_GUI_ACTIVE", 800],
            [GEMM, "TCC_HIT_sum", 3], [GEMM, "TCC_MISS_sum", 1]])
    out = _run(bench.counter_summary, [str(tmp_path / "a"), str(tmp_path / "b")])
    hdr_cells = [c.strip() for c in out.splitlines()[0].strip("|").split("|")]
    row = [c.strip() for c in
           [l for l in out.splitlines() if "grouped_gemm" in l][0].strip("|").split("|")]
    d = dict(zip(hdr_cells, row))
    assert float(d["SQ_WAVE_CYCLES"]) == 2000 and float(d["SQ_WAIT_ANY"]) == 500
    assert float(d["SQ_WAIT_ANY / SQ_WAVE_CYCLES"]) == pytest.approx(0.25)
    assert float(d["TA busy"]) == pytest.approx(8 * 256 * 50 / (256 * 800))
    assert float(d["L2 hit"]) == pytest.approx(0.75)
    assert "FillFunctor" not in out


def test_pmc_summary_scales_by_the_copy(tmp_path, monkeypatch):
    """A copy of 1 GiB that FETCH_SIZE reports as half its bytes: factor 2."""
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    _write(str(tmp_path / "f" / "x_counter_collection.csv"), hdr,
           [[GEMM, "FETCH_SIZE", 1000], [GEMM, "FETCH_SIZE", 3000]])
    _write(str(tmp_path / "w" / "x_counter_collection.csv"), hdr, [[GEMM, "WRITE_SIZE", 10]])
    _write(str(tmp_path / "cf" / "x_counter_collection.csv"), hdr,
           [["copyBuffer", "FETCH_SIZE", 512 * 1024], ["small", "FETCH_SIZE", 1]])
    _write(str(tmp_path / "cw" / "x_counter_collection.csv"), hdr,
           [["copyBuffer", "WRITE_SIZE", 1024 * 1024]])
    out = _run(bench.pmc_summary, str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"),
               str(tmp_path / "cw"), label="grouped_gemm_split<256, 256, 2, 4, 64, 3, 0")
    rec = json.loads([l for l in out.splitlines() if l.startswith("traffic: ")][0][9:])
    assert abs(rec["bytes"] - (2000 * 1024 * 2 + 10 * 1024)) <= 2   # via GB, rounded down
    assert rec["source_sha256"] == bench.source_sha()


def test_roofline_bound_follows_the_algorithmic_work():
    r = bench.roofline(2.5e12, 1e9, 1.0)        # 1 ms of MFMA work, 0.125 ms of bytes
    assert r["bound"] == "mfma" and r["achieved"] == pytest.approx(2500.0)
    assert r["frac"] == pytest.approx(1.0)
    r = bench.roofline(1e9, 8e9, 2.0)           # HBM-bound: 8 GB in 2 ms = 4 TB/s
    assert r["bound"] == "hbm" and r["frac"] == pytest.approx(0.5)


def test_more_than_one_gpu_is_refused():
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(os.path.dirname(bench.__file__), "bench.py"),
                        "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
