"""Host logic of rocprof_summary.py on small hand-made inputs: the kernel-trace table and the
quoted bench.py line of the traced run."""

from __future__ import annotations

import json
import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import rocprof_summary  # noqa: E402


def _db(path, rows):
    con = sqlite3.connect(path)
    con.execute("create table kernels (name text, duration integer)")
    con.executemany("insert into kernels values (?, ?)", rows)
    con.commit()
    con.close()


def test_trace_table_and_bench_quote(tmp_path):
    db = str(tmp_path / "r.db")
    # durations in ns: kernel a 100, 200, 600 us; kernel b 5 us twice
    _db(db, [("a", 100_000), ("b", 5_000), ("a", 200_000), ("b", 5_000), ("a", 600_000)])
    bench_out = tmp_path / "bench.out"
    line = {"metric": "m", "value": 12.5, "unit": "TFLOP/s",
            "config": {"workload": "w1", "path": "fa_fwd", "kernel": "K"},
            "kernel_us": {"mean": 301.0, "median": 200.5, "min": 99.0}}
    bench_out.write_text("profiler chatter\n" + json.dumps(line) + "\nmore chatter\n")
    text = rocprof_summary.trace(db, "CMD", str(bench_out))
    lines = text.splitlines()
    assert lines[1] == "# command: CMD"
    rows = {l.split()[0]: l.split()[1:] for l in lines if l.startswith(("a ", "b "))}
    # calls, mean, median, min, max; the kernel with the larger total comes first
    assert rows["a"] == ["3", "300.0", "200.0", "100.0", "600.0"]
    assert rows["b"] == ["2", "5.0", "5.0", "5.0", "5.0"]
    assert [l.split()[0] for l in lines if l.startswith(("a ", "b "))] == ["a", "b"]
    assert "#   workload w1, path fa_fwd, kernel K" in lines
    assert "#   value 12.5 TFLOP/s, kernel_us mean 301.0 median 200.5 min 99.0" in lines


def test_bench_quote_with_peak_check(tmp_path):
    line = {"metric": "m", "value": 900.0, "unit": "TFLOP/s", "ms_per_step": 0.5,
            "config": {"workload": "w1", "path": "fa_fwd", "kernel": "K"},
            "kernel_us": {"mean": 499.0, "median": 498.0, "min": 490.0},
            "peak_check": {"mfma_loop_tflops": 1800.0, "mfma_loop_clock_ghz": 1.8,
                           "derived_peak_tflops": 2516.6}}
    f = tmp_path / "bench.out"
    f.write_text(json.dumps(line) + "\n")
    q = rocprof_summary.bench_of_run(str(f))
    assert "#   ms_per_step 0.5" in q
    assert q[-1] == ("#   peak_check: bf16 MFMA loop on random operands 1800.0 TFLOP/s at 1.8 GHz "
                     "(derived peak 2516.6), the run's value is 0.500 of it")


def test_bench_quote_missing_line(tmp_path):
    f = tmp_path / "bench.out"
    f.write_text("no json here\n")
    assert rocprof_summary.bench_of_run(str(f))[-1].endswith("not found in bench.out")
    db = str(tmp_path / "r.db")
    _db(db, [("a", 1_000)])
    assert "bench.py line" not in rocprof_summary.trace(db, "CMD")


def test_trace_timed_dispatches(tmp_path):
    """With the traced run's `steps` = K, the last 2K dispatches of each kernel (in start
    order when the table has a start column) are summarised apart from the warm-up."""
    db = str(tmp_path / "t.db")
    con = sqlite3.connect(db)
    con.execute("create table kernels (name text, duration integer, start integer)")
    # kernel a: warm-up 900, 800 us, then the timed 100, 200, 300, 400 us; inserted out of order
    con.executemany("insert into kernels values (?, ?, ?)",
                    [("a", 300_000, 5), ("a", 900_000, 1), ("a", 100_000, 3), ("a", 800_000, 2),
                     ("a", 400_000, 6), ("a", 200_000, 4), ("b", 7_000, 7)])
    con.commit()
    con.close()
    f = tmp_path / "bench.out"
    f.write_text(json.dumps({"metric": "m", "value": 1.0, "unit": "TFLOP/s", "steps": 2,
                             "config": {"workload": "w", "path": "fa_fwd", "kernel": "K"},
                             "kernel_us": {}}) + "\n")
    lines = rocprof_summary.trace(db, "CMD", str(f)).splitlines()
    i = lines.index("# the 4 timed dispatches of each kernel (the last ones of the run):")
    rows = [l.split() for l in lines[i + 2:] if l.startswith(("a ", "b "))]
    assert rows == [["a", "4", "250.0", "250.0"]]   # b has fewer than 2K calls
