"""Host-side logic of bench.py, on the CPU: FLOP and byte counts, the JSON line it assembles
from a timing, the HBM-traffic lookup, and the single-GPU guard.

The timing itself needs a GPU; here `time_gpu` is replaced by a stub returning a fixed
timing, so every field derived from it can be checked exactly.
"""

from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from attention_fa_fwd_amd.inputs import FP8_WORKLOADS, WORKLOADS  # noqa: E402


def _visible_pairs(Sq, Skv, causal, pos, window):
    """Brute-force count of visible (query, key) pairs: key j is visible to query i iff
    j < Skv and, under causal masking, j <= pos + i (and j > pos + i - window if window)."""
    n = 0
    for i in range(Sq):
        for j in range(Skv):
            if causal and j > pos + i:
                continue
            if window and j <= pos + i - window:
                continue
            n += 1
    return n


def test_peaks():
    assert bench.PEAK_TFLOPS == pytest.approx(2516.58, abs=0.01)
    assert bench.PEAK_FP8QK_TFLOPS == pytest.approx(3355.4, abs=0.1)


def test_literal_flops_headline():
    w = WORKLOADS[bench.HEADLINE]
    assert (w["B"], w["Hq"], w["Hkv"], w["Sq"], w["Skv"], w["D"]) == (1, 32, 4, 8192, 8192, 128)
    assert bench.literal_flops(w) == 4.0 * 32 * 8192 * 8192 * 128 / 2 == 549755813888.0


@pytest.mark.parametrize("Sq,Skv,causal,pos,window", [
    (7, 7, True, 0, 0), (5, 9, True, 4, 0), (9, 5, True, 0, 0), (6, 20, True, 30, 0),
    (8, 8, False, 0, 0), (3, 11, False, 0, 0), (10, 10, True, 0, 3), (7, 30, True, 12, 5),
    (12, 6, True, 2, 4), (1, 17, True, 16, 0), (4, 4, True, 0, 100),
])
def test_exact_flops_counts_visible_pairs(Sq, Skv, causal, pos, window):
    w = dict(B=2, Hq=3, Hkv=1, Sq=Sq, Skv=Skv, D=64, causal=causal, input_pos=pos, window=window)
    assert bench.exact_flops(w) == 4.0 * 64 * 2 * 3 * _visible_pairs(Sq, Skv, causal, pos, window)
    if window:
        assert bench.literal_flops(w) == bench.exact_flops(w)


def test_algorithmic_bytes():
    w = WORKLOADS[bench.HEADLINE]
    # q and o (2 bytes each), k and v (2 bytes each), lse (4 bytes).
    assert bench.algorithmic_bytes(w) == 32 * 8192 * 128 * 4 + 4 * 8192 * 128 * 4 + 32 * 8192 * 4
    assert bench.algorithmic_bytes(w) == 152_043_520
    # fp8 q and k: one byte each.
    assert bench.algorithmic_bytes(w, fp8=True) == 32 * 8192 * 128 * 3 + 4 * 8192 * 128 * 3 + 32 * 8192 * 4


def _fake_timing(per_us, steps):
    per_ms = sorted(x / 1000.0 for x in per_us)
    return {"total_ms": sum(per_ms) * steps / len(per_ms), "per_ms": per_ms, "kernel": "stub",
            "warmup_extra": 3, "splits": 4}


def test_bench_line_headline(monkeypatch):
    steps = 10
    monkeypatch.setattr(bench, "time_gpu", lambda *a, **k: _fake_timing([500.0] * steps, steps))
    line = bench.bench_line(bench.HEADLINE, steps, 2, with_cpu=False)
    flops = 549755813888.0
    assert line["metric"] == bench.METRIC
    assert line["unit"] == "TFLOP/s"
    assert line["value"] == round(flops / 500e-6 / 1e12, 2)
    assert line["ms_per_step"] == pytest.approx(0.5)
    assert line["n_gpus"] == 1 and line["steps"] == steps and line["warmup"] == 2
    assert line["higher_is_better"] is True and line["vs_baseline"] is None
    assert line["dtype"] == "bf16"
    assert line["config"]["workload"] == bench.HEADLINE
    r = line["roofline"]
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == round(flops / 500e-6 / 1e12, 2)
    assert r["frac"] == round(r["achieved"] / bench.PEAK_TFLOPS, 4)
    assert line["pct_of_peak"] == round(100 * line["value"] / bench.PEAK_TFLOPS, 2)
    assert "cpu_baseline" not in line
    json.dumps(line)   # one JSON line


def test_bench_line_backward_and_decode(monkeypatch):
    monkeypatch.setattr(bench, "time_gpu", lambda *a, **k: _fake_timing([1000.0] * 4, 4))
    bwd = bench.bench_line(bench.HEADLINE, 4, 0, with_cpu=False, backward=True)
    assert bwd["metric"] == bench.METRIC_BWD
    assert bwd["value"] == round(2.5 * 549755813888.0 / 1e-3 / 1e12, 2)
    assert bwd["roofline"]["traffic"] is None
    dec = "gqa4_decode_b4_kv16384_d128_bf16"
    line = bench.bench_line(dec, 4, 0, with_cpu=False, splitkv=True)
    w = WORKLOADS[dec]
    gbs = bench.algorithmic_bytes(w) / 1e-3 / 1e9
    assert line["unit"] == "GB/s" and line["roofline"]["bound"] == "hbm"
    assert line["value"] == round(gbs, 2)
    assert line["roofline"]["frac"] == round(gbs / bench.HBM_PEAK_GBS, 4)
    fp8 = bench.bench_line("gqa8_causal_s8192_d128_fp8qk_bf16", 4, 0, with_cpu=False)
    assert fp8["metric"] == bench.METRIC_FP8
    assert fp8["roofline"]["peak"] == round(bench.PEAK_FP8QK_TFLOPS, 1)
    assert "gqa8_causal_s8192_d128_fp8qk_bf16" in FP8_WORKLOADS


def test_bench_line_cold(monkeypatch):
    seen = {}

    def stub(*a, **k):
        seen["args"] = a
        return _fake_timing([600.0] * 4, 4)

    monkeypatch.setattr(bench, "time_gpu", stub)
    line = bench.bench_line(bench.HEADLINE, 4, 0, with_cpu=False, cold=True)
    assert seen["args"][-1] is True                     # cold passed through to the timing
    assert line["config"]["caches"].startswith("cold")
    assert line["roofline"]["traffic"] is None          # warm counters do not describe it
    warm = bench.bench_line(bench.HEADLINE, 4, 0, with_cpu=False)
    assert warm["config"]["caches"].startswith("warm")


def test_traffic_lookup_follows_kernel_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    entry = {"workloads": {bench.HEADLINE: {"hbm_bytes_per_launch": 123456}}}
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.traffic_bytes(bench.HEADLINE) is None          # no file
    f.write_text(json.dumps(dict(entry, kernel_source_sha=bench.kernel_source_hash())))
    assert bench.traffic_bytes(bench.HEADLINE) == 123456
    assert bench.traffic_bytes("mha_s1024_d128_fp16") is None   # workload not measured
    f.write_text(json.dumps(dict(entry, kernel_source_sha="0" * 16)))
    assert bench.traffic_bytes(bench.HEADLINE) is None          # kernel changed since


@pytest.mark.parametrize("args", [["--gpus", "2"], ["--gpus", "8"], ["--steps", "0"]])
def test_rejected_arguments(args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert r.stdout == ""
    if args[0] == "--gpus":
        assert "one GPU only" in r.stderr


def test_every_named_workload_resolves(monkeypatch):
    """Each workload bench.py can time (the list, the fp8 list and the context sweep) resolves
    to one shape with the right type flag, and a line built from it carries that name."""
    from attention_fa_fwd_amd.inputs import SWEEP_WORKLOADS

    names = [*WORKLOADS, *FP8_WORKLOADS, *SWEEP_WORKLOADS]
    assert len(set(names)) == len(names)            # no name in two lists
    monkeypatch.setattr(bench, "time_gpu", lambda *a, **k: _fake_timing([250.0] * 2, 2))
    for name in names:
        w, fp8 = bench.workload(name)
        assert fp8 == (name in FP8_WORKLOADS)
        assert bench.literal_flops(w) > 0 and bench.algorithmic_bytes(w, fp8=fp8) > 0
        line = bench.bench_line(name, 2, 0, with_cpu=False)
        assert line["config"]["workload"] == name
    by_len = sorted(SWEEP_WORKLOADS.values(), key=lambda w: w["Sq"])
    assert [w["Sq"] for w in by_len] == [1024, 2048, 4096, 8192, 16384]
    for S, w in zip((1024, 2048, 4096, 8192, 16384), by_len):
        assert (w["B"], w["Hq"], w["Hkv"], w["Sq"], w["Skv"], w["D"], w["causal"]) == (4, 32, 32, S, S, 128, True)
        assert bench.literal_flops(w) == 4.0 * 4 * 32 * S * S * 128 / 2


def test_cpu_baseline_units(monkeypatch):
    """The CPU oracle's rate is reported in the bench line's unit: GB/s of the algorithmic
    bytes for a decoding line, TFLOP/s under the FLOP rule otherwise (here on a tiny
    decoding-like workload registered for the test)."""
    from attention_fa_fwd_amd import inputs

    shape = dict(B=2, Hq=4, Hkv=2, Sq=1, Skv=96, D=64, dtype="fp16", causal=True, input_pos=95)
    monkeypatch.setitem(inputs.WORKLOADS, "tiny_decode_test", shape)
    gb = bench.cpu_baseline("tiny_decode_test", min_s=0.0, unit="GB/s")
    assert gb["unit"] == "GB/s" and gb["kind"] == "oracle" and gb["value"] > 0
    assert "algorithmic byte" in gb["sample"]
    one_group = dict(shape, B=1, Hq=2, Hkv=1)
    # min_s = 0: exactly one group ran
    assert gb["value"] == pytest.approx(bench.algorithmic_bytes(one_group) / 1e9 / gb["wall_s"], rel=0.05) \
        or gb["wall_s"] < 0.01
    tf = bench.cpu_baseline("tiny_decode_test", min_s=0.0)
    assert tf["unit"] == "TFLOP/s" and "FLOP count rule" in tf["sample"]
