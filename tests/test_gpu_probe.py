"""The benchmark's peak check on the GPU: hipDeviceProp gives MI355X's 256 compute units and
2.4 GHz peak engine clock (hence 2516.6 dense bf16 TFLOP/s), and a loop of nothing but bf16
MFMAs (pseudo-random operands) runs at a sizeable fraction of it, at a plausible shader clock."""

from __future__ import annotations

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402

pytestmark = pytest.mark.gpu


def test_peak_check():
    import torch

    torch.cuda.init()
    r = bench.peak_check(iters=20000)
    print("[probe]", r, file=sys.stderr, flush=True)
    assert "error" not in r, r
    assert r["cus"] == 256
    assert r["max_clock_mhz"] == pytest.approx(2400, abs=1)
    assert r["derived_peak_tflops"] == pytest.approx(bench.PEAK_TFLOPS, abs=1)
    assert 0.4 * bench.PEAK_TFLOPS < r["mfma_loop_tflops"] <= 1.01 * bench.PEAK_TFLOPS
    assert 1.0 < r["mfma_loop_clock_ghz"] <= 2.45
