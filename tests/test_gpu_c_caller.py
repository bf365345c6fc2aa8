"""The C ABI from plain C: tests/c/fa_c_caller.c (built by __graft_entry__.build() with gcc,
no C++ and no Python) allocates with the HIP runtime API, calls fa_fwd and writes out and
lse; this test checks them against the fp64 oracle on the same inputs, regenerated here from
the program's formula (element n of tensor t is a hash of (n, t) mapped to [-1, 1) and rounded
to bf16).  Tolerances as everywhere: O <= 1.6e-2 (bf16), LSE <= 1e-3.
"""

from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "c", "fa_c_caller")
B, HQ, HKV, SQ, SKV, D, POS, SCALE = 1, 4, 2, 70, 130, 64, 60, 0.125


def _inputs(n, t):
    """The C program's fill(): hash -> [-1, 1) float32 -> bf16 (nearest even) -> float64."""
    i = np.arange(n, dtype=np.uint64)
    h = (i * np.uint64(2654435761) + np.uint64(t) * np.uint64(0x9E3779B9)) & np.uint64(0xFFFFFFFF)
    h ^= h >> np.uint64(15)
    h = (h * np.uint64(0x2C1B3C6D)) & np.uint64(0xFFFFFFFF)
    h ^= h >> np.uint64(12)
    x = ((h & np.uint64(0xFFFFFF)).astype(np.float32) / np.float32(8388608.0)) - np.float32(1.0)
    bits = x.view(np.uint32).astype(np.uint64)
    bits = (bits + np.uint64(0x7FFF) + ((bits >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def test_c_caller_matches_oracle(tmp_path):
    assert os.path.exists(BIN), "tests/c/fa_c_caller is missing: run __graft_entry__.build()"
    out_file = tmp_path / "fa_c_caller.bin"
    r = subprocess.run([BIN, str(out_file)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "FA_ERR" not in r.stdout and "head dim 96: -4" in r.stdout, r.stdout
    nq, nl = B * HQ * SQ * D, B * HQ * SQ
    raw = out_file.read_bytes()
    assert len(raw) == nq * 2 + nl * 4
    o_bits = np.frombuffer(raw[:nq * 2], np.uint16).astype(np.uint32) << np.uint32(16)
    out = o_bits.view(np.float32).astype(np.float64).reshape(B, HQ, SQ, D)
    lse = np.frombuffer(raw[nq * 2:], np.float32).astype(np.float64).reshape(B, HQ, SQ)
    q = _inputs(nq, 0).reshape(B, HQ, SQ, D)
    k = _inputs(B * HKV * SKV * D, 1).reshape(B, HKV, SKV, D)
    v = _inputs(B * HKV * SKV * D, 2).reshape(B, HKV, SKV, D)
    O, L = oracle.attention_blocked(q, k, v, SCALE, True, POS)
    assert float(np.max(np.abs(out - O))) <= 1.6e-2
    assert float(np.max(np.abs(lse - L))) <= 1e-3
