"""GPU parity of sliding-window causal attention (fa_fwd_window, and fa_fwd_splitkv with a
window) against the fp64 oracle.

Tolerances as for the plain forward pass: max |O - O_oracle| <= 4e-3 (fp16) or 1.6e-2
(bf16), max |LSE - LSE_oracle| <= 1e-3.  Rows whose window holds no key must come out as
O = 0, LSE = -inf, as the oracle reads them.  Cases: windows of one key, shorter than,
equal to and longer than a key tile, not a multiple of the tile, wider than every row's
prefix (plain causal), with an input_pos offset, GQA, both head dims, both dtypes, every
compiled configuration, key splits, and a long workload on sampled rows.
"""

from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import attention_fa_fwd_amd as fa
import oracle
from attention_fa_fwd_amd.inputs import WORKLOADS, make_qkv, make_workload

pytestmark = pytest.mark.gpu

TOL_O = {torch.float16: 4e-3, torch.bfloat16: 1.6e-2}
TOL_LSE = 1e-3
DEV = torch.device("cuda:0")


def _say(*a):
    print("[window]", *a, file=sys.stderr, flush=True)


def _f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def check(q, k, v, scale, pos, W, out, lse, what=""):
    O, L = oracle.attention_blocked(_f64(q), _f64(k), _f64(v), scale, True, pos, window=W)
    o, l = _f64(out), _f64(lse)
    empty = ~np.isfinite(L)
    assert np.all(l[empty] == -np.inf) and np.all(o[empty] == 0.0), f"empty rows {what}"
    assert np.isfinite(o).all() and np.isfinite(l[~empty]).all(), f"non-finite output {what}"
    eo = float(np.max(np.abs(o - O))) if o.size else 0.0
    el = float(np.max(np.abs(l[~empty] - L[~empty]))) if (~empty).any() else 0.0
    assert eo <= TOL_O[q.dtype], f"O max abs err {eo:.3e} {what}"
    assert el <= TOL_LSE, f"LSE max abs err {el:.3e} {what}"


def run_window(q, k, v, scale, pos, W, config=-1):
    out, lse = fa.fa_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=scale, causal=True,
                         input_pos=pos, config=config, window=W)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


WINDOW_CASES = [
    # B, Hq, Hkv, Sq, Skv, D, input_pos, window
    (1, 8, 2, 300, 300, 128, 0, 1),        # one key per row
    (1, 8, 2, 300, 300, 128, 0, 17),       # shorter than a tile, not a multiple
    (1, 8, 2, 300, 300, 128, 0, 32),       # one 32-key tile
    (1, 8, 2, 300, 300, 128, 0, 100),
    (2, 4, 4, 257, 391, 128, 134, 77),     # offset, ragged both
    (1, 4, 4, 200, 200, 128, 0, 1000),     # wider than every prefix: plain causal
    (1, 8, 8, 129, 64, 64, 0, 9),          # Sq > Skv: rows with an empty window
    (1, 4, 1, 333, 500, 64, 100, 64),      # head dim 64 (64-key tiles), MQA
    (1, 4, 2, 1, 4000, 128, 3999, 700),    # decoding row with a window
    (1, 32, 4, 512, 512, 128, 0, 128),
]


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("case", WINDOW_CASES, ids=lambda c: "x".join(map(str, c)))
def test_window_shapes(case, dtype):
    B, Hq, Hkv, Sq, Skv, D, pos, W = case
    _say(case, dtype)
    q, k, v = make_qkv(B, Hq, Hkv, Sq, Skv, D, dtype, seed=sum(case))
    scale = 1.0 / math.sqrt(D)
    out, lse = run_window(q, k, v, scale, pos, W)
    check(q, k, v, scale, pos, W, out, lse, f"{case} {dtype}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_window_every_config(D, dtype):
    q, k, v = make_qkv(1, 16, 2, 333, 400, D, dtype, seed=12)   # GQA 8: every shape applies
    tested = 0
    for cid, name in enumerate(fa.config_names()):
        if not name.startswith(f"D{D}_") or "fp8" in name or "_causal_" not in name or \
                (("_bf16" in name) != (dtype == "bf16")):
            continue
        _say("config", name)
        out, lse = run_window(q, k, v, 0.09, 50, 90, config=cid)
        check(q, k, v, 0.09, 50, 90, out, lse, name)
        tested += 1
    assert tested == (7 if D == 128 else 6)


def test_window_wide_equals_causal_bitwise():
    """A window covering every row's prefix runs the same tiles with the same masks as
    plain causal attention: the outputs are bit-identical."""
    q, k, v = make_qkv(1, 8, 2, 300, 300, 128, "bf16", seed=13)
    a = run_window(q, k, v, 0.1, 0, 300)
    b = fa.fa_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=0.1, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0].cpu()) and torch.equal(a[1], b[1].cpu())


@pytest.mark.parametrize("splits", [2, 3, 16])
def test_window_splitkv(splits):
    q, k, v = make_qkv(1, 8, 2, 130, 2000, 128, "bf16", seed=14)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out, lse = fa.fa_fwd_splitkv(qd, kd, vd, scale=0.1, causal=True, input_pos=1870,
                                 num_splits=splits, window=300)
    torch.cuda.synchronize()
    check(q, k, v, 0.1, 1870, 300, out.cpu(), lse.cpu(), f"splits={splits}")


def test_window_decode_auto_split():
    q, k, v = make_qkv(4, 32, 8, 1, 16384, 128, "bf16", seed=15)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out, lse = fa.fa_fwd_splitkv(qd, kd, vd, scale=1 / math.sqrt(128), causal=True,
                                 input_pos=16383, window=4096)
    torch.cuda.synchronize()
    check(q, k, v, 1 / math.sqrt(128), 16383, 4096, out.cpu(), lse.cpu(), "decode")


def test_window_workload_sampled_rows():
    name = "gqa8_swa4096_causal_s16384_d128_bf16"
    w = WORKLOADS[name]
    _say("workload", name)
    q, k, v, kw = make_workload(name, seed=0)
    out, lse = fa.fa_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=kw["scale"], causal=True,
                         input_pos=kw["input_pos"], window=kw["window"])
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    rng = np.random.default_rng(2)
    B, Hq, Sq = w["B"], w["Hq"], w["Sq"]
    rows = [0, 1, 31, 32, 4095, 4096, 4097, 8191, Sq // 2, Sq - 1]
    samples = [(0, int(rng.integers(Hq)), i) for i in rows]
    samples += [(0, int(rng.integers(Hq)), int(rng.integers(Sq))) for _ in range(40)]
    O, L = oracle.attention_rows(_f64(q), _f64(k), _f64(v), kw["scale"], True, kw["input_pos"],
                                 samples, window=kw["window"])
    o = np.stack([_f64(out[b, h, i]) for b, h, i in samples])
    l = np.array([float(lse[b, h, i]) for b, h, i in samples])
    assert float(np.max(np.abs(o - O))) <= TOL_O[q.dtype]
    assert float(np.max(np.abs(l - L))) <= TOL_LSE
