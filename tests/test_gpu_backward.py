"""GPU parity of the backward pass (fa_bwd) against the fp64 oracle's gradients.

Tolerance (no page or target fixes one): per gradient tensor, max |g - g_oracle| <=
TOL_REL * max(max |g_oracle|, 0.05 * the largest of the three gradients' maxima), with
TOL_REL = 4e-3 (fp16) and 1.6e-2 (bf16).  A CPU simulation
of the kernels' arithmetic (P and dS rounded to the input type before their products, fp32
accumulation, outputs rounded, D from the rounded forward output) stays below 40% of that
(tests/test_tolerance_backward.py).  On the rising-score input, far from N(0,1), the bound
is instead derived elementwise from the same rounding steps (tests/bwd_bound.py).  The
forward pass that provides out and lse is the library's own fa_fwd on the same inputs.
"""

from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import attention_fa_fwd_amd as fa
import oracle
from attention_fa_fwd_amd.inputs import DTYPES, make_qkv, make_rising_scores
from tests.bwd_bound import check_within, rounding_bound, rounding_model

pytestmark = pytest.mark.gpu

TOL_REL = {torch.float16: 4e-3, torch.bfloat16: 1.6e-2}
DEV = torch.device("cuda:0")


def _say(*a):
    print("[bwd]", *a, file=sys.stderr, flush=True)


def make_dout(shape, dtype, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(1000 + int(seed))
    return torch.randn(shape, generator=g, dtype=torch.float32).to(dtype)


def run_bwd(q, k, v, do, scale, causal, pos, window=0):
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    out, lse = fa.fa_fwd(qd, kd, vd, scale=scale, causal=causal, input_pos=pos, window=window)
    dq, dk, dv = fa.fa_bwd(qd, kd, vd, out, lse, dod, scale=scale, causal=causal, input_pos=pos,
                           window=window)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def check(q, k, v, do, scale, causal, pos, window, got, what):
    ref = oracle.attention_backward_blocked(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                                            do.double().numpy(), scale, causal, pos, window)
    # A gradient that is exactly zero (one key per row, say) is compared at the scale of the
    # largest of the three, since its rounding noise comes from products of that size.
    scale_all = max(float(np.max(np.abs(r))) if r.size else 0.0 for r in ref)
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        g = g.double().numpy()
        assert np.isfinite(g).all(), f"{name} non-finite {what}"
        m = float(np.max(np.abs(r))) if r.size else 0.0
        err = float(np.max(np.abs(g - r))) if r.size else 0.0
        bound = TOL_REL[q.dtype] * max(m, 0.05 * scale_all, 1e-6)
        assert err <= bound, f"{name} err {err:.3e} vs max {m:.3e} {what}"


BWD_CASES = [
    # B, Hq, Hkv, Sq, Skv, D, causal, pos, window
    (1, 2, 2, 128, 128, 128, False, 0, 0),
    (1, 2, 2, 128, 128, 64, True, 0, 0),
    (2, 4, 4, 300, 300, 128, True, 0, 0),      # ragged, several blocks
    (1, 8, 2, 257, 391, 128, True, 134, 0),    # ragged both, GQA 4, offset
    (1, 8, 1, 65, 129, 64, False, 0, 0),       # MQA
    (1, 8, 8, 1, 1, 128, True, 0, 0),          # one query, one key
    (1, 4, 4, 1, 700, 128, True, 699, 0),      # decode-like row
    (3, 6, 3, 129, 64, 64, True, 0, 0),        # Sq > Skv
    (1, 8, 2, 300, 300, 128, True, 0, 45),     # sliding window
    (1, 8, 8, 129, 64, 128, True, 0, 9),       # window with empty rows
    (1, 32, 4, 256, 256, 128, True, 0, 0),     # small K/V grid: the group split 8 ways
    (1, 32, 8, 256, 2048, 64, False, 0, 0),    # GQA 4 split over 2 workgroups
    (2, 32, 16, 128, 2048, 64, True, 1920, 0), # GQA 2 with a K/V grid large enough not to split
    (1, 6, 2, 200, 300, 128, True, 40, 0),     # GQA 3: odd group
    (1, 12, 2, 150, 150, 64, True, 0, 0),      # GQA 6
    (1, 21, 3, 96, 200, 128, False, 0, 0),     # GQA 7, non-causal
    # GQA 8 at head dim 128, larger grids
    (2, 32, 4, 1000, 1000, 128, True, 0, 0),   # ragged query tail
    (2, 64, 8, 520, 700, 128, True, 180, 96),  # offset and sliding window
    (4, 64, 8, 300, 200, 128, False, 0, 0),    # non-causal, Sq > Skv
]


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "x".join(map(str, c)))
def test_backward_shapes(case, dtype):
    B, Hq, Hkv, Sq, Skv, D, causal, pos, W = case
    _say(case, dtype)
    q, k, v = make_qkv(B, Hq, Hkv, Sq, Skv, D, dtype, seed=sum(case) + 3)
    do = make_dout(q.shape, DTYPES[dtype], sum(case))
    scale = 1.0 / math.sqrt(D)
    got = run_bwd(q, k, v, do, scale, causal, pos, W)
    check(q, k, v, do, scale, causal, pos, W, got, f"{case} {dtype}")


def test_backward_workspace_sizes():
    """The workspace holds 8 bytes of row statistics per query row (rounded up to 256),
    plus fp32 dk / dv partials for each part of a split head group."""
    stats = lambda B, Hq, Sq: (B * Hq * Sq * 8 + 255) // 256 * 256
    assert fa.bwd_workspace_size(1, 8, 8, 100, 100, 128, True) == stats(1, 8, 100)      # MHA
    assert fa.bwd_workspace_size(1, 32, 4, 256, 256, 128, True) == \
        stats(1, 32, 256) + 8 * 2 * 4 * 256 * 128 * 4                                    # split 8
    assert fa.bwd_workspace_size(1, 32, 8, 256, 2048, 64, False) == \
        stats(1, 32, 256) + 2 * 2 * 8 * 2048 * 64 * 4                                    # split 2
    assert fa.bwd_workspace_size(2, 32, 16, 128, 2048, 64, True) == stats(2, 32, 128)    # none
    assert fa.bwd_workspace_size(0, 8, 8, 100, 100, 128, True) == 0


def test_backward_medium_gqa_causal():
    """A 2048-token causal GQA problem, every element of every gradient."""
    q, k, v = make_qkv(1, 8, 2, 2048, 2048, 128, "bf16", seed=31)
    do = make_dout(q.shape, torch.bfloat16, 31)
    got = run_bwd(q, k, v, do, 1 / math.sqrt(128), True, 0)
    check(q, k, v, do, 1 / math.sqrt(128), True, 0, 0, got, "2048 gqa causal")


def test_backward_headline_sampled():
    """The causal GQA-8 8192-token bf16 workload in the launch configuration bench.py times
    (fa_bwd_into with a preallocated workspace; the group split of 2 the library picks),
    checked on sampled dQ rows of every head and sampled dK / dV rows of one K/V head
    against the fp64 oracle evaluated at those rows."""
    from attention_fa_fwd_amd.inputs import make_workload

    name = "gqa8_causal_s8192_d128_bf16"
    q, k, v, kw = make_workload(name, seed=0)
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    g = torch.Generator(device="cpu")
    g.manual_seed(1)
    do = torch.randn(q.shape, generator=g, dtype=torch.float32).to(q.dtype)
    qd, kd, vd, dod = q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV)
    out, lse = fa.fa_fwd(qd, kd, vd, scale=kw["scale"], causal=True)
    ws = torch.empty(fa.bwd_workspace_size(B, Hq, Hkv, Sq, Skv, D, True), dtype=torch.uint8, device=DEV)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    _say("headline backward", name, "workspace", ws.numel())
    fa.fa_bwd_into(qd, kd, vd, out, lse, dod, dq, dk, dv, ws, scale=kw["scale"], causal=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    qs = [(0, int(rng.integers(Hq)), i) for i in (0, 1, 31, 32, 127, 128, 4095, 8191)]
    qs += [(0, int(rng.integers(Hq)), int(rng.integers(Sq))) for _ in range(24)]
    gk = int(rng.integers(Hkv))
    ks = [(0, gk, j) for j in (0, 1, 127, 128, 4096, 8064, 8191)]
    ks += [(0, gk, int(rng.integers(Skv))) for _ in range(9)]
    rq, rk, rv = oracle.attention_backward_sampled(q.double().numpy(), k.double().numpy(),
                                                   v.double().numpy(), do.double().numpy(),
                                                   kw["scale"], True, 0, qs, ks)
    got = (np.stack([dq[b, h, i].double().cpu().numpy() for b, h, i in qs]),
           np.stack([dk[b, g_, j].double().cpu().numpy() for b, g_, j in ks]),
           np.stack([dv[b, g_, j].double().cpu().numpy() for b, g_, j in ks]))
    top = max(float(np.max(np.abs(r))) for r in (rq, rk, rv))
    for nm, gv, r in zip(("dq", "dk", "dv"), got, (rq, rk, rv)):
        err = float(np.max(np.abs(gv - r)))
        bound = TOL_REL[q.dtype] * max(float(np.max(np.abs(r))), 0.05 * top)
        _say(nm, f"err {err:.3e} bound {bound:.3e}")
        assert err <= bound, f"{nm} err {err:.3e} > {bound:.3e}"


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 64)])
def test_backward_rising_scores(dtype, causal, window):
    """Scores rising along the keys up to about 150, with one outlier key (the forward's
    rising-score input, GQA 2): rows whose softmax is nearly one-hot make dS = P (dP - D) a
    difference of nearly equal numbers, so the gradients' error is set by where the kernels
    round (the stored O that D comes from, P and dS rounded before their products), not by a
    fixed fraction of the gradient.  Every element must lie within the bound derived from those
    rounding steps (tests/bwd_bound.py), and each gradient's largest error within 3x that of a
    CPU model of the same steps (plus 1% of the relative tolerance at the largest gradient)."""
    q, k, v = make_rising_scores(dtype)
    do = make_dout(q.shape, DTYPES[dtype], 77)
    _say("rising scores backward", dtype, "causal", causal, "window", window)
    got = run_bwd(q, k, v, do, 0.5, causal, 0, window)
    ref = oracle.attention_backward_blocked(q.double().numpy(), k.double().numpy(),
                                            v.double().numpy(), do.double().numpy(),
                                            0.5, causal, 0, window)
    bounds = rounding_bound(q, k, v, do, 0.5, causal, 0, window)
    model = rounding_model(q, k, v, do, 0.5, causal, 0, window)
    top = max(float(np.max(np.abs(r))) for r in ref)
    floor = 0.01 * TOL_REL[q.dtype] * top
    for name, err, ratio, lim in check_within(got, ref, bounds, model, factor=3.0, floor=floor):
        m = float(np.max(np.abs(ref[("dq", "dk", "dv").index(name)])))
        _say(name, f"err {err:.3e} (max |g| {m:.3e}), worst err/bound {ratio:.3f}, measured limit {lim:.3e}")
        assert ratio <= 1.0, f"{name}: error {ratio:.2f}x the derived bound"
        assert err <= lim, f"{name}: err {err:.3e} > 3x the rounding model's + floor = {lim:.3e}"


def test_backward_deterministic():
    q, k, v = make_qkv(1, 8, 2, 300, 500, 128, "bf16", seed=32)
    do = make_dout(q.shape, torch.bfloat16, 32)
    a = run_bwd(q, k, v, do, 0.1, True, 200)
    b = run_bwd(q, k, v, do, 0.1, True, 200)
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_backward_errors():
    q, k, v = make_qkv(1, 4, 2, 64, 64, 128, "bf16", seed=33)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    out, lse = fa.fa_fwd(q, k, v)
    do = torch.ones_like(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(fa.FaError) as e:
        fa.fa_bwd_into(q, k, v, out, lse, do, dq, dk, dv, small)
    assert e.value.code == -13
    with pytest.raises(fa.FaError) as e:
        fa.fa_bwd_into(q, k, v, out, lse, do, dq, dk, dk, torch.empty(4096, dtype=torch.uint8, device=DEV))
    assert e.value.code == -9
