"""The backward tolerances are reachable by the kernels' arithmetic, and the derived bound holds.

A CPU model of fa_bwd's rounding steps (tests/bwd_bound.py: fp32 scores from the rounded
inputs, P from an accurate LSE, the forward output as fl(fl(P) V), D from it, P and dS
rounded to the input type before their products, fp32 accumulation, gradients rounded) is
compared with the fp64 oracle:

* on N(0,1) inputs its error must stay below 40% of the relative tolerance the GPU parity
  tests use, so that a failing GPU test points at the kernels rather than at the bound;
* on every input, including the rising-score input whose near one-hot rows make dS a
  difference of nearly equal numbers, it must stay below half of the elementwise bound
  derived from the same rounding steps (``rounding_bound``);
* each of five planted mistakes in the model (D dropped, D's sign flipped, dK without the
  scale, dQ from the wrong key, dV from dS) must exceed that bound somewhere.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from attention_fa_fwd_amd.inputs import make_qkv, make_rising_scores
from tests.bwd_bound import check_within, rounding_bound, rounding_model

TOL_REL = {"fp16": 4e-3, "bf16": 1.6e-2}


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_backward_tolerance_headroom(dtype):
    dt = {"fp16": torch.float16, "bf16": torch.bfloat16}[dtype]
    worst = 0.0
    for seed in range(2):
        q, k, v = make_qkv(1, 4, 4, 192, 192, 128, dtype, seed)
        g = torch.Generator().manual_seed(500 + seed)
        do = torch.randn(q.shape, generator=g).to(dt)
        sim = rounding_model(q, k, v, do, 1 / math.sqrt(128), True)
        ref = oracle.attention_backward_blocked(q.double().numpy(), k.double().numpy(),
                                                v.double().numpy(), do.double().numpy(),
                                                1 / math.sqrt(128), True, 0)
        for a, r in zip(sim, ref):
            worst = max(worst, float(np.max(np.abs(a.double().numpy() - r)) / np.max(np.abs(r))))
    assert worst < 0.4 * TOL_REL[dtype], worst


def _cases(dtype):
    dt = {"fp16": torch.float16, "bf16": torch.bfloat16}[dtype]
    out = []
    for causal in (True, False):
        q, k, v = make_rising_scores(dtype)
        do = torch.randn(q.shape, generator=torch.Generator().manual_seed(7)).to(dt)
        out.append((f"rising causal={causal}", q, k, v, do, 0.5, causal, 0, 0))
    q, k, v = make_qkv(1, 8, 2, 200, 300, 128, dtype, 11)
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(8)).to(dt)
    out.append(("N(0,1) GQA 4, input_pos 40", q, k, v, do, 1 / math.sqrt(128), True, 40, 0))
    q, k, v = make_qkv(1, 4, 4, 150, 150, 64, dtype, 12)
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(9)).to(dt)
    out.append(("N(0,1) window 33", q, k, v, do, 0.125, True, 0, 33))
    return out


def _oracle(q, k, v, do, scale, causal, pos, window):
    return oracle.attention_backward_blocked(q.double().numpy(), k.double().numpy(),
                                             v.double().numpy(), do.double().numpy(),
                                             scale, causal, pos, window)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_derived_bound_holds_for_the_rounding_model(dtype):
    for what, q, k, v, do, scale, causal, pos, window in _cases(dtype):
        ref = _oracle(q, k, v, do, scale, causal, pos, window)
        bounds = rounding_bound(q, k, v, do, scale, causal, pos, window)
        model = rounding_model(q, k, v, do, scale, causal, pos, window)
        for name, err, ratio, _ in check_within(model, ref, bounds):
            assert ratio < 0.5, f"{what} {name}: model error reaches {ratio:.2f} of the bound"


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("mistake", ["no_d", "d_sign", "dk_no_scale", "dq_keys_shifted",
                                     "dv_from_ds"])
def test_derived_bound_catches_planted_mistakes(dtype, mistake):
    caught = []
    for what, q, k, v, do, scale, causal, pos, window in _cases(dtype):
        ref = _oracle(q, k, v, do, scale, causal, pos, window)
        bounds = rounding_bound(q, k, v, do, scale, causal, pos, window)
        bad = rounding_model(q, k, v, do, scale, causal, pos, window, mistake=mistake)
        caught.append(max(r[2] for r in check_within(bad, ref, bounds)) > 1.0)
    # the rising-score causal case and both N(0,1) cases must each catch it
    assert caught[0] and caught[2] and caught[3], caught
