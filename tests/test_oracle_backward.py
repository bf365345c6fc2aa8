"""Pins for the backward oracle (gradients dQ, dK, dV of the attention forward pass).

Independent checks: PyTorch's CPU float64 autograd through scaled_dot_product_attention
with an explicit index mask and repeated K/V heads (a library routine), central finite
differences of <dO, O> computed with the forward oracle, and closed forms (a single key:
dQ = dK = 0, dV = sum of dO over the rows and heads that read it; equal value rows: dQ =
dK = 0).  Copies of the backward with a planted mistake must fail at least one pin.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import key_visibility, kv_head_of, masked_softmax_stats, scaled_scores
from tests import oracle_pins as pins

CASES = [
    # B, Hq, Hkv, Sq, Skv, D, causal, input_pos, window
    (1, 2, 2, 7, 7, 16, False, 0, 0),
    (2, 4, 2, 9, 13, 16, True, 2, 0),
    (1, 4, 1, 6, 11, 32, True, 0, 4),
    (1, 3, 3, 5, 9, 8, True, 3, 0),
]


def _torch_grads(q, k, v, do, scale, causal, pos, window):
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    i = torch.arange(Sq)[:, None] + pos
    j = torch.arange(Skv)[None, :]
    mask = torch.ones(Sq, Skv, dtype=torch.bool)
    if causal:
        mask = j <= i
        if window:
            mask = mask & (j > i - window)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.repeat_interleave(G, dim=1), vt.repeat_interleave(G, dim=1), attn_mask=mask, scale=scale)
    o.backward(torch.tensor(do))
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def pin_torch_autograd(bwd):
    for n, (B, Hq, Hkv, Sq, Skv, D, c, pos, W) in enumerate(CASES):
        q, k, v = pins.tiny_case(B, Hq, Hkv, Sq, Skv, D, 50 + n)
        do = pins.rand(q.shape, 60 + n)
        got = bwd(q, k, v, do, 0.25, c, pos, W)
        ref = _torch_grads(q, k, v, do, 0.25, c, pos, W)
        for g, r, name in zip(got, ref, ("dq", "dk", "dv")):
            assert np.max(np.abs(g - r)) < 1e-11, (name, CASES[n])


def pin_finite_differences(bwd):
    """d<dO, O>/dx by central differences (step 1e-6) with the forward oracle."""
    B, Hq, Hkv, Sq, Skv, D, c, pos, W = 1, 4, 2, 5, 8, 8, True, 1, 3
    q, k, v = pins.tiny_case(B, Hq, Hkv, Sq, Skv, D, 71)
    do = pins.rand(q.shape, 72)
    grads = bwd(q, k, v, do, 0.5, c, pos, W)

    def f(qq, kk, vv):
        O, _ = oracle.attention_blocked(qq, kk, vv, 0.5, c, pos, window=W)
        return float((O * do).sum())

    rng = np.random.default_rng(73)
    h = 1e-6
    for which, g in zip(range(3), grads):
        base = [q, k, v]
        for _ in range(6):
            idx = tuple(int(rng.integers(s)) for s in base[which].shape)
            plus = [x.copy() for x in base]
            minus = [x.copy() for x in base]
            plus[which][idx] += h
            minus[which][idx] -= h
            fd = (f(*plus) - f(*minus)) / (2 * h)
            assert abs(fd - g[idx]) < 1e-6, (which, idx, fd, g[idx])


def pin_single_key(bwd):
    """One key: P = 1 for every row, so dS = 0 (dQ = dK = 0) and dV = sum of dO over all
    rows of all query heads of the group."""
    q, k, v = pins.tiny_case(2, 4, 2, 6, 1, 16, 74)
    do = pins.rand(q.shape, 75)
    dq, dk, dv = bwd(q, k, v, do, 0.3, True, 0, 0)
    assert np.max(np.abs(dq)) < 1e-14 and np.max(np.abs(dk)) < 1e-14
    want = do.reshape(2, 2, 2, 6, 16).sum(axis=(2, 3))[:, :, None, :]
    assert np.max(np.abs(dv - want)) < 1e-12


def pin_equal_values(bwd):
    """All value rows equal: O = v0 whatever the weights, so dQ = dK = 0."""
    q, k, _ = pins.tiny_case(1, 2, 1, 5, 9, 16, 76)
    v = np.broadcast_to(pins.rand((1, 1, 1, 16), 77), (1, 1, 9, 16)).copy()
    do = pins.rand(q.shape, 78)
    dq, dk, dv = bwd(q, k, v, do, 0.4, False, 0, 0)
    assert np.max(np.abs(dq)) < 1e-12 and np.max(np.abs(dk)) < 1e-12


BWD_PINS = [pin_torch_autograd, pin_finite_differences, pin_single_key, pin_equal_values]


def _oracle(q, k, v, do, scale, causal, pos, window):
    return oracle.attention_backward_blocked(q, k, v, do, scale, causal, pos, window)


@pytest.mark.parametrize("pin", BWD_PINS, ids=lambda p: p.__name__)
def test_backward_pins(pin):
    pin(_oracle)


def _sampled_everywhere(q, k, v, do, scale, causal, pos, window):
    """The sampled form evaluated at every row, reshaped to full gradient tensors."""
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    qs = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(Sq)]
    ks = [(b, g, j) for b in range(B) for g in range(Hkv) for j in range(Skv)]
    dq, dk, dv = oracle.attention_backward_sampled(q, k, v, do, scale, causal, pos, qs, ks, window)
    return dq.reshape(q.shape), dk.reshape(k.shape), dv.reshape(v.shape)


@pytest.mark.parametrize("pin", BWD_PINS, ids=lambda p: p.__name__)
def test_backward_pins_sampled_form(pin):
    pin(_sampled_everywhere)


def test_backward_sampled_subset_matches_rows():
    """Any subset of samples returns the same rows as the whole set (no cross-talk)."""
    q, k, v = pins.tiny_case(2, 4, 2, 11, 13, 16, 90)
    do = pins.rand(q.shape, 91)
    full = _sampled_everywhere(q, k, v, do, 0.3, True, 2, 5)
    qs, ks = [(1, 3, 10), (0, 0, 0), (1, 2, 4)], [(1, 1, 12), (0, 0, 3)]
    dq, dk, dv = oracle.attention_backward_sampled(q, k, v, do, 0.3, True, 2, qs, ks, window=5)
    for n, (b, h, i) in enumerate(qs):
        assert np.max(np.abs(dq[n] - full[0][b, h, i])) < 1e-12
    for n, (b, g, j) in enumerate(ks):
        assert np.max(np.abs(dk[n] - full[1][b, g, j])) < 1e-12
        assert np.max(np.abs(dv[n] - full[2][b, g, j])) < 1e-12


def _planted(mistake):
    """A copy of the backward with one planted mistake (for the pins to catch)."""
    def bwd(q, k, v, do, scale, causal, pos, window):
        B, Hq, Sq, D = q.shape
        Hkv, Skv = k.shape[1], k.shape[2]
        dQ, dK, dV = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
        for b in range(B):
            for hq in range(Hq):
                g = kv_head_of(hq, Hq, Hkv)
                vis = key_visibility(np.arange(Sq), Skv, causal, pos, window)
                s = scaled_scores(q[b, hq], k[b, g], scale)
                _, e, l = masked_softmax_stats(s, vis)
                P = e / l
                dP = do[b, hq] @ v[b, g].T
                Dr = (P * dP).sum(axis=1, keepdims=True)
                dS = P * dP if mistake == "no_D" else P * (dP - Dr)
                sc = 1.0 if mistake == "dk_unscaled" else scale
                if mistake == "gqa_overwrite":
                    dV[b, g] = P.T @ do[b, hq]
                else:
                    dV[b, g] += (P @ do[b, hq][:Skv] if mistake == "p_not_transposed" and Sq == Skv
                                 else P.T @ do[b, hq])
                dQ[b, hq] = scale * (dS @ k[b, g])
                dK[b, g] += sc * (dS.T @ q[b, hq])
        return dQ, dK, dV
    return bwd


BWD_MUTANTS = ["no_D", "dk_unscaled", "gqa_overwrite", "p_not_transposed"]


def test_planted_copy_without_mistake_passes():
    for pin in BWD_PINS:
        pin(_planted("none"))


@pytest.mark.parametrize("name", BWD_MUTANTS)
def test_backward_pins_catch_planted_mistake(name):
    caught = []
    for pin in BWD_PINS:
        try:
            pin(_planted(name))
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"planted backward mistake {name} was not caught"


def test_backward_rejects_bad_arguments():
    q, k, v = pins.tiny_case(1, 1, 1, 4, 4, 8, 0)
    with pytest.raises(ValueError):
        oracle.attention_backward_blocked(q, k, v, np.zeros((1, 1, 3, 8)), 0.1)
    with pytest.raises(ValueError):
        oracle.attention_backward_blocked(q, k, v, np.zeros(q.shape), 0.1, False, 0, window=2)
