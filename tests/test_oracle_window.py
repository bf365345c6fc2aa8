"""Pins for the sliding-window form of the oracle (causal attention where query i sees
keys input_pos + i - W + 1 .. input_pos + i).

Independent checks: a closed form (W = 1: each row attends to exactly one key, so O is
that key's value row and LSE its scaled score), PyTorch's CPU float64
scaled_dot_product_attention with an explicit boolean mask built from indices, the
pure-Python loop form, windows wide enough to change nothing, and rows left with no
visible key.  Planted mistakes in the window bound must fail at least one pin.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import oracle.attention as oa
from tests import oracle_pins as pins

TIGHT = 1e-12


def pin_window_one(fn):
    """W = 1: row i sees only key input_pos + i, so O = v[input_pos + i] and
    LSE = scale * q_i . k_{input_pos + i} exactly."""
    q, k, v = pins.tiny_case(1, 4, 2, 9, 20, 64, 31)
    pos = 5
    O, L = fn(q, k, v, 0.3, True, pos, window=1)
    for hq in range(4):
        g = hq // 2
        for i in range(9):
            j = pos + i
            assert np.max(np.abs(O[0, hq, i] - v[0, g, j])) < TIGHT
            assert abs(L[0, hq, i] - 0.3 * float(q[0, hq, i] @ k[0, g, j])) < 1e-12


def pin_window_torch(fn):
    """Against torch's float64 CPU attention with a mask built from indices."""
    q, k, v = pins.tiny_case(2, 6, 3, 23, 40, 64, 32)
    for pos, W in ((0, 5), (17, 8), (3, 30), (10, 1)):
        O, L = fn(q, k, v, 0.2, True, pos, window=W)
        i = torch.arange(23)[:, None] + pos
        j = torch.arange(40)[None, :]
        mask = (j <= i) & (j > i - W)
        qt = torch.from_numpy(q)
        kt = torch.from_numpy(k).repeat_interleave(2, dim=1)
        vt = torch.from_numpy(v).repeat_interleave(2, dim=1)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=0.2)
        s = (qt @ kt.transpose(-1, -2)) * 0.2
        lse = torch.logsumexp(s.masked_fill(~mask, float("-inf")), dim=-1)
        assert np.max(np.abs(O - ref.numpy())) < 1e-12, (pos, W)
        assert np.max(np.abs(L - lse.numpy())) < 1e-12, (pos, W)


def pin_window_naive(fn):
    """Against the pure-Python loop form (written separately, index loops)."""
    q, k, v = pins.tiny_case(1, 2, 1, 7, 13, 64, 33)
    for pos, W in ((0, 3), (4, 6), (2, 1)):
        O, L = fn(q, k, v, 0.25, True, pos, window=W)
        On, Ln = oracle.attention_naive(q, k, v, 0.25, True, pos, window=W)
        assert np.max(np.abs(O - On)) < TIGHT and np.max(np.abs(L - Ln)) < TIGHT


def pin_window_wide_is_causal(fn):
    """A window at least as long as the longest visible prefix changes nothing."""
    q, k, v = pins.tiny_case(1, 4, 4, 12, 30, 128, 34)
    O, L = fn(q, k, v, 0.1, True, 6)
    for W in (18, 19, 1000):
        Ow, Lw = fn(q, k, v, 0.1, True, 6, window=W)
        assert np.max(np.abs(Ow - O)) < TIGHT and np.max(np.abs(Lw - L)) < TIGHT


def pin_window_empty_rows(fn):
    """Sq > Skv with input_pos 0 and W = 4: rows i >= Skv + 3 see no key (O = 0,
    LSE = -inf); row Skv + 2 sees key Skv - 1 only."""
    q, k, v = pins.tiny_case(1, 1, 1, 12, 6, 64, 35)
    O, L = fn(q, k, v, 0.5, True, 0, window=4)
    assert np.all(O[0, 0, 9:] == 0.0) and np.all(L[0, 0, 9:] == -np.inf)
    assert np.max(np.abs(O[0, 0, 8] - v[0, 0, 5])) < TIGHT
    assert np.all(np.isfinite(L[0, 0, :9]))


WINDOW_PINS = [pin_window_one, pin_window_torch, pin_window_naive, pin_window_wide_is_causal,
               pin_window_empty_rows]


@pytest.mark.parametrize("pin", WINDOW_PINS, ids=lambda p: p.__name__)
def test_window_pins_blocked(pin):
    pin(oracle.attention_blocked)


def _rows_form(q, k, v, scale, causal, pos, window=0):
    B, Hq, Sq, D = q.shape
    samples = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(Sq)]
    O, L = oracle.attention_rows(q, k, v, scale, causal, pos, samples, window=window)
    return O.reshape(B, Hq, Sq, D), L.reshape(B, Hq, Sq)


@pytest.mark.parametrize("pin", WINDOW_PINS, ids=lambda p: p.__name__)
def test_window_pins_rows_form(pin):
    pin(_rows_form)


def test_window_key_ranges_merge_to_full():
    q, k, v = pins.tiny_case(1, 4, 2, 30, 50, 64, 36)
    O, L = oracle.attention_blocked(q, k, v, 0.2, True, 12, window=9)
    cuts = [0, 7, 16, 16, 31, 50]
    parts = [oracle.attention_key_range(q, k, v, 0.2, True, 12, a, b, window=9)
             for a, b in zip(cuts[:-1], cuts[1:])]
    Om, Lm = oracle.merge_partials([p[0] for p in parts], [p[1] for p in parts])
    assert np.max(np.abs(Om - O)) < TIGHT and np.max(np.abs(Lm - L)) < TIGHT


def test_window_argument_checks():
    q, k, v = pins.tiny_case(1, 1, 1, 4, 4, 64, 0)
    with pytest.raises(ValueError):
        oracle.attention_blocked(q, k, v, 0.1, False, 0, window=3)
    with pytest.raises(ValueError):
        oracle.attention_blocked(q, k, v, 0.1, True, 0, window=-1)


_vis = oa.key_visibility
WINDOW_MUTANTS = {
    # lower bound off by one (W + 1 keys visible)
    "bound_off_by_one": lambda rows, Skv, c, pos, window=0: _vis(rows, Skv, c, pos, window + 1 if window else 0),
    # window measured from the row index, ignoring input_pos
    "bound_ignores_input_pos": lambda rows, Skv, c, pos, window=0: (
        _vis(rows, Skv, c, pos) & (np.arange(Skv)[None, :] >= np.asarray(rows)[:, None] - window + 1)
        if window else _vis(rows, Skv, c, pos)),
    # window ignored
    "window_ignored": lambda rows, Skv, c, pos, window=0: _vis(rows, Skv, c, pos),
    # window as a strict bound (W - 1 keys visible)
    "bound_strict": lambda rows, Skv, c, pos, window=0: _vis(rows, Skv, c, pos, max(window - 1, 0) if window > 1 else window),
}


@pytest.mark.parametrize("name", sorted(WINDOW_MUTANTS))
def test_window_pins_catch_planted_mistake(name, monkeypatch):
    monkeypatch.setattr(oa, "key_visibility", WINDOW_MUTANTS[name])
    caught = []
    for pin in WINDOW_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(oa.attention_blocked)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"planted window mistake {name} was not caught by any pin"
