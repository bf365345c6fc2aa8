"""Pins for the split-KV forms of the oracle: attention over a key range and the
merge of ranges.

The merge is checked against closed forms (hand-worked weights), invariants
(order of the ranges, ranges with no visible key) and the identity that
merging the ranges of any partition of the keys gives the attention over all
keys, which the one-pass oracle computes (that oracle is itself pinned to brute
force and PyTorch's CPU float64 attention).  Planted mistakes in the merge must
fail at least one of these pins.
"""

from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
from tests import oracle_pins as pins

TIGHT = 1e-12


def _partition(q, k, v, scale, causal, pos, cuts, merge=oracle.merge_partials):
    parts = [oracle.attention_key_range(q, k, v, scale, causal, pos, a, b)
             for a, b in zip(cuts[:-1], cuts[1:])]
    return merge([p[0] for p in parts], [p[1] for p in parts])


# --- pins, each taking the merge function under test ------------------------------

def pin_hand_worked(merge):
    """Two ranges, D = 1: LSE_1 = 0, LSE_2 = ln 3 give weights 1/4 and 3/4, so
    O_1 = 1, O_2 = 5 merge to O = 4 and LSE = ln(1 + 3) = ln 4."""
    O, L = merge(np.array([[[1.0]], [[5.0]]]), np.array([[0.0], [math.log(3.0)]]))
    assert abs(O[0, 0] - 4.0) < TIGHT and abs(L[0] - math.log(4.0)) < TIGHT, (O, L)


def pin_equal_halves(merge):
    """Two ranges with the same O and LSE: O is unchanged and LSE grows by ln 2."""
    o = pins.rand((3, 64), 11)
    lse = pins.rand((3,), 12, 5.0)
    O, L = merge(np.stack([o, o]), np.stack([lse, lse]))
    assert np.max(np.abs(O - o)) < TIGHT and np.max(np.abs(L - (lse + math.log(2.0)))) < TIGHT


def pin_empty_ranges(merge):
    """Ranges with LSE = -inf (no visible key) do not change the result; all empty
    gives O = 0 and LSE = -inf."""
    o = pins.rand((4, 8), 13)
    lse = pins.rand((4,), 14)
    ninf = np.full(4, -np.inf)
    junk = pins.rand((4, 8), 15, 100.0)   # an empty range's O must carry no weight
    O, L = merge(np.stack([junk, o, junk]), np.stack([ninf, lse, ninf]))
    assert np.max(np.abs(O - o)) < TIGHT and np.max(np.abs(L - lse)) < TIGHT
    O, L = merge(np.stack([junk, junk]), np.stack([ninf, ninf]))
    assert np.all(O == 0.0) and np.all(L == -np.inf)


def pin_order_invariant(merge):
    """The merge does not depend on the order of the ranges."""
    o = pins.rand((5, 6, 16), 16)
    lse = pins.rand((5, 6), 17, 20.0)
    O1, L1 = merge(o, lse)
    perm = [3, 0, 4, 1, 2]
    O2, L2 = merge(o[perm], lse[perm])
    assert np.max(np.abs(O1 - O2)) < 1e-12 and np.max(np.abs(L1 - L2)) < 1e-12


def pin_partition_is_full_attention(merge):
    """Merging the ranges of a partition of the keys (with empty and past-the-end
    ranges) gives the attention over all keys: causal GQA with an offset and a
    non-causal case."""
    q, k, v = pins.tiny_case(1, 4, 2, 37, 53, 64, 3)
    for causal, pos, cuts in ((True, 10, [0, 5, 5, 20, 33, 53, 60]),
                              (False, 0, [0, 1, 52, 53]),
                              (True, 0, [0, 16, 32, 48, 64])):
        O, L = oracle.attention_blocked(q, k, v, 0.2, causal, pos)
        Om, Lm = _partition(q, k, v, 0.2, causal, pos, cuts, merge)
        assert np.max(np.abs(Om - O)) < 1e-12, (causal, pos, cuts)
        assert np.max(np.abs(Lm - L)) < 1e-12, (causal, pos, cuts)


def pin_large_lse_spread(merge):
    """LSE values far apart (1000 vs 0): the small range's weight e^-1000 underflows to
    0 without NaN or inf, so the result is the large range's."""
    o = pins.rand((2, 2, 8), 18)
    lse = np.array([[1000.0, 0.0], [0.0, 1000.0]])
    O, L = merge(o, lse)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    assert np.max(np.abs(O[0] - o[0, 0])) < TIGHT and np.max(np.abs(O[1] - o[1, 1])) < TIGHT
    assert np.max(np.abs(L - 1000.0)) < TIGHT


MERGE_PINS = [pin_hand_worked, pin_equal_halves, pin_empty_ranges, pin_order_invariant,
              pin_partition_is_full_attention, pin_large_lse_spread]


@pytest.mark.parametrize("pin", MERGE_PINS, ids=lambda p: p.__name__)
def test_merge_pins(pin):
    pin(oracle.merge_partials)


# --- the key-range form ------------------------------------------------------------

def test_key_range_all_keys_is_full_attention():
    q, k, v = pins.tiny_case(2, 6, 3, 29, 41, 128, 5)
    for causal, pos in ((True, 0), (True, 12), (False, 0)):
        O, L = oracle.attention_blocked(q, k, v, 0.09, causal, pos)
        Or, Lr = oracle.attention_key_range(q, k, v, 0.09, causal, pos, 0, 41)
        assert np.max(np.abs(Or - O)) < TIGHT and np.max(np.abs(Lr - L)) < TIGHT


def test_key_range_brute_force_on_slice():
    """Without a mask, the range [lo, hi) is plain attention over k[lo:hi], v[lo:hi],
    checked against the pure-Python loop form."""
    q, k, v = pins.tiny_case(1, 2, 1, 5, 17, 64, 6)
    lo, hi = 4, 11
    On, Ln = oracle.attention_naive(q, k[:, :, lo:hi], v[:, :, lo:hi], 0.3)
    Or, Lr = oracle.attention_key_range(q, k, v, 0.3, False, 0, lo, hi)
    assert np.max(np.abs(Or - On)) < TIGHT and np.max(np.abs(Lr - Ln)) < TIGHT


def test_key_range_rows_with_no_visible_key():
    """Causal, input_pos 0: row i sees keys <= i, so range [10, 20) is empty for rows
    0..9 (O = 0, LSE = -inf) and row 12 sees keys 10..12 only."""
    q, k, v = pins.tiny_case(1, 1, 1, 16, 20, 64, 7)
    O, L = oracle.attention_key_range(q, k, v, 0.125, True, 0, 10, 20)
    assert np.all(O[0, 0, :10] == 0.0) and np.all(L[0, 0, :10] == -np.inf)
    On, Ln = oracle.attention_naive(q[:, :, 12:13], k[:, :, 10:13], v[:, :, 10:13], 0.125)
    assert np.max(np.abs(O[0, 0, 12] - On[0, 0, 0])) < TIGHT
    assert abs(L[0, 0, 12] - Ln[0, 0, 0]) < TIGHT


# --- planted mistakes in the merge must be caught -----------------------------------

def _merge_closed(o_parts, lse_parts, weight=np.exp, normalise=True, lse_log=True, drop_last=False):
    o_parts = np.asarray(o_parts, np.float64)
    lse_parts = np.asarray(lse_parts, np.float64)
    if drop_last:
        o_parts, lse_parts = o_parts[:-1], lse_parts[:-1]
    m = lse_parts.max(axis=0)
    safe = np.where(np.isfinite(m), m, 0.0)
    w = weight(lse_parts - safe)
    l = w.sum(axis=0)
    acc = (w[..., None] * o_parts).sum(axis=0)
    O = acc / np.where(l > 0, l, 1.0)[..., None] if normalise else acc
    LSE = (m + np.log(l)) if lse_log else m
    return O, LSE


MERGE_MUTANTS = {
    "unnormalised": lambda o, l: _merge_closed(o, l, normalise=False),
    "lse_is_max": lambda o, l: _merge_closed(o, l, lse_log=False),
    "linear_weights": lambda o, l: _merge_closed(o, l, weight=lambda x: np.where(np.isfinite(x), 1.0 + x, 0.0)),
    "exp2_weights": lambda o, l: _merge_closed(o, l, weight=np.exp2),
    "drops_last_range": lambda o, l: _merge_closed(o, l, drop_last=True),
}


def test_closed_form_merge_passes_pins():
    """The closed form LSE = ln sum exp(LSE_s), O = sum exp(LSE_s - LSE) O_s, written
    independently of the oracle's fold, passes every pin (so the mutants below differ
    from it in the planted mistake only)."""
    with np.errstate(divide="ignore"):
        for pin in MERGE_PINS:
            pin(_merge_closed)


@pytest.mark.parametrize("name", sorted(MERGE_MUTANTS))
def test_merge_pins_catch_planted_mistake(name):
    caught = []
    for pin in MERGE_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(MERGE_MUTANTS[name])
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"planted merge mistake {name} was not caught by any pin"


_key_range = oracle.attention_key_range
RANGE_MUTANTS = {
    "end_inclusive": lambda q, k, v, s, c, p, lo, hi: _key_range(q, k, v, s, c, p, lo, hi + 1),
    "start_ignored": lambda q, k, v, s, c, p, lo, hi: _key_range(q, k, v, s, c, p, 0, hi),
    "mask_ignored": lambda q, k, v, s, c, p, lo, hi: _key_range(q, k, v, s, False, p, lo, hi),
}


@pytest.mark.parametrize("name", sorted(RANGE_MUTANTS))
def test_partition_pin_catches_planted_range_mistake(name, monkeypatch):
    monkeypatch.setattr(oracle, "attention_key_range", RANGE_MUTANTS[name])
    with pytest.raises(AssertionError):
        pin_partition_is_full_attention(oracle.merge_partials)
