"""CPU tests of the fp64 oracle: its pins, its three forms, and the pages' printed facts."""

from __future__ import annotations

import functools
import math
import os

import numpy as np
import pytest

import oracle
import oracle.attention as oa
from tests import oracle_pins as pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


# --- the pins, on the oracle used for parity -----------------------------------------

@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_blocked_oracle_pins(pin):
    pin(oracle.attention_blocked)


@pytest.mark.parametrize("pin", [pins.pin_bruteforce, pins.pin_torch_sdpa, pins.pin_causal_row0,
                                 pins.pin_gqa_replicated, pins.pin_input_pos_chunk],
                         ids=lambda p: p.__name__)
def test_online_tiled_oracle_pins(pin):
    pin(functools.partial(oracle.attention_online_tiled, tile_m=16, tile_n=32))


# --- P-g: the online tile-by-tile variant equals the one-pass definition ------------

@pytest.mark.parametrize("tile_m,tile_n", [(16, 16), (64, 64), (32, 64), (64, 32), (128, 64),
                                           (7, 5), (48, 80), (256, 128)])
@pytest.mark.parametrize("causal,pos", [(False, 0), (True, 0), (True, 37), (True, 500)])
def test_online_equals_onepass(tile_m, tile_n, causal, pos):
    q, k, v = pins.tiny_case(1, 4, 2, 150, 171 if pos else 150, 64, 3)
    O1, L1 = oracle.attention_blocked(q, k, v, 0.11, causal, pos)
    for split in (True, False):
        O2, L2 = oracle.attention_online_tiled(q, k, v, 0.11, causal, pos, tile_m, tile_n, split)
        assert np.max(np.abs(O1 - O2)) < 1e-12
        assert np.max(np.abs(L1 - L2)) < 1e-12


def test_rows_form_equals_blocked():
    q, k, v = pins.tiny_case(2, 4, 2, 33, 70, 128, 9)
    O, L = oracle.attention_blocked(q, k, v, 0.1, True, 37)
    samples = [(0, 0, 0), (1, 3, 32), (0, 2, 5), (1, 1, 17)]
    Or, Lr = oracle.attention_rows(q, k, v, 0.1, True, 37, samples)
    for n, (b, h, i) in enumerate(samples):
        assert np.max(np.abs(Or[n] - O[b, h, i])) < 1e-14
        assert abs(Lr[n] - L[b, h, i]) < 1e-14


def test_tile_plan_against_brute_force():
    """The visited and mask-free block counts bound exactly the visible / fully visible
    key blocks (any tiling)."""
    rng = np.random.default_rng(0)
    for _ in range(400):
        tm, tn = int(rng.integers(1, 70)), int(rng.integers(1, 70))
        Sq, Skv = int(rng.integers(1, 300)), int(rng.integers(1, 300))
        causal = bool(rng.integers(0, 2))
        pos = int(rng.integers(0, 300))
        for t in range(-(-Sq // tm)):
            tc, ms = oracle.tile_plan(t, tm, tn, Skv, causal, pos)
            rows = np.arange(t * tm, (t + 1) * tm)  # padded rows included, as the kernel does
            vis = oracle.key_visibility(rows, Skv, causal, pos)
            last_visible = np.nonzero(vis.any(axis=0))[0].max()
            assert tc == last_visible // tn + 1  # every tile with a visible key, none after
            for j in range(min(ms, tc)):  # tiles before mask_start are fully visible, in range
                cols = np.arange(j * tn, (j + 1) * tn)
                assert cols[-1] < Skv and vis[:, cols].all()


# --- the pages' printed facts (tests/golden) ----------------------------------------

def test_golden_gqa_head_map():
    for Hq, Hkv, lo, hi, kv in (map(int, r) for r in _golden_rows("gqa_head_map_32q_4kv.txt")):
        for hq in range(lo, hi + 1):
            assert oracle.kv_head_of(hq, Hq, Hkv) == kv


def test_golden_causal_mask_four_tokens():
    want = np.array([[int(x) for x in r] for r in _golden_rows("causal_mask_4_tokens.txt")], bool)
    assert np.array_equal(oracle.key_visibility(range(4), 4, True, 0), want)
    P = oracle.attention_probs_naive(*pins.tiny_case(1, 1, 1, 4, 4, 64, 0)[:2], 0.125, True, 0)
    assert np.array_equal(P[0, 0] > 0, want)


def test_golden_kloop_split_16k():
    g = {r[0]: float(r[1]) for r in _golden_rows("kloop_split_16k_tile256.txt")}
    S, tm, tn = int(g["seq_len"]), int(g["tile_m"]), int(g["tile_n"])
    unmasked, masked, skipped = oracle.classify_tiles(S, S, tm, tn, causal=True)
    n_rows = S // tm
    total = n_rows * (S // tn)
    assert abs(unmasked / total - g["unmasked_fraction_approx"]) <= g["unmasked_fraction_tolerance"]
    assert masked == n_rows * int(g["masked_tiles_per_row"])
    assert skipped == total - unmasked - masked and skipped > 0


def test_golden_tile_counts():
    for S, tm, n in (map(int, r) for r in _golden_rows("tile_counts.txt")):
        assert -(-S // tm) == n


# --- mistakes planted in the oracle must be caught by the pins ----------------------

MUTANTS = {
    "gqa_strided": ("kv_head_of", lambda hq, Hq, Hkv: hq % Hkv),
    "mask_strict_lt": ("key_visibility", lambda rows, Skv, causal, pos, window=0: (
        np.ones((len(rows), Skv), bool) if not causal else
        np.maximum(np.arange(Skv)[None, :] < np.asarray(rows)[:, None] + pos,
                   np.arange(Skv)[None, :] == 0))),
    "mask_ignores_input_pos": ("key_visibility", lambda rows, Skv, causal, pos, window=0: (
        np.ones((len(rows), Skv), bool) if not causal else
        np.arange(Skv)[None, :] <= np.asarray(rows)[:, None])),
    "mask_transposed": ("key_visibility", lambda rows, Skv, causal, pos, window=0: (
        np.ones((len(rows), Skv), bool) if not causal else
        np.arange(Skv)[None, :] >= np.asarray(rows)[:, None] + pos)),
    "mask_dropped": ("key_visibility", lambda rows, Skv, causal, pos, window=0: np.ones((len(rows), Skv), bool)),
    "scale_dropped": ("scaled_scores", lambda qr, kh, scale: qr @ kh.T),
    "scale_inverted": ("scaled_scores", lambda qr, kh, scale: (qr @ kh.T) / scale),
    "scores_sign": ("scaled_scores", lambda qr, kh, scale: -scale * (qr @ kh.T)),
    "keys_reversed": ("scaled_scores", lambda qr, kh, scale: scale * (qr @ kh[::-1].T)),
    "no_max_shift_lse": ("masked_softmax_stats", lambda s, vis: (
        lambda s2: (s2.max(axis=1, keepdims=True), np.exp(s2), np.exp(s2).sum(axis=1, keepdims=True))
    )(np.where(vis, s, -np.inf))),
    "no_normalisation": ("normalise", lambda e, l, vh: e @ vh),
    "values_reversed": ("normalise", lambda e, l, vh: (e @ vh[::-1]) / l),
    "lse_log2": ("log_sum_exp", lambda m, l: m[:, 0] + np.log2(l[:, 0])),
    "lse_drops_sum": ("log_sum_exp", lambda m, l: m[:, 0]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(oa, attr, fn)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(oa.attention_blocked)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name} was not caught by any pin"


TILED_MUTANTS = {
    # the last visited key block dropped
    "one_block_short": ("tile_plan", lambda t, tm, tn, Skv, c, pos: (
        max(1, _tile_plan(t, tm, tn, Skv, c, pos)[0] - 1), _tile_plan(t, tm, tn, Skv, c, pos)[1])),
    # one more block folded without its mask
    "unmasked_block_too_many": ("tile_plan", lambda t, tm, tn, Skv, c, pos: (
        _tile_plan(t, tm, tn, Skv, c, pos)[0],
        min(_tile_plan(t, tm, tn, Skv, c, pos)[1] + 1, _tile_plan(t, tm, tn, Skv, c, pos)[0]))),
    # visited blocks computed without the query offset
    "plan_ignores_input_pos": ("tile_plan", lambda t, tm, tn, Skv, c, pos: (
        _tile_plan(t, tm, tn, Skv, c, 0)[0], _tile_plan(t, tm, tn, Skv, c, 0)[1])),
    # the running state not rescaled when the maximum grows
    "fold_without_rescale": ("_fold", lambda st, pt: (
        np.maximum(st[0], pt[0]), st[1] + pt[1], st[2] + pt[2])),
    # the block's weights taken relative to zero instead of its own maximum
    "block_not_shifted": ("_block_state", lambda s, vis, vb: (
        np.where(vis, s, -np.inf).max(axis=1),
        np.exp(np.where(vis, s, -np.inf)).sum(axis=1), np.exp(np.where(vis, s, -np.inf)) @ vb)),
}
_tile_plan = oa.tile_plan


@pytest.mark.parametrize("name", sorted(TILED_MUTANTS))
def test_online_pin_catches_planted_tiling_mistake(name, monkeypatch):
    attr, fn = TILED_MUTANTS[name]
    monkeypatch.setattr(oa, attr, fn)
    q, k, v = pins.tiny_case(1, 2, 1, 100, 130, 64, 4)
    O1, L1 = oracle.attention_blocked(q, k, v, 0.125, True, 30)
    O2, L2 = oa.attention_online_tiled(q, k, v, 0.125, True, 30, 32, 16)
    assert max(np.max(np.abs(O1 - O2)), np.max(np.abs(L1 - L2))) > 1e-6


# --- the key span that attention_blocked reads for a block of rows ----------------------

SPAN_MUTANTS = {
    "span_end_short": lambda vis: (oa_span(vis)[0], oa_span(vis)[1] - 1),
    "span_start_late": lambda vis: (min(oa_span(vis)[0] + 1, oa_span(vis)[1] - 1), oa_span(vis)[1]),
}
oa_span = oa.visible_key_span


@pytest.mark.parametrize("rows_per_block", [1, 5, 16])
@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_blocked_oracle_pins_many_blocks(pin, rows_per_block):
    """The pins again with several row blocks per head, each block reading only its own
    visible key span."""
    pin(functools.partial(oracle.attention_blocked, rows_per_block=rows_per_block))


@pytest.mark.parametrize("name", sorted(SPAN_MUTANTS))
def test_pins_catch_planted_span_mistake(name, monkeypatch):
    monkeypatch.setattr(oa, "visible_key_span", SPAN_MUTANTS[name])
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(functools.partial(oa.attention_blocked, rows_per_block=5))
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name} was not caught by any pin"


def test_scale_rejected():
    q, k, v = pins.tiny_case(1, 1, 1, 2, 2, 64, 0)
    for bad in (0.0, -1.0, math.inf, math.nan):
        with pytest.raises(ValueError):
            oracle.attention_blocked(q, k, v, bad)
