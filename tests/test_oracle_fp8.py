"""Pins for the fp8 forms of the oracle: E4M3 decoding and attention over dequantised
fp8 queries and keys.

Independent checks: PyTorch's float8_e4m3fn -> float64 conversion for all 256 codes (a
library routine), hand-decoded codes from the format's definition, PyTorch's rounding of
float32 values to fp8 read back through the decoder, attention over inputs decoded by
PyTorch instead of the oracle, and the invariance of the scores under moving a factor
between the softmax scale and a descale.  Planted mistakes in the decoder must fail.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from attention_fa_fwd_amd.inputs import make_qkv_fp8, make_qkv_fp8qkv, quantize_fp8
from tests import oracle_pins as pins

ALL = np.arange(256, dtype=np.uint8)


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def pin_all_codes(decode):
    a, b = decode(ALL), _torch_decode(ALL)
    same = (a == b) | (np.isnan(a) & np.isnan(b))
    assert same.all(), f"codes differ: {np.nonzero(~same)[0][:8]}"


def pin_hand_values(decode):
    """From the E4M3 definition: 0x38 = 1 (e=7, m=0); 0x7E = 1.75 * 2^8 = 448 (largest);
    0x08 = 2^-6 (smallest normal); 0x01 = 2^-9 (smallest subnormal); 0x07 = 7 * 2^-9;
    0x3C = 1.5; 0xC4 = -3; 0x7F is NaN; 0x80 is -0."""
    cases = {0x38: 1.0, 0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9,
             0x3C: 1.5, 0xC4: -3.0, 0x00: 0.0}
    got = decode(np.array(list(cases), np.uint8))
    assert np.array_equal(got, np.array(list(cases.values()))), got
    assert np.isnan(decode(np.array([0x7F, 0xFF], np.uint8))).all()
    z = decode(np.array([0x80], np.uint8))[0]
    assert z == 0.0 and math.copysign(1.0, z) < 0


def pin_torch_rounding(decode):
    """Values rounded to fp8 by PyTorch decode to PyTorch's own float value of the code."""
    x = torch.from_numpy(pins.rand((4096,), 41, 60.0)).to(torch.float32).clamp(-448, 448)
    codes = x.to(torch.float8_e4m3fn)
    got = decode(codes.view(torch.uint8).numpy())
    assert np.array_equal(got, codes.to(torch.float64).numpy())


DECODE_PINS = [pin_all_codes, pin_hand_values, pin_torch_rounding]


@pytest.mark.parametrize("pin", DECODE_PINS, ids=lambda p: p.__name__)
def test_decode_pins(pin):
    pin(oracle.fp8_e4m3_decode)


def _mut(bias=7, mdiv=8.0, subnormal=True):
    def dec(codes):
        c = np.asarray(codes, np.uint8).astype(np.int64)
        sign = np.where(c & 0x80, -1.0, 1.0)
        e, m = (c >> 3) & 0xF, c & 0x7
        normal = (1.0 + m / mdiv) * np.exp2(e - float(bias))
        mag = np.where(e == 0, m * 2.0 ** -9, normal) if subnormal else normal
        mag = np.where((e == 15) & (m == 7), np.nan, mag)
        return sign * mag
    return dec


DECODE_MUTANTS = {"bias_8": _mut(bias=8), "mantissa_over_16": _mut(mdiv=16.0),
                  "no_subnormals": _mut(subnormal=False)}


@pytest.mark.parametrize("name", sorted(DECODE_MUTANTS))
def test_decode_pins_catch_planted_mistake(name):
    caught = []
    for pin in DECODE_PINS:
        try:
            pin(DECODE_MUTANTS[name])
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"planted decoder mistake {name} was not caught"


def test_fp8_attention_matches_torch_decoded_inputs():
    q8, k8, v, qd, kd = make_qkv_fp8(1, 4, 2, 40, 70, 128, "bf16", seed=3)
    O, L = oracle.attention_fp8_blocked(q8.view(torch.uint8).numpy(), k8.view(torch.uint8).numpy(),
                                        v.double().numpy(), 0.09, qd, kd, True, 10, window=25)
    qf = q8.to(torch.float64).numpy() * qd
    kf = k8.to(torch.float64).numpy() * kd
    O2, L2 = oracle.attention_blocked(qf, kf, v.double().numpy(), 0.09, True, 10, window=25)
    assert np.max(np.abs(O - O2)) < 1e-12 and np.max(np.abs(L - L2)) < 1e-12


def test_fp8_descale_moves_into_scale():
    """S depends on scale * q_descale * k_descale only."""
    q8, k8, v, qd, kd = make_qkv_fp8(1, 2, 1, 30, 30, 128, "fp16", seed=4)
    qc, kc, vv = q8.view(torch.uint8).numpy(), k8.view(torch.uint8).numpy(), v.double().numpy()
    O1, L1 = oracle.attention_fp8_blocked(qc, kc, vv, 0.1, qd, kd, True)
    O2, L2 = oracle.attention_fp8_blocked(qc, kc, vv, 0.05, qd * 2, kd, True)
    O3, L3 = oracle.attention_fp8_blocked(qc, kc, vv, 0.4, qd, kd / 4, True)
    for O, L in ((O2, L2), (O3, L3)):
        assert np.max(np.abs(O - O1)) < 1e-12 and np.max(np.abs(L - L1)) < 1e-12


def test_quantize_fp8_round_trip():
    """The input generator's per-tensor quantisation: the largest magnitude maps to 448
    exactly and every value is within half an fp8 step of the original."""
    x = torch.from_numpy(pins.rand((2, 3, 50, 64), 5)).to(torch.float32)
    codes, d = quantize_fp8(x)
    back = torch.from_numpy(oracle.fp8_e4m3_decode(codes.view(torch.uint8).numpy())) * d
    assert float(back.abs().max()) == pytest.approx(float(x.abs().max()), rel=1e-12)
    err = (back - x.double()).abs()
    tol = torch.maximum(x.double().abs() * 2.0 ** -4, torch.tensor(d * 2.0 ** -10))
    assert bool((err <= tol * (1 + 1e-9)).all())


def test_fp8_rejects_bad_descale():
    q8, k8, v, qd, kd = make_qkv_fp8(1, 1, 1, 4, 4, 128, "bf16", seed=0)
    for bad in (0.0, -1.0, math.inf, math.nan):
        with pytest.raises(ValueError):
            oracle.attention_fp8_blocked(q8.view(torch.uint8).numpy(), k8.view(torch.uint8).numpy(),
                                         v.double().numpy(), 0.1, bad, kd)


# --- fp8 values --------------------------------------------------------------------

def test_fp8v_attention_matches_torch_decoded_inputs():
    """fp8 values: the oracle decodes v's codes and applies v_descale; decoding all three
    inputs with PyTorch's float8_e4m3fn conversion instead gives the same result."""
    q8, k8, v8, qd, kd, vd = make_qkv_fp8qkv(2, 4, 2, 33, 70, 128, seed=6)
    u8 = lambda t: t.view(torch.uint8).numpy()
    O, L = oracle.attention_fp8_blocked(u8(q8), u8(k8), u8(v8), 0.09, qd, kd, True, 37,
                                        v_descale=vd)
    qf = q8.to(torch.float64).numpy() * qd
    kf = k8.to(torch.float64).numpy() * kd
    vf = v8.to(torch.float64).numpy() * vd
    O2, L2 = oracle.attention_blocked(qf, kf, vf, 0.09, True, 37)
    assert np.max(np.abs(O - O2)) < 1e-12 and np.max(np.abs(L - L2)) < 1e-12


def test_fp8v_descale_scales_output_only():
    """O is linear in the values, so doubling v_descale doubles O and leaves LSE as it is."""
    q8, k8, v8, qd, kd, vd = make_qkv_fp8qkv(1, 2, 1, 30, 45, 128, seed=7)
    u8 = lambda t: t.view(torch.uint8).numpy()
    O1, L1 = oracle.attention_fp8_blocked(u8(q8), u8(k8), u8(v8), 0.1, qd, kd, False, v_descale=vd)
    O2, L2 = oracle.attention_fp8_blocked(u8(q8), u8(k8), u8(v8), 0.1, qd, kd, False, v_descale=2 * vd)
    assert np.max(np.abs(O2 - 2 * O1)) < 1e-12 and np.max(np.abs(L2 - L1)) == 0.0


def test_fp8v_rejects_bad_descale():
    q8, k8, v8, qd, kd, vd = make_qkv_fp8qkv(1, 1, 1, 4, 4, 128, seed=0)
    u8 = lambda t: t.view(torch.uint8).numpy()
    for bad in (0.0, -1.0, math.inf, math.nan):
        with pytest.raises(ValueError):
            oracle.attention_fp8_blocked(u8(q8), u8(k8), u8(v8), 0.1, qd, kd, v_descale=bad)
