"""GPU parity of fa_fwd_fp8qkv and fa_fwd_splitkv_fp8qkv (fp8 E4M3 queries, keys and values,
fp16 / bf16 output) against the fp64 oracle over the dequantised inputs.

Q K^T is exact in fp8 x fp8 -> fp32; every E4M3 value widens exactly to bf16 / fp16, so
P V has the error sources of the fp16 / bf16 path (P rounded to the output type, O rounded
once) and the same tolerances apply: max |O - O_oracle| <= 4e-3 (fp16) or 1.6e-2 (bf16),
max |LSE - LSE_oracle| <= 1e-3.  The fp8 rounding of the inputs is part of the problem:
the oracle decodes the very codes the kernels read.
"""

from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import attention_fa_fwd_amd as fa
import oracle
from attention_fa_fwd_amd.inputs import FP8_WORKLOADS, make_fp8_workload, make_qkv_fp8qkv

pytestmark = pytest.mark.gpu

TOL_O = {torch.float16: 4e-3, torch.bfloat16: 1.6e-2}
TOL_LSE = 1e-3
DEV = torch.device("cuda:0")
DT = {"fp16": torch.float16, "bf16": torch.bfloat16}


def _say(*a):
    print("[fp8qkv]", *a, file=sys.stderr, flush=True)


def _codes(t):
    return t.view(torch.uint8).numpy()


def oracle_qkv(q8, k8, v8, scale, qd, kd, vd, causal, pos, window=0):
    return oracle.attention_fp8_blocked(_codes(q8), _codes(k8), _codes(v8), scale, qd, kd, causal,
                                        pos, window=window, v_descale=vd)


def run(q8, k8, v8, qd, kd, vd, dt, scale, causal, pos, window=0, config=-1):
    out, lse = fa.fa_fwd_fp8qkv(q8.to(DEV), k8.to(DEV), v8.to(DEV), qd, kd, vd, out_dtype=dt,
                                scale=scale, causal=causal, input_pos=pos, window=window,
                                config=config)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def run_split(q8, k8, v8, qd, kd, vd, dt, scale, pos, window, splits):
    out, lse = fa.fa_fwd_splitkv_fp8qkv(q8.to(DEV), k8.to(DEV), v8.to(DEV), qd, kd, vd, out_dtype=dt,
                                        scale=scale, causal=True, input_pos=pos, num_splits=splits,
                                        window=window)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def check(O, L, out, lse, dtype, what):
    o, l = out.double().numpy(), lse.double().numpy()
    empty = ~np.isfinite(L)
    assert np.all(l[empty] == -np.inf) and np.all(o[empty] == 0.0), what
    assert np.isfinite(o).all() and np.isfinite(l[~empty]).all(), f"non-finite {what}"
    eo = float(np.max(np.abs(o - O))) if o.size else 0.0
    el = float(np.max(np.abs(l[~empty] - L[~empty]))) if (~empty).any() else 0.0
    _say(what, f"O err {eo:.2e} LSE err {el:.2e}")
    assert eo <= TOL_O[dtype], f"O max abs err {eo:.3e} {what}"
    assert el <= TOL_LSE, f"LSE max abs err {el:.3e} {what}"


CASES = [
    # B, Hq, Hkv, Sq, Skv, causal, pos, window
    (1, 2, 2, 128, 128, False, 0, 0),
    (2, 4, 4, 300, 300, True, 0, 0),          # several tiles + ragged tail
    (1, 8, 2, 257, 391, True, 134, 0),        # ragged both, GQA 4, offset
    (1, 8, 1, 65, 129, False, 0, 0),          # MQA
    (1, 8, 8, 1, 1, True, 0, 0),              # one query, one key
    (1, 4, 4, 1, 700, True, 699, 0),          # decode-like row
    (1, 8, 2, 300, 300, True, 0, 45),         # sliding window
    (1, 32, 4, 256, 256, True, 0, 0),
    (1, 6, 2, 200, 300, True, 40, 0),         # GQA 3
]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("odt", ["fp16", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_fp8qkv_shapes(case, odt, D):
    B, Hq, Hkv, Sq, Skv, causal, pos, W = case
    _say(case, odt, D)
    q8, k8, v8, qd, kd, vd = make_qkv_fp8qkv(B, Hq, Hkv, Sq, Skv, D, seed=sum(case) + 11 + D)
    scale = 1.0 / math.sqrt(D)
    out, lse = run(q8, k8, v8, qd, kd, vd, DT[odt], scale, causal, pos, W)
    O, L = oracle_qkv(q8, k8, v8, scale, qd, kd, vd, causal, pos, W)
    check(O, L, out, lse, DT[odt], f"{case} {odt} D{D}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("odt", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8qkv_every_config(odt, causal, D):
    """Every compiled fp8 Q/K/V configuration of the head dim (seven shapes at 128, six at
    64, per output type and causality), forced on one GQA-8 input."""
    q8, k8, v8, qd, kd, vd = make_qkv_fp8qkv(1, 16, 2, 333, 333, D, seed=31)
    pos = 7 if causal else 0
    O, L = oracle_qkv(q8, k8, v8, 0.09, qd, kd, vd, causal, pos)
    tested = 0
    for cid, name in enumerate(fa.config_names()):
        if "_fp8qkv_" not in name or (("_causal_" in name) != causal) or not name.endswith(odt):
            continue
        if not name.startswith(f"D{D}_"):
            continue
        _say("config", name)
        out, lse = run(q8, k8, v8, qd, kd, vd, DT[odt], 0.09, causal, pos, config=cid)
        check(O, L, out, lse, DT[odt], name)
        tested += 1
    assert tested == (7 if D == 128 else 6)


def test_fp8qkv_v_descale_doubles_output_exactly():
    """v_descale is applied to the fp32 result before rounding: doubling it doubles O bit for
    bit (a power of two) and leaves LSE unchanged."""
    q8, k8, v8, qd, kd, vd = make_qkv_fp8qkv(1, 8, 2, 200, 260, 128, seed=32)
    a = run(q8, k8, v8, qd, kd, vd, torch.bfloat16, 0.1, True, 60)
    b = run(q8, k8, v8, qd, kd, 2 * vd, torch.bfloat16, 0.1, True, 60)
    assert torch.equal(b[0], a[0] * 2) and torch.equal(a[1], b[1])


SPLIT_CASES = [
    # B, Hq, Hkv, Sq, Skv, input_pos, window, num_splits (0 = the library's choice)
    (2, 8, 2, 1, 3000, 2999, 0, 0),       # decoding rows
    (2, 8, 2, 1, 3000, 2999, 0, 5),
    (1, 8, 2, 130, 2000, 1870, 0, 3),     # a chunk of queries against a cache
    (1, 8, 2, 130, 2000, 1870, 300, 16),  # with a sliding window
    (1, 4, 4, 64, 333, 0, 0, 2),          # causal from 0, ragged key tail
]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("odt", ["fp16", "bf16"])
@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "x".join(map(str, c)))
def test_fp8qkv_splitkv_shapes(case, odt, D):
    B, Hq, Hkv, Sq, Skv, pos, W, splits = case
    _say("split", case, odt, D)
    q8, k8, v8, qd, kd, vd = make_qkv_fp8qkv(B, Hq, Hkv, Sq, Skv, D, seed=(sum(case) + D) % 89)
    scale = 1.0 / math.sqrt(D)
    out, lse = run_split(q8, k8, v8, qd, kd, vd, DT[odt], scale, pos, W, splits)
    O, L = oracle_qkv(q8, k8, v8, scale, qd, kd, vd, True, pos, W)
    check(O, L, out, lse, DT[odt], f"split {case} {odt} D{D}")


def test_fp8qkv_splitkv_one_split_is_fa_fwd_fp8qkv():
    q8, k8, v8, qd, kd, vd = make_qkv_fp8qkv(1, 8, 2, 100, 700, 128, seed=33)
    a = run_split(q8, k8, v8, qd, kd, vd, torch.bfloat16, 0.09, 600, 0, 1)
    b = run(q8, k8, v8, qd, kd, vd, torch.bfloat16, 0.09, True, 600)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_fp8qkv_decode_workload_library_split():
    """Decoding against an fp8 K/V cache (B=4, GQA 4, one query row against 16384 keys) in the
    launch configuration bench.py times (the library's split count): every output row."""
    name = "gqa4_decode_b4_kv16384_d128_fp8qkv_bf16"
    w = FP8_WORKLOADS[name]
    q8, k8, v8, kw = make_fp8_workload(name, seed=0)
    splits = fa.splitkv_num_splits_fp8qkv(w["B"], w["Hq"], w["Hkv"], w["Sq"], w["Skv"], w["D"], True,
                                          kw["input_pos"], torch.bfloat16)
    assert splits > 1
    out, lse = run_split(q8, k8, v8, kw["q_descale"], kw["k_descale"], kw["v_descale"],
                         torch.bfloat16, kw["scale"], kw["input_pos"], 0, splits)
    O, L = oracle_qkv(q8, k8, v8, kw["scale"], kw["q_descale"], kw["k_descale"], kw["v_descale"],
                      True, kw["input_pos"])
    check(O, L, out, lse, torch.bfloat16, f"{name} splits={splits}")


def test_fp8qkv_rejects_bad_arguments():
    q8, k8, v8, qd, kd, vd = make_qkv_fp8qkv(1, 2, 2, 8, 8, 128, seed=34)
    q8, k8, v8 = q8.to(DEV), k8.to(DEV), v8.to(DEV)
    for bad in (0.0, -1.0, math.inf, math.nan):
        with pytest.raises(fa.FaError) as e:
            fa.fa_fwd_fp8qkv(q8, k8, v8, qd, kd, bad)
        assert e.value.code == -6
    q96 = torch.zeros(1, 2, 8, 96, dtype=torch.float8_e4m3fn, device=DEV)
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_fp8qkv(q96, q96, q96, 1.0, 1.0, 1.0)
    assert e.value.code == -4
