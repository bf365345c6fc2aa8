"""GPU parity of fa_fwd_fp8 (fp8 E4M3 queries and keys, fp16 / bf16 values) against the
fp64 oracle over the dequantised inputs; the named fp8 workloads include fp8 values too
(fa_fwd_fp8qkv, whose own tests are in test_gpu_fp8qkv.py).

The scores come from exact products of fp8 values accumulated in fp32, so the output
error has the same sources as the fp16 / bf16 path (P and O rounded to the value type) and
the same tolerances apply: max |O - O_oracle| <= 4e-3 (fp16) or 1.6e-2 (bf16), max |LSE -
LSE_oracle| <= 1e-3.
"""

from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import attention_fa_fwd_amd as fa
import oracle
from attention_fa_fwd_amd.inputs import FP8_WORKLOADS, make_fp8_workload, make_qkv_fp8

pytestmark = pytest.mark.gpu

TOL_O = {torch.float16: 4e-3, torch.bfloat16: 1.6e-2}
TOL_LSE = 1e-3
DEV = torch.device("cuda:0")


def _say(*a):
    print("[fp8]", *a, file=sys.stderr, flush=True)


def _codes(t):
    return t.view(torch.uint8).numpy()


def oracle_fp8(q8, k8, v, scale, qd, kd, causal, pos, window=0):
    return oracle.attention_fp8_blocked(_codes(q8), _codes(k8), v.double().numpy(), scale, qd, kd,
                                        causal, pos, window=window)


def run(q8, k8, v, qd, kd, scale, causal, pos, window=0, config=-1):
    out, lse = fa.fa_fwd_fp8(q8.to(DEV), k8.to(DEV), v.to(DEV), qd, kd, scale=scale, causal=causal,
                             input_pos=pos, window=window, config=config)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def check(O, L, out, lse, dtype, what):
    o, l = out.double().numpy(), lse.double().numpy()
    empty = ~np.isfinite(L)
    assert np.all(l[empty] == -np.inf) and np.all(o[empty] == 0.0), what
    assert np.isfinite(o).all() and np.isfinite(l[~empty]).all(), f"non-finite {what}"
    eo = float(np.max(np.abs(o - O))) if o.size else 0.0
    el = float(np.max(np.abs(l[~empty] - L[~empty]))) if (~empty).any() else 0.0
    assert eo <= TOL_O[dtype], f"O max abs err {eo:.3e} {what}"
    assert el <= TOL_LSE, f"LSE max abs err {el:.3e} {what}"


FP8_CASES = [
    # B, Hq, Hkv, Sq, Skv, causal, pos, window
    (1, 2, 2, 128, 128, False, 0, 0),
    (2, 4, 4, 300, 300, True, 0, 0),          # several tiles + ragged tail
    (1, 8, 2, 257, 391, True, 134, 0),        # ragged both, GQA 4, offset
    (1, 8, 1, 65, 129, False, 0, 0),          # MQA
    (1, 8, 8, 1, 1, True, 0, 0),              # one query, one key
    (1, 4, 4, 1, 700, True, 699, 0),          # decode-like row
    (1, 8, 2, 300, 300, True, 0, 45),         # sliding window
    (1, 32, 4, 256, 256, True, 0, 0),
]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("vdt", ["fp16", "bf16"])
@pytest.mark.parametrize("case", FP8_CASES, ids=lambda c: "x".join(map(str, c)))
def test_fp8_shapes(case, vdt, D):
    B, Hq, Hkv, Sq, Skv, causal, pos, W = case
    _say(case, vdt, D)
    q8, k8, v, qd, kd = make_qkv_fp8(B, Hq, Hkv, Sq, Skv, D, vdt, seed=sum(case) + 7 + D)
    scale = 1.0 / math.sqrt(D)
    out, lse = run(q8, k8, v, qd, kd, scale, causal, pos, W)
    O, L = oracle_fp8(q8, k8, v, scale, qd, kd, causal, pos, W)
    check(O, L, out, lse, v.dtype, f"{case} {vdt} D{D}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("vdt", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_every_config(vdt, causal, D):
    """Every compiled fp8 configuration of the head dim (seven shapes at 128, six at 64),
    forced on one GQA-8 input."""
    q8, k8, v, qd, kd = make_qkv_fp8(1, 16, 2, 333, 333, D, vdt, seed=21)   # GQA 8: every shape applies
    pos = 7 if causal else 0
    O, L = oracle_fp8(q8, k8, v, 0.09, qd, kd, causal, pos)
    tested = 0
    for cid, name in enumerate(fa.config_names()):
        if "_fp8qk_" not in name or (("_causal_" in name) != causal) or not name.endswith(vdt):
            continue
        if not name.startswith(f"D{D}_"):
            continue
        _say("config", name)
        out, lse = run(q8, k8, v, qd, kd, 0.09, causal, pos, config=cid)
        check(O, L, out, lse, v.dtype, name)
        tested += 1
    assert tested == (7 if D == 128 else 6)


def test_fp8_descale_invariance():
    """Moving a factor of 2 from scale into q_descale gives bit-identical results (the
    kernel folds both into one fp32 constant computed in double)."""
    q8, k8, v, qd, kd = make_qkv_fp8(1, 8, 2, 200, 200, 128, "bf16", seed=22)
    a = run(q8, k8, v, qd, kd, 0.1, True, 0)
    b = run(q8, k8, v, qd * 2, kd, 0.05, True, 0)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("name", sorted(FP8_WORKLOADS))
def test_fp8_named_workload(name):
    """Full-size fp8 workloads (fp8 queries and keys; with "fp8v", fp8 values too) in the
    dispatch table's configuration: every element of O and LSE against the oracle."""
    w = FP8_WORKLOADS[name]
    _say("workload", name)
    q8, k8, v, kw = make_fp8_workload(name, seed=0)
    if w.get("fp8v"):
        out, lse = fa.fa_fwd_fp8qkv(q8.to(DEV), k8.to(DEV), v.to(DEV), kw["q_descale"], kw["k_descale"],
                                    kw["v_descale"], out_dtype=torch.bfloat16, scale=kw["scale"],
                                    causal=kw["causal"], input_pos=kw["input_pos"])
        torch.cuda.synchronize()
        out, lse = out.cpu(), lse.cpu()
        O, L = oracle.attention_fp8_blocked(_codes(q8), _codes(k8), _codes(v), kw["scale"],
                                            kw["q_descale"], kw["k_descale"], kw["causal"],
                                            kw["input_pos"], v_descale=kw["v_descale"])
        dt = torch.bfloat16
    else:
        out, lse = run(q8, k8, v, kw["q_descale"], kw["k_descale"], kw["scale"], kw["causal"],
                       kw["input_pos"], kw["window"])
        O, L = oracle_fp8(q8, k8, v, kw["scale"], kw["q_descale"], kw["k_descale"], kw["causal"],
                          kw["input_pos"])
        dt = v.dtype
    check(O, L, out, lse, dt, name)


FP8_SPLIT_CASES = [
    # B, Hq, Hkv, Sq, Skv, input_pos, window, num_splits (0 = the library's choice)
    (2, 8, 2, 1, 3000, 2999, 0, 0),       # decoding rows
    (2, 8, 2, 1, 3000, 2999, 0, 5),
    (1, 8, 2, 130, 2000, 1870, 0, 3),     # a chunk of queries against a cache
    (1, 8, 2, 130, 2000, 1870, 300, 16),  # with a sliding window
    (1, 4, 4, 64, 333, 0, 0, 2),          # causal from 0, ragged key tail
]


def run_split(q8, k8, v, qd, kd, scale, pos, W, splits):
    out, lse = fa.fa_fwd_splitkv_fp8(q8.to(DEV), k8.to(DEV), v.to(DEV), qd, kd, scale=scale,
                                     causal=True, input_pos=pos, num_splits=splits, window=W)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("vdt", ["fp16", "bf16"])
@pytest.mark.parametrize("case", FP8_SPLIT_CASES, ids=lambda c: "x".join(map(str, c)))
def test_fp8_splitkv_shapes(case, vdt, D):
    """fa_fwd_splitkv_fp8: fp8 queries and keys over split key ranges, merged."""
    B, Hq, Hkv, Sq, Skv, pos, W, splits = case
    _say("splitkv", case, vdt, D)
    q8, k8, v, qd, kd = make_qkv_fp8(B, Hq, Hkv, Sq, Skv, D, vdt, seed=(sum(case) + D) % 97)
    scale = 1.0 / math.sqrt(D)
    out, lse = run_split(q8, k8, v, qd, kd, scale, pos, W, splits)
    O, L = oracle_fp8(q8, k8, v, scale, qd, kd, True, pos, W)
    check(O, L, out, lse, v.dtype, f"{case} {vdt} D{D}")


def test_fp8_splitkv_one_split_is_fa_fwd_fp8():
    """One split runs the plain kernel: bit-identical to fa_fwd_fp8."""
    q8, k8, v, qd, kd = make_qkv_fp8(1, 8, 2, 100, 700, 128, "bf16", seed=23)
    a = run_split(q8, k8, v, qd, kd, 0.09, 600, 0, 1)
    b = run(q8, k8, v, qd, kd, 0.09, True, 600)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_fp8_splitkv_decode_workload():
    """The fp8 decoding workload (B=4, GQA 4, one query row against 16384 fp8 keys) in the
    launch configuration bench.py times (the library's split count), every output row."""
    name = "gqa4_decode_b4_kv16384_d128_fp8qk_bf16"
    _say("workload", name)
    q8, k8, v, kw = make_fp8_workload(name, seed=0)
    w = FP8_WORKLOADS[name]
    splits = fa.splitkv_num_splits_fp8(w["B"], w["Hq"], w["Hkv"], w["Sq"], w["Skv"], w["D"], True,
                                       kw["input_pos"], v.dtype)
    assert splits > 1
    out, lse = run_split(q8, k8, v, kw["q_descale"], kw["k_descale"], kw["scale"], kw["input_pos"],
                         0, splits)
    O, L = oracle_fp8(q8, k8, v, kw["scale"], kw["q_descale"], kw["k_descale"], True,
                      kw["input_pos"])
    check(O, L, out, lse, v.dtype, name)

