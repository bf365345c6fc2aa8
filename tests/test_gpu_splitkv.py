"""GPU parity of the split-KV entry point (fa_fwd_splitkv, through the C ABI) against the
fp64 oracle.

The same tolerances as the plain forward pass: max |O - O_oracle| <= 4e-3 (fp16) or
1.6e-2 (bf16), max |LSE - LSE_oracle| <= 1e-3, no NaN or Inf.  Cases cover more ranges
than key tiles (empty ranges), rows with no visible key in some ranges (causal), one
query row against a long cache (decoding), ragged tails, GQA, both head dims, every
compiled configuration, a workspace full of NaN on entry, and the library's own split
choice on the decoding workload.
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
    print("[splitkv]", *a, file=sys.stderr, flush=True)


def _f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def run_split(q, k, v, scale, causal, pos, num_splits, config=-1, poison=True):
    """fa_fwd_splitkv with a workspace that holds NaN on entry (every partial the merge
    reads must have been written by the attention kernel)."""
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    splits = num_splits or fa.splitkv_num_splits(B, Hq, Hkv, Sq, Skv, D, causal, pos, q.dtype, config)
    nbytes = fa.splitkv_workspace_size(B, Hq, Sq, D, splits)
    ws = None
    if nbytes:
        ws = torch.full((nbytes // 4,), float("nan") if poison else 0.0, dtype=torch.float32, device=DEV)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    fa.fa_fwd_splitkv_into(q, k, v, out, lse, ws, num_splits=num_splits, scale=scale, causal=causal,
                           input_pos=pos, config=config)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def check_full(q, k, v, scale, causal, pos, out, lse, what=""):
    O, L = oracle.attention_blocked(_f64(q), _f64(k), _f64(v), scale, causal, pos)
    o, l = _f64(out), _f64(lse)
    assert np.isfinite(o).all() and np.isfinite(l).all(), f"non-finite output {what}"
    eo = float(np.max(np.abs(o - O))) if o.size else 0.0
    el = float(np.max(np.abs(l - L))) if l.size else 0.0
    assert eo <= TOL_O[q.dtype], f"O max abs err {eo:.3e} {what}"
    assert el <= TOL_LSE, f"LSE max abs err {el:.3e} {what}"
    return eo, el


SPLIT_CASES = [
    # B, Hq, Hkv, Sq, Skv, D, causal, pos, split counts
    ((1, 8, 2, 257, 391, 128, True, 134), (2, 3, 7, 64)),   # ragged, GQA 4, offset; 64 > tiles
    ((1, 32, 4, 1, 16384, 128, True, 16383), (0, 4, 256)),   # decoding: one row, long cache
    ((2, 4, 4, 300, 300, 64, True, 0), (2, 5)),              # causal: rows with empty ranges
    ((1, 4, 4, 63, 65, 128, False, 0), (2, 3)),              # ragged key tail in the last range
    ((1, 8, 8, 1, 1, 128, True, 0), (4,)),                   # one key: all ranges but one empty
    ((1, 4, 2, 17, 1, 64, True, 0), (3,)),
    ((3, 6, 3, 129, 64, 64, True, 0), (2,)),                 # Sq > Skv
    ((1, 8, 1, 65, 129, 64, False, 0), (3,)),                # MQA, head dim 64
    ((1, 8, 4, 200, 200, 128, True, 500), (2, 6)),           # every key visible to every row
]


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "x".join(map(str, c[0])))
def test_split_shapes(case, dtype):
    shape, splits = case
    B, Hq, Hkv, Sq, Skv, D, causal, pos = shape
    q, k, v = make_qkv(B, Hq, Hkv, Sq, Skv, D, dtype, seed=sum(shape) + 1)
    scale = 1.0 / math.sqrt(D)
    for s in splits:
        _say("shape", shape, dtype, "splits", s)
        out, lse = run_split(q, k, v, scale, causal, pos, s)
        check_full(q, k, v, scale, causal, pos, out, lse, f"{shape} {dtype} splits={s}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_every_config_split(D, dtype, causal):
    """Every compiled configuration that fits the call, with 3 ranges."""
    q, k, v = make_qkv(1, 16, 2, 333, 333, D, dtype, seed=9)   # GQA 8: every shape applies
    pos = 7 if causal else 0
    tested = 0
    for cid, name in enumerate(fa.config_names()):
        if not name.startswith(f"D{D}_") or "fp8" in name or (("_causal_" in name) != causal) or \
                (("_bf16" in name) != (dtype == "bf16")):
            continue
        _say("config", name)
        if "_KS2_" in name:
            # two key parts run one key range: a forced one with 3 ranges is refused
            with pytest.raises(fa.FaError) as e:
                run_split(q, k, v, 0.09, causal, pos, 3, config=cid)
            assert e.value.code == -10
            continue
        out, lse = run_split(q, k, v, 0.09, causal, pos, 3, config=cid)
        check_full(q, k, v, 0.09, causal, pos, out, lse, name)
        tested += 1
    assert tested == (7 if D == 128 else 6)


def test_one_split_is_the_plain_kernel():
    """num_splits = 1 runs the plain forward kernel: bit-identical to fa_fwd."""
    q, k, v = make_qkv(1, 8, 2, 300, 420, 128, "bf16", seed=3)
    a_out, a_lse = run_split(q, k, v, 0.1, True, 120, 1)
    b_out, b_lse = fa.fa_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=0.1, causal=True, input_pos=120)
    torch.cuda.synchronize()
    assert torch.equal(a_out, b_out.cpu()) and torch.equal(a_lse, b_lse.cpu())


def test_split_deterministic():
    q, k, v = make_qkv(1, 8, 2, 100, 2000, 128, "fp16", seed=4)
    a = run_split(q, k, v, 0.1, True, 1900, 9)
    b = run_split(q, k, v, 0.1, True, 1900, 9, poison=False)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_decode_workload_auto_split():
    """The decoding workload (one query row per sequence, 32 workgroups unsplit) with the
    library's split choice, compared with the oracle on every element."""
    name = "gqa4_decode_b4_kv16384_d128_bf16"
    w = WORKLOADS[name]
    q, k, v, kw = make_workload(name, seed=0)
    s = fa.splitkv_num_splits(w["B"], w["Hq"], w["Hkv"], w["Sq"], w["Skv"], w["D"], kw["causal"],
                              kw["input_pos"], q.dtype)
    _say(name, "auto splits", s)
    assert s > 1
    out, lse = run_split(q, k, v, kw["scale"], kw["causal"], kw["input_pos"], 0)
    check_full(q, k, v, kw["scale"], kw["causal"], kw["input_pos"], out, lse, name)


def test_cross_attention_workload_auto_split():
    """The non-causal cross-attention workload (256 queries, 16K keys; fa_fwd runs it with two
    key parts per workgroup) through fa_fwd_splitkv with the library's split choice, which
    runs the one-part twin over several key ranges: every element against the oracle."""
    name = "gqa4_xattn_q256_kv16384_d128_bf16"
    w = WORKLOADS[name]
    q, k, v, kw = make_workload(name, seed=0)
    names = fa.config_names()
    assert "_KS2_" in names[fa.select_config(w["B"], w["Hq"], w["Hkv"], w["Sq"], w["Skv"], w["D"],
                                             False, 0, q.dtype)]
    s = fa.splitkv_num_splits(w["B"], w["Hq"], w["Hkv"], w["Sq"], w["Skv"], w["D"], False, 0, q.dtype)
    _say(name, "auto splits", s)
    assert s > 1
    out, lse = run_split(q, k, v, kw["scale"], False, 0, 0)
    check_full(q, k, v, kw["scale"], False, 0, out, lse, name)


def test_split_workspace_errors():
    q, k, v = make_qkv(1, 4, 2, 64, 256, 128, "bf16", seed=2)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    need = fa.splitkv_workspace_size(1, 4, 64, 128, 4)
    small = torch.empty(need - 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_splitkv_into(q, k, v, out, lse, small, num_splits=4)
    assert e.value.code == -13
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_splitkv_into(q, k, v, out, lse, None, num_splits=4)
    assert e.value.code == -1
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_splitkv_into(q, k, v, out, lse, None, num_splits=1000)
    assert e.value.code == -12


def test_split_on_side_stream():
    q, k, v = make_qkv(1, 8, 2, 1, 3000, 128, "bf16", seed=6)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    s = torch.cuda.Stream()
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    ws = torch.empty(fa.splitkv_workspace_size(1, 8, 1, 128, 16), dtype=torch.uint8, device=DEV)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        fa.fa_fwd_splitkv_into(q, k, v, out, lse, ws, num_splits=16, scale=0.1, causal=True,
                               input_pos=2999)
    s.synchronize()
    check_full(q.cpu(), k.cpu(), v.cpu(), 0.1, True, 2999, out.cpu(), lse.cpu(), "side stream")
