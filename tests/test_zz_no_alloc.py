"""GPU test of fa_fwd_splitkv_noalloc, the split-KV entry point without a workspace argument
(its partials live in the library's fixed per-GPU scratch), called through the C ABI.

Two calls in a row, the second on a smaller problem, each compared with fa_fwd_splitkv (the
entry point with a caller-owned workspace) at the same split count and configuration --
the same kernels, so the results must be bit-identical -- and with the fp64 oracle within
the forward tolerances (O: 4e-3 fp16, 1.6e-2 bf16; LSE: 1e-3).
"""

from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import attention_fa_fwd_amd as fa
import oracle
from attention_fa_fwd_amd.inputs import make_qkv

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TOL_O = {torch.float16: 4e-3, torch.bfloat16: 1.6e-2}


def _say(*a):
    print("[noalloc]", *a, file=sys.stderr, flush=True)


def _f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _one_call(shape, dtype, num_splits, seed):
    B, Hq, Hkv, Sq, Skv, D, pos = shape
    q, k, v = make_qkv(B, Hq, Hkv, Sq, Skv, D, dtype, seed=seed)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    splits = num_splits or fa.splitkv_num_splits(B, Hq, Hkv, Sq, Skv, D, True, pos, q.dtype)
    assert splits > 1
    assert fa.splitkv_workspace_size(B, Hq, Sq, D, splits) <= fa.NOALLOC_SCRATCH_BYTES
    _say("shape", shape, dtype, "splits", splits)
    out, lse = fa.fa_fwd_splitkv_noalloc(qd, kd, vd, causal=True, input_pos=pos, num_splits=num_splits)
    ref_out, ref_lse = fa.fa_fwd_splitkv(qd, kd, vd, causal=True, input_pos=pos, num_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), "differs from fa_fwd_splitkv"
    O, L = oracle.attention_blocked(_f64(q), _f64(k), _f64(v), 1.0 / math.sqrt(D), True, pos)
    eo = float(np.max(np.abs(_f64(out) - O)))
    el = float(np.max(np.abs(_f64(lse) - L)))
    _say(f"O err {eo:.2e} LSE err {el:.2e}")
    assert eo <= TOL_O[q.dtype] and el <= 1e-3


def test_noalloc_two_calls_second_smaller():
    # the decoding shape (one query per sequence, 16K cache), the library's split count
    _one_call((4, 32, 8, 1, 16384, 128, 16383), "bf16", 0, seed=21)
    # then a smaller problem with a ragged tail and another head dim, 5 ranges
    _one_call((1, 8, 2, 37, 3000, 64, 2963), "fp16", 5, seed=22)


def test_noalloc_rejects_partials_beyond_the_scratch():
    q, k, v = make_qkv(1, 32, 32, 4096, 4096, 128, "bf16", seed=23)
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_splitkv_noalloc(q.to(DEV), k.to(DEV), v.to(DEV), num_splits=2)
    assert e.value.code == -15
