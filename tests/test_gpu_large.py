"""GPU parity at tensor sizes past 2^31 elements (byte offsets past 4 GiB).

Index arithmetic that overflows 32 bits would show up here first: each case puts one tensor
past 2^31 elements and checks rows whose offsets lie beyond that boundary against the fp64
oracle.  The large tensors are drawn on the GPU by torch's seeded generator (N(0,1), rounded
to bf16); only the rows an oracle needs are copied back.  The cases stay cheap by making the
other dimension small: a long query tensor against 100 keys, or a long key / value cache
seen through a sliding window of a few dozen keys, so the oracle needs only a key slice.

Tolerances as everywhere: O <= 1.6e-2 (bf16), LSE <= 1e-3, gradients as in
test_gpu_backward.py.  About 20 GiB of device memory.
"""

from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import attention_fa_fwd_amd as fa
import oracle

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
D = 128
BIG = 1 << 31


def _say(*a):
    print("[large]", *a, file=sys.stderr, flush=True)


def _randn(shape, seed):
    """Seeded N(0,1) drawn on the GPU, rounded to bf16; one head at a time to bound the fp32
    temporary."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    out = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
    for b in range(shape[0]):
        for h in range(shape[1]):
            out[b, h] = torch.randn(shape[2:], generator=g, device=DEV, dtype=torch.float32).to(torch.bfloat16)
    return out


def _f64(t):
    return t.detach().cpu().double().numpy()


def _check(o_gpu, l_gpu, O, L, what):
    eo = float(np.max(np.abs(_f64(o_gpu) - O)))
    el = float(np.max(np.abs(_f64(l_gpu) - L)))
    assert eo <= 1.6e-2, f"O err {eo:.3e} {what}"
    assert el <= 1e-3, f"LSE err {el:.3e} {what}"


def test_long_query_tensor():
    """q and out of 2 x (2^23 + 37) x 128 elements (> 2^31); 100 keys, causal, input_pos 60.
    Rows checked: the first of head 0, rows astride element offset 2^31 and the last rows."""
    Sq, Skv, pos, scale = (1 << 23) + 37, 100, 60, 1.0 / math.sqrt(D)
    assert 2 * Sq * D > BIG
    _say("fa_fwd", (1, 2, 1, Sq, Skv, D), "bf16 causal pos", pos)
    q = _randn((1, 2, Sq, D), 11)
    k = _randn((1, 1, Skv, D), 12)
    v = _randn((1, 1, Skv, D), 13)
    out, lse = fa.fa_fwd(q, k, v, scale=scale, causal=True, input_pos=pos)
    torch.cuda.synchronize()
    kc, vc = _f64(k), _f64(v)
    r_boundary = BIG // D - Sq          # head-1 row whose first element sits at offset 2^31
    for h, r0, n in [(0, 0, 32), (1, r_boundary - 16, 32), (1, Sq - 40, 40)]:
        O, L = oracle.attention_blocked(_f64(q[:, h:h + 1, r0:r0 + n]), kc, vc, scale, True, pos + r0)
        _check(out[:, h:h + 1, r0:r0 + n], lse[:, h:h + 1, r0:r0 + n], O, L, (h, r0, n))


def test_key_range_past_1gib_of_one_workgroup():
    """A query tile whose key range holds more than 2^30 bytes of K and of V: 40 rows of two
    query heads against (2^22 + 12345) keys (1.08 GB of K, as much of V), non-causal and causal
    with the last row on the last key (input_pos = Skv - Sq).  The kernel addresses a range's
    tiles from one buffer resource and moves it up once 2^30 bytes of the range have been
    streamed (here after 131073 of its 131458 key tiles); every element is compared with the
    oracle."""
    Hq, Sq, Skv, scale = 2, 40, (1 << 22) + 12345, 1.0 / math.sqrt(D)
    assert Skv * D * 2 > (1 << 30)
    _say("fa_fwd long key range", (1, Hq, 1, Sq, Skv, D), "bf16")
    q = _randn((1, Hq, Sq, D), 41)
    k = _randn((1, 1, Skv, D), 42)
    v = _randn((1, 1, Skv, D), 43)
    qd, kd, vd = _f64(q), _f64(k), _f64(v)
    for causal, pos in ((False, 0), (True, Skv - Sq)):
        O, L = oracle.attention_blocked(qd, kd, vd, scale, causal, pos)
        out, lse = fa.fa_fwd(q, k, v, scale=scale, causal=causal, input_pos=pos)
        torch.cuda.synchronize()
        _check(out, lse, O, L, f"causal={causal}")


def _window_case(Hq, Sq, Skv, W, seed):
    pos = Skv - Sq
    q = _randn((1, Hq, Sq, D), seed)
    k = _randn((1, 1, Skv, D), seed + 1)
    v = _randn((1, 1, Skv, D), seed + 2)
    lo = pos - W + 1                    # first key any row can see
    return q, k, v, pos, lo


def test_long_cache_window_forward():
    """k and v of (2^24 + 51) x 128 elements (> 2^31) seen through a 64-key window by 40 rows
    at the end of the cache (input_pos = Skv - Sq): fa_fwd_window and fa_fwd_splitkv."""
    Hq, Sq, Skv, W, scale = 4, 40, (1 << 24) + 51, 64, 0.09
    assert Skv * D > BIG
    _say("fa_fwd_window / fa_fwd_splitkv", (1, Hq, 1, Sq, Skv, D), "bf16 window", W)
    q, k, v, pos, lo = _window_case(Hq, Sq, Skv, W, 21)
    O, L = oracle.attention_blocked(_f64(q), _f64(k[:, :, lo:]), _f64(v[:, :, lo:]), scale, True,
                                    pos - lo, window=W)
    out, lse = fa.fa_fwd(q, k, v, scale=scale, causal=True, input_pos=pos, window=W)
    torch.cuda.synchronize()
    _check(out, lse, O, L, "fa_fwd_window")
    for splits in (0, 3):
        out, lse = fa.fa_fwd_splitkv(q, k, v, scale=scale, causal=True, input_pos=pos,
                                     num_splits=splits, window=W)
        torch.cuda.synchronize()
        _check(out, lse, O, L, f"fa_fwd_splitkv {splits}")


def test_long_cache_window_backward():
    """Gradients with k, v, dk, dv past 2^31 elements: 48 rows at the end of a (2^24 + 77)-key
    cache through a 96-key window.  dk and dv are checked on the visible key slice against
    the oracle (keys past row 2^24, i.e. past element 2^31, are among them) and are exactly
    zero on keys no query sees (sampled rows)."""
    Hq, Sq, Skv, W, scale = 2, 48, (1 << 24) + 77, 96, 1.0 / math.sqrt(D)
    assert Skv * D > BIG
    _say("fa_bwd", (1, Hq, 1, Sq, Skv, D), "bf16 window", W)
    q, k, v, pos, lo = _window_case(Hq, Sq, Skv, W, 31)
    g = torch.Generator(device="cpu")
    g.manual_seed(32)
    do = torch.randn((1, Hq, Sq, D), generator=g).to(torch.bfloat16).to(DEV)
    out, lse = fa.fa_fwd(q, k, v, scale=scale, causal=True, input_pos=pos, window=W)
    dq, dk, dv = fa.fa_bwd(q, k, v, out, lse, do, scale=scale, causal=True, input_pos=pos, window=W)
    torch.cuda.synchronize()
    ref = oracle.attention_backward_blocked(_f64(q), _f64(k[:, :, lo:]), _f64(v[:, :, lo:]), _f64(do),
                                            scale, True, pos - lo, W)
    got = (dq, dk[:, :, lo:], dv[:, :, lo:])
    top = max(float(np.max(np.abs(r))) for r in ref)
    for name, gv, r in zip(("dq", "dk", "dv"), got, ref):
        gd = _f64(gv)
        err = float(np.max(np.abs(gd - r)))
        bound = 1.6e-2 * max(float(np.max(np.abs(r))), 0.05 * top)
        assert err <= bound, f"{name} err {err:.3e} > {bound:.3e}"
    assert lo < BIG // D < Skv
    for r0 in (0, 1 << 23, lo - 128):
        for t in (dk, dv):
            assert torch.count_nonzero(t[:, :, r0:r0 + 64]).item() == 0, r0
