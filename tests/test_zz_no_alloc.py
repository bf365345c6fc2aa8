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


SHORT_SHAPES = [
    # B, Hq, Hkv, Sq, Skv, D, input_pos: decoding and short query lengths
    (4, 32, 8, 1, 16384, 128, 16383),   # decoding, GQA 4
    (2, 16, 2, 3, 4099, 128, 4096),     # three queries, ragged cache, GQA 8
    (3, 8, 8, 4, 2500, 64, 2496),       # four queries, MHA, head dim 64
    (1, 12, 2, 2, 700, 128, 698),       # GQA 6 (two heads per workgroup)
]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_noalloc_many_calls_in_a_row(dtype):
    """Twelve calls in a row over four decoding-like shapes (GQA 4, 8 and 6, MHA, head dims
    64 and 128, ragged caches), each bit-identical to fa_fwd_splitkv at the same split count,
    and the last call of each shape within tolerance of the oracle: the shared scratch
    carries nothing from one call into the next."""
    for rep in range(3):
        for i, (B, Hq, Hkv, Sq, Skv, D, pos) in enumerate(SHORT_SHAPES):
            q, k, v = make_qkv(B, Hq, Hkv, Sq, Skv, D, dtype, seed=40 + 7 * rep + i)
            qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
            splits = fa.splitkv_num_splits(B, Hq, Hkv, Sq, Skv, D, True, pos, q.dtype)
            if splits < 2:
                splits = 4
            _say("call", rep, (B, Hq, Hkv, Sq, Skv, D, pos), dtype, "splits", splits)
            out, lse = fa.fa_fwd_splitkv_noalloc(qd, kd, vd, causal=True, input_pos=pos,
                                                 num_splits=splits)
            ref_out, ref_lse = fa.fa_fwd_splitkv(qd, kd, vd, causal=True, input_pos=pos,
                                                 num_splits=splits)
            torch.cuda.synchronize()
            assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), "differs from fa_fwd_splitkv"
            if rep == 2:
                O, L = oracle.attention_blocked(_f64(q), _f64(k), _f64(v), 1.0 / math.sqrt(D), True, pos)
                assert float(np.max(np.abs(_f64(out) - O))) <= TOL_O[q.dtype]
                assert float(np.max(np.abs(_f64(lse) - L))) <= 1e-3


def test_noalloc_graph_replay():
    """The decoding call captured in a HIP graph (what callers that cannot allocate do) and
    replayed four times with new inputs copied in between (eager work and synchronisation
    between replays): every replay equals an eager fa_fwd_splitkv call on the same inputs."""
    B, Hq, Hkv, Sq, Skv, D, pos = SHORT_SHAPES[0]
    splits = fa.splitkv_num_splits(B, Hq, Hkv, Sq, Skv, D, True, pos, torch.bfloat16)
    q, k, v = (t.to(DEV) for t in make_qkv(B, Hq, Hkv, Sq, Skv, D, "bf16", seed=60))
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):   # first call eagerly (symbol lookup), then capture
        fa.fa_fwd_splitkv_noalloc_into(q, k, v, out, lse, num_splits=splits, causal=True,
                                       input_pos=pos)
    torch.cuda.current_stream(DEV).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fa.fa_fwd_splitkv_noalloc_into(q, k, v, out, lse, num_splits=splits, causal=True,
                                       input_pos=pos)
    torch.cuda.synchronize()
    for rep in range(4):
        nq, nk, nv = make_qkv(B, Hq, Hkv, Sq, Skv, D, "bf16", seed=61 + rep)
        q.copy_(nq.to(DEV))
        k.copy_(nk.to(DEV))
        v.copy_(nv.to(DEV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref_out, ref_lse = fa.fa_fwd_splitkv(q, k, v, causal=True, input_pos=pos, num_splits=splits)
        torch.cuda.synchronize()
        _say("graph replay", rep)
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"replay {rep}"
