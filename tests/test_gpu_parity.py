"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle.

Tolerances: max |O_gpu - O_oracle| <= 4e-3 (fp16) or 1.6e-2 (bf16); max |LSE_gpu -
LSE_oracle| <= 1e-3; no NaN or Inf.  Every comparison is element by element: small
shapes, every compiled configuration forced on one input, and the named full-size
workloads for seeds 0, 1 and 2, in the configuration the dispatch picks (the one the
benchmark times).
"""

from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import attention_fa_fwd_amd as fa
import oracle
from attention_fa_fwd_amd.inputs import WORKLOADS, make_qkv, make_rising_scores, make_workload

pytestmark = pytest.mark.gpu

TOL_O = {torch.float16: 4e-3, torch.bfloat16: 1.6e-2}
TOL_LSE = 1e-3
DT = {"fp16": torch.float16, "bf16": torch.bfloat16}


def _say(*a):
    print("[parity]", *a, file=sys.stderr, flush=True)


def _f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def run_gpu(q, k, v, scale, causal, pos, config=-1, window=0):
    dev = torch.device("cuda:0")
    out, lse = fa.fa_fwd(q.to(dev), k.to(dev), v.to(dev), scale=scale, causal=causal,
                         input_pos=pos, config=config, window=window)
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


SMALL = [
    # B, Hq, Hkv, Sq, Skv, D, causal, pos
    (1, 2, 2, 128, 128, 64, False, 0),
    (1, 2, 2, 128, 128, 64, True, 0),
    (2, 4, 4, 300, 300, 128, True, 0),        # several tiles + ragged tail
    (1, 8, 2, 257, 391, 128, True, 134),      # ragged both, GQA 4, offset
    (1, 8, 1, 65, 129, 64, False, 0),         # MQA
    (1, 8, 8, 1, 1, 128, True, 0),            # single query, single key
    (1, 4, 4, 1, 700, 128, True, 699),        # decode-like row, full visibility
    (1, 4, 2, 17, 1, 64, True, 0),            # one key for every row
    (1, 4, 4, 63, 65, 128, False, 0),
    (1, 8, 4, 200, 200, 128, True, 500),      # input_pos + i beyond Skv: all keys visible
    (3, 6, 3, 129, 64, 64, True, 0),          # Sq > Skv
    (1, 32, 4, 256, 256, 128, True, 0),
    (1, 6, 2, 200, 300, 128, True, 40),       # GQA 3: odd group, one head per wave group
    (1, 10, 2, 100, 180, 128, False, 0),      # GQA 5
    (2, 12, 2, 150, 150, 64, True, 0),        # GQA 6: pairs of heads per workgroup
    (1, 24, 2, 96, 160, 128, True, 64),       # GQA 12: four heads per workgroup, three groups
    (1, 14, 2, 70, 70, 128, True, 0),         # GQA 7
]


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_small_shapes(shape, dtype):
    B, Hq, Hkv, Sq, Skv, D, causal, pos = shape
    _say("small", shape, dtype)
    q, k, v = make_qkv(B, Hq, Hkv, Sq, Skv, D, dtype, seed=sum(shape))
    scale = 1.0 / math.sqrt(D)
    out, lse = run_gpu(q, k, v, scale, causal, pos)
    check_full(q, k, v, scale, causal, pos, out, lse, f"{shape} {dtype}")


def forced_configs(D, dtype, causal):
    """(id, name) of every compiled fp16 / bf16 configuration for head dim D, dtype and
    causality (the fp8 ones have their own tests)."""
    out = []
    for cid, name in enumerate(fa.config_names()):
        if not name.startswith(f"D{D}_") or "fp8" in name:
            continue
        if ("_causal_" in name) != causal or (("_bf16" in name) != (dtype == "bf16")):
            continue
        out.append((cid, name))
    return out


# Compiled shapes per head dim: 7 for head dim 128 (32-key tiles), 6 for head dim 64
# (64-key tiles), among them the eight-wave ones the dispatch takes for large grids; the
# non-causal lists add the three two-key-part ("KS2") shapes.
N_SHAPES = {128: 7, 64: 6}
N_KS2 = 3

# Key lengths with a ragged last tile and an even number of tiles (32-key tiles for head dim
# 128, 64-key tiles for head dim 64), so the two-key-part configurations apply.
SKV_EVEN_TILES = {128: 300, 64: 333}


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_every_config_on_same_input(D, dtype, causal):
    """Every compiled configuration that fits the call agrees with the oracle."""
    skv = 333 if causal else SKV_EVEN_TILES[D]
    q, k, v = make_qkv(1, 16, 2, 333, skv, D, dtype, seed=5)   # GQA 8: every shape applies
    pos = 7 if causal else 0
    configs = forced_configs(D, dtype, causal)
    assert len(configs) == N_SHAPES[D] + (0 if causal else N_KS2)
    for cid, name in configs:
        _say("config", name)
        out, lse = run_gpu(q, k, v, 0.09, causal, pos, config=cid)
        check_full(q, k, v, 0.09, causal, pos, out, lse, name)


# The eight-wave head-dim-64 configurations are taken by the dispatch for these full-size
# workloads (grids of at least 256 workgroups).
D64_EIGHT_WAVE = {
    "mha_causal_s4096_d64_fp16": "D64_BN64_Mw1x32_WPH8_HPW1_causal_fp16",
    "gqa4_causal_s4096_d64_bf16": "D64_BN64_Mw1x32_WPH2_HPW4_causal_bf16",
    "gqa2_s2048_d64_fp16": "D64_BN64_Mw1x32_WPH4_HPW2_full_fp16",
}


def test_dispatch_takes_the_eight_wave_head_dim_64_configs():
    names = fa.config_names()
    for name, want in D64_EIGHT_WAVE.items():
        w = WORKLOADS[name]
        cid = fa.select_config(w["B"], w["Hq"], w["Hkv"], w["Sq"], w["Skv"], w["D"], w["causal"],
                               w["input_pos"], DT[w["dtype"]])
        assert names[cid] == want, (name, names[cid])


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_named_workload(name, seed):
    """Full-size workloads in the dispatch table's configuration: every element of O and
    LSE against the oracle."""
    _say("workload", name, "seed", seed)
    q, k, v, kw = make_workload(name, seed=seed)
    out, lse = run_gpu(q, k, v, kw["scale"], kw["causal"], kw["input_pos"], window=kw["window"])
    O, L = oracle.attention_blocked(_f64(q), _f64(k), _f64(v), kw["scale"], kw["causal"],
                                    kw["input_pos"], window=kw["window"])
    o, l = _f64(out), _f64(lse)
    assert np.isfinite(o).all() and np.isfinite(l).all(), f"non-finite output {name}"
    err_o, err_l = np.abs(o - O), np.abs(l - L)
    eo, el = float(err_o.max()), float(err_l.max())
    at = np.unravel_index(int(err_o.argmax()), err_o.shape)
    _say(f"{name} seed {seed}: O max {eo:.3e} mean {float(err_o.mean()):.3e} at {tuple(map(int, at))}; "
         f"LSE max {el:.3e} mean {float(err_l.mean()):.3e}")
    assert eo <= TOL_O[q.dtype], f"{name} seed {seed}: O max abs err {eo:.3e} at {at}"
    assert el <= TOL_LSE, f"{name} seed {seed}: LSE max abs err {el:.3e}"


def test_causal_row0_is_exact():
    """Query 0 sees only key 0: P = 1, l = 1, so O_0 = V_0 bit for bit."""
    for dtype in ("fp16", "bf16"):
        q, k, v = make_qkv(2, 8, 4, 100, 100, 128, dtype, seed=11)
        out, lse = run_gpu(q, k, v, 0.1, True, 0)
        G = 2
        for h in range(8):
            assert torch.equal(out[:, h, 0], v[:, h // G, 0])
            want = 0.1 * (q[:, h, 0].double() * k[:, h // G, 0].double()).sum(-1)
            assert torch.allclose(lse[:, h, 0].double(), want, atol=1e-4, rtol=0)


def test_constant_keys_give_mean_of_values():
    q, k, v = make_qkv(1, 4, 4, 150, 150, 64, "bf16", seed=12)
    k[:] = k[:, :, :1]
    out, _ = run_gpu(q, k, v, 0.125, True, 0)
    csum = torch.cumsum(v.double(), dim=2)
    mean = csum / torch.arange(1, 151, dtype=torch.float64)[None, None, :, None]
    assert float((out.double() - mean).abs().max()) <= TOL_O[torch.bfloat16]


def test_repeated_launches_bitwise_identical():
    q, k, v = make_qkv(1, 32, 4, 1000, 1000, 128, "bf16", seed=13)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    ref = fa.fa_fwd(qd, kd, vd, causal=True)
    for _ in range(3):
        o, l = fa.fa_fwd(qd, kd, vd, causal=True)
        assert torch.equal(o, ref[0]) and torch.equal(l, ref[1])


def test_prepared_call_matches_fa_fwd_into():
    """fa_fwd_prepared (arguments checked once, one C call per launch) gives bit-identical
    results to fa_fwd_into, plain and with a window, re-launched after the inputs change;
    an invalid argument raises when the call is prepared."""
    dev = torch.device("cuda:0")
    q, k, v = make_qkv(1, 8, 2, 300, 300, 128, "bf16", seed=15)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    for window in (0, 70):
        out, lse = torch.empty_like(qd), torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)
        call = fa.fa_fwd_prepared(qd, kd, vd, out, lse, causal=True, window=window)
        for it in range(3):
            qd.copy_(q.to(dev) * (1 + it))
            call()
            ref = fa.fa_fwd(qd, kd, vd, causal=True, window=window)
            torch.cuda.synchronize()
            assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]), (window, it)
    with pytest.raises(fa.FaError):
        fa.fa_fwd_prepared(qd, kd, vd, out, lse, scale=-1.0)()
    with pytest.raises(ValueError):
        fa.fa_fwd_prepared(qd, kd, vd, out, lse, causal=False, window=4)


def test_empty_and_errors_on_gpu():
    dev = torch.device("cuda:0")
    q = torch.zeros(1, 4, 0, 128, dtype=torch.bfloat16, device=dev)
    k = torch.zeros(1, 4, 5, 128, dtype=torch.bfloat16, device=dev)
    out, lse = fa.fa_fwd(q, k, k)
    assert out.shape == (1, 4, 0, 128) and lse.shape == (1, 4, 0)
    q = torch.zeros(1, 3, 4, 128, dtype=torch.bfloat16, device=dev)
    k = torch.zeros(1, 2, 4, 128, dtype=torch.bfloat16, device=dev)
    with pytest.raises(fa.FaError):
        fa.fa_fwd(q, k, k)
    q = torch.zeros(1, 2, 4, 96, dtype=torch.bfloat16, device=dev)
    with pytest.raises(fa.FaError):
        fa.fa_fwd(q, q, q)
    q = torch.zeros(1, 2, 4, 128, dtype=torch.bfloat16, device=dev)
    with pytest.raises(fa.FaError):
        fa.fa_fwd(q, q, q, scale=-1.0)
    with pytest.raises(fa.FaError):
        fa.fa_fwd(q, q, q, input_pos=-1)


def test_runs_on_a_side_stream():
    q, k, v = make_qkv(1, 8, 8, 200, 200, 128, "fp16", seed=14)
    dev = torch.device("cuda:0")
    s = torch.cuda.Stream(device=dev)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        out, lse = fa.fa_fwd(qd, kd, vd, causal=True)
    s.synchronize()
    check_full(q, k, v, 1 / math.sqrt(128), True, 0, out.cpu(), lse.cpu(), "side stream")


def test_concurrent_threads_and_streams():
    """The library keeps no state between calls: four host threads, each on its own stream and
    problem, interleave 20 calls of fa_fwd / fa_fwd_splitkv / fa_bwd; every result matches,
    bit for bit, the same call run alone."""
    import threading

    dev = torch.device("cuda:0")
    problems = [
        (1, 8, 2, 300, 300, 128, "bf16", True, 0),
        (2, 4, 4, 1, 900, 128, "fp16", True, 899),
        (1, 6, 3, 129, 257, 64, "fp16", False, 0),
        (1, 8, 1, 200, 200, 128, "bf16", True, 40),
    ]
    inputs = []
    for n, (B, Hq, Hkv, Sq, Skv, D, dt, causal, pos) in enumerate(problems):
        q, k, v = make_qkv(B, Hq, Hkv, Sq, Skv, D, dt, seed=60 + n)
        g = torch.Generator(device="cpu")
        g.manual_seed(70 + n)
        do = torch.randn(q.shape, generator=g).to(q.dtype)
        inputs.append(tuple(t.to(dev) for t in (q, k, v, do)) + (causal, pos))

    def run(i):
        q, k, v, do, causal, pos = inputs[i]
        out, lse = fa.fa_fwd(q, k, v, causal=causal, input_pos=pos)
        o2, l2 = fa.fa_fwd_splitkv(q, k, v, causal=causal, input_pos=pos, num_splits=3)
        grads = fa.fa_bwd(q, k, v, out, lse, do, causal=causal, input_pos=pos)
        return (out, lse, o2, l2) + tuple(grads)

    torch.cuda.synchronize()
    alone = [tuple(t.clone() for t in run(i)) for i in range(len(problems))]
    torch.cuda.synchronize()
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream(device=dev)
            with torch.cuda.stream(s):
                for _ in range(20):
                    got = run(i)
            s.synchronize()
            for a, b in zip(alone[i], got):
                if not torch.equal(a, b):
                    errors.append(f"problem {i}: result differs from the call run alone")
                    return
        except Exception as e:  # collected and reported by the main thread
            errors.append(f"problem {i}: {e!r}")

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(problems))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors


def test_hip_graph_capture_and_replay():
    """fa_fwd, fa_bwd and the split-KV decode path captured in one HIP graph (torch.cuda.graph):
    the library only launches kernels on the given stream, so the calls are capturable.  The
    graph is replayed four times; before each replay the inputs are overwritten eagerly, and
    every replay's outputs must equal, bit for bit, the same calls run eagerly."""
    dev = torch.device("cuda:0")
    B, Hq, Hkv, S, D = 1, 8, 2, 256, 128
    dB, dHq, dHkv, dSkv = 2, 8, 2, 2048
    bf = torch.bfloat16
    q = torch.empty((B, Hq, S, D), dtype=bf, device=dev)
    k = torch.empty((B, Hkv, S, D), dtype=bf, device=dev)
    v, do = torch.empty_like(k), torch.empty_like(q)
    out, lse = torch.empty_like(q), torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(16, fa.bwd_workspace_size(B, Hq, Hkv, S, S, D, True)), dtype=torch.uint8, device=dev)
    qd = torch.empty((dB, dHq, 1, D), dtype=bf, device=dev)
    kd = torch.empty((dB, dHkv, dSkv, D), dtype=bf, device=dev)
    vd = torch.empty_like(kd)
    od, ld = torch.empty_like(qd), torch.empty((dB, dHq, 1), dtype=torch.float32, device=dev)
    wsd = torch.empty(fa.splitkv_workspace_size(dB, dHq, 1, D, 8), dtype=torch.uint8, device=dev)

    def calls(o, l, gq, gk, gv, odec, ldec):
        fa.fa_fwd_into(q, k, v, o, l, causal=True)
        fa.fa_bwd_into(q, k, v, o, l, do, gq, gk, gv, ws, causal=True)
        fa.fa_fwd_splitkv_into(qd, kd, vd, odec, ldec, wsd, num_splits=8, causal=True,
                               input_pos=dSkv - 1)

    gen = torch.Generator(device=dev)

    def refill(seed):
        gen.manual_seed(seed)
        for t in (q, k, v, do, qd, kd, vd):
            t.copy_(torch.randn(t.shape, generator=gen, device=dev, dtype=torch.float32))

    refill(0)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        calls(out, lse, dq, dk, dv, od, ld)       # warm-up outside the capture
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls(out, lse, dq, dk, dv, od, ld)
    torch.cuda.synchronize()
    for rep in range(4):
        refill(100 + rep)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = [torch.empty_like(t) for t in (out, lse, dq, dk, dv, od, ld)]
        calls(*ref)
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "lse", "dq", "dk", "dv", "out_dec", "lse_dec"),
                              (out, lse, dq, dk, dv, od, ld), ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_rising_scores_and_outlier(dtype, causal):
    """Scores that rise along the keys, so a row's maximum jumps by about 17 (in base-2 exponent
    units) from one 32-key tile to the next, plus one late outlier key 60 units above the rest:
    the lazily kept running maximum must be raised tile after tile, with the accumulator and
    the row sum rescaled each time, and the outlier must not overflow p.  Scores reach about
    120 (natural units), far outside the N(0,1) workloads.  fa_fwd and fa_fwd_splitkv.
    (The backward pass on the same inputs is checked in test_gpu_backward.py against a bound
    derived from where its arithmetic rounds.)"""
    q, k, v = make_rising_scores(dtype)
    out, lse = run_gpu(q, k, v, 0.5, causal, 0)
    eo, el = check_full(q, k, v, 0.5, causal, 0, out, lse, f"rising scores {dtype} causal={causal}")
    _say("rising scores", dtype, causal, f"O err {eo:.2e} LSE err {el:.2e}", f"max LSE {float(lse.max()):.1f}")
    assert float(lse.max()) > 100.0   # the scores really are that large
    # The split-KV path on the same inputs (partials merged across key ranges).
    dev = torch.device("cuda:0")
    o2, l2 = fa.fa_fwd_splitkv(q.to(dev), k.to(dev), v.to(dev), scale=0.5, causal=causal, num_splits=5)
    torch.cuda.synchronize()
    check_full(q, k, v, 0.5, causal, 0, o2.cpu(), l2.cpu(), f"rising scores split-KV {dtype}")
