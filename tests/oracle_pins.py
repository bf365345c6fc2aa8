"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each ``pin_*`` function takes the attention function under test (same
signature as ``oracle.attention_blocked``) and raises AssertionError when it
disagrees with brute force, an independent library routine, a closed form or
an invariant.  The test suite runs them on the real oracle, and runs them
again on copies with planted mistakes to show that each mistake is caught.
"""

from __future__ import annotations

import math

import numpy as np
import torch

import oracle

TIGHT = 1e-12


def rand(shape, seed, scale=1.0):
    g = np.random.default_rng(seed)
    return g.standard_normal(shape) * scale


def tiny_case(B, Hq, Hkv, Sq, Skv, D, seed):
    return rand((B, Hq, Sq, D), seed), rand((B, Hkv, Skv, D), seed + 1), \
        rand((B, Hkv, Skv, D), seed + 2)


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0
    assert err <= tol, f"{what}: max abs error {err:.3e} > {tol:.1e}"


# Small shapes that cover: single key, single query, ragged lengths, Sq != Skv,
# GQA and MQA, D of 64 and 128, causal with and without an offset.
TINY_SHAPES = [
    # B, Hq, Hkv, Sq, Skv, D, causal, input_pos
    (1, 1, 1, 1, 1, 64, False, 0),
    (1, 1, 1, 1, 1, 64, True, 0),
    (1, 2, 2, 3, 3, 64, True, 0),
    (2, 4, 2, 17, 17, 64, True, 0),
    (1, 4, 1, 17, 65, 64, True, 5),
    (1, 2, 1, 65, 17, 64, True, 0),
    (2, 2, 2, 17, 64, 128, False, 0),
    (1, 4, 2, 2, 65, 128, True, 63),
    (1, 2, 2, 64, 64, 128, True, 0),
]


def pin_bruteforce(attn):
    """P-a: equals the pure-Python brute-force definition on tiny shapes."""
    for n, (B, Hq, Hkv, Sq, Skv, D, causal, pos) in enumerate(TINY_SHAPES):
        if Sq * Skv * D > 80000:
            continue
        q, k, v = tiny_case(B, Hq, Hkv, Sq, Skv, D, 10 * n)
        scale = 1.0 / math.sqrt(D)
        O, L = attn(q, k, v, scale, causal, pos)
        O0, L0 = oracle.attention_naive(q, k, v, scale, causal, pos)
        _close(O, O0, TIGHT, f"O vs brute force {TINY_SHAPES[n]}")
        _close(L, L0, TIGHT, f"LSE vs brute force {TINY_SHAPES[n]}")


def _torch_reference(q, k, v, scale, causal, pos):
    """PyTorch CPU float64 scaled_dot_product_attention with an explicit mask.

    GQA is expressed by repeating each K/V head over its group of query heads;
    LSE is torch.logsumexp of the masked, scaled scores.
    """
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    G = qt.shape[1] // kt.shape[1]
    kt = kt.repeat_interleave(G, dim=1)
    vt = vt.repeat_interleave(G, dim=1)
    Sq, Skv = qt.shape[2], kt.shape[2]
    if causal:
        i = torch.arange(Sq)[:, None]
        j = torch.arange(Skv)[None, :]
        mask = j <= i + pos
    else:
        mask = torch.ones(Sq, Skv, dtype=torch.bool)
    O = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    s = torch.matmul(qt, kt.transpose(-1, -2).contiguous()) * scale
    s = s.masked_fill(~mask, float("-inf"))
    L = torch.logsumexp(s, dim=-1)
    return O.numpy(), L.numpy()


def pin_torch_sdpa(attn):
    """P-b: equals PyTorch's CPU float64 SDPA (an independent library routine)."""
    shapes = TINY_SHAPES + [(1, 8, 2, 200, 300, 128, True, 100), (1, 4, 4, 130, 130, 64, False, 0)]
    for n, (B, Hq, Hkv, Sq, Skv, D, causal, pos) in enumerate(shapes):
        q, k, v = tiny_case(B, Hq, Hkv, Sq, Skv, D, 100 + n)
        scale = 0.3 + 0.1 * n
        O, L = attn(q, k, v, scale, causal, pos)
        O1, L1 = _torch_reference(q, k, v, scale, causal, pos)
        _close(O, O1, TIGHT, f"O vs torch SDPA {shapes[n]}")
        _close(L, L1, TIGHT, f"LSE vs torch logsumexp {shapes[n]}")


def pin_constant_k(attn):
    """P-d: with every key equal to k_0, O_i is the mean of the visible V rows and
    LSE_i = scale q_i.k_0 + ln |V(i)|."""
    for causal, pos in ((True, 0), (True, 3), (False, 0)):
        B, Hq, Hkv, Sq, Skv, D = 1, 4, 2, 9, 12, 64
        q, k, v = tiny_case(B, Hq, Hkv, Sq, Skv, D, 7)
        k[:] = k[:, :, :1, :]
        scale = 0.125
        O, L = attn(q, k, v, scale, causal, pos)
        for hq in range(Hq):
            g = hq // (Hq // Hkv)
            for i in range(Sq):
                n = Skv if not causal else min(Skv, pos + i + 1)
                _close(O[0, hq, i], v[0, g, :n].mean(axis=0), 1e-12, "constant-K mean")
                want = scale * float(q[0, hq, i] @ k[0, g, 0]) + math.log(n)
                _close(L[0, hq, i], want, 1e-12, "constant-K LSE")


def pin_causal_row0(attn):
    """P-e: causal with input_pos = 0, query 0 sees only key 0: O_0 = V_0 and
    LSE_0 = scale q_0.k_0."""
    B, Hq, Hkv, Sq, Skv, D = 2, 4, 2, 5, 7, 128
    q, k, v = tiny_case(B, Hq, Hkv, Sq, Skv, D, 3)
    O, L = attn(q, k, v, 0.2, True, 0)
    for b in range(B):
        for hq in range(Hq):
            g = hq // 2
            _close(O[b, hq, 0], v[b, g, 0], 1e-13, "causal row 0 output")
            _close(L[b, hq, 0], 0.2 * float(q[b, hq, 0] @ k[b, g, 0]), 1e-13, "causal row 0 LSE")


def pin_gqa_replicated(attn):
    """P-f: GQA equals MHA with each K/V head repeated over its contiguous group
    of query heads ("Grouped-query attention"), and differs from a strided map."""
    B, Hq, Hkv, Sq, Skv, D = 1, 8, 2, 6, 10, 64
    q, k, v = tiny_case(B, Hq, Hkv, Sq, Skv, D, 21)
    O, L = attn(q, k, v, 0.125, True, 2)
    kr = np.repeat(k, Hq // Hkv, axis=1)
    vr = np.repeat(v, Hq // Hkv, axis=1)
    O2, L2 = oracle.attention_naive(q, kr, vr, 0.125, True, 2)
    _close(O, O2, TIGHT, "GQA vs replicated K/V heads")
    _close(L, L2, TIGHT, "GQA LSE vs replicated K/V heads")
    ks = np.tile(k, (1, Hq // Hkv, 1, 1))  # strided: head hq reads kv head hq % Hkv
    vs = np.tile(v, (1, Hq // Hkv, 1, 1))
    O3, _ = oracle.attention_naive(q, ks, vs, 0.125, True, 2)
    assert np.max(np.abs(O - O3)) > 1e-3, "GQA map must be contiguous, not strided"


def pin_input_pos_chunk(attn):
    """P-h: a query chunk at input_pos = p equals rows p.. of the full causal
    problem whose queries contain the chunk at rows p.. ."""
    B, Hq, Hkv, Skv, D = 1, 2, 1, 40, 64
    p, n = 25, 9
    qf, k, v = tiny_case(B, Hq, Hkv, Skv, Skv, D, 31)
    Of, Lf = attn(qf, k, v, 0.125, True, 0)
    Oc, Lc = attn(qf[:, :, p:p + n], k, v, 0.125, True, p)
    _close(Oc, Of[:, :, p:p + n], TIGHT, "input_pos chunk output")
    _close(Lc, Lf[:, :, p:p + n], TIGHT, "input_pos chunk LSE")


def pin_key_permutation(attn):
    """P-i: without a mask, permuting keys jointly in K and V changes nothing."""
    B, Hq, Hkv, Sq, Skv, D = 1, 2, 2, 7, 13, 64
    q, k, v = tiny_case(B, Hq, Hkv, Sq, Skv, D, 41)
    perm = np.random.default_rng(5).permutation(Skv)
    O, L = attn(q, k, v, 0.125, False, 0)
    O2, L2 = attn(q, k[:, :, perm], v[:, :, perm], 0.125, False, 0)
    _close(O, O2, TIGHT, "key permutation output")
    _close(L, L2, TIGHT, "key permutation LSE")


def pin_tiny_scale_mean(attn):
    """P-i: as scale -> 0 the softmax is uniform over the visible keys."""
    B, Hq, Hkv, Sq, Skv, D = 1, 2, 1, 6, 6, 64
    q, k, v = tiny_case(B, Hq, Hkv, Sq, Skv, D, 51)
    O, L = attn(q, k, v, 1e-12, True, 0)
    for i in range(Sq):
        _close(O[0, 0, i], v[0, 0, :i + 1].mean(axis=0), 1e-9, "uniform softmax at tiny scale")
        _close(L[0, 0, i], math.log(i + 1), 1e-9, "LSE at tiny scale = ln |V(i)|")


def pin_one_hot_v(attn):
    """P-c/P-i: with V = identity rows, O reads back the attention weights P,
    whose rows sum to 1 and vanish on masked keys."""
    B, Hq, Hkv, Sq, Skv, D = 1, 2, 1, 5, 64, 64
    q, k, _ = tiny_case(B, Hq, Hkv, Sq, Skv, D, 61)
    v = np.broadcast_to(np.eye(Skv, D), (B, Hkv, Skv, D)).copy()
    O, _ = attn(q, k, v, 0.125, True, 30)
    P = oracle.attention_probs_naive(q, k, 0.125, True, 30)
    _close(O, P, TIGHT, "one-hot V reads back P")
    _close(P.sum(axis=-1), 1.0, TIGHT, "softmax rows sum to 1")
    for i in range(Sq):
        assert np.all(P[0, :, i, 30 + i + 1:] == 0.0)


ALL_PINS = [pin_bruteforce, pin_torch_sdpa, pin_constant_k, pin_causal_row0, pin_gqa_replicated,
            pin_input_pos_chunk, pin_key_permutation, pin_tiny_scale_mean, pin_one_hot_v]
