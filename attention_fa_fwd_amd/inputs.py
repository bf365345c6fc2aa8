"""Seeded synthetic inputs and the named workload shapes.

This module holds no attention arithmetic: it draws N(0, 1) tensors on the CPU
with a seeded generator and rounds them to the storage dtype.  Both the HIP
path (tests, benchmark) and the fp64 oracle read the same rounded tensors.

Recipe: ``torch.Generator('cpu').manual_seed(seed)``; float32 ``randn`` for q,
then k, then v, each at its full [B, H, S, D] shape; ``.to(dtype)``
(round-to-nearest-even); contiguous BHSD layout.
"""

from __future__ import annotations

import math

import torch

DTYPES = {"fp16": torch.float16, "bf16": torch.bfloat16}

# Named workloads: the shapes on which the attention forward pass is checked and
# measured.  Sizes follow the sequence-length sweeps of the pages (B, heads, head
# dim 128 or 64, causal and non-causal, multi-head and grouped-query).
WORKLOADS = {
    "mha_s128_d64_fp16": dict(B=1, Hq=2, Hkv=2, Sq=128, Skv=128, D=64, dtype="fp16",
                              causal=False, input_pos=0),
    "mha_s1024_d128_fp16": dict(B=1, Hq=32, Hkv=32, Sq=1024, Skv=1024, D=128, dtype="fp16",
                                causal=False, input_pos=0),
    "mha_causal_s4096_d128_fp16": dict(B=1, Hq=32, Hkv=32, Sq=4096, Skv=4096, D=128,
                                       dtype="fp16", causal=True, input_pos=0),
    "gqa8_causal_s8192_d128_bf16": dict(B=1, Hq=32, Hkv=4, Sq=8192, Skv=8192, D=128,
                                        dtype="bf16", causal=True, input_pos=0),
    "gqa4_prefill_q1024_kv16384_d128_bf16": dict(B=2, Hq=32, Hkv=8, Sq=1024, Skv=16384, D=128,
                                                  dtype="bf16", causal=True, input_pos=15360),
    # Sliding-window causal attention over a 16K sequence, window 4096 keys.
    "gqa8_swa4096_causal_s16384_d128_bf16": dict(B=1, Hq=32, Hkv=4, Sq=16384, Skv=16384, D=128,
                                                  dtype="bf16", causal=True, input_pos=0,
                                                  window=4096),
    # Head dim 64 ("TiledAttention" Table 5 shape family) at sizes whose grids fill the GPU,
    # so the dispatch takes the eight-wave head-dim-64 workgroups: 8 positions x 1 head
    # (MHA), 2 positions x 4 heads (GQA 4) and 4 positions x 2 heads (GQA 2).
    "mha_causal_s4096_d64_fp16": dict(B=1, Hq=32, Hkv=32, Sq=4096, Skv=4096, D=64,
                                      dtype="fp16", causal=True, input_pos=0),
    "gqa4_causal_s4096_d64_bf16": dict(B=1, Hq=32, Hkv=8, Sq=4096, Skv=4096, D=64,
                                       dtype="bf16", causal=True, input_pos=0),
    "gqa2_s2048_d64_fp16": dict(B=1, Hq=32, Hkv=16, Sq=2048, Skv=2048, D=64, dtype="fp16",
                                causal=False, input_pos=0),
    # Non-causal attention of 256 queries over 16K keys (a cross-attention shape, GQA 4): 64
    # four-wave workgroups, one wave per SIMD on the CUs they use, so fa_fwd's dispatch takes
    # two key parts per workgroup; fa_fwd_splitkv splits the keys across workgroups instead
    # (both are timed: "splitkv_line").
    "gqa4_xattn_q256_kv16384_d128_bf16": dict(B=1, Hq=32, Hkv=8, Sq=256, Skv=16384, D=128,
                                              dtype="bf16", causal=False, input_pos=0,
                                              splitkv_line=True),
    # One new token per sequence against a 16K-token cache: the under-filled grid that
    # split-KV is for (32 workgroups unsplit).
    "gqa4_decode_b4_kv16384_d128_bf16": dict(B=4, Hq=32, Hkv=8, Sq=1, Skv=16384, D=128,
                                              dtype="bf16", causal=True, input_pos=16383),
}


# A sequence-length sweep of causal MHA at B=4, H=32, D=128, fp16: the shape of the length
# sweep in "Tuning Flash Attention for peak performance in NVIDIA CUDA Tile" (Tables 1-6),
# timed for context only.
SWEEP_WORKLOADS = {
    f"mha_causal_b4_s{S}_d128_fp16": dict(B=4, Hq=32, Hkv=32, Sq=S, Skv=S, D=128, dtype="fp16",
                                          causal=True, input_pos=0)
    for S in (1024, 2048, 4096, 8192, 16384)
}

# Workloads with fp8 E4M3 queries and keys (per-tensor descale factors) and fp16 / bf16
# values -- or fp8 values too ("fp8v") -- the headline, causal multi-head and decoding shapes.
FP8_WORKLOADS = {
    "gqa8_causal_s8192_d128_fp8qk_bf16": dict(B=1, Hq=32, Hkv=4, Sq=8192, Skv=8192, D=128,
                                              dtype="bf16", causal=True, input_pos=0),
    "mha_causal_s4096_d128_fp8qk_fp16": dict(B=1, Hq=32, Hkv=32, Sq=4096, Skv=4096, D=128,
                                             dtype="fp16", causal=True, input_pos=0),
    # Decoding against an fp8 key cache (the bf16 decode workload's shape).
    "gqa4_decode_b4_kv16384_d128_fp8qk_bf16": dict(B=4, Hq=32, Hkv=8, Sq=1, Skv=16384, D=128,
                                                   dtype="bf16", causal=True, input_pos=16383),
    # fp8 queries, keys and values (bf16 output): decoding against an fp8 K/V cache, and
    # the headline prefill shape.
    "gqa4_decode_b4_kv16384_d128_fp8qkv_bf16": dict(B=4, Hq=32, Hkv=8, Sq=1, Skv=16384, D=128,
                                                    dtype="bf16", causal=True, input_pos=16383,
                                                    fp8v=True),
    "gqa8_causal_s8192_d128_fp8qkv_bf16": dict(B=1, Hq=32, Hkv=4, Sq=8192, Skv=8192, D=128,
                                               dtype="bf16", causal=True, input_pos=0, fp8v=True),
    # Head dim 64 in fp8: the GQA-4 causal shape of the head-dim-64 bf16 workload.
    "gqa4_causal_s4096_d64_fp8qk_bf16": dict(B=1, Hq=32, Hkv=8, Sq=4096, Skv=4096, D=64,
                                             dtype="bf16", causal=True, input_pos=0),
    "gqa4_causal_s4096_d64_fp8qkv_bf16": dict(B=1, Hq=32, Hkv=8, Sq=4096, Skv=4096, D=64,
                                              dtype="bf16", causal=True, input_pos=0, fp8v=True),
}


def default_scale(D: int) -> float:
    """1/sqrt(D), the default softmax scale."""
    return 1.0 / math.sqrt(D)


def _randn_qkv(B, Hq, Hkv, Sq, Skv, D, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = torch.randn((B, Hq, Sq, D), generator=g, dtype=torch.float32)
    k = torch.randn((B, Hkv, Skv, D), generator=g, dtype=torch.float32)
    v = torch.randn((B, Hkv, Skv, D), generator=g, dtype=torch.float32)
    return q, k, v


def make_qkv(B, Hq, Hkv, Sq, Skv, D, dtype, seed=0):
    """Seeded q [B,Hq,Sq,D], k and v [B,Hkv,Skv,D] on the CPU, rounded to ``dtype``."""
    if isinstance(dtype, str):
        dtype = DTYPES[dtype]
    q, k, v = _randn_qkv(B, Hq, Hkv, Sq, Skv, D, seed)
    return q.to(dtype).contiguous(), k.to(dtype).contiguous(), v.to(dtype).contiguous()


FP8_MAX = 448.0   # largest finite fp8 E4M3 (OCP "E4M3FN") value


def quantize_fp8(x):
    """Per-tensor fp8 E4M3 quantisation of a float32 tensor: descale = amax / 448 and
    codes = round-to-nearest-even(x / descale) (torch's conversion), so that
    descale * codes approximates x.  Returns (codes as torch.float8_e4m3fn, descale)."""
    amax = float(x.abs().max()) if x.numel() else 1.0
    descale = (amax / FP8_MAX) if amax > 0 else 1.0
    return (x / descale).to(torch.float8_e4m3fn).contiguous(), descale


def make_qkv_fp8(B, Hq, Hkv, Sq, Skv, D, v_dtype, seed=0):
    """The same seeded draws as ``make_qkv``, with q and k quantised to fp8 E4M3 per
    tensor and v rounded to ``v_dtype``.  Returns (q8, k8, v, q_descale, k_descale)."""
    if isinstance(v_dtype, str):
        v_dtype = DTYPES[v_dtype]
    q, k, v = _randn_qkv(B, Hq, Hkv, Sq, Skv, D, seed)
    q8, qd = quantize_fp8(q)
    k8, kd = quantize_fp8(k)
    return q8, k8, v.to(v_dtype).contiguous(), qd, kd


def make_qkv_fp8qkv(B, Hq, Hkv, Sq, Skv, D, seed=0):
    """The same seeded draws as ``make_qkv``, with q, k and v each quantised to fp8 E4M3 per
    tensor.  Returns (q8, k8, v8, q_descale, k_descale, v_descale)."""
    q, k, v = _randn_qkv(B, Hq, Hkv, Sq, Skv, D, seed)
    q8, qd = quantize_fp8(q)
    k8, kd = quantize_fp8(k)
    v8, vd = quantize_fp8(v)
    return q8, k8, v8, qd, kd, vd


def make_rising_scores(dtype, B=1, Hq=4, Hkv=2, S=320, D=128, seed=5):
    """Queries and keys built so that scores rise steadily along the keys, plus one outlier.

    With a random unit direction u: q = 3 u + 0.1 N(0,1) noise; key j = r_j u + 0.1 noise with
    r_j rising linearly from 0 to 80 over the S keys, except key 250 (when S > 250), set to
    100 u; v is N(0,1).  At scale 0.5 the scores reach about 150, so a row's maximum grows
    from one key block to the next and the outlier dominates every row that sees it.
    Returns (q, k, v) rounded to ``dtype``."""
    if isinstance(dtype, str):
        dtype = DTYPES[dtype]
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    u = torch.randn(D, generator=g)
    u = u / u.norm()
    q = 3.0 * u + 0.1 * torch.randn((B, Hq, S, D), generator=g)
    ramp = torch.linspace(0.0, 80.0, S)
    k = ramp[None, None, :, None] * u + 0.1 * torch.randn((B, Hkv, S, D), generator=g)
    if S > 250:
        k[:, :, 250, :] = 100.0 * u
    v = torch.randn((B, Hkv, S, D), generator=g)
    return tuple(t.to(dtype).contiguous() for t in (q, k, v))


def make_workload(name, seed=0):
    """Inputs and call arguments for a named workload: (q, k, v, kwargs)."""
    w = dict(WORKLOADS[name] if name in WORKLOADS else SWEEP_WORKLOADS[name])
    q, k, v = make_qkv(w["B"], w["Hq"], w["Hkv"], w["Sq"], w["Skv"], w["D"], w["dtype"], seed)
    kw = dict(scale=default_scale(w["D"]), causal=w["causal"], input_pos=w["input_pos"],
              window=w.get("window", 0))
    return q, k, v, kw


def make_fp8_workload(name, seed=0):
    """Inputs and call arguments for a named fp8 workload: (q8, k8, v, kwargs).  For an
    fp8 Q/K/V workload v is fp8 codes too and kwargs holds v_descale; its "dtype" is the
    output's."""
    w = dict(FP8_WORKLOADS[name])
    kw = dict(scale=default_scale(w["D"]), causal=w["causal"], input_pos=w["input_pos"],
              window=w.get("window", 0))
    if w.get("fp8v"):
        q8, k8, v, qd, kd, vd = make_qkv_fp8qkv(w["B"], w["Hq"], w["Hkv"], w["Sq"], w["Skv"],
                                                w["D"], seed)
        kw["v_descale"] = vd
    else:
        q8, k8, v, qd, kd = make_qkv_fp8(w["B"], w["Hq"], w["Hkv"], w["Sq"], w["Skv"], w["D"],
                                         w["dtype"], seed)
    kw.update(q_descale=qd, k_descale=kd)
    return q8, k8, v, kw
