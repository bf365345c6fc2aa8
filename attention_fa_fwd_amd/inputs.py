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
    # One new token per sequence against a 16K-token cache: the under-filled grid that
    # split-KV is for (32 workgroups unsplit).
    "gqa4_decode_b4_kv16384_d128_bf16": dict(B=4, Hq=32, Hkv=8, Sq=1, Skv=16384, D=128,
                                              dtype="bf16", causal=True, input_pos=16383),
}


def default_scale(D: int) -> float:
    """1/sqrt(D), the default softmax scale."""
    return 1.0 / math.sqrt(D)


def make_qkv(B, Hq, Hkv, Sq, Skv, D, dtype, seed=0):
    """Seeded q [B,Hq,Sq,D], k and v [B,Hkv,Skv,D] on the CPU, rounded to ``dtype``."""
    if isinstance(dtype, str):
        dtype = DTYPES[dtype]
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = torch.randn((B, Hq, Sq, D), generator=g, dtype=torch.float32).to(dtype)
    k = torch.randn((B, Hkv, Skv, D), generator=g, dtype=torch.float32).to(dtype)
    v = torch.randn((B, Hkv, Skv, D), generator=g, dtype=torch.float32).to(dtype)
    return q.contiguous(), k.contiguous(), v.contiguous()


def make_workload(name, seed=0):
    """Inputs and call arguments for a named workload: (q, k, v, kwargs)."""
    w = dict(WORKLOADS[name])
    q, k, v = make_qkv(w["B"], w["Hq"], w["Hkv"], w["Sq"], w["Skv"], w["D"], w["dtype"], seed)
    kw = dict(scale=default_scale(w["D"]), causal=w["causal"], input_pos=w["input_pos"],
              window=w.get("window", 0))
    return q, k, v, kw
