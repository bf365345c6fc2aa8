"""GPU parity of the two-key-part forward configurations ("KS2"): a workgroup's waves in two
sets, each running the online softmax over one half of the key tiles, the two states merged
through LDS before the epilogue.  The dispatch takes them for non-causal calls over at least
4096 keys whose four-wave grid leaves one wave per SIMD and whose key tiles split evenly;
split-KV calls fall back to the one-part twin.  Every output is compared with the fp64 oracle at the forward
tolerances (max |O - O_oracle| <= 4e-3 fp16 / 1.6e-2 bf16, max |LSE - LSE_oracle| <= 1e-3).
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

TOL_O = {torch.float16: 4e-3, torch.bfloat16: 1.6e-2}
TOL_LSE = 1e-3
DEV = torch.device("cuda:0")
DT = {"fp16": 0, "bf16": 1}
BN = {128: 32, 64: 64}


def _say(*a):
    print("[keyparts]", *a, file=sys.stderr, flush=True)


def _f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def check_full(q, k, v, scale, out, lse, what):
    O, L = oracle.attention_blocked(_f64(q), _f64(k), _f64(v), scale, False, 0)
    o, l = _f64(out), _f64(lse)
    assert np.isfinite(o).all() and np.isfinite(l).all(), f"non-finite output {what}"
    eo = float(np.max(np.abs(o - O))) if o.size else 0.0
    el = float(np.max(np.abs(l - L))) if l.size else 0.0
    _say(what, f"O err {eo:.2e} LSE err {el:.2e}")
    assert eo <= TOL_O[q.dtype], f"O max abs err {eo:.3e} {what}"
    assert el <= TOL_LSE, f"LSE max abs err {el:.3e} {what}"


def ks2_configs(D, dtype):
    names = fa.config_names()
    return [(i, n) for i, n in enumerate(names)
            if n.startswith(f"D{D}_") and "_KS2_full_" in n and n.endswith(dtype)]


def test_dispatch_takes_key_parts_for_one_wave_per_simd_grids():
    names = fa.config_names()
    # Non-causal MHA with 4K keys: 256 four-wave workgroups, 128 key tiles.
    c = fa.select_config(1, 32, 32, 1024, 4096, 128, False, 0, DT["fp16"])
    assert names[c] == "D128_BN32_Mw1x32_WPH4_HPW1_KS2_full_fp16"
    # GQA 4 and GQA 2, small grids, even tile counts.
    c = fa.select_config(1, 16, 4, 256, 8192, 128, False, 0, DT["bf16"])
    assert names[c] == "D128_BN32_Mw1x32_WPH1_HPW4_KS2_full_bf16"
    c = fa.select_config(2, 8, 4, 300, 4096, 64, False, 0, DT["fp16"])
    assert names[c] == "D64_BN64_Mw1x32_WPH2_HPW2_KS2_full_fp16"
    c = fa.select_config(1, 32, 32, 1024, 4100, 128, False, 0, DT["fp16"])   # 129 tiles: odd
    assert names[c] == "D128_BN32_Mw1x32_WPH4_HPW1_full_fp16"
    c = fa.select_config(1, 32, 32, 1024, 4130, 128, False, 0, DT["fp16"])   # 130, ragged
    assert "_KS2_" in names[c]
    # Under 4096 keys (the short MHA workload among them), a causal call, or a grid of more
    # than one four-wave workgroup per CU keeps one part.
    c = fa.select_config(1, 32, 32, 1024, 1024, 128, False, 0, DT["fp16"])
    assert names[c] == "D128_BN32_Mw1x32_WPH4_HPW1_full_fp16"
    c = fa.select_config(1, 32, 32, 1024, 4064, 128, False, 0, DT["fp16"])
    assert "_KS2_" not in names[c]
    c = fa.select_config(1, 32, 32, 1024, 4096, 128, True, 0, DT["fp16"])
    assert "_KS2_" not in names[c]
    c = fa.select_config(2, 32, 32, 1024, 4096, 128, False, 0, DT["fp16"])  # 512 workgroups
    assert "_KS2_" not in names[c]


# B, Hq, Hkv, Sq, Skv, D -- even key-tile counts, ragged query and key ends
CASES = [
    (1, 4, 4, 128, 64, 128),        # two tiles: one per part
    (1, 4, 4, 37, 300, 128),        # one ragged query block, ragged last key tile
    (2, 8, 2, 200, 640, 128),       # GQA 4, several query blocks
    (1, 6, 3, 130, 1000, 128),      # GQA 2
    (1, 4, 4, 100, 128, 64),        # two 64-key tiles
    (2, 8, 4, 257, 333, 64),        # GQA 2, ragged both
    (1, 8, 2, 64, 1000, 64),        # GQA 4, 16 tiles
]


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_every_key_part_config(case, dtype):
    """Each two-part configuration that fits the call's head group, forced, against the
    oracle; and the plain call (whatever the dispatch takes) as well."""
    B, Hq, Hkv, Sq, Skv, D = case
    assert ((Skv + BN[D] - 1) // BN[D]) % 2 == 0
    q, k, v = make_qkv(B, Hq, Hkv, Sq, Skv, D, dtype, seed=sum(case))
    scale = 1.0 / math.sqrt(D)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    tested = 0
    for cid, name in ks2_configs(D, dtype):
        hpw = int(name.split("_HPW")[1].split("_")[0])
        if (Hq // Hkv) % hpw:
            continue
        out, lse = fa.fa_fwd(qd, kd, vd, scale=scale, causal=False, config=cid)
        torch.cuda.synchronize()
        check_full(q, k, v, scale, out, lse, f"{case} {dtype} {name}")
        tested += 1
    assert tested >= 1
    out, lse = fa.fa_fwd(qd, kd, vd, scale=scale, causal=False)
    torch.cuda.synchronize()
    check_full(q, k, v, scale, out, lse, f"{case} {dtype} dispatch")


def test_key_parts_refused_where_they_do_not_fit():
    """A forced two-part configuration with an odd number of key tiles, or with several key
    ranges, is refused (FA_ERR_INVALID_CONFIG) before any launch."""
    cid = fa.config_names().index("D128_BN32_Mw1x32_WPH4_HPW1_KS2_full_bf16")
    q, k, v = (t.to(DEV) for t in make_qkv(1, 4, 4, 64, 96, 128, "bf16", seed=1))   # 3 tiles
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd(q, k, v, causal=False, config=cid)
    assert e.value.code == -10
    q, k, v = (t.to(DEV) for t in make_qkv(1, 4, 4, 64, 128, 128, "bf16", seed=1))   # 4 tiles
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd_splitkv(q, k, v, causal=False, num_splits=2, config=cid)
    assert e.value.code == -10
    out, lse = fa.fa_fwd_splitkv(q, k, v, causal=False, num_splits=1, config=cid)
    torch.cuda.synchronize()
    check_full(*(t.cpu() for t in (q, k, v)), 1.0 / math.sqrt(128), out, lse, "forced, one split")


@pytest.mark.parametrize("num_splits", [0, 1, 2, 5])
def test_splitkv_falls_back_to_one_part(num_splits):
    """On a shape the dispatch gives two key parts, split-KV with several ranges runs the
    one-part twin (and the library's split count is the twin's), one range keeps the parts:
    every result agrees with the oracle."""
    B, Hq, Hkv, Sq, Skv, D = 1, 8, 2, 64, 4096, 128
    names = fa.config_names()
    assert "_KS2_" in names[fa.select_config(B, Hq, Hkv, Sq, Skv, D, False, 0, DT["bf16"])]
    auto = fa.splitkv_num_splits(B, Hq, Hkv, Sq, Skv, D, False, 0, torch.bfloat16)
    assert auto > 1
    q, k, v = make_qkv(B, Hq, Hkv, Sq, Skv, D, "bf16", seed=7)
    out, lse = fa.fa_fwd_splitkv(q.to(DEV), k.to(DEV), v.to(DEV), causal=False, num_splits=num_splits)
    torch.cuda.synchronize()
    check_full(q, k, v, 1.0 / math.sqrt(D), out, lse, f"splits={num_splits}")
    out2, lse2 = fa.fa_fwd_splitkv_noalloc(q.to(DEV), k.to(DEV), v.to(DEV), causal=False,
                                           num_splits=num_splits)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), out2.cpu()) and torch.equal(lse.cpu(), lse2.cpu())


def test_dispatched_key_parts_full_size():
    """A full-size call the dispatch gives two key parts (non-causal MHA, 1024 queries
    against 4096 keys, fp16): every element against the oracle, and bit-identical on a
    second call."""
    names = fa.config_names()
    assert "_KS2_" in names[fa.select_config(1, 32, 32, 1024, 4096, 128, False, 0, DT["fp16"])]
    q, k, v = make_qkv(1, 32, 32, 1024, 4096, 128, "fp16", seed=3)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    a = fa.fa_fwd(qd, kd, vd, causal=False)
    b = fa.fa_fwd(qd, kd, vd, causal=False)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    check_full(q, k, v, 1.0 / math.sqrt(128), a[0], a[1], "full size")
