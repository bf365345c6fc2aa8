"""CPU tests of the C ABI: the library loads, exports what include/fa_fwd.h declares, and
rejects bad arguments with the documented codes before any HIP call (no GPU needed)."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

import attention_fa_fwd_amd as fa

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "fa_fwd.h")

# Fake, well-aligned, non-overlapping device addresses: validation only compares them.
P = 1 << 30
Q, K, V, O, L = P, 2 * P, 3 * P, 4 * P, 5 * P
GOOD = dict(q=Q, k=K, v=V, out=O, lse=L, B=1, Hq=4, Hkv=2, Sq=8, Skv=8, D=64, scale=0.125,
            causal=1, input_pos=0, dtype=0)


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M)


def _header_enum(name):
    text = open(HEADER).read()
    return {m.group(1): int(m.group(2)) for m in re.finditer(r"(FA_\w+)\s*=\s*(-?\d+)", text)}


@pytest.fixture(scope="module")
def lib():
    return fa.load_library()


def call(lib, **over):
    a = dict(GOOD, **over)
    return lib.fa_fwd(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Sq"],
                      a["Skv"], a["D"], a["scale"], a["causal"], a["input_pos"], a["dtype"], None)


def test_exports_every_declared_symbol(lib):
    names = _header_functions()
    assert set(names) >= {"fa_fwd", "fa_fwd_config", "fa_select_config", "fa_num_configs",
                          "fa_config_name", "fa_strerror"}
    for n in names:
        assert hasattr(lib, n), f"{n} declared in fa_fwd.h but not exported"


def test_status_codes_match_header(lib):
    codes = _header_enum("fa_status")
    assert codes["FA_OK"] == 0
    for name, code in codes.items():
        if name.startswith("FA_ERR"):
            msg = lib.fa_strerror(code)
            assert msg and b"unknown" not in msg, name
    assert b"unknown" in lib.fa_strerror(12345)


@pytest.mark.parametrize("over,code", [
    (dict(q=0), -1), (dict(lse=0), -1),
    (dict(B=-1), -2), (dict(Hkv=0), -2), (dict(Skv=0), -2), (dict(Sq=-3), -2),
    (dict(B=1 << 21, Hq=1 << 11, Hkv=1 << 11), -2), (dict(B=1 << 10, Hq=1 << 10, Hkv=1 << 10, Sq=1 << 30), -2),
    (dict(Hq=3), -3),
    (dict(D=96), -4), (dict(D=256), -4),
    (dict(dtype=2), -5),
    (dict(scale=0.0), -6), (dict(scale=-1.0), -6), (dict(scale=float("inf")), -6),
    (dict(scale=float("nan")), -6),
    (dict(input_pos=-1), -7), (dict(input_pos=2 ** 31 - 4), -7),
    (dict(q=Q + 8), -8), (dict(out=O + 4), -8), (dict(lse=L + 2), -8),
    (dict(out=Q), -9), (dict(lse=K + 64), -9), (dict(lse=O), -9),
])
def test_validation_codes(lib, over, code):
    assert call(lib, **over) == code


def test_validation_order(lib):
    # several faults at once: the first check in header order wins
    assert call(lib, q=0, Hq=3, D=7) == -1
    assert call(lib, B=-1, Hq=3, D=7) == -2
    assert call(lib, Hq=3, D=7, dtype=9) == -3
    assert call(lib, D=7, dtype=9, scale=0.0) == -4


def test_empty_problem_is_a_noop(lib):
    assert call(lib, B=0) == 0
    assert call(lib, Sq=0) == 0
    assert call(lib, Hq=0) == 0
    # empty tensors may come with NULL pointers (torch gives them data_ptr() == 0)
    assert call(lib, Sq=0, q=0, out=0, lse=0) == 0
    assert call(lib, B=0, q=0, k=0, v=0, out=0, lse=0) == 0
    assert call(lib, Sq=0, k=0) == -1   # K/V are not empty


def test_config_table(lib):
    n = fa.num_configs()
    names = fa.config_names()
    assert n == len(names) >= 16 and len(set(names)) == n
    assert lib.fa_config_name(-1) is None and lib.fa_config_name(n) is None
    for D in (64, 128):
        for dtype in (0, 1):
            for causal in (0, 1):
                for Hq, Hkv in ((32, 32), (32, 8), (32, 4), (8, 1), (6, 3)):
                    c = fa.select_config(2, Hq, Hkv, 1000, 1000, D, causal, 0, dtype)
                    nm = names[c]
                    assert nm.startswith(f"D{D}_") and ("_bf16" if dtype else "_fp16") in nm
                    assert ("_causal_" if causal else "_full_") in nm
                    hpw = int(re.search(r"HPW(\d+)", nm).group(1))
                    assert (Hq // Hkv) % hpw == 0


def test_forced_config_checks(lib):
    a = dict(GOOD)
    args = [a[x] for x in ("q", "k", "v", "out", "lse", "B", "Hq", "Hkv", "Sq", "Skv", "D", "scale",
                           "causal", "input_pos", "dtype")] + [None]
    assert lib.fa_fwd_config(*args, fa.num_configs()) == -10
    assert lib.fa_fwd_config(*args, -2) == -10
    names = fa.config_names()
    wrong_dim = next(i for i, nm in enumerate(names) if nm.startswith("D128_"))
    assert lib.fa_fwd_config(*args, wrong_dim) == -10   # D=64 call, D=128 kernel
    hpw4 = next(i for i, nm in enumerate(names) if "HPW4" in nm and nm.startswith("D64_")
                and "_causal_fp16" in nm)
    assert lib.fa_fwd_config(*args, hpw4) == -10        # group of 2 cannot pack 4 heads


def test_binding_rejects_cpu_tensors():
    import torch

    q = torch.zeros(1, 1, 4, 64, dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        fa.fa_fwd(q, q, q)


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        fa.load_library(str(tmp_path / "missing.so"))
