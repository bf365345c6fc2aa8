"""CPU tests of the C ABI: the library loads, exports what include/fa_fwd.h declares, and
rejects bad arguments with the documented codes before any HIP call (no GPU needed)."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

import attention_fa_fwd_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa_fwd.h")

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


# --- split-KV entry points -----------------------------------------------------------

W = 6 * P   # fake workspace address, 16-byte aligned, clear of every tensor


def call_split(lib, num_splits=2, config=-1, ws=W, ws_bytes=1 << 28, window=0, **over):
    a = dict(GOOD, **over)
    return lib.fa_fwd_splitkv(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                              a["Sq"], a["Skv"], a["D"], a["scale"], a["causal"], a["input_pos"],
                              window, a["dtype"], num_splits, config, ws, ws_bytes, None)


def call_window(lib, window=4, config=-1, **over):
    a = dict(GOOD, **over)
    return lib.fa_fwd_window(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                             a["Sq"], a["Skv"], a["D"], a["scale"], a["input_pos"], window,
                             a["dtype"], None, config)


def test_splitkv_workspace_size(lib):
    assert fa.splitkv_workspace_size(1, 32, 1024, 128, 2) == 2 * 32 * 1024 * 129 * 4
    assert fa.splitkv_workspace_size(2, 3, 5, 64, 7) == 7 * 2 * 3 * 5 * 65 * 4
    assert fa.splitkv_workspace_size(1, 32, 1024, 128, 1) == 0
    assert fa.splitkv_workspace_size(1, 32, 1024, 128, 0) == 0
    assert fa.splitkv_workspace_size(0, 32, 1024, 128, 4) == 0
    assert fa.splitkv_workspace_size(1, 32, 1024, 96, 4) == 0


def test_splitkv_auto_split_count(lib):
    # A grid with a workgroup per CU is not split (256 workgroups at 1024 tokens, and the
    # full causal 8K grid); decoding (8 workgroups) is split to ~512 workgroups; ranges
    # keep >= 8 key tiles; a small prefill (128 workgroups) is not split because its fp32
    # partials would move more bytes than its K/V.
    assert fa.splitkv_num_splits(1, 32, 32, 1024, 1024, 128, False, 0, 0) == 1
    assert fa.splitkv_num_splits(1, 32, 4, 8192, 8192, 128, True, 0, 1) == 1
    assert fa.splitkv_num_splits(1, 32, 4, 1, 16384, 128, True, 16383, 1) == 64
    assert fa.splitkv_num_splits(4, 32, 8, 1, 16384, 128, True, 16383, 1) == 16
    assert fa.splitkv_num_splits(16, 32, 8, 1, 4096, 128, True, 4095, 1) == 4
    assert fa.splitkv_num_splits(1, 1, 1, 1, 64, 128, True, 63, 1) == 1     # 2 tiles: too short
    assert fa.splitkv_num_splits(1, 1, 1, 1, 4096, 64, False, 0, 0) == 4096 // 64 // 8
    assert fa.splitkv_num_splits(1, 8, 8, 2048, 2048, 128, True, 0, 0) == 1
    with pytest.raises(fa.FaError):
        fa.splitkv_num_splits(1, 3, 2, 1, 64, 128, True, 0, 1)


@pytest.mark.parametrize("over,kw,code", [
    (dict(Hq=3), {}, -3),                                    # fa_fwd's checks come first
    ({}, dict(config=10 ** 6), -10),
    ({}, dict(num_splits=-1), -12), ({}, dict(num_splits=257), -12),
    ({}, dict(ws=0), -1),
    ({}, dict(ws=W + 8), -8),
    ({}, dict(ws_bytes=2 * 4 * 8 * 65 * 4 - 1), -13),
    ({}, dict(ws=O - 64), -9), ({}, dict(ws=L), -9), ({}, dict(ws=Q + 16), -9),
])
def test_splitkv_validation(lib, over, kw, code):
    assert call_split(lib, **kw, **over) == code


def test_splitkv_validation_order_and_noops(lib):
    assert call_split(lib, num_splits=-1, ws=0, D=96) == -4
    assert call_split(lib, num_splits=300, ws=0) == -12
    # empty problems launch nothing and need no workspace
    assert call_split(lib, Sq=0, ws=0, ws_bytes=0) == 0
    assert call_split(lib, B=0, ws=0, ws_bytes=0, num_splits=0) == 0
    # exactly the documented workspace size is enough to pass validation; the call would
    # then launch, which needs a GPU, so only the size rule is checked here
    need = fa.splitkv_workspace_size(1, 4, 8, 64, 2)
    assert call_split(lib, ws_bytes=need - 1) == -13


def call_noalloc(lib, num_splits=2, config=-1, window=0, **over):
    a = dict(GOOD, **over)
    return lib.fa_fwd_splitkv_noalloc(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"],
                                      a["Hkv"], a["Sq"], a["Skv"], a["D"], a["scale"], a["causal"],
                                      a["input_pos"], window, a["dtype"], num_splits, config, None)


def test_noalloc_scratch_size_header_and_binding():
    text = open(HEADER).read()
    m = re.search(r"#define FA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == fa.NOALLOC_SCRATCH_BYTES


def test_noalloc_validation(lib):
    """The workspace-free split-KV entry point checks what fa_fwd_splitkv checks, in the same
    order, and then that the partials fit its fixed scratch -- all before any HIP call."""
    assert call_noalloc(lib, q=0) == -1
    assert call_noalloc(lib, Hq=3) == -3
    assert call_noalloc(lib, D=96) == -4
    assert call_noalloc(lib, scale=0.0) == -6
    assert call_noalloc(lib, out=Q) == -9
    assert call_noalloc(lib, config=10 ** 6) == -10
    assert call_noalloc(lib, num_splits=-1) == -12 and call_noalloc(lib, num_splits=257) == -12
    assert call_noalloc(lib, window=4, causal=0) == -14
    assert call_noalloc(lib, Sq=0) == 0 and call_noalloc(lib, B=0, num_splits=0) == 0
    # B=1, Hq=32, Sq=4096, D=128 at 2 splits needs 135 MB of partials: over the 64 MiB scratch
    big = dict(B=1, Hq=32, Hkv=32, Sq=4096, Skv=4096, D=128)
    need = fa.splitkv_workspace_size(1, 32, 4096, 128, 2)
    assert need > fa.NOALLOC_SCRATCH_BYTES
    assert call_noalloc(lib, num_splits=2, **big) == -15
    assert call_noalloc(lib, num_splits=256, B=1, Hq=8, Hkv=8, Sq=64, Skv=4096, D=128) == -15
    assert b"scratch" in lib.fa_strerror(-15)


# --- sliding window ------------------------------------------------------------------

def test_window_validation(lib):
    assert call_window(lib, window=0) == -14
    assert call_window(lib, window=-3) == -14
    assert call_split(lib, window=-1) == -14
    assert call_split(lib, window=5, causal=0) == -14
    # order: input_pos before window, window before alignment
    assert call_window(lib, window=0, input_pos=-1) == -7
    assert call_window(lib, window=0, q=Q + 8) == -14
    assert call_split(lib, window=3, causal=0, out=O + 4) == -14
    # the window entry point checks everything fa_fwd checks
    assert call_window(lib, Hq=3) == -3
    assert call_window(lib, D=96) == -4
    assert call_window(lib, config=10 ** 6) == -10
    # empty problems launch nothing
    assert call_window(lib, Sq=0, q=0, out=0, lse=0) == 0


def test_window_split_count(lib):
    # decoding against a 16K cache with a 4K (1K) window: the window bounds the key tiles,
    # so the ranges keep >= 8 of them
    assert fa.splitkv_num_splits(4, 32, 8, 1, 16384, 128, True, 16383, 1, window=4096) == 16
    assert fa.splitkv_num_splits(4, 32, 8, 1, 16384, 128, True, 16383, 1, window=1024) == 4
    with pytest.raises(fa.FaError):
        fa.splitkv_num_splits(4, 32, 8, 1, 16384, 128, False, 0, 1, window=1024)


# --- fp8 queries and keys ------------------------------------------------------------

def call_fp8(lib, qd=0.01, kd=0.02, window=0, config=-1, **over):
    a = dict(GOOD, **dict(dict(D=128), **over))
    return lib.fa_fwd_fp8(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                          a["Sq"], a["Skv"], a["D"], a["scale"], qd, kd, a["causal"], a["input_pos"],
                          window, a["dtype"], None, config)


def test_fp8_validation(lib):
    assert call_fp8(lib, D=96) == -4                      # head dim 64 or 128
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert call_fp8(lib, qd=bad) == -6
        assert call_fp8(lib, kd=bad) == -6
    assert call_fp8(lib, scale=0.0, qd=0.0) == -6
    assert call_fp8(lib, window=3, causal=0) == -14
    assert call_fp8(lib, dtype=2) == -5
    assert call_fp8(lib, Sq=0, q=0, out=0, lse=0) == 0   # empty: no launch
    # q and k are 1 byte per element: out placed right after q (B*Hq*Sq*D bytes) is legal,
    # one byte earlier overlaps
    qbytes = 1 * 4 * 8 * 128
    assert call_fp8(lib, out=Q + qbytes, Sq=0) == 0
    assert call_fp8(lib, out=Q + qbytes - 16) == -9


def call_split_fp8(lib, num_splits=2, ws=W, ws_bytes=1 << 28, qd=0.01, kd=0.02, window=0,
                   config=-1, **over):
    a = dict(GOOD, **dict(dict(D=128), **over))
    return lib.fa_fwd_splitkv_fp8(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["Hq"],
                                  a["Hkv"], a["Sq"], a["Skv"], a["D"], a["scale"], qd, kd,
                                  a["causal"], a["input_pos"], window, a["dtype"], num_splits,
                                  config, ws, ws_bytes, None)


def test_fp8_splitkv_validation(lib):
    """fa_fwd_splitkv_fp8 runs fa_fwd_fp8's checks, then the split and workspace checks
    (no call here reaches a launch)."""
    assert call_split_fp8(lib, D=96) == -4
    assert call_split_fp8(lib, qd=float("nan")) == -6
    assert call_split_fp8(lib, kd=0.0) == -6
    assert call_split_fp8(lib, window=5, causal=0) == -14
    assert call_split_fp8(lib, num_splits=-1) == -12
    assert call_split_fp8(lib, num_splits=257) == -12
    assert call_split_fp8(lib, ws=None) == -1
    assert call_split_fp8(lib, ws=W + 8) == -8
    need = fa.splitkv_workspace_size(1, 4, 8, 128, 2)
    assert call_split_fp8(lib, ws_bytes=need - 1) == -13
    assert call_split_fp8(lib, ws=Q) == -9                # workspace overlapping q
    assert call_split_fp8(lib, Sq=0, q=0, out=0, lse=0) == 0
    names = fa.config_names()
    bf16 = names.index("D128_BN32_Mw1x32_WPH1_HPW4_causal_bf16")
    assert call_split_fp8(lib, config=bf16, dtype=1) == -10


def test_fp8_splitkv_num_splits(lib):
    """The split rule of fa_splitkv_num_splits with 3 bytes per K/V element: the decoding
    shape (32 workgroups) gets 16 ranges; a full grid gets 1."""
    f = lib.fa_splitkv_num_splits_fp8
    assert f(4, 32, 8, 1, 16384, 128, 1, 16383, 0, 1, -1) == 16
    assert f(1, 32, 4, 8192, 8192, 128, 1, 0, 0, 1, -1) == 1
    assert f(4, 32, 8, 1, 16384, 64, 1, 16383, 0, 1, -1) == 16
    assert f(4, 32, 8, 1, 16384, 96, 1, 16383, 0, 1, -1) == -4
    assert f(4, 32, 8, 1, 16384, 128, 1, 16383, 0, 3, -1) == -5
    assert fa.splitkv_num_splits_fp8(4, 32, 8, 1, 16384, 128, True, 16383, 1) == 16


def test_fp8_configs(lib):
    names = fa.config_names()
    fp8 = [i for i, nm in enumerate(names) if "_fp8qk_" in nm]
    assert len(fp8) == 52
    assert sum(names[i].startswith("D128_BN32_") for i in fp8) == 28
    assert sum(names[i].startswith("D64_BN64_") for i in fp8) == 24
    c = fa.select_config_fp8(1, 32, 4, 8192, 128, True, 1)
    assert names[c] == "D128_BN32_Mw1x32_WPH1_HPW8_causal_fp8qk_bf16"
    c = fa.select_config_fp8(1, 32, 32, 4096, 128, True, 0)
    assert names[c] == "D128_BN32_Mw1x32_WPH8_HPW1_causal_fp8qk_fp16"
    # a bf16 configuration is not applicable to an fp8 call, nor the reverse
    bf16 = names.index("D128_BN32_Mw1x32_WPH2_HPW4_causal_bf16")
    assert call_fp8(lib, config=bf16, dtype=1) == -10
    args = [GOOD[x] for x in ("q", "k", "v", "out", "lse", "B", "Hq", "Hkv", "Sq", "Skv")] + \
        [128, GOOD["scale"], 1, 0, 1, None]
    assert lib.fa_fwd_config(*args, fp8[0]) == -10
    c = fa.select_config_fp8(1, 32, 4, 8192, 64, True, 1)
    assert names[c] == "D64_BN64_Mw1x32_WPH2_HPW4_causal_fp8qk_bf16"
    with pytest.raises(fa.FaError):
        fa.select_config_fp8(1, 32, 4, 8192, 96, True, 1)


def test_header_compiles_as_c99():
    """include/fa_fwd.h is a C header: the plain-C test caller (which includes it) passes a
    C99 syntax check with warnings as errors."""
    import shutil
    import subprocess

    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("gcc not available")
    src = os.path.join(ROOT, "tests", "c", "fa_c_caller.c")
    r = subprocess.run([cc, "-std=c99", "-fsyntax-only", "-Wall", "-Wextra", "-Werror",
                        "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{ROOT}/include", src],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
