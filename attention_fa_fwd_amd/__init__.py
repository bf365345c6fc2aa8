"""MI355X (gfx950) FlashAttention-style attention forward pass.

A thin ctypes binding over the C ABI in ``include/fa_fwd.h`` (``libfa_fwd.so``,
built in-tree by ``attention_fa_fwd_amd.build``).  This module only marshals
torch tensors into pointers and sizes and passes the current HIP stream; every
step of the computation runs in the HIP kernels.  There is no fallback: if the
library is missing or the tensors are not on a GPU, the call raises.
"""

from __future__ import annotations

import ctypes
import math
import os
import threading

__all__ = ["fa_fwd", "fa_fwd_into", "fa_fwd_prepared", "fa_bwd", "fa_bwd_into", "bwd_workspace_size", "fa_fwd_fp8",
           "fa_fwd_fp8_into", "select_config_fp8", "fa_fwd_splitkv_fp8", "fa_fwd_splitkv_fp8_into",
           "splitkv_num_splits_fp8", "fa_fwd_splitkv", "fa_fwd_splitkv_into", "splitkv_num_splits",
           "fa_fwd_splitkv_noalloc", "fa_fwd_splitkv_noalloc_into", "NOALLOC_SCRATCH_BYTES",
           "fa_fwd_fp8qkv", "fa_fwd_fp8qkv_into", "fa_fwd_splitkv_fp8qkv", "fa_fwd_splitkv_fp8qkv_into",
           "splitkv_num_splits_fp8qkv",
           "splitkv_workspace_size", "select_config", "config_names", "num_configs", "FaError",
           "load_library", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_fwd.so")

FA_DTYPE_FP16 = 0
FA_DTYPE_BF16 = 1
# Size of the fixed split-KV scratch of fa_fwd_splitkv_noalloc (FA_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 64 << 20

_lib = None
_lock = threading.Lock()

_c_int, _c_float, _vp = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
_FWD_ARGS = [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float,
             _c_int, _c_int, _c_int, _vp]


class FaError(RuntimeError):
    """A nonzero status from the C ABI."""

    def __init__(self, code: int, message: str):
        super().__init__(f"fa_fwd failed ({code}): {message}")
        self.code = code


def _declare(lib):
    lib.fa_fwd.argtypes = _FWD_ARGS
    lib.fa_fwd.restype = _c_int
    lib.fa_fwd_config.argtypes = _FWD_ARGS + [_c_int]
    lib.fa_fwd_config.restype = _c_int
    lib.fa_bwd.argtypes = [_vp] * 9 + [_c_int] * 6 + [_c_float] + [_c_int] * 4 + [_vp, ctypes.c_size_t,
                                                                              _vp]
    lib.fa_bwd.restype = _c_int
    lib.fa_bwd_workspace_size.argtypes = [_c_int] * 7
    lib.fa_bwd_workspace_size.restype = ctypes.c_size_t
    lib.fa_fwd_fp8.argtypes = _FWD_ARGS[:12] + [_c_float, _c_float, _c_int, _c_int, _c_int, _c_int,
                                                _vp, _c_int]
    lib.fa_fwd_fp8.restype = _c_int
    lib.fa_select_config_fp8.argtypes = [_c_int] * 7
    lib.fa_select_config_fp8.restype = _c_int
    lib.fa_fwd_window.argtypes = _FWD_ARGS[:12] + [_c_int, _c_int, _c_int, _vp, _c_int]
    lib.fa_fwd_window.restype = _c_int
    lib.fa_fwd_splitkv.argtypes = _FWD_ARGS[:14] + [_c_int, _c_int, _c_int, _c_int, _vp,
                                                    ctypes.c_size_t, _vp]
    lib.fa_fwd_splitkv.restype = _c_int
    lib.fa_fwd_fp8qkv.argtypes = _FWD_ARGS[:12] + [_c_float] * 3 + [_c_int] * 4 + [_vp, _c_int]
    lib.fa_fwd_fp8qkv.restype = _c_int
    lib.fa_fwd_splitkv_fp8qkv.argtypes = _FWD_ARGS[:12] + [_c_float] * 3 + [_c_int] * 6 + [
        _vp, ctypes.c_size_t, _vp]
    lib.fa_fwd_splitkv_fp8qkv.restype = _c_int
    lib.fa_splitkv_num_splits_fp8qkv.argtypes = [_c_int] * 11
    lib.fa_splitkv_num_splits_fp8qkv.restype = _c_int
    lib.fa_fwd_splitkv_noalloc.argtypes = _FWD_ARGS[:14] + [_c_int, _c_int, _c_int, _c_int, _vp]
    lib.fa_fwd_splitkv_noalloc.restype = _c_int
    lib.fa_fwd_splitkv_fp8.argtypes = _FWD_ARGS[:12] + [_c_float, _c_float] + [_c_int] * 6 + [
        _vp, ctypes.c_size_t, _vp]
    lib.fa_fwd_splitkv_fp8.restype = _c_int
    lib.fa_splitkv_num_splits_fp8.argtypes = [_c_int] * 11
    lib.fa_splitkv_num_splits_fp8.restype = _c_int
    lib.fa_splitkv_num_splits.argtypes = [_c_int] * 11
    lib.fa_splitkv_num_splits.restype = _c_int
    lib.fa_splitkv_workspace_size.argtypes = [_c_int] * 5
    lib.fa_splitkv_workspace_size.restype = ctypes.c_size_t
    lib.fa_select_config.argtypes = [_c_int] * 9
    lib.fa_select_config.restype = _c_int
    lib.fa_num_configs.argtypes = []
    lib.fa_num_configs.restype = _c_int
    lib.fa_config_name.argtypes = [_c_int]
    lib.fa_config_name.restype = ctypes.c_char_p
    lib.fa_strerror.argtypes = [_c_int]
    lib.fa_strerror.restype = ctypes.c_char_p
    return lib


def load_library(path: str = LIB_PATH):
    """Load ``libfa_fwd.so`` and declare the C signatures.

    The in-tree library is loaded once and cached; another ``path`` is loaded
    on its own.  Raises RuntimeError if the file does not exist.
    """
    global _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"HIP attention library not built: {path} is missing "
            "(run `python -m attention_fa_fwd_amd.build` or __graft_entry__.build())")
    if path != LIB_PATH:
        return _declare(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            _lib = _declare(ctypes.CDLL(path))
        return _lib


def _dtype_code(dtype) -> int:
    import torch

    if dtype == torch.float16:
        return FA_DTYPE_FP16
    if dtype == torch.bfloat16:
        return FA_DTYPE_BF16
    raise TypeError(f"unsupported dtype {dtype}: expected torch.float16 or torch.bfloat16")


def _check(rc: int):
    if rc != 0:
        raise FaError(rc, load_library().fa_strerror(rc).decode())


def _check_tensors(q, k, v, out, lse):
    """Shapes, dtypes, devices and contiguity of one call; returns (B, Hq, Hkv, Sq, Skv, D)."""
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("lse", lse)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, S, D]")
    if k.dtype != q.dtype or v.dtype != q.dtype or out.dtype != q.dtype:
        raise TypeError("q, k, v and out must share one dtype")
    if lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Skv, Dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or Dk != D:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != (B, Hq, Sq):
        raise ValueError("out must match q and lse must be [B, Hq, Sq]")
    return B, Hq, Hkv, Sq, Skv, D


def _check_window(causal, window):
    if window < 0 or (window > 0 and not causal):
        raise ValueError("window must be >= 0 and a sliding window needs causal=True")


def fa_fwd_into(q, k, v, out, lse, scale=None, causal=True, input_pos=0, config=-1, stream=None,
                window=0):
    """Run the kernel into caller-provided ``out`` [B,Hq,Sq,D] and ``lse`` [B,Hq,Sq] (fp32).

    All tensors must be contiguous and on the same GPU.  ``stream`` is a raw
    hipStream_t value; by default torch's current stream on q's device.
    ``window`` > 0 restricts causal attention to a sliding window of that many keys
    (query i sees keys input_pos + i - window + 1 .. input_pos + i; fa_fwd_window).
    """
    import torch

    lib = load_library()
    B, Hq, Hkv, Sq, Skv, D = _check_tensors(q, k, v, out, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    _check_window(causal, window)
    with torch.cuda.device(q.device):
        if window > 0:
            rc = lib.fa_fwd_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   lse.data_ptr(), B, Hq, Hkv, Sq, Skv, D, float(scale),
                                   int(input_pos), int(window), _dtype_code(q.dtype), stream,
                                   int(config))
        else:
            rc = lib.fa_fwd_config(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   lse.data_ptr(), B, Hq, Hkv, Sq, Skv, D, float(scale),
                                   1 if causal else 0, int(input_pos), _dtype_code(q.dtype),
                                   stream, int(config))
    _check(rc)
    return out, lse


def fa_fwd_prepared(q, k, v, out, lse, scale=None, causal=True, input_pos=0, config=-1, stream=None,
                    window=0):
    """``fa_fwd_into`` with its argument checks and marshalling done once: returns a callable
    that, each time it is called, enqueues the same forward pass (same tensors, scale, masking,
    configuration and stream) with one C call.  For launch loops whose per-call host time
    matters (a short problem runs in a few microseconds on the GPU).  The callable holds
    references to the tensors; their storage must not be resized or replaced while it is used.
    A nonzero status raises FaError as in fa_fwd_into."""
    import torch

    lib = load_library()
    B, Hq, Hkv, Sq, Skv, D = _check_tensors(q, k, v, out, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    _check_window(causal, window)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq, Hkv,
            Sq, Skv, D, float(scale))
    if window > 0:
        fn, args = lib.fa_fwd_window, ptrs + (int(input_pos), int(window), _dtype_code(q.dtype),
                                              stream, int(config))
    else:
        fn, args = lib.fa_fwd_config, ptrs + (1 if causal else 0, int(input_pos),
                                              _dtype_code(q.dtype), stream, int(config))
    keep = (q, k, v, out, lse)

    def call():
        rc = fn(*args)
        if rc != 0:
            _check(rc)
        return keep[3], keep[4]

    return call


def splitkv_num_splits(B, Hq, Hkv, Sq, Skv, D, causal, input_pos, dtype, config=-1, window=0) -> int:
    """Split count fa_fwd_splitkv picks for num_splits=0 (dtype: torch dtype or FA code)."""
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    rc = load_library().fa_splitkv_num_splits(B, Hq, Hkv, Sq, Skv, D, 1 if causal else 0,
                                              input_pos, window, code, config)
    _check(rc if rc < 0 else 0)
    return rc


def splitkv_workspace_size(B, Hq, Sq, D, num_splits) -> int:
    """Workspace bytes fa_fwd_splitkv needs for ``num_splits`` key ranges."""
    return int(load_library().fa_splitkv_workspace_size(B, Hq, Sq, D, num_splits))


def fa_fwd_splitkv_into(q, k, v, out, lse, workspace, num_splits=0, scale=None, causal=True,
                        input_pos=0, config=-1, stream=None, window=0):
    """Split-KV forward into caller-provided ``out``, ``lse`` and ``workspace``.

    ``workspace`` is a contiguous GPU tensor of at least
    ``splitkv_workspace_size(B, Hq, Sq, D, splits)`` bytes (None when one split runs).
    ``num_splits`` = 0 lets the library choose.
    """
    import torch

    lib = load_library()
    B, Hq, Hkv, Sq, Skv, D = _check_tensors(q, k, v, out, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    if workspace is not None:
        if not workspace.is_cuda or workspace.device != q.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on q's device")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    else:
        ws_ptr, ws_bytes = None, 0
    with torch.cuda.device(q.device):
        rc = lib.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                lse.data_ptr(), B, Hq, Hkv, Sq, Skv, D, float(scale),
                                1 if causal else 0, int(input_pos), int(window),
                                _dtype_code(q.dtype), int(num_splits), int(config), ws_ptr,
                                ws_bytes, stream)
    _check(rc)
    return out, lse


def fa_fwd_splitkv(q, k, v, scale=None, causal=True, input_pos=0, num_splits=0, config=-1,
                   window=0):
    """Split-KV attention forward: the same result as ``fa_fwd`` (up to rounding order),
    computed over ``num_splits`` key ranges (0 = the library's choice) and merged.
    Allocates the workspace with torch; returns (out, lse)."""
    import torch

    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    B, Hq, Sq, D = q.shape
    _, Hkv, Skv, _ = k.shape
    if num_splits == 0:
        num_splits = splitkv_num_splits(B, Hq, Hkv, Sq, Skv, D, causal, input_pos, q.dtype, config,
                                        window)
    nbytes = splitkv_workspace_size(B, Hq, Sq, D, num_splits)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device) if nbytes else None
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    return fa_fwd_splitkv_into(q, k, v, out, lse, ws, num_splits=num_splits, scale=scale,
                               causal=causal, input_pos=input_pos, config=config, window=window)


def fa_fwd_splitkv_noalloc_into(q, k, v, out, lse, num_splits=0, scale=None, causal=True,
                                input_pos=0, config=-1, stream=None, window=0):
    """Split-KV forward into caller-provided ``out`` and ``lse`` with no workspace: the
    partials live in the library's fixed scratch (``NOALLOC_SCRATCH_BYTES`` per GPU), so
    the call allocates nothing.  Calls that overlap in time on one GPU share that scratch
    and must not run concurrently."""
    import torch

    lib = load_library()
    B, Hq, Hkv, Sq, Skv, D = _check_tensors(q, k, v, out, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        rc = lib.fa_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                        lse.data_ptr(), B, Hq, Hkv, Sq, Skv, D, float(scale),
                                        1 if causal else 0, int(input_pos), int(window),
                                        _dtype_code(q.dtype), int(num_splits), int(config), stream)
    _check(rc)
    return out, lse


def fa_fwd_splitkv_noalloc(q, k, v, scale=None, causal=True, input_pos=0, num_splits=0, config=-1,
                           window=0):
    """``fa_fwd_splitkv`` without a workspace (the library's fixed scratch holds the
    partials); allocates only ``out`` and ``lse``.  Returns (out, lse)."""
    import torch

    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    return fa_fwd_splitkv_noalloc_into(q, k, v, out, lse, num_splits=num_splits, scale=scale,
                                       causal=causal, input_pos=input_pos, config=config,
                                       window=window)


def fa_fwd(q, k, v, scale=None, causal=True, input_pos=0, config=-1, window=0):
    """Attention forward: returns (out [B,Hq,Sq,D] in q's dtype, lse [B,Hq,Sq] fp32).

    q: [B,Hq,Sq,D]; k, v: [B,Hkv,Skv,D]; fp16 or bf16 on one GPU.  ``scale``
    defaults to 1/sqrt(D); ``causal`` to True; under causal masking query i
    sees key j iff j <= input_pos + i.  Inputs are made contiguous.
    """
    import torch

    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    return fa_fwd_into(q, k, v, out, lse, scale=scale, causal=causal, input_pos=input_pos,
                       config=config, window=window)


def select_config(B, Hq, Hkv, Sq, Skv, D, causal, input_pos, dtype) -> int:
    """Configuration id the dispatch table picks (dtype: torch dtype or FA code)."""
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    rc = load_library().fa_select_config(B, Hq, Hkv, Sq, Skv, D, 1 if causal else 0, input_pos, code)
    _check(rc if rc < 0 else 0)
    return rc


def num_configs() -> int:
    return load_library().fa_num_configs()


def config_names():
    lib = load_library()
    return [lib.fa_config_name(i).decode() for i in range(lib.fa_num_configs())]


def _check_fp8_tensors(q8, k8, v, out, lse):
    """Device, contiguity, dtype and shape checks of the fp8 entry points; returns the sizes."""
    import torch

    for name, t in (("q8", q8), ("k8", k8), ("v", v), ("out", out), ("lse", lse)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.device != q8.device:
            raise ValueError(f"{name} is on {t.device}, q8 on {q8.device}")
    if q8.dtype != torch.float8_e4m3fn or k8.dtype != torch.float8_e4m3fn:
        raise TypeError("q8 and k8 must be torch.float8_e4m3fn")
    if out.dtype != v.dtype:
        raise TypeError("out must have v's dtype")
    if lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    B, Hq, Sq, D = q8.shape
    Bk, Hkv, Skv, Dk = k8.shape
    if tuple(v.shape) != tuple(k8.shape) or Bk != B or Dk != D:
        raise ValueError(f"shape mismatch q{tuple(q8.shape)} k{tuple(k8.shape)} v{tuple(v.shape)}")
    if tuple(out.shape) != tuple(q8.shape) or tuple(lse.shape) != (B, Hq, Sq):
        raise ValueError("out must be [B, Hq, Sq, D] and lse [B, Hq, Sq]")
    return B, Hq, Hkv, Sq, Skv, D


def fa_fwd_fp8_into(q8, k8, v, out, lse, q_descale, k_descale, scale=None, causal=True,
                    input_pos=0, window=0, config=-1, stream=None):
    """fp8 E4M3 q8 [B,Hq,Sq,D], k8 [B,Hkv,Skv,D] (torch.float8_e4m3fn) with per-tensor
    descale factors; v [B,Hkv,Skv,D] and out in fp16 / bf16; lse fp32 (fa_fwd_fp8)."""
    import torch

    lib = load_library()
    B, Hq, Hkv, Sq, Skv, D = _check_fp8_tensors(q8, k8, v, out, lse)
    _check_window(causal, window)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if stream is None:
        stream = torch.cuda.current_stream(q8.device).cuda_stream
    with torch.cuda.device(q8.device):
        rc = lib.fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v.data_ptr(), out.data_ptr(),
                            lse.data_ptr(), B, Hq, Hkv, Sq, Skv, D, float(scale),
                            float(q_descale), float(k_descale), 1 if causal else 0,
                            int(input_pos), int(window), _dtype_code(v.dtype), stream,
                            int(config))
    _check(rc)
    return out, lse


def fa_fwd_fp8(q8, k8, v, q_descale, k_descale, scale=None, causal=True, input_pos=0, window=0,
               config=-1):
    """Attention with fp8 E4M3 queries and keys (real values q_descale * q8, k_descale * k8)
    and fp16 / bf16 values: returns (out in v's dtype, lse fp32)."""
    import torch

    q8, k8, v = q8.contiguous(), k8.contiguous(), v.contiguous()
    out = torch.empty(q8.shape, dtype=v.dtype, device=q8.device)
    lse = torch.empty(q8.shape[:3], dtype=torch.float32, device=q8.device)
    return fa_fwd_fp8_into(q8, k8, v, out, lse, q_descale, k_descale, scale=scale, causal=causal,
                           input_pos=input_pos, window=window, config=config)


def splitkv_num_splits_fp8(B, Hq, Hkv, Sq, Skv, D, causal, input_pos, v_dtype, config=-1,
                           window=0) -> int:
    """Split count fa_fwd_splitkv_fp8 picks for num_splits=0 (v_dtype: torch dtype or code)."""
    code = v_dtype if isinstance(v_dtype, int) else _dtype_code(v_dtype)
    rc = load_library().fa_splitkv_num_splits_fp8(B, Hq, Hkv, Sq, Skv, D, 1 if causal else 0,
                                                  int(input_pos), int(window), code, int(config))
    _check(rc if rc < 0 else 0)
    return rc


def fa_fwd_splitkv_fp8_into(q8, k8, v, out, lse, workspace, q_descale, k_descale, num_splits=0,
                            scale=None, causal=True, input_pos=0, window=0, config=-1,
                            stream=None):
    """Split-KV forward with fp8 E4M3 q8, k8 and fp16 / bf16 v into caller-provided
    ``out``, ``lse`` and ``workspace`` (``splitkv_workspace_size`` bytes; None when one
    split runs)."""
    import torch

    lib = load_library()
    B, Hq, Hkv, Sq, Skv, D = _check_fp8_tensors(q8, k8, v, out, lse)
    _check_window(causal, window)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if stream is None:
        stream = torch.cuda.current_stream(q8.device).cuda_stream
    if workspace is not None:
        if not workspace.is_cuda or workspace.device != q8.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on q8's device")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    else:
        ws_ptr, ws_bytes = None, 0
    with torch.cuda.device(q8.device):
        rc = lib.fa_fwd_splitkv_fp8(q8.data_ptr(), k8.data_ptr(), v.data_ptr(), out.data_ptr(),
                                    lse.data_ptr(), B, Hq, Hkv, Sq, Skv, D, float(scale),
                                    float(q_descale), float(k_descale), 1 if causal else 0,
                                    int(input_pos), int(window), _dtype_code(v.dtype),
                                    int(num_splits), int(config), ws_ptr, ws_bytes, stream)
    _check(rc)
    return out, lse


def fa_fwd_splitkv_fp8(q8, k8, v, q_descale, k_descale, scale=None, causal=True, input_pos=0,
                       num_splits=0, window=0, config=-1):
    """Split-KV attention with fp8 E4M3 queries and keys; allocates out, lse and the
    workspace with torch."""
    import torch

    q8, k8, v = q8.contiguous(), k8.contiguous(), v.contiguous()
    B, Hq, Sq, D = q8.shape
    Hkv, Skv = k8.shape[1], k8.shape[2]
    if num_splits == 0:
        num_splits = splitkv_num_splits_fp8(B, Hq, Hkv, Sq, Skv, D, causal, input_pos, v.dtype,
                                            config, window)
    out = torch.empty(q8.shape, dtype=v.dtype, device=q8.device)
    lse = torch.empty(q8.shape[:3], dtype=torch.float32, device=q8.device)
    nbytes = splitkv_workspace_size(B, Hq, Sq, D, num_splits)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q8.device) if nbytes else None
    return fa_fwd_splitkv_fp8_into(q8, k8, v, out, lse, ws, q_descale, k_descale,
                                   num_splits=num_splits, scale=scale, causal=causal,
                                   input_pos=input_pos, window=window, config=config)


def _check_fp8qkv_tensors(q8, k8, v8, out, lse):
    """Checks of the fp8 Q/K/V entry points: q8, k8, v8 float8_e4m3fn; out fp16 / bf16;
    lse fp32; all contiguous on one GPU.  Returns (B, Hq, Hkv, Sq, Skv, D)."""
    import torch

    for name, t in (("q8", q8), ("k8", k8), ("v8", v8), ("out", out), ("lse", lse)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.device != q8.device:
            raise ValueError(f"{name} is on {t.device}, q8 on {q8.device}")
    if any(t.dtype != torch.float8_e4m3fn for t in (q8, k8, v8)):
        raise TypeError("q8, k8 and v8 must be torch.float8_e4m3fn")
    if out.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("out must be float16 or bfloat16")
    if lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    B, Hq, Sq, D = q8.shape
    Bk, Hkv, Skv, Dk = k8.shape
    if tuple(v8.shape) != tuple(k8.shape) or Bk != B or Dk != D:
        raise ValueError(f"shape mismatch q{tuple(q8.shape)} k{tuple(k8.shape)} v{tuple(v8.shape)}")
    if tuple(out.shape) != tuple(q8.shape) or tuple(lse.shape) != (B, Hq, Sq):
        raise ValueError("out must be [B, Hq, Sq, D] and lse [B, Hq, Sq]")
    return B, Hq, Hkv, Sq, Skv, D


def fa_fwd_fp8qkv_into(q8, k8, v8, out, lse, q_descale, k_descale, v_descale, scale=None,
                       causal=True, input_pos=0, window=0, config=-1, stream=None):
    """fp8 E4M3 q8, k8, v8 (torch.float8_e4m3fn) with per-tensor descale factors into
    caller-provided out (fp16 / bf16) and lse fp32 (fa_fwd_fp8qkv)."""
    import torch

    lib = load_library()
    B, Hq, Hkv, Sq, Skv, D = _check_fp8qkv_tensors(q8, k8, v8, out, lse)
    _check_window(causal, window)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if stream is None:
        stream = torch.cuda.current_stream(q8.device).cuda_stream
    with torch.cuda.device(q8.device):
        rc = lib.fa_fwd_fp8qkv(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), out.data_ptr(),
                               lse.data_ptr(), B, Hq, Hkv, Sq, Skv, D, float(scale),
                               float(q_descale), float(k_descale), float(v_descale),
                               1 if causal else 0, int(input_pos), int(window),
                               _dtype_code(out.dtype), stream, int(config))
    _check(rc)
    return out, lse


def fa_fwd_fp8qkv(q8, k8, v8, q_descale, k_descale, v_descale, out_dtype=None, scale=None,
                  causal=True, input_pos=0, window=0, config=-1):
    """Attention with fp8 E4M3 queries, keys and values (real values descale * codes):
    returns (out in out_dtype, default bfloat16; lse fp32)."""
    import torch

    q8, k8, v8 = q8.contiguous(), k8.contiguous(), v8.contiguous()
    out = torch.empty(q8.shape, dtype=out_dtype or torch.bfloat16, device=q8.device)
    lse = torch.empty(q8.shape[:3], dtype=torch.float32, device=q8.device)
    return fa_fwd_fp8qkv_into(q8, k8, v8, out, lse, q_descale, k_descale, v_descale, scale=scale,
                              causal=causal, input_pos=input_pos, window=window, config=config)


def splitkv_num_splits_fp8qkv(B, Hq, Hkv, Sq, Skv, D, causal, input_pos, out_dtype, config=-1,
                              window=0) -> int:
    """Split count fa_fwd_splitkv_fp8qkv picks for num_splits=0."""
    code = out_dtype if isinstance(out_dtype, int) else _dtype_code(out_dtype)
    rc = load_library().fa_splitkv_num_splits_fp8qkv(B, Hq, Hkv, Sq, Skv, D, 1 if causal else 0,
                                                     int(input_pos), int(window), code,
                                                     int(config))
    _check(rc if rc < 0 else 0)
    return rc


def fa_fwd_splitkv_fp8qkv_into(q8, k8, v8, out, lse, workspace, q_descale, k_descale, v_descale,
                               num_splits=0, scale=None, causal=True, input_pos=0, window=0,
                               config=-1, stream=None):
    """Split-KV forward with fp8 E4M3 q8, k8, v8 into caller-provided out, lse and workspace
    (``splitkv_workspace_size`` bytes; None when one split runs)."""
    import torch

    lib = load_library()
    B, Hq, Hkv, Sq, Skv, D = _check_fp8qkv_tensors(q8, k8, v8, out, lse)
    _check_window(causal, window)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if stream is None:
        stream = torch.cuda.current_stream(q8.device).cuda_stream
    if workspace is not None:
        if not workspace.is_cuda or workspace.device != q8.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on q8's device")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    else:
        ws_ptr, ws_bytes = None, 0
    with torch.cuda.device(q8.device):
        rc = lib.fa_fwd_splitkv_fp8qkv(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(),
                                       out.data_ptr(), lse.data_ptr(), B, Hq, Hkv, Sq, Skv, D,
                                       float(scale), float(q_descale), float(k_descale),
                                       float(v_descale), 1 if causal else 0, int(input_pos),
                                       int(window), _dtype_code(out.dtype), int(num_splits),
                                       int(config), ws_ptr, ws_bytes, stream)
    _check(rc)
    return out, lse


def fa_fwd_splitkv_fp8qkv(q8, k8, v8, q_descale, k_descale, v_descale, out_dtype=None, scale=None,
                          causal=True, input_pos=0, num_splits=0, window=0, config=-1):
    """Split-KV attention with fp8 E4M3 queries, keys and values; allocates out, lse and the
    workspace with torch."""
    import torch

    q8, k8, v8 = q8.contiguous(), k8.contiguous(), v8.contiguous()
    B, Hq, Sq, D = q8.shape
    Hkv, Skv = k8.shape[1], k8.shape[2]
    dt = out_dtype or torch.bfloat16
    if num_splits == 0:
        num_splits = splitkv_num_splits_fp8qkv(B, Hq, Hkv, Sq, Skv, D, causal, input_pos, dt,
                                               config, window)
    out = torch.empty(q8.shape, dtype=dt, device=q8.device)
    lse = torch.empty(q8.shape[:3], dtype=torch.float32, device=q8.device)
    nbytes = splitkv_workspace_size(B, Hq, Sq, D, num_splits)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q8.device) if nbytes else None
    return fa_fwd_splitkv_fp8qkv_into(q8, k8, v8, out, lse, ws, q_descale, k_descale, v_descale,
                                      num_splits=num_splits, scale=scale, causal=causal,
                                      input_pos=input_pos, window=window, config=config)


def select_config_fp8(B, Hq, Hkv, Sq, D, causal, v_dtype) -> int:
    """Configuration fa_fwd_fp8 picks (v_dtype: torch dtype or FA code)."""
    code = v_dtype if isinstance(v_dtype, int) else _dtype_code(v_dtype)
    rc = load_library().fa_select_config_fp8(B, Hq, Hkv, Sq, D, 1 if causal else 0, code)
    _check(rc if rc < 0 else 0)
    return rc


def fa_bwd_into(q, k, v, out, lse, dout, dq, dk, dv, workspace, scale=None, causal=True,
                input_pos=0, window=0, stream=None):
    """Backward pass into caller-provided dq [B,Hq,Sq,D], dk, dv [B,Hkv,Skv,D] (q's dtype).

    ``out`` and ``lse`` are the forward pass's results for the same arguments;
    ``workspace`` holds at least ``bwd_workspace_size(...)`` bytes.
    """
    import torch

    lib = load_library()
    B, Hq, Hkv, Sq, Skv, D = _check_tensors(q, k, v, out, lse)
    for name, t, ref in (("dout", dout, q), ("dq", dq, q), ("dk", dk, k), ("dv", dv, k)):
        if not t.is_cuda or t.device != q.device or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor on q's device")
        if tuple(t.shape) != tuple(ref.shape) or t.dtype != q.dtype:
            raise ValueError(f"{name} must have shape {tuple(ref.shape)} and dtype {q.dtype}")
    _check_window(causal, window)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    if workspace is not None:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    else:
        ws_ptr, ws_bytes = None, 0
    with torch.cuda.device(q.device):
        rc = lib.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                        dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv,
                        Sq, Skv, D, float(scale), 1 if causal else 0, int(input_pos), int(window),
                        _dtype_code(q.dtype), ws_ptr, ws_bytes, stream)
    _check(rc)
    return dq, dk, dv


def bwd_workspace_size(B, Hq, Hkv, Sq, Skv, D, causal=True):
    """Workspace bytes fa_bwd needs: the row statistics plus, for a small K/V grid with a
    head group to split, fp32 partial dk / dv sums."""
    return int(load_library().fa_bwd_workspace_size(B, Hq, Hkv, Sq, Skv, D, 1 if causal else 0))


def fa_bwd(q, k, v, out, lse, dout, scale=None, causal=True, input_pos=0, window=0):
    """Gradients (dq, dk, dv) of the forward pass for upstream gradient ``dout``;
    allocates the outputs and the workspace with torch."""
    import torch

    q, k, v, out, dout = (t.contiguous() for t in (q, k, v, out, dout))
    B, Hq, Sq, D = q.shape
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nbytes = bwd_workspace_size(B, Hq, k.shape[1], Sq, k.shape[2], D, causal)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    return fa_bwd_into(q, k, v, out, lse.contiguous(), dout, dq, dk, dv, ws, scale=scale,
                       causal=causal, input_pos=input_pos, window=window)
