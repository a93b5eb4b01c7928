"""ctypes binding of libfa (``include/fa.h``).

Argument marshalling only: every step of the forward pass runs in the HIP
kernels of ``libfa.so``.  PyTorch supplies device memory and the current
stream.  If the library is missing this module raises at load time; there is
no CPU fallback.
"""
from __future__ import annotations

import ctypes
import math
from pathlib import Path

import torch

_LIB_PATH = Path(__file__).resolve().parent / "libfa.so"

FA_F32, FA_BF16, FA_F16 = 0, 1, 2
FA_OK = 0
STATUS_NAMES = {0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_HEAD_DIM",
                4: "FA_ERR_DTYPE", 5: "FA_ERR_SCALE", 6: "FA_ERR_ALIGN", 7: "FA_ERR_ALIAS",
                8: "FA_ERR_LAUNCH"}
_DTYPE_CODES = {torch.float32: FA_F32, torch.bfloat16: FA_BF16, torch.float16: FA_F16}

# Every symbol include/fa.h declares.
EXPORTED = ("fa_fwd", "fa_strerror", "fa_version")

_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {strerror(status)}")


def library_path() -> Path:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libfa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not _LIB_PATH.exists():
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with `python -m exact_attention_13_amd.build`")
        lib = ctypes.CDLL(str(_LIB_PATH))
        lib.fa_fwd.restype = ctypes.c_int
        lib.fa_fwd.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_void_p] + [ctypes.c_int64] * 4 + [
            ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        lib.fa_strerror.restype = ctypes.c_char_p
        lib.fa_strerror.argtypes = [ctypes.c_int]
        lib.fa_version.restype = ctypes.c_int
        lib.fa_version.argtypes = []
        _lib = lib
    return _lib


def strerror(status: int) -> str:
    return load().fa_strerror(int(status)).decode()


def version() -> int:
    return int(load().fa_version())


def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, stream) -> int:
    """Raw C call with integer pointers; returns the fa_status code."""
    return int(load().fa_fwd(q, k, v, o, lse, int(B), int(H), int(N), int(d), float(scale),
                             int(bool(causal)), int(dtype), stream))


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float | None = None,
        causal: bool = False, out: torch.Tensor | None = None,
        lse: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None):
    """O = softmax(Q K^T * scale) V and LSE for [B, H, N, d] CUDA tensors.

    Returns ``(o, lse)``: ``o`` has q's dtype and shape, ``lse`` is fp32
    [B, H, N].  Runs asynchronously on ``stream`` (default: the current
    stream).  ``scale`` defaults to 1/sqrt(d).
    """
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must be [B, H, N, d] tensors of one shape")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DTYPE_CODES:
        raise TypeError("q, k, v must share one dtype: float32, bfloat16 or float16")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be GPU tensors")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of q's shape and dtype")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                B, H, N, d, scale, causal, _DTYPE_CODES[q.dtype], stream.cuda_stream)
    if st != FA_OK:
        raise FaError(st)
    return out, lse
