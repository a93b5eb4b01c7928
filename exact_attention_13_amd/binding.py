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
                8: "FA_ERR_LAUNCH", 9: "FA_ERR_WORKSPACE", 10: "FA_ERR_SCRATCH"}
# Bytes of fa_fwd_ex_noalloc's static device scratch (FA_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024
_DTYPE_CODES = {torch.float32: FA_F32, torch.bfloat16: FA_BF16, torch.float16: FA_F16}

# Every symbol include/fa.h declares.
EXPORTED = ("fa_bwd", "fa_bwd_ex", "fa_bwd_ex_default_splits", "fa_bwd_ex_workspace_bytes",
            "fa_fwd", "fa_fwd_ex", "fa_fwd_ex_default_splits", "fa_fwd_ex_noalloc",
            "fa_fwd_ex_workspace_bytes", "fa_lse_combine", "fa_strerror", "fa_version")

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
        lib.fa_fwd_ex.restype = ctypes.c_int
        lib.fa_fwd_ex.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 6 + [
            ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_void_p]
        lib.fa_fwd_ex_noalloc.restype = ctypes.c_int
        lib.fa_fwd_ex_noalloc.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 6 + [
            ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p]
        lib.fa_fwd_ex_workspace_bytes.restype = ctypes.c_int64
        lib.fa_fwd_ex_workspace_bytes.argtypes = [ctypes.c_int64] * 6
        lib.fa_fwd_ex_default_splits.restype = ctypes.c_int64
        lib.fa_fwd_ex_default_splits.argtypes = [ctypes.c_int64] * 6 + [ctypes.c_int, ctypes.c_int]
        lib.fa_lse_combine.restype = ctypes.c_int
        lib.fa_lse_combine.argtypes = [ctypes.c_void_p] * 2 + [ctypes.c_int64] * 3 + [
            ctypes.c_void_p] * 2 + [ctypes.c_int, ctypes.c_void_p]
        lib.fa_bwd.restype = ctypes.c_int
        lib.fa_bwd.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int64] * 4 + [
            ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        lib.fa_bwd_ex.restype = ctypes.c_int
        lib.fa_bwd_ex.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int64] * 6 + [
            ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_void_p]
        lib.fa_bwd_ex_workspace_bytes.restype = ctypes.c_int64
        lib.fa_bwd_ex_workspace_bytes.argtypes = [ctypes.c_int64] * 7
        lib.fa_bwd_ex_default_splits.restype = ctypes.c_int64
        lib.fa_bwd_ex_default_splits.argtypes = [ctypes.c_int64] * 6 + [ctypes.c_int, ctypes.c_int]
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


def _launch_stream(stream, device) -> torch.cuda.Stream:
    """The stream a call runs on; tensors the binding allocates for the call are
    allocated under it, so the caching allocator hands their memory to later
    work only behind the call's kernels (a scratch tensor allocated under
    another stream could be reused while the kernels still read it)."""
    return stream if stream is not None else torch.cuda.current_stream(device)


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
    stream = _launch_stream(stream, q.device)
    with torch.cuda.stream(stream):
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of q's shape and dtype")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor")
    st = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                B, H, N, d, scale, causal, _DTYPE_CODES[q.dtype], stream.cuda_stream)
    if st != FA_OK:
        raise FaError(st)
    return out, lse


def fa_fwd_ex(q, k, v, o, lse, B, H, H_kv, N_q, N_kv, d, scale, causal, dtype, num_splits,
              workspace, workspace_bytes, stream) -> int:
    """Raw C call with integer pointers; returns the fa_status code."""
    return int(load().fa_fwd_ex(q, k, v, o, lse, int(B), int(H), int(H_kv), int(N_q), int(N_kv),
                                int(d), float(scale), int(bool(causal)), int(dtype),
                                int(num_splits), workspace, int(workspace_bytes), stream))


def fa_fwd_ex_noalloc(q, k, v, o, lse, B, H, H_kv, N_q, N_kv, d, scale, causal, dtype,
                      num_splits, stream) -> int:
    """Raw C call with integer pointers; returns the fa_status code."""
    return int(load().fa_fwd_ex_noalloc(q, k, v, o, lse, int(B), int(H), int(H_kv), int(N_q),
                                        int(N_kv), int(d), float(scale), int(bool(causal)),
                                        int(dtype), int(num_splits), stream))


def workspace_bytes(B, H, N_q, N_kv, d, num_splits) -> int:
    return int(load().fa_fwd_ex_workspace_bytes(int(B), int(H), int(N_q), int(N_kv), int(d),
                                                int(num_splits)))


def default_splits(B, H, H_kv, N_q, N_kv, d, causal, dtype) -> int:
    return int(load().fa_fwd_ex_default_splits(int(B), int(H), int(H_kv), int(N_q), int(N_kv),
                                               int(d), int(bool(causal)), int(dtype)))


def fa_lse_combine(o_part, lse_part, splits, rows, d, o, lse, dtype, stream) -> int:
    """Raw C call with integer pointers; returns the fa_status code."""
    return int(load().fa_lse_combine(o_part, lse_part, int(splits), int(rows), int(d), o, lse,
                                     int(dtype), stream))


def fwd_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float | None = None,
           causal: bool = False, num_splits: int | None = None,
           out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
           workspace: torch.Tensor | None = None,
           stream: torch.cuda.Stream | None = None):
    """Attention with q [B, H, N_q, d] and k, v [B, H_kv, N_kv, d].

    Query head h reads K/V head h // (H // H_kv); causal masking is aligned
    to the end of the keys (key j hidden from query i when
    j > i + N_kv - N_q).  ``num_splits`` (default: the library's choice)
    splits the keys into ranges merged by logsumexp; the workspace it needs
    is allocated here unless given.  Returns ``(o, lse)``.
    """
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, H, N_q, d]; k and v one [B, H_kv, N_kv, d] shape")
    B, H, N_q, d = q.shape
    Bk, H_kv, N_kv, dk = k.shape
    if Bk != B or dk != d:
        raise ValueError("q, k, v must share B and d")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DTYPE_CODES:
        raise TypeError("q, k, v must share one dtype: float32, bfloat16 or float16")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be GPU tensors")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    dt = _DTYPE_CODES[q.dtype]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if num_splits is None:
        num_splits = default_splits(B, H, H_kv, N_q, N_kv, d, causal, dt)
    stream = _launch_stream(stream, q.device)
    with torch.cuda.stream(stream):
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((B, H, N_q), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of q's shape and dtype")
    if lse.shape != (B, H, N_q) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N_q] tensor")
    need = workspace_bytes(B, H, N_q, N_kv, d, num_splits)
    if need < 0:
        raise FaError(2)
    if workspace is None and need > 0:
        with torch.cuda.stream(stream):
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                   B, H, H_kv, N_q, N_kv, d, scale, causal, dt, num_splits, ws_ptr, ws_len,
                   stream.cuda_stream)
    if st != FA_OK:
        raise FaError(st)
    return out, lse


def lse_combine(o_part: torch.Tensor, lse_part: torch.Tensor, dtype: torch.dtype,
                out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                stream: torch.cuda.Stream | None = None):
    """Merge per-range results: o_part fp32 [S, rows, d], lse_part fp32 [S, rows].

    Returns ``(o, lse)`` with o [rows, d] of ``dtype`` and lse fp32 [rows].
    """
    if o_part.dim() != 3 or lse_part.shape != o_part.shape[:2]:
        raise ValueError("o_part must be [S, rows, d] and lse_part [S, rows]")
    if o_part.dtype != torch.float32 or lse_part.dtype != torch.float32:
        raise TypeError("partials are float32")
    if not (o_part.is_cuda and lse_part.is_cuda):
        raise ValueError("partials must be GPU tensors")
    if not (o_part.is_contiguous() and lse_part.is_contiguous()):
        raise ValueError("partials must be contiguous")
    if dtype not in _DTYPE_CODES:
        raise TypeError("dtype must be float32, bfloat16 or float16")
    S, rows, d = o_part.shape
    stream = _launch_stream(stream, o_part.device)
    with torch.cuda.stream(stream):
        if out is None:
            out = torch.empty((rows, d), dtype=dtype, device=o_part.device)
        if lse is None:
            lse = torch.empty((rows,), dtype=torch.float32, device=o_part.device)
    if out.shape != (rows, d) or out.dtype != dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [rows, d] tensor of dtype")
    if lse.shape != (rows,) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [rows] tensor")
    st = fa_lse_combine(o_part.data_ptr(), lse_part.data_ptr(), S, rows, d, out.data_ptr(),
                        lse.data_ptr(), _DTYPE_CODES[dtype], stream.cuda_stream)
    if st != FA_OK:
        raise FaError(st)
    return out, lse


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, scale, causal, dtype,
           stream) -> int:
    """Raw C call with integer pointers; returns the fa_status code."""
    return int(load().fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, int(B), int(H), int(N),
                             int(d), float(scale), int(bool(causal)), int(dtype), stream))


def fa_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, H_kv, N_q, N_kv, d, scale, causal,
              dtype, num_splits, workspace, workspace_bytes, stream) -> int:
    """Raw C call with integer pointers; returns the fa_status code."""
    return int(load().fa_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, delta, int(B), int(H),
                                int(H_kv), int(N_q), int(N_kv), int(d), float(scale),
                                int(bool(causal)), int(dtype), int(num_splits), workspace,
                                int(workspace_bytes), stream))


def bwd_workspace_bytes(B, H, H_kv, N_q, N_kv, d, num_splits) -> int:
    return int(load().fa_bwd_ex_workspace_bytes(int(B), int(H), int(H_kv), int(N_q), int(N_kv),
                                                int(d), int(num_splits)))


def bwd_default_splits(B, H, H_kv, N_q, N_kv, d, causal, dtype) -> int:
    return int(load().fa_bwd_ex_default_splits(int(B), int(H), int(H_kv), int(N_q), int(N_kv),
                                               int(d), int(bool(causal)), int(dtype)))


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
        lse: torch.Tensor, dout: torch.Tensor, scale: float | None = None,
        causal: bool = False, stream: torch.cuda.Stream | None = None,
        num_splits: int | None = None):
    """Gradients (dq, dk, dv) of the forward pass for fp32/bf16/fp16 tensors.

    q, o, dout: [B, H, N_q, d]; k, v: [B, H_kv, N_kv, d] with H_kv dividing H
    (``fa_bwd`` when the shapes are all equal, else ``fa_bwd_ex``).  ``o`` and
    ``lse`` are what ``fwd`` / ``fwd_ex`` returned for the same inputs.
    ``num_splits`` is the number of parts each group's query heads are cut
    into for dK/dV (None: ``fa_bwd_ex_default_splits``).  Returns
    ``(dq, dk, dv)`` shaped like q, k, v; the row dot products
    D = rowsum(dO * O) and the parts' workspace are allocated here.
    """
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or not (q.shape == o.shape == dout.shape):
        raise ValueError("q, o, dout must be [B, H, N_q, d] and k, v [B, H_kv, N_kv, d]")
    if not (q.dtype == k.dtype == v.dtype == o.dtype == dout.dtype) or q.dtype not in _DTYPE_CODES:
        raise TypeError("the backward pass takes float32, bfloat16 or float16 tensors of one dtype")
    tensors = (q, k, v, o, dout, lse)
    if not all(t.is_cuda and t.is_contiguous() for t in tensors):
        raise ValueError("inputs must be contiguous GPU tensors")
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError("q and k must share B and d")
    if lse.shape != (B, H, Nq) or lse.dtype != torch.float32:
        raise ValueError("lse must be a float32 [B, H, N_q] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    stream = _launch_stream(stream, q.device)
    with torch.cuda.stream(stream):
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        delta = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
            lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr())
    code = _DTYPE_CODES[q.dtype]
    if k.shape == q.shape and num_splits is None:
        st = fa_bwd(*ptrs, B, H, Nq, d, scale, causal, code, stream.cuda_stream)
    else:
        if num_splits is None:
            num_splits = bwd_default_splits(B, H, Hkv, Nq, Nk, d, causal, code)
        nbytes = bwd_workspace_bytes(B, H, Hkv, Nq, Nk, d, num_splits) if Hkv > 0 else 0
        ws = None
        if nbytes > 0:
            with torch.cuda.stream(stream):
                ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
        st = fa_bwd_ex(*ptrs, B, H, Hkv, Nq, Nk, d, scale, causal, code, num_splits,
                       ws.data_ptr() if ws is not None else None, nbytes, stream.cuda_stream)
    if st != FA_OK:
        raise FaError(st)
    return dq, dk, dv
