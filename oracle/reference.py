"""ctypes wrapper around ``fa_oracle.c`` (fp64 three-pass attention).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

The wrapper only marshals arguments: inputs are handed to C as their stored
bits (fp32, bf16 or fp16), the C side widens them exactly and does every
arithmetic step in double.  ``scale`` is the fp32 value that the GPU library
receives, widened to double, so both sides use the same number.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "fa_oracle.c"
_LIB = _HERE / "liboracle.so"

DTYPE_CODES = {"f32": 0, "bf16": 1, "f16": 2}
FLAT_ROWS_ALL = None

_lib = None


def build(force: bool = True) -> Path:
    """Compile ``fa_oracle.c`` with gcc into ``oracle/liboracle.so``."""
    global _lib
    if force or not _LIB.exists():
        tmp = _LIB.with_suffix(".so.tmp")
        cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
               "-pthread", "-o", str(tmp), str(_SRC), "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not _LIB.exists() and not os.environ.get("FA_ORACLE_LIB"):
            build(force=True)
        # FA_ORACLE_LIB lets the mutation test load a deliberately broken
        # build of this same source; nothing else sets it.
        lib = ctypes.CDLL(os.environ.get("FA_ORACLE_LIB") or str(_LIB))
        lib.oracle_fwd_f64.restype = ctypes.c_int
        lib.oracle_fwd_f64.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_fwd_gqa_f64.restype = ctypes.c_int
        lib.oracle_fwd_gqa_f64.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_combine_f64.restype = ctypes.c_int
        lib.oracle_combine_f64.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_void_p]
        lib.oracle_bwd_f64.restype = ctypes.c_int
        lib.oracle_bwd_f64.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
            ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_bwd_dq_rows_f64.restype = ctypes.c_int
        lib.oracle_bwd_dq_rows_f64.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
            ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        lib.oracle_bwd_gqa_f64.restype = ctypes.c_int
        lib.oracle_bwd_gqa_f64.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_int]
        lib.oracle_bwd_dq_rows_gqa_f64.restype = ctypes.c_int
        lib.oracle_bwd_dq_rows_gqa_f64.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_void_p]
        lib.oracle_widen.restype = ctypes.c_double
        lib.oracle_widen.argtypes = [ctypes.c_int, ctypes.c_uint32]
        _lib = lib
    return _lib


def _stored_bits(x):
    """Return (contiguous numpy array of stored bits, dtype name)."""
    try:
        import torch
    except ImportError:  # pragma: no cover
        torch = None
    if torch is not None and isinstance(x, torch.Tensor):
        x = x.detach().cpu().contiguous()
        if x.dtype == torch.float32:
            return x.numpy(), "f32"
        if x.dtype == torch.bfloat16:
            return x.view(torch.int16).numpy().view(np.uint16), "bf16"
        if x.dtype == torch.float16:
            return x.view(torch.int16).numpy().view(np.uint16), "f16"
        raise TypeError(f"unsupported tensor dtype {x.dtype}")
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, "f32"
    if x.dtype == np.float16:
        return x.view(np.uint16), "f16"
    raise TypeError(f"unsupported array dtype {x.dtype}")


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def fwd(q, k, v, scale: float, causal: bool, rows=None, threads: int | None = None):
    """Exact attention in fp64.

    q, k, v: [B, H, N, d] torch tensors (fp32 / bf16 / fp16) or numpy arrays
    (float32 / float16).  ``rows`` (optional) lists flat row indices
    ``(b*H + h)*N + i``; the result then has one row per entry.

    Returns ``(o, lse)`` as float64 numpy arrays: ``o`` is [B, H, N, d] (or
    [len(rows), d]) and ``lse`` is [B, H, N] (or [len(rows)]).
    """
    qb, dt = _stored_bits(q)
    kb, dtk = _stored_bits(k)
    vb, dtv = _stored_bits(v)
    if not (dt == dtk == dtv):
        raise TypeError("q, k, v must share one dtype")
    if not (qb.shape == kb.shape == vb.shape) or qb.ndim != 4:
        raise ValueError("q, k, v must all be [B, H, N, d] of one shape")
    B, H, N, d = (int(s) for s in qb.shape)
    scale64 = float(np.float32(scale))
    if rows is None:
        nrows = B * H * N
        rows_arr = None
        rows_ptr = None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = int(rows_arr.size)
        rows_ptr = rows_arr.ctypes.data
    o = np.zeros((max(nrows, 0), max(d, 1)), dtype=np.float64)
    lse = np.zeros((max(nrows, 0),), dtype=np.float64)
    if nrows > 0:
        rc = _load().oracle_fwd_f64(
            qb.ctypes.data, kb.ctypes.data, vb.ctypes.data, DTYPE_CODES[dt],
            B, H, N, d, scale64, int(bool(causal)), rows_ptr, nrows,
            o.ctypes.data, lse.ctypes.data, int(threads or default_threads()))
        if rc != 0:
            raise RuntimeError(f"oracle_fwd_f64 failed with code {rc}")
    if rows is None:
        return o.reshape(B, H, N, d), lse.reshape(B, H, N)
    return o[:, :d], lse


def fwd_gqa(q, k, v, scale: float, causal: bool, rows=None, threads: int | None = None):
    """Exact attention in fp64 with grouped K/V heads and N_q != N_kv.

    q: [B, H, N_q, d]; k, v: [B, H_kv, N_kv, d] (H_kv divides H; query head
    h reads K/V head h // (H // H_kv)).  Causal masking hides key j from
    query i when j > i + N_kv - N_q.  ``rows`` lists flat indices
    ``(b*H + h)*N_q + i``.  Returns ``(o, lse)`` as float64 numpy arrays:
    [B, H, N_q, d] and [B, H, N_q] (or one row per entry of ``rows``).
    """
    qb, dt = _stored_bits(q)
    kb, dtk = _stored_bits(k)
    vb, dtv = _stored_bits(v)
    if not (dt == dtk == dtv):
        raise TypeError("q, k, v must share one dtype")
    if qb.ndim != 4 or kb.ndim != 4 or kb.shape != vb.shape:
        raise ValueError("q must be [B, H, N_q, d]; k and v one [B, H_kv, N_kv, d] shape")
    B, H, Nq, d = (int(s) for s in qb.shape)
    Bk, Hkv, Nk, dk = (int(s) for s in kb.shape)
    if Bk != B or dk != d or Hkv == 0 or H % Hkv:
        raise ValueError("q, k, v must share B and d, and H_kv must divide H")
    scale64 = float(np.float32(scale))
    if rows is None:
        nrows, rows_ptr = B * H * Nq, None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows, rows_ptr = int(rows_arr.size), rows_arr.ctypes.data
    o = np.zeros((max(nrows, 0), max(d, 1)), dtype=np.float64)
    lse = np.zeros((max(nrows, 0),), dtype=np.float64)
    if nrows > 0:
        rc = _load().oracle_fwd_gqa_f64(
            qb.ctypes.data, kb.ctypes.data, vb.ctypes.data, DTYPE_CODES[dt],
            B, H, Hkv, Nq, Nk, d, scale64, int(bool(causal)), rows_ptr, nrows,
            o.ctypes.data, lse.ctypes.data, int(threads or default_threads()))
        if rc != 0:
            raise RuntimeError(f"oracle_fwd_gqa_f64 failed with code {rc}")
    if rows is None:
        return o.reshape(B, H, Nq, d), lse.reshape(B, H, Nq)
    return o[:, :d], lse


def combine(o_parts, lse_parts):
    """Merge per-range results in fp64: o_parts [S, rows, d], lse_parts [S, rows].

    Returns ``(o [rows, d], lse [rows])`` as float64 numpy arrays.
    """
    op = np.ascontiguousarray(np.asarray(o_parts, dtype=np.float64))
    lp = np.ascontiguousarray(np.asarray(lse_parts, dtype=np.float64))
    if op.ndim != 3 or lp.shape != op.shape[:2]:
        raise ValueError("o_parts must be [S, rows, d] and lse_parts [S, rows]")
    S, rows, d = op.shape
    o = np.zeros((rows, d), dtype=np.float64)
    lse = np.zeros((rows,), dtype=np.float64)
    rc = _load().oracle_combine_f64(op.ctypes.data, lp.ctypes.data, S, rows, d,
                                    o.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"oracle_combine_f64 failed with code {rc}")
    return o, lse


def _four(q, k, v, dout):
    qb, dt = _stored_bits(q)
    kb, dtk = _stored_bits(k)
    vb, dtv = _stored_bits(v)
    gb, dtg = _stored_bits(dout)
    if not (dt == dtk == dtv == dtg):
        raise TypeError("q, k, v, dout must share one dtype")
    if qb.ndim != 4 or kb.ndim != 4 or qb.shape != gb.shape or kb.shape != vb.shape:
        raise ValueError("q, dout must be [B, H, N_q, d] and k, v [B, H_kv, N_kv, d]")
    B, H, _, d = (int(s) for s in qb.shape)
    Bk, Hkv, _, dk = (int(s) for s in kb.shape)
    if Bk != B or dk != d or (Hkv == 0) != (H == 0) or (Hkv and H % Hkv):
        raise ValueError("q, k, v must share B and d, and H_kv must divide H")
    return qb, kb, vb, gb, dt


def bwd(q, k, v, dout, scale: float, causal: bool, threads: int | None = None):
    """Gradients of sum(dout * O) w.r.t. q, k, v in fp64.

    q, dout: [B, H, N_q, d]; k, v: [B, H_kv, N_kv, d] with H_kv dividing H
    (query head h reads K/V head h // (H // H_kv)); the causal mask is the
    forward oracle's (key j visible to row i when j <= i + N_kv - N_q).
    Returns ``(dq, dk, dv)`` as float64 numpy arrays shaped like q, k, v.
    """
    qb, kb, vb, gb, dt = _four(q, k, v, dout)
    B, H, Nq, d = (int(s) for s in qb.shape)
    Hkv, Nk = int(kb.shape[1]), int(kb.shape[2])
    dq = np.zeros((B, H, Nq, d), dtype=np.float64)
    dk = np.zeros((B, Hkv, Nk, d), dtype=np.float64)
    dv = np.zeros_like(dk)
    rc = _load().oracle_bwd_gqa_f64(qb.ctypes.data, kb.ctypes.data, vb.ctypes.data,
                                    gb.ctypes.data, DTYPE_CODES[dt], B, H, Hkv, Nq, Nk, d,
                                    float(np.float32(scale)), int(bool(causal)), dq.ctypes.data,
                                    dk.ctypes.data, dv.ctypes.data,
                                    int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle_bwd_gqa_f64 failed with code {rc}")
    return dq, dk, dv


def bwd_dq_rows(q, k, v, dout, scale: float, causal: bool, rows):
    """dQ for the flat query rows ``(b*H + h)*N_q + i`` only: [len(rows), d] float64."""
    qb, kb, vb, gb, dt = _four(q, k, v, dout)
    B, H, Nq, d = (int(s) for s in qb.shape)
    Hkv, Nk = int(kb.shape[1]), int(kb.shape[2])
    rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    dq = np.zeros((rows_arr.size, d), dtype=np.float64)
    rc = _load().oracle_bwd_dq_rows_gqa_f64(qb.ctypes.data, kb.ctypes.data, vb.ctypes.data,
                                            gb.ctypes.data, DTYPE_CODES[dt], B, H, Hkv, Nq, Nk,
                                            d, float(np.float32(scale)), int(bool(causal)),
                                            rows_arr.ctypes.data, rows_arr.size, dq.ctypes.data)
    if rc != 0:
        raise RuntimeError(f"oracle_bwd_dq_rows_gqa_f64 failed with code {rc}")
    return dq


def widen(dtype: str, bits: int) -> float:
    """The oracle's own widening of one stored element to double."""
    return _load().oracle_widen(DTYPE_CODES[dtype], int(bits) & 0xFFFFFFFF)
