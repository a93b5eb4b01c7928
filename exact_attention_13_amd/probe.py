"""ctypes binding of libfa_probe.so: the dense MFMA rate of the current GPU.

The benchmark reports an attention kernel's FLOP rate against MI355X's
published dense peak and, beside it, against this measured rate of a plain
MFMA loop (independent 32x32 MFMAs back to back on every SIMD, two waves per
SIMD), which runs at the clock the chip holds under MFMA load.  The probe is
not part of libfa and computes nothing of the attention path.  Its delay
kernel lets the benchmark queue timed launches so that they run back to back.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

_PATH = Path(__file__).resolve().parent / "libfa_probe.so"
_DTYPES = {"f32": 0, "bf16": 1, "f16": 2}
_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not _PATH.exists():
            raise RuntimeError(f"{_PATH} is missing: build it with `python -m exact_attention_13_amd.build`")
        lib = ctypes.CDLL(str(_PATH))
        lib.fa_probe_mfma_tflops.restype = ctypes.c_int
        lib.fa_probe_mfma_tflops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                             ctypes.POINTER(ctypes.c_double)]
        lib.fa_probe_delay.restype = ctypes.c_int
        lib.fa_probe_delay.argtypes = [ctypes.c_int, ctypes.c_void_p]
        _lib = lib
    return _lib


def mfma_tflops(dtype: str, iters: int = 4000, launches: int = 5, stream=None) -> float:
    """Best of `launches` timed launches of the MFMA loop for `dtype`
    ("f32", "bf16" or "f16"), in TFLOP/s.  `stream` is a torch.cuda.Stream or
    None (the default stream).  Synchronises the stream."""
    out = ctypes.c_double(0.0)
    handle = stream.cuda_stream if stream is not None else None
    st = load().fa_probe_mfma_tflops(_DTYPES[dtype], int(iters), int(launches), handle, ctypes.byref(out))
    if st != 0:
        raise RuntimeError(f"fa_probe_mfma_tflops failed with HIP error {st}")
    return float(out.value)


def delay(microseconds: int, stream=None) -> None:
    """Occupy `stream` (a torch.cuda.Stream or None) for about `microseconds`
    (0 .. 1e6) with a kernel that waits on the GPU's real-time counter, so that
    the launches made next queue up behind it.  Asynchronous."""
    handle = stream.cuda_stream if stream is not None else None
    st = load().fa_probe_delay(int(microseconds), handle)
    if st != 0:
        raise RuntimeError(f"fa_probe_delay failed with HIP error {st}")
