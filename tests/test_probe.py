"""The benchmark's MFMA-rate probe (libfa_probe.so, not part of libfa).

CPU: the library loads, exports its one entry point, and rejects bad
arguments before any HIP call.  GPU: the measured rate of the plain MFMA
loop lies between a floor that any working MI355X exceeds and the published
dense peak of the type at 2.4 GHz (bf16 / fp16 2.5 PFLOP/s, fp32 157.3 TFLOP/s)
plus a small allowance for timer granularity.
"""
import ctypes
import subprocess

import pytest

from exact_attention_13_amd import probe


def test_probe_loads_and_exports():
    lib = probe.load()
    assert isinstance(lib, ctypes.CDLL)
    out = subprocess.run(["nm", "-D", "--defined-only", str(probe._PATH)],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert exported == {"fa_probe_mfma_tflops"}


@pytest.mark.parametrize("args", [(3, 10, 1), (-1, 10, 1), (1, 0, 1), (1, 10, 0)])
def test_probe_rejects_bad_arguments(args):
    out = ctypes.c_double(-1.0)
    st = probe.load().fa_probe_mfma_tflops(args[0], args[1], args[2], None, ctypes.byref(out))
    assert st != 0
    assert out.value == -1.0
    assert probe.load().fa_probe_mfma_tflops(1, 10, 1, None, None) != 0


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,floor,peak", [("bf16", 1000.0, 2516.6), ("f16", 1000.0, 2516.6),
                                              ("f32", 60.0, 157.3)])
def test_probe_rate_is_plausible(dtype, floor, peak):
    r = probe.mfma_tflops(dtype, iters=2000, launches=3)
    print(f"MFMA loop {dtype}: {r:.1f} TFLOP/s", flush=True)
    assert floor < r <= peak * 1.02
