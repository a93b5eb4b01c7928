"""The benchmark's MFMA-rate probe (libfa_probe.so, not part of libfa).

CPU: the library loads, exports its two entry points, and rejects bad
arguments before any HIP call.  GPU: the measured rate of the plain MFMA
loop lies between a floor that any working MI355X exceeds and the published
dense peak of the type at 2.4 GHz (bf16 / fp16 2.5 PFLOP/s, fp32 157.3 TFLOP/s)
plus a small allowance for timer granularity; the delay kernel holds its
stream for at least the time asked (events around it) and not far beyond.
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
    assert exported == {"fa_probe_mfma_tflops", "fa_probe_delay"}


@pytest.mark.parametrize("args", [(3, 10, 1), (-1, 10, 1), (1, 0, 1), (1, 10, 0)])
def test_probe_rejects_bad_arguments(args):
    out = ctypes.c_double(-1.0)
    st = probe.load().fa_probe_mfma_tflops(args[0], args[1], args[2], None, ctypes.byref(out))
    assert st != 0
    assert out.value == -1.0
    assert probe.load().fa_probe_mfma_tflops(1, 10, 1, None, None) != 0


@pytest.mark.parametrize("us", [-1, 1000001])
def test_delay_rejects_bad_times(us):
    assert probe.load().fa_probe_delay(us, None) != 0


@pytest.mark.gpu
@pytest.mark.parametrize("us", [200, 5000])
def test_delay_holds_the_stream(us):
    import torch
    stream = torch.cuda.Stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    probe.delay(10, stream)  # first launch loads the code object
    torch.cuda.synchronize()
    a.record(stream)
    probe.delay(us, stream)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    print(f"delay {us} us: {ms * 1e3:.1f} us", flush=True)
    assert us * 1e-3 <= ms <= us * 1e-3 * 1.5 + 0.1


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,floor,peak", [("bf16", 1000.0, 2516.6), ("f16", 1000.0, 2516.6),
                                              ("f32", 60.0, 157.3)])
def test_probe_rate_is_plausible(dtype, floor, peak):
    r = probe.mfma_tflops(dtype, iters=2000, launches=3)
    print(f"MFMA loop {dtype}: {r:.1f} TFLOP/s", flush=True)
    assert floor < r <= peak * 1.02
