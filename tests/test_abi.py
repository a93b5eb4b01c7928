"""The C-ABI library: it loads, exports what include/fa.h declares, and
rejects bad arguments on the host before anything touches a GPU.

CPU only: every call here returns from the validation step, so no kernel is
launched and no GPU is needed.  Pointers are fake but aligned host addresses
(validation never dereferences them).
"""
import ctypes
import re
import subprocess
from pathlib import Path

import pytest

from exact_attention_13_amd import binding as libfa

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "fa.h"


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_\w+)\s*\(", text)))


def test_library_is_built_and_loads():
    assert libfa.library_path().exists()
    lib = libfa.load()
    assert isinstance(lib, ctypes.CDLL)


def test_exports_every_declared_symbol():
    declared = declared_functions()
    assert declared == sorted(libfa.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", str(libfa.library_path())],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared:
        assert name in exported, name
        assert hasattr(libfa.load(), name)


def test_version_and_strerror():
    assert libfa.version() == 100
    for code in range(9):
        msg = libfa.strerror(code)
        assert msg and "unknown" not in msg
    assert "unknown" in libfa.strerror(99)


# Fake, 256-byte aligned, non-overlapping "device" addresses.
BASE = 1 << 40
Q, K, V, O, L = (BASE + i * (1 << 32) for i in range(5))
OK_ARGS = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, N=128, d=64, scale=0.125,
               causal=0, dtype=libfa.FA_BF16, stream=None)


def call(**kw):
    a = dict(OK_ARGS)
    a.update(kw)
    return libfa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"],
                        a["d"], a["scale"], a["causal"], a["dtype"], a["stream"])


@pytest.mark.parametrize("name", ["q", "k", "v", "o"])
def test_null_pointer(name):
    assert call(**{name: None}) == 1


@pytest.mark.parametrize("kw", [dict(B=-1), dict(H=-3), dict(N=-5),
                                dict(N=1 << 31), dict(B=1 << 20, H=1 << 20),
                                dict(B=1 << 16, H=1 << 14, N=1 << 24)])
def test_bad_shape(kw):
    assert call(**kw) == 2


@pytest.mark.parametrize("d", [0, 1, 32, 63, 96, 256, -64])
def test_bad_head_dim(d):
    assert call(d=d) == 3


@pytest.mark.parametrize("dt", [-1, 3, 7])
def test_bad_dtype(dt):
    assert call(dtype=dt) == 4


@pytest.mark.parametrize("s", [0.0, -0.125, float("inf"), float("nan"), -float("inf")])
def test_bad_scale(s):
    assert call(scale=s) == 5


@pytest.mark.parametrize("kw", [dict(q=Q + 8), dict(k=K + 2), dict(v=V + 4), dict(o=O + 12),
                                dict(lse=L + 2)])
def test_misaligned(kw):
    assert call(**kw) == 6


@pytest.mark.parametrize("kw", [dict(o=Q), dict(o=K + 64), dict(o=V - 64),
                                dict(lse=O + 16), dict(lse=Q), dict(lse=V + 1024)])
def test_aliasing(kw):
    assert call(**kw) == 7


def test_inputs_may_alias_each_other():
    # q, k, v are read-only; self-attention on one buffer is fine.  N = 0 so
    # that the call returns after validation without a launch.
    assert call(k=Q, v=Q, N=0) == 0


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0)])
def test_empty_problem_is_a_noop(kw):
    assert call(**kw) == 0


def test_validation_order_prefers_null_then_shape():
    assert call(q=None, d=7, scale=-1.0) == 1
    assert call(N=-1, d=7) == 2
