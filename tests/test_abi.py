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
    assert libfa.version() == 500
    for code in range(11):
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


# --------------------------------------------------------------------------
# fa_fwd_ex, its helpers and fa_lse_combine (validation only, no launch)
# --------------------------------------------------------------------------

WS = BASE + 5 * (1 << 32)
EX_ARGS = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=4, H_kv=2, N_q=16, N_kv=4096, d=128,
               scale=0.125, causal=0, dtype=libfa.FA_BF16, num_splits=4, workspace=WS,
               workspace_bytes=1 << 30, stream=None)


def call_ex(**kw):
    a = dict(EX_ARGS)
    a.update(kw)
    return libfa.fa_fwd_ex(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["H_kv"],
                           a["N_q"], a["N_kv"], a["d"], a["scale"], a["causal"], a["dtype"],
                           a["num_splits"], a["workspace"], a["workspace_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(k=None), 1), (dict(v=None), 1),
    (dict(H_kv=3), 2), (dict(H_kv=0), 2), (dict(H_kv=-2), 2), (dict(N_kv=-1), 2),
    (dict(N_q=-1), 2), (dict(N_kv=1 << 31), 2), (dict(d=96), 3), (dict(dtype=5), 4),
    (dict(scale=float("nan")), 5), (dict(workspace=WS + 8), 9), (dict(q=Q + 4), 6),
    (dict(num_splits=0), 9), (dict(num_splits=-3), 9), (dict(workspace=None), 9),
    (dict(workspace_bytes=1000), 9), (dict(workspace=O), 7), (dict(workspace=K + 256), 7),
    (dict(lse=WS), 7), (dict(o=V + 64), 7),
])
def test_fwd_ex_rejects(kw, status):
    assert call_ex(**kw) == status


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0, H_kv=0), dict(N_q=0),
                                dict(B=0, workspace=None, num_splits=8)])
def test_fwd_ex_empty_is_a_noop(kw):
    assert call_ex(**kw) == 0


def test_fwd_ex_no_keys_allows_null_kv():
    # validation passes; N_q = 0 keeps the call from launching
    assert call_ex(k=None, v=None, N_kv=0, N_q=0) == 0
    assert call_ex(k=None, v=None, N_kv=0, N_q=0, num_splits=1, workspace=None) == 0
    # fa_fwd keeps requiring every pointer
    assert call(k=None, N=0) == 1


def call_noalloc(**kw):
    a = dict(EX_ARGS)
    a.update(kw)
    return libfa.fa_fwd_ex_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                                   a["H_kv"], a["N_q"], a["N_kv"], a["d"], a["scale"],
                                   a["causal"], a["dtype"], a["num_splits"], a["stream"])


# fa_fwd_ex_noalloc validates like fa_fwd_ex, before it looks up (or uses)
# the GPU's static scratch; partials beyond that scratch are FA_ERR_SCRATCH.
@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(k=None), 1), (dict(H_kv=3), 2),
    (dict(N_q=-1), 2), (dict(N_kv=1 << 31), 2), (dict(d=96), 3), (dict(dtype=5), 4),
    (dict(scale=0.0), 5), (dict(q=Q + 4), 6), (dict(o=V + 64), 7), (dict(lse=O), 7),
    (dict(num_splits=0), 9),
    # 64 ranges of 262144 rows of d = 128: 8.6 GB of partials
    (dict(B=1, H=64, H_kv=64, N_q=4096, N_kv=65536, num_splits=64), 10),
])
def test_fwd_ex_noalloc_rejects(kw, status):
    assert call_noalloc(**kw) == status


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0, H_kv=0), dict(N_q=0),
                                dict(B=0, num_splits=8)])
def test_fwd_ex_noalloc_empty_is_a_noop(kw):
    assert call_noalloc(**kw) == 0


def test_noalloc_scratch_size_matches_header():
    text = HEADER.read_text()
    m = re.search(r"#define FA_NOALLOC_SCRATCH_BYTES \((\d+) \* 1024 \* 1024\)", text)
    assert m and int(m.group(1)) * 1024 * 1024 == libfa.NOALLOC_SCRATCH_BYTES
    assert libfa.strerror(10).startswith("the split partials exceed the static scratch")


def test_workspace_bytes():
    # one range needs no workspace
    assert libfa.workspace_bytes(1, 4, 16, 4096, 128, 1) == 0
    assert libfa.workspace_bytes(1, 4, 16, 64, 128, 8) == 0
    # 4096 keys in 4 ranges: 4 * rows * (d + 1) fp32
    assert libfa.workspace_bytes(1, 4, 16, 4096, 128, 4) == 4 * 64 * 129 * 4
    # ranges are whole multiples of 64 keys: 4096 keys cannot make 1000 ranges
    assert libfa.workspace_bytes(1, 4, 16, 4096, 128, 1000) == 64 * 64 * 129 * 4
    # 300 keys (5 chunks of 64) asked for 4 ranges: chunks of 128 keys -> 3 ranges
    assert libfa.workspace_bytes(2, 2, 3, 300, 64, 4) == 3 * 12 * 65 * 4
    assert libfa.workspace_bytes(1, 1, 1, 100, 64, 0) == 0


def test_default_splits():
    bf16, f32 = libfa.FA_BF16, libfa.FA_F32
    # a full grid is not split (the headline bf16 shape)
    assert libfa.default_splits(1, 16, 16, 16384, 16384, 64, False, bf16) == 1
    # one fp32 head of 512 rows: the small-problem kernel, unsplit, is faster
    assert libfa.default_splits(1, 1, 1, 512, 512, 64, False, f32) == 1
    assert libfa.default_splits(1, 1, 1, 512, 512, 128, True, f32) == 1
    assert libfa.default_splits(2, 4, 4, 256, 256, 64, False, f32) == 1
    # its longer key chains are split: 2048 keys at d = 64, 1024 at d = 128
    assert libfa.default_splits(1, 1, 1, 512, 2048, 64, False, f32) == 32
    assert libfa.default_splits(4, 1, 1, 256, 1024, 128, False, f32) == 16
    assert libfa.default_splits(1, 1, 1, 1, 16384, 64, False, f32) >= 64
    # a full fp32 grid is not split
    assert libfa.default_splits(4, 8, 8, 2048, 2048, 64, False, f32) == 1
    # decoding against a long cache is split into many ranges
    s = libfa.default_splits(8, 32, 8, 1, 16384, 128, False, bf16)
    assert 8 <= s <= 256
    assert libfa.default_splits(1, 4, 3, 1, 100, 64, False, bf16) == 1  # invalid grouping
    # a short d = 64 grid runs 32-row workgroups that fill the chip unsplit
    assert libfa.default_splits(1, 16, 16, 2048, 2048, 64, False, bf16) == 1
    # eight-wave d = 64 tiles (96 of them): one workgroup per compute unit
    assert libfa.default_splits(1, 24, 24, 2048, 2048, 64, False, bf16) == 3
    # d = 128 grids of 128 row blocks run unsplit
    assert libfa.default_splits(2, 8, 8, 1024, 1024, 128, False, bf16) == 1
    # a few query rows over a short key sequence: 128-key ranges
    assert libfa.default_splits(1, 1, 1, 512, 512, 64, False, bf16) == 4
    assert libfa.default_splits(4, 1, 1, 256, 1024, 128, False, bf16) == 8
    # ... but not with more rows; short d = 64 grids of 32-row workgroups
    # that fill the chip are not split
    assert libfa.default_splits(1, 8, 8, 512, 512, 64, False, bf16) == 2
    assert libfa.default_splits(2, 8, 8, 1024, 1024, 64, False, bf16) == 1


@pytest.mark.parametrize("kw,status", [
    (dict(o_part=None), 1), (dict(lse_part=None), 1), (dict(o=None), 1),
    (dict(splits=0), 2), (dict(rows=-1), 2), (dict(d=32), 3), (dict(dtype=9), 4),
    (dict(o_part=Q + 4), 6), (dict(o=O + 2), 6), (dict(lse_part=K + 2), 6),
    (dict(o=Q + 64), 7), (dict(lse=K), 7), (dict(lse=O + 128), 7),
])
def test_lse_combine_rejects(kw, status):
    a = dict(o_part=Q, lse_part=K, splits=4, rows=100, d=64, o=O, lse=L, dtype=libfa.FA_F16,
             stream=None)
    a.update(kw)
    assert libfa.fa_lse_combine(a["o_part"], a["lse_part"], a["splits"], a["rows"], a["d"],
                                a["o"], a["lse"], a["dtype"], a["stream"]) == status


def test_lse_combine_empty_is_a_noop():
    assert libfa.fa_lse_combine(Q, K, 3, 0, 64, O, L, libfa.FA_F32, None) == 0


# --------------------------------------------------------------------------
# fa_bwd (validation only, no launch)
# --------------------------------------------------------------------------

OB, GB, DQ, DK, DV, DL = (BASE + (6 + i) * (1 << 32) for i in range(6))
BWD_ARGS = dict(q=Q, k=K, v=V, o=OB, dout=GB, lse=L, dq=DQ, dk=DK, dv=DV, delta=DL, B=1, H=2,
                N=256, d=64, scale=0.125, causal=1, dtype=libfa.FA_BF16, stream=None)


def call_bwd(**kw):
    a = dict(BWD_ARGS)
    a.update(kw)
    return libfa.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"],
                        a["dv"], a["delta"], a["B"], a["H"], a["N"], a["d"], a["scale"],
                        a["causal"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(dout=None), 1), (dict(lse=None), 1), (dict(dv=None), 1),
    (dict(delta=None), 1), (dict(N=-1), 2), (dict(N=1 << 31), 2), (dict(d=32), 3),
    (dict(dtype=-1), 4), (dict(dtype=3), 4), (dict(scale=0.0), 5),
    (dict(dq=DQ + 8), 6), (dict(o=OB + 4), 6), (dict(delta=DL + 2), 6),
    (dict(dq=Q), 7), (dict(dk=DQ + 64), 7), (dict(dv=GB), 7), (dict(delta=L), 7),
    (dict(delta=DV + 128), 7), (dict(dk=K - 16), 7),
])
def test_bwd_rejects(kw, status):
    assert call_bwd(**kw) == status


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0)])
def test_bwd_empty_is_a_noop(kw):
    assert call_bwd(**kw) == 0


# --------------------------------------------------------------------------
# fa_bwd_ex (validation only, no launch)
# --------------------------------------------------------------------------

BWDX_ARGS = dict(q=Q, k=K, v=V, o=OB, dout=GB, lse=L, dq=DQ, dk=DK, dv=DV, delta=DL, B=1, H=4,
                 H_kv=2, N_q=100, N_kv=300, d=128, scale=0.088, causal=1, dtype=libfa.FA_F16,
                 num_splits=1, workspace=None, workspace_bytes=0, stream=None)
# two head parts of the [1, 2, 300, 128] K/V heads: fp32 partial dK and dV
BWDX_WS_BYTES = 2 * 2 * 1 * 2 * 300 * 128 * 4


def call_bwd_ex(**kw):
    a = dict(BWDX_ARGS)
    a.update(kw)
    return libfa.fa_bwd_ex(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"],
                           a["dv"], a["delta"], a["B"], a["H"], a["H_kv"], a["N_q"], a["N_kv"],
                           a["d"], a["scale"], a["causal"], a["dtype"], a["num_splits"],
                           a["workspace"], a["workspace_bytes"], a["stream"])


def split2(**kw):
    """Arguments of a two-part call with a workspace of the right size."""
    return {**dict(num_splits=2, workspace=WS, workspace_bytes=BWDX_WS_BYTES), **kw}


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(dout=None), 1), (dict(lse=None), 1),
    (dict(dq=None), 1), (dict(delta=None), 1), (dict(k=None), 1), (dict(v=None), 1),
    (dict(dk=None), 1), (dict(dv=None), 1),
    (dict(k=None, N_q=0), 1), (dict(q=None, N_kv=0), 1),
    (dict(H_kv=-1), 2), (dict(N_q=-1), 2), (dict(N_kv=-2), 2), (dict(H_kv=3), 2),
    (dict(H_kv=0), 2), (dict(N_kv=1 << 31), 2), (dict(N_q=1 << 31), 2),
    (dict(d=96), 3), (dict(dtype=7), 4), (dict(scale=float("nan")), 5),
    (dict(dk=DK + 8), 6), (dict(v=V + 2), 6), (dict(lse=L + 1), 6),
    # dK/dV are [B, H_kv, N_kv, d] (300 * 128 * 2 * 2 bytes), dQ [B, H, N_q, d]
    (dict(dk=K + 150_000), 7), (dict(dv=DK + 153_584), 7), (dict(dq=OB + 102_384), 7),
    (dict(delta=L + 1596), 7),
    # head parts: count, workspace presence, size, alignment and overlap
    (dict(num_splits=0), 9), (dict(num_splits=-3), 9), (dict(num_splits=0, H=2, H_kv=2), 9),
    (dict(num_splits=2), 9), (split2(workspace=None), 9),
    (split2(workspace_bytes=BWDX_WS_BYTES - 1), 9), (split2(workspace=WS + 8), 9),
    # num_splits beyond the group size of 2 still needs only two parts
    (dict(num_splits=9, workspace=WS, workspace_bytes=BWDX_WS_BYTES - 16), 9),
    (split2(workspace=DK - 1024), 7), (split2(workspace=Q + 16), 7),
    (split2(workspace=L + 512), 7), (split2(workspace=DL - BWDX_WS_BYTES + 16), 7),
    # the workspace is checked after the other arguments
    (split2(workspace=None, d=96), 3), (split2(workspace=None, dk=DK + 8), 6),
])
def test_bwd_ex_rejects(kw, status):
    assert call_bwd_ex(**kw) == status


def test_bwd_workspace_bytes():
    # 2 * parts * B * H_kv * N_kv * d * 4 with parts = min(num_splits, H / H_kv)
    assert libfa.bwd_workspace_bytes(1, 4, 2, 100, 300, 128, 2) == BWDX_WS_BYTES
    assert libfa.bwd_workspace_bytes(1, 4, 2, 100, 300, 128, 9) == BWDX_WS_BYTES
    assert libfa.bwd_workspace_bytes(2, 32, 8, 50, 1000, 64, 3) == 2 * 3 * 2 * 8 * 1000 * 64 * 4
    # one part: no workspace
    assert libfa.bwd_workspace_bytes(1, 4, 2, 100, 300, 128, 1) == 0
    assert libfa.bwd_workspace_bytes(1, 4, 4, 100, 300, 128, 8) == 0
    assert libfa.bwd_workspace_bytes(1, 4, 2, 0, 300, 128, 2) == 0
    assert libfa.bwd_workspace_bytes(1, 4, 2, 100, 0, 128, 2) == 0
    # invalid sizes give 0, overflow -1
    assert libfa.bwd_workspace_bytes(1, 4, 2, 100, 300, 96, 2) == 0
    assert libfa.bwd_workspace_bytes(-1, 4, 2, 100, 300, 128, 2) == 0
    assert libfa.bwd_workspace_bytes(1 << 40, 4, 2, 1, 1 << 30, 128, 2) == -1


def test_bwd_default_splits():
    bf16, f32 = libfa.FA_BF16, libfa.FA_F32
    # no grouping, or a full grid without a mask: one part
    assert libfa.bwd_default_splits(1, 16, 16, 16384, 16384, 64, True, bf16) == 1
    assert libfa.bwd_default_splits(8, 32, 8, 4096, 4096, 128, False, bf16) == 1
    # a causal mask, or a short grid, asks for parts, at most the group size
    s = libfa.bwd_default_splits(2, 32, 8, 8192, 8192, 128, True, bf16)
    assert 1 < s <= 4
    assert libfa.bwd_default_splits(1, 8, 1, 1024, 1024, 64, False, f32) == 8
    assert libfa.bwd_default_splits(1, 8, 2, 4096, 4096, 64, False, f32) == 4
    # parts of equal size only: 512 d = 64 workgroups want 3 parts (two per
    # slot of 768), and a group of 4 takes 4 rather than 1 + 1 + 2 heads
    assert libfa.bwd_default_splits(1, 16, 4, 16384, 16384, 64, False, bf16) == 4
    assert libfa.bwd_default_splits(1, 12, 4, 4096, 4096, 64, False, bf16) == 3
    # invalid arguments: 1
    assert libfa.bwd_default_splits(1, 4, 3, 100, 100, 64, True, bf16) == 1
    assert libfa.bwd_default_splits(1, 4, 2, 100, 100, 96, True, bf16) == 1
    assert libfa.bwd_default_splits(1, 4, 2, 0, 100, 64, True, bf16) == 1


@pytest.mark.parametrize("kw", [
    dict(B=0), dict(H=0, H_kv=0), dict(N_q=0, N_kv=0),
    dict(N_q=0, N_kv=0, q=None, o=None, dout=None, lse=None, dq=None, delta=None,
         k=None, v=None, dk=None, dv=None)])
def test_bwd_ex_empty_is_a_noop(kw):
    assert call_bwd_ex(**kw) == 0
