"""Parity of fa_fwd_ex (split keys, grouped K/V heads, N_q != N_kv) and of
fa_lse_combine with the fp64 oracle (MI355X only).

Every case goes through the C ABI (``binding.fwd_ex`` -> ``fa_fwd_ex``,
``binding.lse_combine`` -> ``fa_lse_combine``) on seeded inputs and is
compared element by element with ``oracle.fwd_gqa`` / ``oracle.combine`` on
the same bits, to the same bar as the plain forward pass:
  * fp32: max |O - O_ref| <= 1e-4, max |LSE - LSE_ref| <= 1e-4;
  * bf16/fp16: max |O - O_ref| <= 2e-2, rel-L2 <= 5e-3, max |dLSE| <= 2e-2.
Rows with no visible key must be exactly O = 0 and LSE = -inf.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_attention_13_amd import binding
from exact_attention_13_amd.inputs import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_ex(q, k, v, scale, causal, num_splits=None, workspace=None):
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    o, lse = binding.fwd_ex(qd, kd, vd, scale, causal, num_splits=num_splits,
                            workspace=workspace)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def assert_close(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what=""):
    o = o_gpu.to(torch.float64).numpy().reshape(o_ref.shape)
    l = lse_gpu.to(torch.float64).numpy().reshape(lse_ref.shape)
    empty = np.isneginf(lse_ref)
    # rows without a visible key: exactly zero output and -inf LSE
    assert np.array_equal(np.isneginf(l), empty), f"{what}: -inf LSE pattern differs"
    assert np.all(o[empty] == 0.0), f"{what}: empty rows not zero"
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    full = ~empty
    err = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    lerr = float(np.max(np.abs(l[full] - lse_ref[full]))) if full.any() else 0.0
    if dtype == "f32":
        assert err <= 1e-4, f"{what}: max|dO| = {err:.3e}"
        assert lerr <= 1e-4, f"{what}: max|dLSE| = {lerr:.3e}"
    else:
        ref_norm = np.linalg.norm(o_ref)
        rel = float(np.linalg.norm(o - o_ref) / ref_norm) if ref_norm > 0 else 0.0
        assert err <= 2e-2, f"{what}: max|dO| = {err:.3e}"
        assert rel <= 5e-3, f"{what}: rel-L2 = {rel:.3e}"
        assert lerr <= 2e-2, f"{what}: max|dLSE| = {lerr:.3e}"


def case(dtype, B, H, Hkv, Nq, Nkv, d, causal, seed, dist="normal"):
    w = Workload("case", dtype, B, H, Nq, d, causal, seed, dist, Hkv=Hkv, Nkv=Nkv)
    return w, make_inputs(w)


# --------------------------------------------------------------------------
# The extended call reduces to fa_fwd
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,d,causal", [("f32", 64, False), ("bf16", 64, True),
                                            ("f16", 128, False), ("bf16", 128, True)])
def test_unsplit_square_equals_fa_fwd_bitwise(dtype, d, causal):
    w, (q, k, v) = case(dtype, 2, 3, 3, 333, 333, d, causal, seed=500)
    _note(f"ex == fwd {dtype} d={d} causal={causal}")
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    o1, l1 = binding.fwd(qd, kd, vd, w.scale, causal)
    o2, l2 = binding.fwd_ex(qd, kd, vd, w.scale, causal, num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# --------------------------------------------------------------------------
# Split over keys
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_split_keys_small(dtype, d, causal):
    # (1000, 6): ranges of 192 keys, not a multiple of the 128-key tiles of
    # the d = 64 kernel, so a tile crosses into the next range and must mask
    for i, (n, splits) in enumerate([(65, 2), (200, 3), (513, 5), (1000, 16), (129, 300),
                                     (1000, 6)]):
        w, (q, k, v) = case(dtype, 1 + i % 2, 2, 2, n, n, d, causal, seed=600 + i)
        _note(f"split {dtype} d={d} causal={causal} N={n} splits={splits}")
        o, lse = run_ex(q, k, v, w.scale, causal, num_splits=splits)
        o_ref, lse_ref = oracle.fwd_gqa(q, k, v, w.scale, causal)
        assert_close(o, lse, o_ref, lse_ref, dtype, f"N={n} S={splits}")


def test_split_is_deterministic_and_workspace_bounded():
    w, (q, k, v) = case("bf16", 2, 4, 2, 300, 2000, 128, True, seed=610)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    need = binding.workspace_bytes(2, 4, 300, 2000, 128, 7)
    assert need > 0
    guard = 4096
    ws = torch.full((need + guard,), 0x5A, dtype=torch.uint8, device=DEV)
    _note("split determinism / workspace guard")
    o1, l1 = binding.fwd_ex(qd, kd, vd, w.scale, True, num_splits=7, workspace=ws)
    o2, l2 = binding.fwd_ex(qd, kd, vd, w.scale, True, num_splits=7, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.all(ws[need:] == 0x5A), "split kernels wrote past the workspace size"
    o_ref, lse_ref = oracle.fwd_gqa(q, k, v, w.scale, True)
    assert_close(o1.cpu(), l1.cpu(), o_ref, lse_ref, "bf16")


# --------------------------------------------------------------------------
# Grouped K/V heads and N_q != N_kv
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_grouped_heads_and_lengths(dtype, d, causal):
    shapes = [  # (B, H, Hkv, Nq, Nkv, splits)
        (2, 4, 2, 129, 129, 1),
        (1, 6, 3, 70, 300, 1),
        (2, 8, 1, 17, 517, 3),
        (1, 4, 4, 300, 90, 1),     # more queries than keys
        (1, 4, 2, 300, 90, 2),
        (3, 4, 1, 1, 2049, 1),     # decoding, unsplit
        (3, 8, 2, 1, 2049, 6),     # decoding, split
        (2, 16, 2, 3, 700, 4),     # a few new tokens, 8 heads per K/V head
        (1, 2, 1, 64, 64, 1),
    ]
    for i, (B, H, Hkv, Nq, Nkv, s) in enumerate(shapes):
        w, (q, k, v) = case(dtype, B, H, Hkv, Nq, Nkv, d, causal, seed=700 + i)
        _note(f"gqa {dtype} d={d} causal={causal} B={B} H={H} Hkv={Hkv} Nq={Nq} Nkv={Nkv} S={s}")
        o, lse = run_ex(q, k, v, w.scale, causal, num_splits=s)
        o_ref, lse_ref = oracle.fwd_gqa(q, k, v, w.scale, causal)
        assert_close(o, lse, o_ref, lse_ref, dtype, f"case {i}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_default_splits_and_zero_keys(dtype):
    w, (q, k, v) = case(dtype, 2, 8, 2, 4, 3000, 64, False, seed=720)
    s = binding.default_splits(2, 8, 2, 4, 3000, 64, False, binding._DTYPE_CODES[TORCH[dtype]])
    assert s > 1
    _note(f"default splits {dtype} S={s}")
    o, lse = run_ex(q, k, v, w.scale, False)
    o_ref, lse_ref = oracle.fwd_gqa(q, k, v, w.scale, False)
    assert_close(o, lse, o_ref, lse_ref, dtype, "default splits")
    # no keys at all: every row is empty
    k0 = torch.zeros((2, 2, 0, 64), dtype=TORCH[dtype])
    _note(f"zero keys {dtype}")
    o, lse = run_ex(q, k0, k0, w.scale, False)
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_large_logits_split(dtype):
    w, (q, k, v) = case(dtype, 1, 4, 2, 260, 3000, 128, True, seed=730, dist="large_logit")
    _note(f"large-logit split {dtype}")
    o, lse = run_ex(q, k, v, w.scale, True, num_splits=9)
    o_ref, lse_ref = oracle.fwd_gqa(q, k, v, w.scale, True)
    assert_close(o, lse, o_ref, lse_ref, dtype)


# --------------------------------------------------------------------------
# fa_lse_combine on its own
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
def test_lse_combine(dtype, d):
    g = np.random.default_rng(740 + d)
    for S, rows in [(1, 37), (2, 1000), (7, 333), (64, 129)]:
        op = g.standard_normal((S, rows, d)).astype(np.float32)
        lp = (5.0 * g.standard_normal((S, rows))).astype(np.float32)
        empty = g.random((S, rows)) < 0.2          # ranges with no key
        lp[empty] = -np.inf
        op[empty] = 0.0
        lp[:, :3] = -np.inf                         # rows with no key anywhere
        op[:, :3] = 0.0
        _note(f"combine {dtype} d={d} S={S} rows={rows}")
        o, lse = binding.lse_combine(torch.from_numpy(op).to(DEV), torch.from_numpy(lp).to(DEV),
                                     TORCH[dtype])
        torch.cuda.synchronize()
        o_ref, lse_ref = oracle.combine(op, lp)
        assert_close(o.cpu(), lse.cpu(), o_ref, lse_ref, dtype, f"S={S}")


# --------------------------------------------------------------------------
# The split / grouped workloads at full size
# --------------------------------------------------------------------------

def test_workload_C1s_full_oracle():
    w = WORKLOADS["C1s"]
    q, k, v = make_inputs(w)
    _note("workload C1s full")
    o, lse = run_ex(q, k, v, w.scale, w.causal)
    o_ref, lse_ref = oracle.fwd_gqa(q, k, v, w.scale, w.causal)
    assert_close(o, lse, o_ref, lse_ref, w.dtype, "C1s")


def test_workload_D1_full_oracle():
    w = WORKLOADS["D1"]
    q, k, v = make_inputs(w)
    _note("workload D1 full")
    o, lse = run_ex(q, k, v, w.scale, w.causal)
    o_ref, lse_ref = oracle.fwd_gqa(q, k, v, w.scale, w.causal)
    assert_close(o, lse, o_ref, lse_ref, w.dtype, "D1")


@pytest.mark.parametrize("name", ["G1", "G2"])
def test_workload_grouped_every_row(name):
    # Full size, every row against the oracle (G1: 16 query heads on 4 K/V
    # heads at 16384 rows; G2: 8 x 16 causal heads on 2 K/V heads at 4096),
    # with O and LSE pre-filled with NaN so that a tile the grid skipped
    # fails.  The oracle runs a few query heads at a time (rows are flat
    # indices (b H + h) N + i), printing its progress.
    w = WORKLOADS[name]
    q, k, v = make_inputs(w)
    _note(f"workload {name} every row")
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((w.B, w.H, w.N), float("nan"), dtype=torch.float32, device=DEV)
    binding.fwd_ex(qd, kd, vd, w.scale, w.causal, num_splits=1, out=o, lse=lse)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    del qd, kd, vd
    o_ref = np.empty((w.B * w.H * w.N, w.d))
    lse_ref = np.empty((w.B * w.H * w.N,))
    step = 4
    for b in range(w.B):
        for h0 in range(0, w.H, step):
            lo = (b * w.H + h0) * w.N
            hi = (b * w.H + min(w.H, h0 + step)) * w.N
            rows = np.arange(lo, hi, dtype=np.int64)
            o_ref[lo:hi], lse_ref[lo:hi] = oracle.fwd_gqa(q, k, v, w.scale, w.causal, rows=rows)
            _note(f"  oracle {name} b={b} heads {h0}..{min(w.H, h0 + step) - 1}")
    assert_close(o.reshape(-1, w.d), lse.reshape(-1), o_ref, lse_ref, w.dtype, name)
