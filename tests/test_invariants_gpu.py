"""Properties the method fixes, checked on the HIP forward pass (MI355X only).

The same invariants that pin the oracle are run here on the kernels, through
the C ABI, with closed-form expected values computed in fp64 from the stored
input bits (no oracle involved) and, where a case has no closed form, the
oracle as well:

  * value rows all ones: every output row is exactly the all-ones row (the
    weights of a row sum to one), "FlashAttention dissected", section "The
    mathematical breakthrough: Tiling and Online Softmax";
  * Q = 0: every score is 0, so a row's output is the mean of the value rows
    it sees (all rows, or the prefix 0..i under the causal mask) and its
    logsumexp is ln(number of visible keys);
  * one dominant logit: a row whose score against one key exceeds every
    other score by far returns that key's value row, with LSE equal to that
    score;
  * causal row 0 sees only key 0: O_0 = V_0 and LSE_0 = scale q_0 . k_0.

The dominant logit is placed in the last key tile of the row, after earlier
tiles have settled the kernel's reference maximum, at three gaps above the
row's other scores (in exp2 units): 12 (the bf16/fp16 fast path, which
skips the row maximum while a lane's partial sum stays below 2^15, keeps the
weight 2^12), 18 (the weight crosses that bound late and the tile takes the
exact path: new maximum, rescale of O and l) and 100 (a one-hot row: closed
form).  "CUDA Flash Attention: Online Softmax with Shared Memory Tiling",
section "Design decisions" (the guard against overflow and -inf - -inf).

Tolerances are the forward pass's (fp32: max |err| <= 1e-4 on O and LSE;
bf16 / fp16: max |err| <= 2e-2 and rel-L2 <= 5e-3 on O, max |err| <= 2e-2 on
LSE).  Outputs are pre-filled with NaN so that a row the kernel never writes
fails.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_attention_13_amd import binding
from exact_attention_13_amd.inputs import Workload, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
LN2 = math.log(2.0)

# (B, H, N): several key tiles and a ragged tail for every instance (d = 64
# bf16/fp16 tiles are 512 query rows x 128 keys, d = 128 ones 128 x 32, fp32
# ones 128 x 64); the fp32 small-problem kernel (16 rows per workgroup) takes
# grids of fewer than 128 workgroups of 128 rows, so (1, 2, 1000) runs it and
# (2, 8, 1000) does not.
SHAPES = [(1, 2, 1000), (2, 8, 1000)]


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run(q, k, v, scale, causal):
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    B, H, N, d = q.shape
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=DEV)
    binding.fwd(qd, kd, vd, scale, causal, out=o, lse=lse)
    torch.cuda.synchronize()
    return o.cpu().double().numpy(), lse.cpu().double().numpy()


def check(o, lse, o_ref, lse_ref, dtype, what):
    assert np.all(np.isfinite(o)), f"{what}: non-finite or unwritten O"
    assert np.all(np.isfinite(lse)), f"{what}: non-finite or unwritten LSE"
    err = float(np.max(np.abs(o - o_ref)))
    lerr = float(np.max(np.abs(lse - lse_ref)))
    if dtype == "f32":
        assert err <= 1e-4, f"{what}: max|dO| = {err:.3e}"
        assert lerr <= 1e-4, f"{what}: max|dLSE| = {lerr:.3e}"
    else:
        rel = float(np.linalg.norm(o - o_ref) / np.linalg.norm(o_ref))
        assert err <= 2e-2, f"{what}: max|dO| = {err:.3e}"
        assert rel <= 5e-3, f"{what}: rel-L2 = {rel:.3e}"
        assert lerr <= 2e-2, f"{what}: max|dLSE| = {lerr:.3e}"


def stored(t):
    return t.double().numpy()


CASES = [(dt, d, c, s) for dt in ("f32", "bf16", "f16") for d in (64, 128)
         for c in (False, True) for s in SHAPES]
IDS = [f"{dt}-d{d}-{'causal' if c else 'full'}-{s[0]}x{s[1]}x{s[2]}" for dt, d, c, s in CASES]


@pytest.mark.parametrize("dtype,d,causal,shape", CASES, ids=IDS)
def test_ones_values_give_ones(dtype, d, causal, shape):
    B, H, N = shape
    w = Workload("inv", dtype, B, H, N, d, causal, 4000 + d + N)
    q, k, _ = make_inputs(w)
    v = torch.ones_like(q)
    _note(f"V = 1: {dtype} d={d} causal={causal} {shape}")
    o, lse = run(q, k, v, w.scale, causal)
    _, lse_ref = oracle.fwd(q, k, v, w.scale, causal)
    check(o, lse, np.ones_like(o), lse_ref, dtype, "V = 1")


@pytest.mark.parametrize("dtype,d,causal,shape", CASES, ids=IDS)
def test_zero_queries_give_visible_mean(dtype, d, causal, shape):
    B, H, N = shape
    w = Workload("inv", dtype, B, H, N, d, causal, 4100 + d + N)
    _, k, v = make_inputs(w)
    q = torch.zeros_like(k)
    _note(f"Q = 0: {dtype} d={d} causal={causal} {shape}")
    o, lse = run(q, k, v, w.scale, causal)
    vs = stored(v)
    if causal:
        count = np.arange(1, N + 1, dtype=np.float64)
        o_ref = np.cumsum(vs, axis=2) / count[None, None, :, None]
        lse_ref = np.broadcast_to(np.log(count), (B, H, N))
    else:
        o_ref = np.broadcast_to(vs.mean(axis=2, keepdims=True), vs.shape)
        lse_ref = np.full((B, H, N), math.log(N))
    check(o, lse, o_ref, lse_ref, dtype, "Q = 0")


CAUSAL = [(c, i) for c, i in zip(CASES, IDS) if c[2]]


@pytest.mark.parametrize("dtype,d,causal,shape", [c for c, _ in CAUSAL], ids=[i for _, i in CAUSAL])
def test_causal_row_zero_is_first_value(dtype, d, causal, shape):
    B, H, N = shape
    w = Workload("inv", dtype, B, H, N, d, True, 4200 + d + N)
    q, k, v = make_inputs(w)
    _note(f"causal row 0: {dtype} d={d} {shape}")
    o, lse = run(q, k, v, w.scale, True)
    qs, ks, vs = stored(q), stored(k), stored(v)
    o0_ref = vs[:, :, 0, :]
    lse0_ref = float(np.float32(w.scale)) * np.einsum("bhc,bhc->bh", qs[:, :, 0], ks[:, :, 0])
    check(o[:, :, 0, :], lse[:, :, 0], o0_ref, lse0_ref, dtype, "row 0")
    o_ref, lse_ref = oracle.fwd(q, k, v, w.scale, True)
    check(o, lse, o_ref, lse_ref, dtype, "all rows")


def dominant_inputs(dtype, d, causal, shape, gap_exp2, seed):
    """Inputs where row i* = N-1 of every head scores key j* = N-2 about
    gap_exp2 (in exp2 units) above every other key it sees.  Returns
    (q, k, v, actual gaps in exp2 units per head)."""
    B, H, N = shape
    w = Workload("inv", dtype, B, H, N, d, causal, seed)
    q, k, v = make_inputs(w)
    scale = float(np.float32(w.scale))
    istar, jstar = N - 1, N - 2
    qs, ks = stored(q), stored(k)
    kn = ks.copy()
    for b in range(B):
        for h in range(H):
            qi = qs[b, h, istar]
            s = scale * (ks[b, h] @ qi)
            s[jstar] = -np.inf
            target = s.max() + gap_exp2 * LN2
            kn[b, h, jstar] = qi * (target / (scale * float(qi @ qi)))
    k = torch.from_numpy(kn.astype(np.float32)).to(TORCH[dtype])
    ks = stored(k)
    gaps = np.empty((B, H))
    for b in range(B):
        for h in range(H):
            s = scale * (ks[b, h] @ qs[b, h, istar])
            top = s[jstar]
            s[jstar] = -np.inf
            gaps[b, h] = (top - s.max()) / LN2
    return w, q, k, v, gaps


@pytest.mark.parametrize("gap", [12.0, 18.0, 100.0])
@pytest.mark.parametrize("dtype,d,causal,shape", CASES, ids=IDS)
def test_late_dominant_logit(dtype, d, causal, shape, gap):
    w, q, k, v, gaps = dominant_inputs(dtype, d, causal, shape, gap, 4300 + d + int(gap))
    assert np.all(np.abs(gaps - gap) < 1.5), f"constructed gaps {gaps.ravel()}"
    _note(f"dominant logit gap {gap}: {dtype} d={d} causal={causal} {shape}")
    o, lse = run(q, k, v, w.scale, causal)
    o_ref, lse_ref = oracle.fwd(q, k, v, w.scale, causal)
    check(o, lse, o_ref, lse_ref, dtype, f"gap {gap}")
    if gap >= 100.0:
        # one-hot row: O = V[j*] and LSE = s_{i* j*} to far below rounding
        N = q.shape[2]
        qs, ks, vs = stored(q), stored(k), stored(v)
        s_top = float(np.float32(w.scale)) * np.einsum("bhc,bhc->bh", qs[:, :, N - 1],
                                                       ks[:, :, N - 2])
        check(o[:, :, N - 1], lse[:, :, N - 1], vs[:, :, N - 2], s_top, dtype, "one-hot row")
