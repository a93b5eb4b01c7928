"""Parity of the HIP backward pass (fa_bwd) with the fp64 oracle (MI355X only).

Every case runs fa_fwd then fa_bwd through the C ABI on seeded inputs and a
seeded upstream gradient dO, and compares dQ, dK, dV element by element with
``oracle.bwd`` (fp64 gradients of sum(dO * O) computed from the same stored
bits).

Tolerance (no accuracy target is stated for gradients; this one is derived
from the arithmetic).  The kernels round P and dS to the input type for the MFMA
operands, and round dQ, dK, dV once from fp32 accumulators; each of these
three roundings is relative, at most one unit roundoff of the type (bf16
2^-8, fp16 2^-11).  With u = 2^-9 for bf16 (half its unit roundoff) and
2^-11 for fp16, measured errors are about 1.3 u (rel-L2).  The bound is
    ||G - G_ref||_2 <= 5 u ||G_ref||_2 + 1e-5 sqrt(n)
    max |G - G_ref| <= 10 u max|G_ref| + 1e-4
for every gradient G.  The absolute floor covers gradients that vanish in
exact arithmetic (one key: the softmax is constant, so dQ = dK = 0, while
the kernels carry rounding residues of the recomputed weights).

fp32 inputs keep P and dS in fp32 (fp32 MFMA), so the error is the fp32
accumulation over up to N terms (about sqrt(N) 2^-24 relative, 2^-17 for
N = 16384) plus v_exp_f32's last-bit error: the same bound with u = 2^-17.

One more source is not relative to the gradient: D_i = dO_i . O_i is formed
from the O the forward pass stored (the backward pass takes it as an input),
while the oracle differentiates the exact O.  The error of that input,
dD_i = dO_i . (O_stored,i - O_exact,i), is known exactly in a test (both O are
at hand), and to first order it moves dQ_i by -scale dD_i sum_j P_ij k_j and
dK_j by -scale sum_i P_ij dD_i q_i.  ``stored_o_allowance`` turns that into a
per-element allowance (absolute values of those terms, with the exact fp64
weights) for the tests whose inputs make it visible (large logits with few
query rows: dQ_i and dK are then small next to |dO_i| |O_i|); the
element-wise bound adds each element's own allowance, the L2 bound the
allowance's L2 norm.  For ordinary inputs the allowance is orders of
magnitude below the relative bound.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_attention_13_amd import binding
from exact_attention_13_amd.inputs import WORKLOADS, Workload, make_inputs, make_upstream, sample_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
UNIT = {"bf16": 2.0 ** -9, "f16": 2.0 ** -11, "f32": 2.0 ** -17}
TORCH = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def upstream(w, seed):
    return make_upstream(w, seed)


def run_bwd(w, q, k, v, dout):
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, dout))
    o, lse = binding.fwd(qd, kd, vd, w.scale, w.causal)
    dq, dk, dv = binding.bwd(qd, kd, vd, o, lse, gd, w.scale, w.causal)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def assert_grad_close(got, ref, dtype, what, extra=None):
    """Element-wise and L2 comparison; ``extra`` is an optional per-element
    allowance (an array shaped like ``ref``) added to the element-wise bound,
    its L2 norm to the L2 bound."""
    g = got.to(torch.float64).numpy().reshape(ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite gradient"
    u = UNIT[dtype]
    diff = g - ref
    ex = np.zeros_like(ref) if extra is None else np.asarray(extra).reshape(ref.shape)
    l2 = float(np.linalg.norm(diff))
    bound = 5 * u * float(np.linalg.norm(ref)) + 1e-5 * np.sqrt(ref.size) + float(np.linalg.norm(ex))
    assert l2 <= bound, f"{what}: ||dG|| = {l2:.3e} > {bound:.3e}"
    if diff.size:
        mbound = 10 * u * float(np.abs(ref).max()) + 1e-4 + ex
        over = np.abs(diff) - mbound
        k = int(np.argmax(over))
        assert over.flat[k] <= 0, (f"{what}: |dG| = {abs(diff.flat[k]):.3e} > "
                                   f"{mbound.flat[k]:.3e} at flat index {k}")


def stored_o_allowance(q, k, dout, o_stored, o_ref, lse_ref, scale, causal):
    """Per-element allowances (for dQ and dK) for the error that forming D
    from the stored O causes, from the exact dD_i and the exact weights (see
    the module docstring).  q, dout, o_*: [B, H, N_q, d]; k: [B, H_kv, N_kv, d];
    lse_ref: [B, H, N_q].  Small shapes only (the weights are formed)."""
    qs = q.to(torch.float64).numpy()
    ks = k.to(torch.float64).numpy()
    g = dout.to(torch.float64).numpy()
    os_ = o_stored.to(torch.float64).numpy().reshape(o_ref.shape)
    dd = np.abs((g * (os_ - o_ref)).sum(-1))  # |dD_i|, [B, H, N_q]
    B, H, nq, d = qs.shape
    hkv, nk = ks.shape[1], ks.shape[2]
    grp = H // hkv
    a_q = np.zeros_like(qs)
    a_k = np.zeros_like(ks)
    s64 = float(np.float32(scale))
    i = np.arange(nq)[:, None]
    j = np.arange(nk)[None, :]
    hidden = j > i + (nk - nq) if causal else np.zeros((nq, nk), dtype=bool)
    for b in range(B):
        for h in range(H):
            kh = ks[b, h // grp]
            s = s64 * (qs[b, h] @ kh.T)
            with np.errstate(invalid="ignore"):  # rows with no visible key: lse = -inf
                p = np.where(hidden, 0.0, np.exp(np.where(hidden, -np.inf, s) - lse_ref[b, h][:, None]))
            a_q[b, h] = s64 * dd[b, h][:, None] * np.abs(p @ kh)
            a_k[b, h // grp] += s64 * (p.T @ (dd[b, h][:, None] * np.abs(qs[b, h])))
    return a_q, a_k


SMALL_N = [1, 31, 32, 33, 100, 128, 129, 257, 512]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_small_shapes(dtype, d, causal):
    for i, n in enumerate(SMALL_N):
        B, H = (1, 2) if i % 2 else (2, 1)
        w = Workload("case", dtype, B, H, n, d, causal, 1100 + i)
        q, k, v = make_inputs(w)
        dout = upstream(w, 1200 + i)
        _note(f"bwd {dtype} d={d} causal={causal} B={B} H={H} N={n}")
        dq, dk, dv = run_bwd(w, q, k, v, dout)
        rq, rk, rv = oracle.bwd(q, k, v, dout, w.scale, causal)
        for got, ref, name in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
            assert_grad_close(got, ref, dtype, f"N={n} {name}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_d64_dq_short_grid_switch(dtype, causal):
    # d = 64 dQ grids of fewer than 256 workgroups of 256 rows take 128-row
    # workgroups (one 32-row block per wave).  Both sides of the switch
    # (255 and 256 problems of one block), multi-block heads on the short
    # side, ragged tails.
    for i, (B, H, n) in enumerate(((1, 255, 40), (1, 256, 40), (3, 5, 700), (1, 1, 129))):
        w = Workload("case", dtype, B, H, n, 64, causal, 1350 + i)
        q, k, v = make_inputs(w)
        dout = upstream(w, 1360 + i)
        _note(f"bwd dQ short grid {dtype} causal={causal} B={B} H={H} N={n}")
        dq, dk, dv = run_bwd(w, q, k, v, dout)
        rq, rk, rv = oracle.bwd(q, k, v, dout, w.scale, causal)
        for got, ref, name in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
            assert_grad_close(got, ref, dtype, f"B={B} H={H} N={n} {name}")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_bwd_large_logits(dtype):
    # scores with std ~ 9: most weights are tiny, a few dominate each row
    w = Workload("case", dtype, 1, 2, 333, 128, True, 1300, "large_logit")
    q, k, v = make_inputs(w)
    dout = upstream(w, 1301)
    _note(f"bwd large-logit {dtype}")
    dq, dk, dv = run_bwd(w, q, k, v, dout)
    rq, rk, rv = oracle.bwd(q, k, v, dout, w.scale, True)
    for got, ref, name in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
        assert_grad_close(got, ref, dtype, name)


def test_bwd_deterministic_and_delta():
    w = Workload("case", "bf16", 2, 2, 700, 64, True, 1400)
    q, k, v = make_inputs(w)
    dout = upstream(w, 1401)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, dout))
    o, lse = binding.fwd(qd, kd, vd, w.scale, True)
    _note("bwd determinism")
    r1 = binding.bwd(qd, kd, vd, o, lse, gd, w.scale, True)
    r2 = binding.bwd(qd, kd, vd, o, lse, gd, w.scale, True)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
    # the scratch delta holds the row dot products dO . O of the stored values
    delta = torch.empty((2, 2, 700), dtype=torch.float32, device=DEV)
    outs = [torch.empty_like(qd) for _ in range(3)]
    st = binding.fa_bwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), gd.data_ptr(),
                        lse.data_ptr(), *(t.data_ptr() for t in outs), delta.data_ptr(),
                        2, 2, 700, 64, w.scale, True, binding.FA_BF16,
                        torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    ref = (o.cpu().double() * dout.double()).sum(-1)
    np.testing.assert_allclose(delta.cpu().double().numpy(), ref.numpy(), rtol=1e-5, atol=1e-5)


def test_bwd_medium_full_oracle():
    w = Workload("case", "bf16", 1, 2, 2048, 128, True, 1500)
    q, k, v = make_inputs(w)
    dout = upstream(w, 1501)
    _note("bwd medium full")
    dq, dk, dv = run_bwd(w, q, k, v, dout)
    rq, rk, rv = oracle.bwd(q, k, v, dout, w.scale, True)
    for got, ref, name in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
        assert_grad_close(got, ref, "bf16", name)


def whole_heads(w):
    """(b, h) of the heads a full-size test compares element by element: the
    first and the last head of the workload."""
    return [(0, 0), (w.B - 1, w.H - 1)]


@pytest.mark.parametrize("name", ["C2", "C2r"])
def test_bwd_workload_full_oracle(name):
    # fp32 workloads: every gradient of every head against the oracle.
    w = WORKLOADS[name]
    q, k, v = make_inputs(w)
    dout = upstream(w, 1600)
    _note(f"bwd workload {name} full")
    dq, dk, dv = run_bwd(w, q, k, v, dout)
    rq, rk, rv = oracle.bwd(q, k, v, dout, w.scale, w.causal)
    for got, ref, g in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
        assert_grad_close(got, ref, w.dtype, f"{name} {g}")


@pytest.mark.parametrize("name", ["C3", "C4", "C5"])
def test_bwd_workload_whole_heads_and_sampled_rows(name):
    # Full size.  Two whole heads (the first and the last) against the
    # oracle run on that head's slice, element by element for dQ, dK and dV
    # (heads are independent, so the slice is the exact sub-problem); dQ rows
    # sampled across every head; and for every head what holds at any size:
    # the key gradients sum to zero and the value gradients to the sum of
    # the dO rows.
    w = WORKLOADS[name]
    q, k, v = make_inputs(w)
    dout = upstream(w, 1600)
    _note(f"bwd workload {name}")
    dq, dk, dv = run_bwd(w, q, k, v, dout)
    for b, h in whole_heads(w):
        _note(f"bwd workload {name} head ({b}, {h})")
        sl = (slice(b, b + 1), slice(h, h + 1))
        rq, rk, rv = oracle.bwd(q[sl], k[sl], v[sl], dout[sl], w.scale, w.causal)
        for got, ref, g in ((dq[sl], rq, "dQ"), (dk[sl], rk, "dK"), (dv[sl], rv, "dV")):
            assert_grad_close(got, ref, w.dtype, f"{name} head ({b}, {h}) {g}")
    rows = sample_rows(w, 256)
    ref = oracle.bwd_dq_rows(q, k, v, dout, w.scale, w.causal, rows)
    got = dq.reshape(-1, w.d)[torch.from_numpy(rows)]
    assert_grad_close(got, ref, w.dtype, f"{name} dQ rows")
    u = UNIT[w.dtype]
    dk64, dv64 = dk.double(), dv.double()
    sum_k = dk64.sum(dim=2)
    assert float(sum_k.norm()) <= 5 * u * float(dk64.norm()), f"{name}: sum of dK rows"
    sum_v = dv64.sum(dim=2)
    sum_g = dout.double().sum(dim=2)
    assert float((sum_v - sum_g).norm()) <= 5 * u * float(dv64.norm()), f"{name}: sum of dV rows"


# --------------------------------------------------------------------------
# Grouped K/V heads and N_q != N_kv (fa_bwd_ex)
# --------------------------------------------------------------------------

def run_bwd_ex(w, q, k, v, dout, splits=1, parts=None):
    # splits: the forward's key ranges; parts: the backward's head parts
    # (None: the library's default)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, dout))
    o, lse = binding.fwd_ex(qd, kd, vd, w.scale, w.causal, num_splits=splits)
    dq, dk, dv = binding.bwd(qd, kd, vd, o, lse, gd, w.scale, w.causal, num_splits=parts)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


GROUPED = [  # (H, H_kv, N_q, N_kv)
    (4, 2, 100, 100), (4, 1, 77, 300), (6, 2, 300, 77), (8, 8, 33, 65), (2, 1, 1, 1000),
    (4, 4, 129, 129), (16, 2, 40, 257),
]


# Head parts per group: 1 (one workgroup sums the whole group) and 3, which
# cuts groups of 4 into parts of 1, 1, 2 heads and groups of 8 into 2, 3, 3
# (groups of 2 into 2 parts).
@pytest.mark.parametrize("parts", [1, 3])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_grouped_shapes(dtype, d, causal, parts):
    for i, (H, Hkv, Nq, Nk) in enumerate(GROUPED):
        w = Workload("case", dtype, 2 if i % 2 else 1, H, Nq, d, causal, 1700 + i, "normal", Hkv, Nk)
        q, k, v = make_inputs(w)
        dout = upstream(w, 1800 + i)
        _note(f"bwd_ex {dtype} d={d} causal={causal} B={w.B} H={H} H_kv={Hkv} N_q={Nq} "
              f"N_kv={Nk} parts={parts}")
        dq, dk, dv = run_bwd_ex(w, q, k, v, dout, parts=parts)
        rq, rk, rv = oracle.bwd(q, k, v, dout, w.scale, causal)
        for got, ref, name in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
            assert_grad_close(got, ref, dtype, f"{(H, Hkv, Nq, Nk)} {name}")
        if causal and Nq > Nk:
            assert torch.all(dq[:, :, : Nq - Nk] == 0)


def test_bwd_grouped_after_split_forward():
    # the forward's key split changes only how O and LSE were formed
    w = Workload("case", "bf16", 2, 8, 3, 128, False, 1900, "normal", 2, 4000)
    q, k, v = make_inputs(w)
    dout = upstream(w, 1901)
    _note("bwd_ex after a split forward")
    dq, dk, dv = run_bwd_ex(w, q, k, v, dout, splits=8)
    rq, rk, rv = oracle.bwd(q, k, v, dout, w.scale, False)
    for got, ref, name in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
        assert_grad_close(got, ref, "bf16", name)


def test_bwd_ex_empty_sides_are_zero_filled():
    # N_q = 0: no query uses the keys, so dK = dV = 0; N_kv = 0: dQ = 0.
    st = torch.cuda.current_stream().cuda_stream
    kv = torch.randn((1, 2, 70, 64), device=DEV).to(torch.bfloat16)
    dk = torch.full_like(kv, float("nan"))
    dv = torch.full_like(kv, float("nan"))
    _note("bwd_ex N_q = 0")
    for parts in (1, 2):  # no queries: one part whatever num_splits asks, no workspace
        dk.fill_(float("nan"))
        dv.fill_(float("nan"))
        s = binding.fa_bwd_ex(0, kv.data_ptr(), kv.data_ptr(), 0, 0, 0, 0, dk.data_ptr(),
                              dv.data_ptr(), 0, 1, 4, 2, 0, 70, 64, 0.125, True, binding.FA_BF16,
                              parts, None, 0, st)
        assert s == 0
        torch.cuda.synchronize()
        assert torch.all(dk == 0) and torch.all(dv == 0)
    q = torch.randn((1, 4, 50, 64), device=DEV).to(torch.bfloat16)
    o, g = torch.zeros_like(q), torch.randn_like(q)
    lse = torch.full((1, 4, 50), float("-inf"), device=DEV)
    dq = torch.full_like(q, float("nan"))
    delta = torch.empty_like(lse)
    _note("bwd_ex N_kv = 0")
    s = binding.fa_bwd_ex(q.data_ptr(), 0, 0, o.data_ptr(), g.data_ptr(), lse.data_ptr(),
                          dq.data_ptr(), 0, 0, delta.data_ptr(), 1, 4, 2, 50, 0, 64, 0.125, False,
                          binding.FA_BF16, 2, None, 0, st)
    assert s == 0
    torch.cuda.synchronize()
    assert torch.all(dq == 0)


def test_bwd_grouped_deterministic():
    w = Workload("case", "f16", 1, 8, 600, 128, True, 1950, "normal", 2, 700)
    q, k, v = make_inputs(w)
    dout = upstream(w, 1951)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, dout))
    o, lse = binding.fwd_ex(qd, kd, vd, w.scale, True, num_splits=1)
    for parts in (1, 2, 4):
        _note(f"bwd_ex determinism parts={parts}")
        r1 = binding.bwd(qd, kd, vd, o, lse, gd, w.scale, True, num_splits=parts)
        r2 = binding.bwd(qd, kd, vd, o, lse, gd, w.scale, True, num_splits=parts)
        torch.cuda.synchronize()
        for a, b in zip(r1, r2):
            assert torch.equal(a, b)
        if parts == 1:
            one = r1
        else:
            # dQ does not depend on the parts; dK, dV differ by summation order
            assert torch.equal(r1[0], one[0])
            for a, b in zip(r1[1:], one[1:]):
                assert float((a.float() - b.float()).abs().max()) <= 4 * 2.0 ** -11 * float(
                    b.float().abs().max())


def test_bwd_workload_g2_sampled_rows_and_invariants():
    # G2: bf16 B=8, 16 query heads on 2 K/V heads, N=4096, d=128, causal.
    # dQ rows sampled against the oracle; per K/V head the key gradients sum
    # to zero and the value gradients to the sum of its group's dO rows.
    w = WORKLOADS["G2"]
    q, k, v = make_inputs(w)
    dout = upstream(w, 2000)
    parts = binding.bwd_default_splits(w.B, w.H, w.h_kv, w.N, w.n_kv, w.d, w.causal,
                                       binding.FA_BF16)
    _note(f"bwd workload G2, default head parts {parts}")
    dq, dk, dv = run_bwd_ex(w, q, k, v, dout)
    # the first and the last K/V head with their groups of query heads,
    # element by element against the oracle on that slice
    grp = w.H // w.h_kv
    for b, g in ((0, 0), (w.B - 1, w.h_kv - 1)):
        _note(f"bwd workload G2 K/V head ({b}, {g})")
        qs_ = (slice(b, b + 1), slice(g * grp, (g + 1) * grp))
        ks_ = (slice(b, b + 1), slice(g, g + 1))
        rq, rk, rv = oracle.bwd(q[qs_], k[ks_], v[ks_], dout[qs_], w.scale, w.causal)
        for got, ref, name in ((dq[qs_], rq, "dQ"), (dk[ks_], rk, "dK"), (dv[ks_], rv, "dV")):
            assert_grad_close(got, ref, w.dtype, f"G2 K/V head ({b}, {g}) {name}")
    rows = sample_rows(w, 256)
    ref = oracle.bwd_dq_rows(q, k, v, dout, w.scale, w.causal, rows)
    got = dq.reshape(-1, w.d)[torch.from_numpy(rows)]
    assert_grad_close(got, ref, w.dtype, "G2 dQ rows")
    u = UNIT[w.dtype]
    dk64, dv64 = dk.double(), dv.double()
    assert float(dk64.sum(dim=2).norm()) <= 5 * u * float(dk64.norm()), "G2: sum of dK rows"
    grp = w.H // w.h_kv
    sum_g = dout.double().sum(dim=2).reshape(w.B, w.h_kv, grp, w.d).sum(dim=2)
    assert float((dv64.sum(dim=2) - sum_g).norm()) <= 5 * u * float(dv64.norm()), "G2: dV rows"
    # one part per group (a single workgroup sums the group) agrees to rounding
    _note("bwd workload G2, one head part")
    _, dk1, dv1 = run_bwd_ex(w, q, k, v, dout, parts=1)
    for a, b, name in ((dk, dk1, "dK"), (dv, dv1, "dV")):
        assert float((a.double() - b.double()).norm()) <= 2 * u * float(b.double().norm()), name


def test_bwd_f32_deterministic_and_delta():
    w = Workload("case", "f32", 2, 2, 333, 128, True, 2100)
    q, k, v = make_inputs(w)
    dout = upstream(w, 2101)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, dout))
    o, lse = binding.fwd(qd, kd, vd, w.scale, True)
    _note("bwd f32 determinism")
    r1 = binding.bwd(qd, kd, vd, o, lse, gd, w.scale, True)
    r2 = binding.bwd(qd, kd, vd, o, lse, gd, w.scale, True)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
    delta = torch.empty((2, 2, 333), dtype=torch.float32, device=DEV)
    outs = [torch.empty_like(qd) for _ in range(3)]
    st = binding.fa_bwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), gd.data_ptr(),
                        lse.data_ptr(), *(t.data_ptr() for t in outs), delta.data_ptr(),
                        2, 2, 333, 128, w.scale, True, binding.FA_F32,
                        torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    ref = (o.cpu().double() * dout.double()).sum(-1)
    np.testing.assert_allclose(delta.cpu().double().numpy(), ref.numpy(), rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("dtype,d,parts", [("bf16", 128, 2), ("f16", 64, 4), ("f32", 64, 2)])
def test_bwd_canaries_untouched_and_not_read(dtype, d, parts):
    # Every buffer (inputs, gradients, delta, the head-part workspace) sits at
    # the front of a larger allocation whose tail is NaN.  Writes must leave
    # the tails alone, and reads must not reach them (a read would put NaN
    # into a gradient).
    B, H, Hkv, Nq, Nk = 1, 4, 1, 150, 333
    w = Workload("case", dtype, B, H, Nq, d, True, 2300, "normal", Hkv, Nk)
    q, k, v = make_inputs(w)
    dout = upstream(w, 2301)
    tdt = TORCH[dtype]
    pad = 4096
    nq, nk, nl = B * H * Nq * d, B * Hkv * Nk * d, B * H * Nq

    def fenced(n, dt, src=None):
        buf = torch.full((n + pad,), float("nan"), dtype=dt, device=DEV)
        if src is not None:
            buf[:n] = src.reshape(-1).to(DEV)
        return buf

    qb, gb = fenced(nq, tdt, q), fenced(nq, tdt, dout)
    kb, vb = fenced(nk, tdt, k), fenced(nk, tdt, v)
    ob, lb = fenced(nq, tdt), fenced(nl, torch.float32)
    shape_q, shape_k = (B, H, Nq, d), (B, Hkv, Nk, d)
    binding.fwd_ex(qb[:nq].view(shape_q), kb[:nk].view(shape_k), vb[:nk].view(shape_k), w.scale,
                   True, num_splits=1, out=ob[:nq].view(shape_q), lse=lb[:nl].view(B, H, Nq))
    dqb, dkb, dvb, deltab = fenced(nq, tdt), fenced(nk, tdt), fenced(nk, tdt), fenced(nl, torch.float32)
    wsn = binding.bwd_workspace_bytes(B, H, Hkv, Nq, Nk, d, parts)
    assert wsn == 2 * parts * nk * 4
    wsb = torch.full((wsn + 4 * pad,), 0xFF, dtype=torch.uint8, device=DEV)  # NaN as fp32
    code = {"f32": binding.FA_F32, "bf16": binding.FA_BF16, "f16": binding.FA_F16}[dtype]
    _note(f"bwd canaries {dtype} d={d} parts={parts}")
    st = binding.fa_bwd_ex(qb.data_ptr(), kb.data_ptr(), vb.data_ptr(), ob.data_ptr(),
                           gb.data_ptr(), lb.data_ptr(), dqb.data_ptr(), dkb.data_ptr(),
                           dvb.data_ptr(), deltab.data_ptr(), B, H, Hkv, Nq, Nk, d, w.scale, True,
                           code, parts, wsb.data_ptr(), wsn,
                           torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    for buf, n, name in ((dqb, nq, "dq"), (dkb, nk, "dk"), (dvb, nk, "dv"), (deltab, nl, "delta")):
        assert torch.isnan(buf[n:]).all(), f"{name}: tail written"
    assert bool((wsb[wsn:] == 0xFF).all()), "workspace: tail written"
    rq, rk, rv = oracle.bwd(q, k, v, dout, w.scale, True)
    for buf, n, shape, ref, name in ((dqb, nq, shape_q, rq, "dQ"), (dkb, nk, shape_k, rk, "dK"),
                                     (dvb, nk, shape_k, rv, "dV")):
        assert_grad_close(buf[:n].view(shape).cpu(), ref, dtype, name)


# The dQ kernel takes the same grouped heavy-first causal order: shapes whose
# grid splits evenly over the eight dies (d = 64 dQ tiles hold 256 rows,
# d = 128 and fp32 ones 128), 3, 5 and 2 units per die.
@pytest.mark.parametrize("dtype,B,H,N,d", [("bf16", 2, 12, 520, 64), ("bf16", 2, 20, 300, 128),
                                           ("f32", 1, 16, 260, 64)])
def test_bwd_causal_tile_order_groups(dtype, B, H, N, d):
    w = Workload("case", dtype, B, H, N, d, True, 2400 + H)
    q, k, v = make_inputs(w)
    dout = upstream(w, 2401 + H)
    _note(f"bwd causal order {dtype} B={B} H={H} N={N} d={d}")
    dq, dk, dv = run_bwd(w, q, k, v, dout)
    rq, rk, rv = oracle.bwd(q, k, v, dout, w.scale, True)
    for got, ref, name in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
        assert_grad_close(got, ref, dtype, f"{(dtype, B, H, N, d)} {name}")


# Gradients of tensors past 4 GiB (head offsets beyond 2^31 and 2^32 bytes):
# the inputs and dO repeat a seeded block of 97 heads along H; the first
# block is checked against the oracle and every later head must equal its
# image in the first block bitwise (97 does not divide the 2^32-byte head
# count, so an offset wrapped at 32 bits would read other data).
def test_bwd_tensors_past_4gib():
    P, H, N, d = 97, 33000, 512, 128
    w = Workload("big", "bf16", 1, P, N, d, True, 2500)
    q, k, v = make_inputs(w)
    dout = upstream(w, 2501)
    assert H * N * d * 2 > 2 ** 32
    _note(f"bwd past 4 GiB H={H} N={N} d={d}")

    def periodic(x):
        reps = -(-H // P)
        return x.to(DEV).repeat(1, reps, 1, 1)[:, :H].contiguous()

    qd, kd, vd, gd = periodic(q), periodic(k), periodic(v), periodic(dout)
    o, lse = binding.fwd(qd, kd, vd, w.scale, True)
    dq, dk, dv = binding.bwd(qd, kd, vd, o, lse, gd, w.scale, True)
    torch.cuda.synchronize()
    del qd, kd, vd, gd, o, lse
    rq, rk, rv = oracle.bwd(q, k, v, dout, w.scale, True)
    for got, ref, name in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
        assert_grad_close(got[:, :P].cpu(), ref, "bf16", f"first block {name}")
        assert torch.equal(got, periodic(got[:, :P])), f"{name}: a head past the first block differs"


# Calls on a side stream while the current stream at once allocates and
# fills memory: the scratch the binding allocates for a call (the forward's
# key-range workspace, the backward's row dot products and head-part
# workspace) is allocated under the call's stream, so the caching allocator
# cannot hand it to the current stream's work while the kernels still use it.
def test_side_stream_scratch_is_not_reused_early():
    w = Workload("side", "bf16", 2, 8, 2000, 128, True, 2600, Hkv=2)
    q, k, v = make_inputs(w)
    dout = upstream(w, 2601)
    _note("side-stream scratch")
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, dout))
    o_ref, lse_ref = binding.fwd_ex(qd, kd, vd, w.scale, True, num_splits=4)
    g_ref = binding.bwd(qd, kd, vd, o_ref, lse_ref, gd, w.scale, True, num_splits=4)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    o, lse = binding.fwd_ex(qd, kd, vd, w.scale, True, num_splits=4, stream=side)
    junk = [torch.full((1 << 22,), float("nan"), device=DEV) for _ in range(8)]
    g = binding.bwd(qd, kd, vd, o, lse, gd, w.scale, True, stream=side, num_splits=4)
    junk += [torch.full((1 << 22,), float("nan"), device=DEV) for _ in range(8)]
    side.synchronize()
    torch.cuda.synchronize()
    assert len(junk) == 16
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    for a, b, name in zip(g, g_ref, ("dQ", "dK", "dV")):
        assert torch.equal(a, b), f"{name} on the side stream differs"
