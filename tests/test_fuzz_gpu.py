"""Seeded random shapes through the extended entry points (MI355X only).

Eighty cases drawn from two fixed seeds over everything the extended calls
combine: element type, head size, causal mask, batch, grouped K/V heads,
query and key lengths (one query row, more queries than keys, lengths off
every tile size), key ranges of the forward split and head parts of the
backward.  Each case runs fa_fwd_ex then fa_bwd_ex and compares O, LSE, dQ,
dK and dV with the fp64 oracle on the same inputs, to the bounds of the
other parity tests (the gradient bounds with the per-element allowance for
D formed from the stored O, which large logits with few query rows make
visible).
"""
import numpy as np
import pytest
import torch

import oracle
from exact_attention_13_amd import binding
from exact_attention_13_amd.inputs import Workload, make_inputs, make_upstream
from test_parity_bwd_gpu import assert_grad_close, stored_o_allowance
from test_parity_ex_gpu import assert_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def draw_cases(count=40, seed=20240611):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        dtype = str(rng.choice(["f32", "bf16", "f16"]))
        d = int(rng.choice([64, 128]))
        causal = bool(rng.integers(2))
        B = int(rng.integers(1, 3))
        h_kv = int(rng.choice([1, 2, 3]))
        grp = int(rng.choice([1, 2, 4]))
        n_q = 1 if rng.random() < 0.15 else int(rng.integers(2, 400))
        n_kv = int(rng.integers(1, 600))
        splits = int(rng.choice([1, 1, 2, 5]))
        parts = int(rng.choice([1, 2, 3]))
        dist = "large_logit" if rng.random() < 0.2 else "normal"
        cases.append((i, dtype, d, causal, B, h_kv * grp, h_kv, n_q, n_kv, splits, parts, dist))
    return cases


# Two fixed draws of forty: the second spans the same space with other
# shapes (among them the short-grid tiles' switches).
CASES = draw_cases() + [(40 + c[0],) + c[1:] for c in draw_cases(40, seed=777001)]


@pytest.mark.parametrize("case", CASES, ids=[f"case{c[0]}" for c in CASES])
def test_random_shapes(case):
    i, dtype, d, causal, B, H, h_kv, n_q, n_kv, splits, parts, dist = case
    w = Workload("fuzz", dtype, B, H, n_q, d, causal, 3000 + i, dist, Hkv=h_kv, Nkv=n_kv)
    q, k, v = make_inputs(w)
    dout = make_upstream(w, 3100 + i)
    print(f"fuzz {case}", flush=True)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, dout))
    o, lse = binding.fwd_ex(qd, kd, vd, w.scale, causal, num_splits=splits)
    dq, dk, dv = binding.bwd(qd, kd, vd, o, lse, gd, w.scale, causal, num_splits=parts)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.fwd_gqa(q, k, v, w.scale, causal)
    assert_close(o.cpu(), lse.cpu(), o_ref, lse_ref, dtype, f"case {i} forward")
    rq, rk, rv = oracle.bwd(q, k, v, dout, w.scale, causal)
    a_q, a_k = stored_o_allowance(q, k, dout, o.cpu(), o_ref, lse_ref, w.scale, causal)
    for got, ref, name, a in ((dq, rq, "dQ", a_q), (dk, rk, "dK", a_k), (dv, rv, "dV", None)):
        assert_grad_close(got.cpu(), ref, dtype, f"case {i} {name}", extra=a)
