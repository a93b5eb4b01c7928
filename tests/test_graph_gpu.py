"""The entry points inside a captured HIP graph, and from several host
threads at once (MI355X only).

libfa's calls allocate nothing, clear nothing and never synchronise, so a
caller can capture them (with the buffers torch allocates around them) into
one graph and replay it.  Every replay here is compared bitwise with eager
calls on the same inputs (the kernels are deterministic), with new inputs
copied into the captured buffers and unrelated eager work between replays;
the first replay is also checked against the fp64 oracle.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_attention_13_amd import binding
from exact_attention_13_amd.inputs import Workload, make_inputs, make_upstream

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# (name, workload, forward key ranges, backward head parts): the square path
# (fa_fwd, fa_bwd) and the extended one with a split forward and head parts
# (fa_fwd_ex and fa_bwd_ex, both with workspaces allocated during capture).
CASES = [
    ("square", Workload("graph_sq", "bf16", 2, 4, 700, 64, True, 71), 1, None),
    ("extended", Workload("graph_ex", "f16", 1, 8, 300, 128, True, 73, Hkv=2, Nkv=1000), 4, 2),
]


def _step(w, q, k, v, g, splits, parts):
    if w.extended:
        o, lse = binding.fwd_ex(q, k, v, w.scale, w.causal, num_splits=splits)
    else:
        o, lse = binding.fwd(q, k, v, w.scale, w.causal)
    dq, dk, dv = binding.bwd(q, k, v, o, lse, g, w.scale, w.causal, num_splits=parts)
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("name,w,splits,parts", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(name, w, splits, parts):
    _note(f"graph capture {name}")
    inputs = [make_inputs(w.with_(seed=w.seed + 10 * r)) + (make_upstream(w, w.seed + 10 * r + 1),)
              for r in range(3)]
    static = [t.to(DEV) for t in inputs[0]]

    # warm-up on a side stream, as torch asks before capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(w, *static, splits, parts)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = _step(w, *static, splits, parts)

    for r in (0, 1, 2, 0):
        for dst, src in zip(static, inputs[r]):
            dst.copy_(src)
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs]
        # unrelated eager work between replays, then the eager reference
        junk = torch.randn(1 << 20, device=DEV).sum()
        fresh = [t.to(DEV) for t in inputs[r]]
        ref = _step(w, *fresh, splits, parts)
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for a, b, what in zip(got, ref, ("O", "LSE", "dQ", "dK", "dV")):
            assert torch.equal(a, b), f"{name} replay with inputs {r}: {what} differs from eager"
        if r == 0:
            q, k, v, _ = inputs[0]
            if w.extended:
                o_ref, lse_ref = oracle.fwd_gqa(q, k, v, w.scale, w.causal)
            else:
                o_ref, lse_ref = oracle.fwd(q, k, v, w.scale, w.causal)
            o = got[0].cpu().double().numpy().reshape(o_ref.shape)
            assert float(np.max(np.abs(o - o_ref))) <= 2e-2
            rel = np.linalg.norm(o - o_ref) / np.linalg.norm(o_ref)
            assert rel <= 5e-3, f"{name}: rel-L2 {rel:.2e}"


def test_concurrent_host_threads():
    # The library holds no mutable global state: calls from several host
    # threads at once, each on its own stream with its own buffers (split
    # forward with a workspace, backward with head parts), give the results
    # of one thread calling alone, bitwise.
    import threading

    w = Workload("threads", "bf16", 1, 8, 600, 64, True, 75, Hkv=2, Nkv=900)
    q, k, v = make_inputs(w)
    g = make_upstream(w, 76)
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    ref = _step(w, qd, kd, vd, gd, 3, 2)
    torch.cuda.synchronize()
    results, errors = {}, []

    def worker(t):
        try:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.default_stream())
            with torch.cuda.stream(s):
                outs = [_step(w, qd, kd, vd, gd, 3, 2) for _ in range(4)]
            s.synchronize()
            results[t] = outs
        except Exception as e:  # reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=60)
    assert not errors, errors
    assert sorted(results) == [0, 1, 2, 3]
    for t, outs in results.items():
        for got in outs:
            for a, b, what in zip(got, ref, ("O", "LSE", "dQ", "dK", "dV")):
                assert torch.equal(a, b), f"thread {t}: {what} differs"
