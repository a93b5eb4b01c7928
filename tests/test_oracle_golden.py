"""The oracle reproduces its stored outputs (regression guard, not a pin)."""
import json
from pathlib import Path

import numpy as np

import oracle
from exact_attention_13_amd.inputs import Workload, make_inputs, make_upstream

GOLDEN = Path(__file__).resolve().parent / "golden" / "oracle_small.json"


def test_oracle_matches_stored_outputs(oracle_lib):
    for case in json.loads(GOLDEN.read_text()):
        dtype, B, H, N, d, causal, seed, dist = case["workload"]
        w = Workload(case["name"], dtype, B, H, N, d, causal, seed, dist)
        q, k, v = make_inputs(w)
        o, lse = oracle.fwd(q, k, v, w.scale, w.causal)
        np.testing.assert_allclose(o.ravel(), case["o"], rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(lse.ravel(), case["lse"], rtol=1e-14, atol=1e-15)


EXTENDED = Path(__file__).resolve().parent / "golden" / "oracle_extended.json"


def test_oracle_matches_stored_extended_outputs(oracle_lib):
    # grouped K/V heads with N_q != N_kv (forward) and gradients
    for case in json.loads(EXTENDED.read_text()):
        dtype, B, H, N, d, causal, seed, dist, hkv, nkv = case["workload"]
        w = Workload(case["name"], dtype, B, H, N, d, causal, seed, dist, Hkv=hkv, Nkv=nkv)
        q, k, v = make_inputs(w)
        if case["kind"] == "fwd":
            o, lse = oracle.fwd_gqa(q, k, v, w.scale, w.causal)
            got = {"o": o, "lse": lse}
        else:
            dq, dk, dv = oracle.bwd(q, k, v, make_upstream(w, w.seed + 100), w.scale, w.causal)
            got = {"dq": dq, "dk": dk, "dv": dv}
        for key, val in got.items():
            np.testing.assert_allclose(val.ravel(), case[key], rtol=1e-13, atol=1e-15)
