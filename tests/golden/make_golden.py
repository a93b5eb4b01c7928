"""Writes tests/golden/oracle_small.json and oracle_extended.json: oracle outputs on tiny seeded inputs.

Calls only the oracle and the seeded input recipe.  The fixture guards the
oracle against unintended changes; it is not a pin (the pins are in
tests/test_oracle_pins.py).  Regenerate with: python tests/golden/make_golden.py
"""
import json
import sys
from pathlib import Path

ROOT = Path(__file__).resolve().parents[2]
sys.path.insert(0, str(ROOT))

import oracle  # noqa: E402
from exact_attention_13_amd.inputs import Workload, make_inputs, make_upstream  # noqa: E402

CASES = [Workload("g-f32", "f32", 1, 2, 37, 8, False, 7),
         Workload("g-bf16-causal", "bf16", 1, 2, 37, 8, True, 8),
         Workload("g-f16-large", "f16", 1, 1, 29, 16, True, 9, "large_logit")]


# grouped K/V heads and N_q != N_kv (forward), and gradients (square and grouped)
EXTENDED = [("fwd", Workload("g-gqa-bf16", "bf16", 1, 4, 11, 8, True, 10, Hkv=2, Nkv=19)),
            ("bwd", Workload("g-bwd-f32", "f32", 1, 2, 13, 8, True, 11)),
            ("bwd", Workload("g-bwd-gqa-bf16", "bf16", 1, 4, 9, 8, True, 12, Hkv=2, Nkv=14))]


def extended():
    out = []
    for kind, w in EXTENDED:
        q, k, v = make_inputs(w)
        spec = [w.dtype, w.B, w.H, w.N, w.d, w.causal, w.seed, w.dist, w.h_kv, w.n_kv]
        if kind == "fwd":
            o, lse = oracle.fwd_gqa(q, k, v, w.scale, w.causal)
            out.append({"name": w.name, "kind": kind, "workload": spec,
                        "o": [float(x) for x in o.ravel()], "lse": [float(x) for x in lse.ravel()]})
        else:
            dq, dk, dv = oracle.bwd(q, k, v, make_upstream(w, w.seed + 100), w.scale, w.causal)
            out.append({"name": w.name, "kind": kind, "workload": spec,
                        "dq": [float(x) for x in dq.ravel()], "dk": [float(x) for x in dk.ravel()],
                        "dv": [float(x) for x in dv.ravel()]})
    path = Path(__file__).with_name("oracle_extended.json")
    path.write_text(json.dumps(out))
    print(path)


def main():
    out = []
    for w in CASES:
        q, k, v = make_inputs(w)
        o, lse = oracle.fwd(q, k, v, w.scale, w.causal)
        out.append({"name": w.name, "workload": [w.dtype, w.B, w.H, w.N, w.d, w.causal, w.seed, w.dist],
                    "o": [float(x) for x in o.ravel()], "lse": [float(x) for x in lse.ravel()]})
    path = Path(__file__).with_name("oracle_small.json")
    path.write_text(json.dumps(out))
    print(path)


if __name__ == "__main__":
    main()
    extended()
