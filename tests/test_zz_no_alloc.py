"""fa_fwd_ex_noalloc: the split forward pass with its partials in the
library's static device scratch (MI355X only).

Each case calls fa_fwd_ex_noalloc through the C ABI and fa_fwd_ex (with a
workspace the test allocates) on the same inputs and split count: the same
kernels run, so O and LSE must agree bitwise, and both must match the fp64
oracle to the forward pass's tolerances.  Calls come in pairs, the second on
a smaller problem, so the second call reads its partials from a scratch that
still holds the first call's.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_attention_13_amd import binding
from exact_attention_13_amd.inputs import Workload, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CODE = {"f32": binding.FA_F32, "bf16": binding.FA_BF16, "f16": binding.FA_F16}


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_pair(w, splits):
    q, k, v = make_inputs(w)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    rows = w.B * w.H * w.N
    st = torch.cuda.current_stream().cuda_stream
    o1 = torch.full_like(qd, float("nan"))
    l1 = torch.full((rows,), float("nan"), dtype=torch.float32, device=DEV)
    o2 = torch.full_like(qd, float("nan"))
    l2 = torch.full((rows,), float("nan"), dtype=torch.float32, device=DEV)
    args = (w.B, w.H, w.h_kv, w.N, w.n_kv, w.d, w.scale, w.causal, CODE[w.dtype], splits)
    wsb = binding.load().fa_fwd_ex_workspace_bytes(w.B, w.H, w.N, w.n_kv, w.d, splits)
    assert 0 < wsb <= binding.NOALLOC_SCRATCH_BYTES
    ws = torch.empty((wsb,), dtype=torch.uint8, device=DEV)
    s1 = binding.fa_fwd_ex_noalloc(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o1.data_ptr(),
                                   l1.data_ptr(), *args, st)
    s2 = binding.fa_fwd_ex(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o2.data_ptr(),
                           l2.data_ptr(), *args, ws.data_ptr(), wsb, st)
    torch.cuda.synchronize()
    assert s1 == 0 and s2 == 0, (s1, s2)
    assert torch.equal(o1, o2), "O differs from fa_fwd_ex"
    assert torch.equal(l1, l2), "LSE differs from fa_fwd_ex"
    o_ref, lse_ref = oracle.fwd_gqa(q, k, v, w.scale, w.causal)
    o = o1.cpu().double().numpy()
    lse = l1.cpu().double().numpy().reshape(lse_ref.shape)
    err = float(np.abs(o - o_ref).max())
    lerr = float(np.abs(lse - lse_ref).max())
    if w.dtype == "f32":
        assert err <= 1e-4 and lerr <= 1e-4, (err, lerr)
    else:
        rel = float(np.linalg.norm(o - o_ref) / np.linalg.norm(o_ref))
        assert err <= 2e-2 and rel <= 5e-3 and lerr <= 2e-2, (err, rel, lerr)


# (first, second): the second call is smaller than the first.
PAIRS = [
    # decoding: one query row per head, grouped K/V heads, 8 key ranges
    (Workload("dec", "bf16", 8, 32, 1, 128, False, 51, Hkv=8, Nkv=16384),
     Workload("dec2", "bf16", 2, 8, 1, 128, False, 52, Hkv=2, Nkv=3000)),
    # a short prefill split over keys, causal, fp16 then fp32
    (Workload("pre", "f16", 1, 4, 300, 64, True, 53, Hkv=2, Nkv=2000),
     Workload("pre2", "f32", 1, 2, 100, 64, True, 54, Hkv=1, Nkv=700)),
]


@pytest.mark.parametrize("pair", range(len(PAIRS)))
def test_noalloc_matches_workspace_call_twice(pair):
    first, second = PAIRS[pair]
    for w in (first, second):
        _note(f"noalloc {w}")
        run_pair(w, 8)


def test_noalloc_rejects_partials_beyond_scratch():
    # 64 ranges of 8192 rows of d = 128 need 270 MB of partials: refused
    # before any launch, outputs untouched
    w = Workload("big", "bf16", 1, 8, 1024, 128, False, 55, Nkv=65536)
    q = torch.zeros((1, 8, 1024, 128), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((1, 8, 65536, 128), dtype=torch.bfloat16, device=DEV)
    o = torch.full_like(q, 7.0)
    s = binding.fa_fwd_ex_noalloc(q.data_ptr(), kv.data_ptr(), kv.data_ptr(), o.data_ptr(), None,
                                  1, 8, 8, 1024, 65536, 128, w.scale, False, binding.FA_BF16, 64,
                                  torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert s == 10
    assert bool((o == 7.0).all())
