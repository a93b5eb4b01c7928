"""Parity of the HIP forward pass with the fp64 oracle (MI355X only).

Every case runs the library through its C ABI (``binding.fwd`` -> ``fa_fwd``)
on seeded synthetic inputs and compares O and LSE element by element with the
three-pass fp64 oracle on the same bits.

Tolerances of the forward output (the stated accuracy targets; LSE's own bound
follows that of O):
  * fp32 inputs: max |O - O_ref| <= 1e-4 and max |LSE - LSE_ref| <= 1e-4;
  * bf16/fp16 inputs: max |O - O_ref| <= 2e-2 and
    ||O - O_ref||_2 / ||O_ref||_2 <= 5e-3, max |LSE - LSE_ref| <= 2e-2.
Every workload is compared with the oracle at its full size, row by row
(the longest single-head case, 131072 keys, on a row sample).
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_attention_13_amd import binding
from exact_attention_13_amd.inputs import WORKLOADS, Workload, make_inputs, sample_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(q, k, v, scale, causal, stream=None):
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    o, lse = binding.fwd(qd, kd, vd, scale, causal, stream=stream)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def assert_close(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what=""):
    o = o_gpu.to(torch.float64).numpy().reshape(o_ref.shape)
    l = lse_gpu.to(torch.float64).numpy().reshape(lse_ref.shape)
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    err = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    lerr = float(np.max(np.abs(l - lse_ref))) if l.size else 0.0
    if dtype == "f32":
        assert err <= 1e-4, f"{what}: max|dO| = {err:.3e}"
        assert lerr <= 1e-4, f"{what}: max|dLSE| = {lerr:.3e}"
    else:
        rel = float(np.linalg.norm(o - o_ref) / max(np.linalg.norm(o_ref), 1e-300))
        assert err <= 2e-2, f"{what}: max|dO| = {err:.3e}"
        assert rel <= 5e-3, f"{what}: rel-L2 = {rel:.3e}"
        assert lerr <= 2e-2, f"{what}: max|dLSE| = {lerr:.3e}"
    return err, lerr


def small_case(dtype, B, H, N, d, causal, seed, dist="normal"):
    w = Workload("case", dtype, B, H, N, d, causal, seed, dist)
    return w, make_inputs(w)


# --------------------------------------------------------------------------
# Small shapes: full oracle, several tiles plus ragged tails
# --------------------------------------------------------------------------

SMALL_N = [1, 2, 31, 63, 64, 65, 127, 128, 129, 200, 383, 513]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_small_shapes(dtype, d, causal):
    for i, n in enumerate(SMALL_N):
        B, H = (1, 2) if i % 2 else (2, 3)
        w, (q, k, v) = small_case(dtype, B, H, n, d, causal, seed=1000 + i)
        _note(f"small {dtype} d={d} causal={causal} B={B} H={H} N={n}")
        o, lse = run_gpu(q, k, v, w.scale, causal)
        o_ref, lse_ref = oracle.fwd(q, k, v, w.scale, causal)
        assert_close(o, lse, o_ref, lse_ref, dtype, f"N={n}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_f32_grid_sizes(d, causal):
    # fp32 problems of at most 128 workgroups of 128 rows (255 causal) take
    # the small-problem kernel (16 rows per workgroup, eight waves splitting
    # the keys in 16-key tiles); larger ones the 128-row kernel.  Both sides
    # of both switches, ragged tails, key counts that leave waves without
    # tiles.
    for B, H, N, seed in ((1, 1, 700, 1600), (2, 16, 1000, 1601), (1, 31, 513, 1602),
                          (1, 3, 100, 1603), (1, 2, 17, 1604), (1, 128, 100, 1605),
                          (1, 129, 100, 1606), (5, 51, 70, 1607), (1, 256, 90, 1608),
                          (1, 2, 2100, 1609), (1, 16, 2048, 1610)):
        w, (q, k, v) = small_case("f32", B, H, N, d, causal, seed=seed)
        _note(f"f32 grid d={d} causal={causal} B={B} H={H} N={N}")
        o, lse = run_gpu(q, k, v, w.scale, causal)
        o_ref, lse_ref = oracle.fwd(q, k, v, w.scale, causal)
        assert_close(o, lse, o_ref, lse_ref, "f32", f"B={B} H={H} N={N}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_h16_d64_short_grid_switch(dtype, causal):
    # d = 64 grids of at most 64 eight-wave workgroups of 512 rows take
    # one-wave 32-row workgroups.  Both sides of the switch (64 and 65
    # problems of one block), a multi-block head on the short side, ragged
    # tails, and rows past the last key block of a causal wave.
    for B, H, N, seed in ((1, 64, 100, 1650), (1, 65, 100, 1651), (3, 21, 97, 1652),
                          (2, 4, 1500, 1653), (1, 1, 33, 1654)):
        w, (q, k, v) = small_case(dtype, B, H, N, 64, causal, seed=seed)
        _note(f"h16 short grid {dtype} causal={causal} B={B} H={H} N={N}")
        o, lse = run_gpu(q, k, v, w.scale, causal)
        o_ref, lse_ref = oracle.fwd(q, k, v, w.scale, causal)
        assert_close(o, lse, o_ref, lse_ref, dtype, f"B={B} H={H} N={N}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_large_logits_small(dtype, causal):
    # scores with std ~ 9: the running max moves often, rescaling is exercised
    w, (q, k, v) = small_case(dtype, 2, 2, 777, 128, causal, seed=77, dist="large_logit")
    _note(f"large-logit {dtype} causal={causal}")
    o, lse = run_gpu(q, k, v, w.scale, causal)
    o_ref, lse_ref = oracle.fwd(q, k, v, w.scale, causal)
    assert_close(o, lse, o_ref, lse_ref, dtype)


# --------------------------------------------------------------------------
# The workloads at full size
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["C1", "C2", "C2r"])
def test_workload_full_oracle(name):
    w = WORKLOADS[name]
    q, k, v = make_inputs(w)
    _note(f"workload {name} full")
    o, lse = run_gpu(q, k, v, w.scale, w.causal)
    o_ref, lse_ref = oracle.fwd(q, k, v, w.scale, w.causal)
    assert_close(o, lse, o_ref, lse_ref, w.dtype, name)


@pytest.mark.parametrize("name", ["C3", "C4", "C5"])
def test_workload_every_row(name):
    # Full size, every row against the oracle (about 10 s for C3 and 20 s
    # each for C4 and C5 of fp64 work on 16 host threads).  O and LSE start
    # as NaN, so a query tile the grid skipped or a row no wave stored fails
    # even if its neighbours are right; C3 (128 causal units of 32 query
    # tiles, 16 units per die) runs the grouped heavy-first tile order at its
    # full size.
    w = WORKLOADS[name]
    q, k, v = make_inputs(w)
    _note(f"workload {name} every row")
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    o = torch.full_like(qd, float("nan"))
    lse = torch.full((w.B, w.H, w.N), float("nan"), dtype=torch.float32, device=DEV)
    binding.fwd(qd, kd, vd, w.scale, w.causal, out=o, lse=lse)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    del qd, kd, vd
    # the oracle a few heads at a time (heads are independent problems)
    o_ref = np.empty((w.B, w.H, w.N, w.d))
    lse_ref = np.empty((w.B, w.H, w.N))
    step = 4
    for b in range(w.B):
        for h0 in range(0, w.H, step):
            sl = (slice(b, b + 1), slice(h0, h0 + step))
            o_ref[sl], lse_ref[sl] = oracle.fwd(q[sl], k[sl], v[sl], w.scale, w.causal)
            _note(f"  oracle {name} b={b} heads {h0}..{min(w.H, h0 + step) - 1}")
    assert_close(o, lse, o_ref, lse_ref, w.dtype, name)
    # and per (batch, head, 128-row query block): a block whose rows were
    # computed against the wrong head or range stands out even when the
    # tensor-wide rel-L2 is small
    blk = 128
    nb = -(-w.N // blk)
    og = o.to(torch.float64).numpy()
    for b in range(w.B):
        for h in range(w.H):
            for t in range(nb):
                sl = slice(t * blk, min(w.N, (t + 1) * blk))
                ref = o_ref[b, h, sl]
                err = np.linalg.norm(og[b, h, sl] - ref) / max(np.linalg.norm(ref), 1e-300)
                bound = 1e-4 * 10 if w.dtype == "f32" else 2e-2
                assert err <= bound, f"{name}: block (b={b}, h={h}, rows {sl}) rel-L2 {err:.3e}"


# --------------------------------------------------------------------------
# Edge cases of the boundary
# --------------------------------------------------------------------------

def test_null_lse_gives_same_output():
    w, (q, k, v) = small_case("bf16", 1, 2, 300, 64, True, seed=5)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    o1 = torch.empty_like(qd)
    o2 = torch.empty_like(qd)
    lse = torch.empty((1, 2, 300), dtype=torch.float32, device=DEV)
    st = torch.cuda.current_stream().cuda_stream
    B, H, N, d = q.shape
    assert binding.fa_fwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o1.data_ptr(),
                          lse.data_ptr(), B, H, N, d, w.scale, 1, binding.FA_BF16, st) == 0
    assert binding.fa_fwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o2.data_ptr(),
                          None, B, H, N, d, w.scale, 1, binding.FA_BF16, st) == 0
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_canaries_untouched_and_not_read(dtype):
    # Every buffer sits at the front of a larger allocation whose tail is NaN.
    # Outputs must leave the tail alone; inputs must not read it (a read would
    # put NaN into O).
    B, H, N, d = 2, 3, 333, 128
    w, (q, k, v) = small_case(dtype, B, H, N, d, True, seed=9)
    tdt = TORCH[dtype]
    pad = 4096
    n = q.numel()

    def poisoned(src):
        buf = torch.full((n + pad,), float("nan"), dtype=tdt, device=DEV)
        buf[:n] = src.reshape(-1).to(DEV)
        return buf, buf[:n].view(B, H, N, d)

    (qb, qd), (kb, kd), (vb, vd) = poisoned(q), poisoned(k), poisoned(v)
    ob = torch.full((n + pad,), float("nan"), dtype=tdt, device=DEV)
    lb = torch.full((B * H * N + pad,), float("nan"), dtype=torch.float32, device=DEV)
    o, lse = ob[:n].view(B, H, N, d), lb[:B * H * N].view(B, H, N)
    binding.fwd(qd, kd, vd, w.scale, True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isnan(ob[n:]).all() and torch.isnan(lb[B * H * N:]).all()
    o_ref, lse_ref = oracle.fwd(q, k, v, w.scale, True)
    assert_close(o.cpu(), lse.cpu(), o_ref, lse_ref, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_tail_reads_zeros_over_stale_lds(dtype, d, causal):
    # Keys past the end must reach the P.V product as zero rows (their
    # weights are 0, and 0 * NaN would be NaN).  A first launch of the same
    # kernel on all-NaN K/V (every CU busy) leaves NaN in the LDS stages;
    # the second problem's last key tile is ragged and lands in a stage
    # that its workgroup has not written before (65 keys: 32-key tiles 0, 1
    # full, tile 2 one key; 100 keys: 64-key steps), so its rows past the
    # end must be written as zeros by the loads themselves, not left over.
    tdt = TORCH[dtype]
    Bp, Hp, Np = 4, 64, 1024
    nan = torch.full((Bp, Hp, Np, d), float("nan"), dtype=tdt, device=DEV)
    qp = torch.randn(Bp, Hp, Np, d, device=DEV).to(tdt)
    op = torch.empty_like(qp)
    for n in (65, 100):
        _note(f"stale-LDS ragged {dtype} d={d} causal={causal} N={n}")
        binding.fwd(qp, nan, nan, 0.1, causal, out=op)
        w, (q, k, v) = small_case(dtype, 8, 64, n, d, causal, seed=2100 + n)
        o, lse = run_gpu(q, k, v, w.scale, causal)
        o_ref, lse_ref = oracle.fwd(q, k, v, w.scale, causal)
        assert_close(o, lse, o_ref, lse_ref, dtype, f"N={n}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_deterministic_bitwise(dtype):
    w, (q, k, v) = small_case(dtype, 1, 4, 1000, 64, False, seed=11)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    o1, l1 = binding.fwd(qd, kd, vd, w.scale, False)
    o2, l2 = binding.fwd(qd, kd, vd, w.scale, False)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_side_stream():
    w, (q, k, v) = small_case("f16", 1, 2, 260, 128, False, seed=13)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        qd, kd, vd = (t.to(DEV) for t in (q, k, v))
        o, lse = binding.fwd(qd, kd, vd, w.scale, False, stream=s)
    s.synchronize()
    o_ref, lse_ref = oracle.fwd(q, k, v, w.scale, False)
    assert_close(o.cpu(), lse.cpu(), o_ref, lse_ref, "f16")


def test_nondefault_scale_and_self_attention():
    # q = k = v (one buffer), scale not 1/sqrt(d)
    w, (q, _, _) = small_case("bf16", 1, 1, 190, 64, True, seed=15)
    qd = q.to(DEV)
    o, lse = binding.fwd(qd, qd, qd, 0.37, True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.fwd(q, q, q, 0.37, True)
    assert_close(o.cpu(), lse.cpu(), o_ref, lse_ref, "bf16")


def test_long_sequence_single_head():
    # one head, 131072 keys: the longest row in the suite (causal, d = 128)
    w = Workload("long", "bf16", 1, 1, 131072, 128, True, 17)
    q, k, v = make_inputs(w)
    _note("long single head N=131072")
    o, lse = run_gpu(q, k, v, w.scale, True)
    rows = sample_rows(w, 48)
    o_ref, lse_ref = oracle.fwd(q, k, v, w.scale, True, rows=rows)
    idx = torch.from_numpy(rows)
    assert_close(o.reshape(-1, 128)[idx], lse.reshape(-1)[idx], o_ref, lse_ref, "bf16")


def test_library_is_the_hip_build():
    binding.load()
    with open("/proc/self/maps") as f:
        maps = f.read()
    assert str(binding.library_path()) in maps


# Causal launches whose grid splits evenly over the eight dies take the
# grouped heavy-first tile order (groups of up to 4 units inside each die's
# range, a shorter last group, or fewer units than a group); every tile must
# still be computed exactly once.  Cases: (dtype, B, H, N, d) chosen so that
# each die holds 1, 3, 6 or 5 units (d = 64 tiles hold 512 rows, d = 128 and
# fp32 tiles 128), with ragged last tiles in some.
ORDER_CASES = [("bf16", 2, 4, 1024, 64), ("bf16", 2, 12, 1024, 64), ("f16", 4, 12, 600, 64),
               ("bf16", 2, 20, 500, 128), ("f16", 1, 16, 256, 128), ("f32", 2, 20, 384, 64)]


@pytest.mark.parametrize("dtype,B,H,N,d", ORDER_CASES)
def test_causal_tile_order_groups(dtype, B, H, N, d):
    w, (q, k, v) = small_case(dtype, B, H, N, d, True, seed=41 + H + N)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    print(f"causal order {dtype} B={B} H={H} N={N} d={d}", flush=True)
    o, lse = binding.fwd(qd, kd, vd, w.scale, True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.fwd(q, k, v, w.scale, True)
    assert_close(o.cpu(), lse.cpu(), o_ref, lse_ref, dtype, f"{(dtype, B, H, N, d)}")


# Tensors past 4 GiB: head base offsets beyond 2^31 and 2^32 bytes.  The
# inputs repeat a seeded block of 97 heads along H on the device (97 does not
# divide the 2^31 / 2^32-byte head counts, so an offset that wrapped at 32
# bits would land on a head with other data).  The first block is checked
# against the full oracle; every later head must equal its image in the first
# block bitwise (a head's result depends only on its own data).
PERIOD = 97


def periodic(base, H):
    reps = -(-H // base.shape[1])
    return base.to(DEV).repeat(1, reps, 1, 1)[:, :H].contiguous()


@pytest.mark.parametrize("dtype,H,d", [("bf16", 65600, 64), ("f32", 33000, 64)])
def test_tensors_past_4gib(dtype, H, d):
    N = 512
    w, (q, k, v) = small_case(dtype, 1, PERIOD, N, d, False, seed=61)
    e = 4 if dtype == "f32" else 2
    assert H * N * d * e > 2 ** 32
    _note(f"past 4 GiB {dtype} H={H} N={N} d={d}")
    qd, kd, vd = periodic(q, H), periodic(k, H), periodic(v, H)
    o, lse = binding.fwd(qd, kd, vd, w.scale, False)
    torch.cuda.synchronize()
    del qd, kd, vd
    o_ref, lse_ref = oracle.fwd(q, k, v, w.scale, False)
    assert_close(o[:, :PERIOD].cpu(), lse[:, :PERIOD].cpu(), o_ref, lse_ref, dtype, "first block")
    assert torch.equal(o, periodic(o[:, :PERIOD], H)), "a head past the first block differs"
    assert torch.equal(lse, periodic(lse[:, :PERIOD].unsqueeze(-1), H).squeeze(-1))
