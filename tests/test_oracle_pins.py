"""Pins of the fp64 oracle to facts fixed outside the oracle itself.

Each test ties the three-pass oracle (``oracle/fa_oracle.c``) to something it
does not compute itself: a closed form, an invariant of softmax attention, an
independent library routine, exhaustive conversion tables, or the tile-by-tile
online recurrence that the pages describe.  They are chosen so that a plausible
slip anywhere in the oracle (a dropped term, a wrong sign or index, a
transposed operand, an off-by-one causal bound, a wrong head offset, a wrong
16-bit decode) fails at least one of them.  CPU only.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import online_ref

RNG = np.random.default_rng(2024)


def _rand(shape, dtype=torch.float32, scale=1.0, seed=0):
    g = np.random.default_rng(seed)
    x = (scale * g.standard_normal(shape)).astype(np.float32)
    return torch.from_numpy(x).to(dtype)


def _f64(t):
    return t.to(torch.float64).numpy()


# --------------------------------------------------------------------------
# Exact widening of stored elements (the oracle's own bf16/fp16 decoders)
# --------------------------------------------------------------------------

def test_widen_f16_exhaustive_against_numpy(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32)
    ref = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    got = np.array([oracle.widen("f16", int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_widen_bf16_exhaustive_against_torch(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32)
    ref = torch.from_numpy(bits.astype(np.uint16).view(np.int16)).view(torch.bfloat16)
    ref = ref.to(torch.float64).numpy()
    got = np.array([oracle.widen("bf16", int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# --------------------------------------------------------------------------
# Closed forms
# --------------------------------------------------------------------------

def test_two_key_closed_form(oracle_lib):
    # d = 1, N = 2, scale = 1: query 0 sees scores (0, 1) -> weights
    # 1/(1+e) and e/(1+e); LSE = ln(1 + e).  Causal row 0 sees key 0 only.
    q = torch.tensor([[[[1.0], [1.0]]]])
    k = torch.tensor([[[[0.0], [1.0]]]])
    v = torch.tensor([[[[3.0], [-5.0]]]])
    o, lse = oracle.fwd(q, k, v, 1.0, False)
    e = math.e
    assert o[0, 0, 0, 0] == pytest.approx((3.0 - 5.0 * e) / (1.0 + e), rel=1e-15)
    assert lse[0, 0, 0] == pytest.approx(math.log1p(e), rel=1e-15)
    o, lse = oracle.fwd(q, k, v, 1.0, True)
    assert o[0, 0, 0, 0] == 3.0 and lse[0, 0, 0] == 0.0
    assert o[0, 0, 1, 0] == pytest.approx((3.0 - 5.0 * e) / (1.0 + e), rel=1e-15)


def test_score_range_beyond_exp_range_stays_finite(oracle_lib):
    # Scores -800, 0, 800 (scale 1, d = 1): exp(1600) overflows a double, so
    # only a softmax that subtracts the row maximum (the "safe" form whose
    # three passes the pages describe) returns the one-hot answer here:
    # O = V[2], LSE = 800.  Causal row 1 sees scores -800, 0 -> O = V[1].
    q = torch.ones((1, 1, 3, 1))
    k = torch.tensor([[[[-800.0], [0.0], [800.0]]]])
    v = torch.tensor([[[[1.0], [2.0], [4.0]]]])
    o, lse = oracle.fwd(q, k, v, 1.0, False)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    np.testing.assert_array_equal(o[0, 0, :, 0], [4.0, 4.0, 4.0])
    np.testing.assert_array_equal(lse[0, 0], [800.0, 800.0, 800.0])
    o, lse = oracle.fwd(q, k, v, 1.0, True)
    np.testing.assert_array_equal(o[0, 0, :, 0], [1.0, 2.0, 4.0])
    np.testing.assert_array_equal(lse[0, 0], [-800.0, 0.0, 800.0])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one(oracle_lib, dtype, causal):
    # V = 1 everywhere: every output is the sum of the softmax weights.
    B, H, N, d = 2, 3, 37, 16
    q = _rand((B, H, N, d), dtype, seed=1)
    k = _rand((B, H, N, d), dtype, seed=2)
    v = torch.ones((B, H, N, d), dtype=dtype)
    o, lse = oracle.fwd(q, k, v, 1.0 / math.sqrt(d), causal)
    assert np.max(np.abs(o - 1.0)) <= 1e-14
    # and LSE normalises the same scores: sum_j exp(s_ij - lse_i) = 1
    s = (1.0 / math.sqrt(d)) * np.einsum("bhid,bhjd->bhij", _f64(q), _f64(k))
    if causal:
        s = np.where(np.triu(np.ones((N, N), bool), 1), -np.inf, s)
    tot = np.exp(s - lse[..., None]).sum(-1)
    assert np.max(np.abs(tot - 1.0)) <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_column_mean(oracle_lib, causal):
    # Q = 0 makes every score 0: O_i is the plain mean of the visible V rows
    # and LSE_i = ln(#visible).
    B, H, N, d = 1, 2, 50, 8
    q = torch.zeros((B, H, N, d))
    k = _rand((B, H, N, d), seed=3)
    v = _rand((B, H, N, d), seed=4)
    o, lse = oracle.fwd(q, k, v, 0.35, causal)
    vv = _f64(v)
    if causal:
        ref = np.cumsum(vv, axis=2) / np.arange(1, N + 1)[None, None, :, None]
        ref_lse = np.log(np.arange(1, N + 1, dtype=np.float64))[None, None, :]
    else:
        ref = np.broadcast_to(vv.mean(axis=2, keepdims=True), vv.shape)
        ref_lse = np.full((B, H, N), math.log(N))
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, np.broadcast_to(ref_lse, lse.shape), rtol=0, atol=1e-14)


@pytest.mark.parametrize("jstar", [0, 5, 31])
@pytest.mark.parametrize("causal", [False, True])
def test_single_dominant_logit_returns_that_value_row(oracle_lib, jstar, causal):
    # Key j* = t*u with q_i = u: its score beats every other by > 60, so the
    # softmax is one-hot to far below 1e-20 and O_i = V_j*, LSE_i = s_ij*.
    N, d = 32, 8
    scale = float(np.float32(1.0 / math.sqrt(d)))
    k = _rand((1, 1, N, d), scale=0.5, seed=5)
    u = torch.zeros(d)
    u[2] = 1.0
    t = 256.0
    k[0, 0, jstar] = t * u
    q = u.expand(1, 1, N, d).contiguous()
    v = _rand((1, 1, N, d), seed=6)
    o, lse = oracle.fwd(q, k, v, scale, causal)
    rows = range(jstar, N) if causal else range(N)
    others = [j for j in range(N) if j != jstar]
    gap = scale * t - scale * float(k[0, 0, others, 2].abs().max())
    assert gap > 60
    for i in rows:
        np.testing.assert_allclose(o[0, 0, i], _f64(v[0, 0, jstar]), rtol=0, atol=1e-20)
        assert lse[0, 0, i] == pytest.approx(scale * t, rel=1e-15)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_causal_row_zero_is_first_value_row(oracle_lib, dtype):
    B, H, N, d = 2, 2, 19, 8
    q, k, v = (_rand((B, H, N, d), dtype, seed=s) for s in (7, 8, 9))
    scale = 0.25
    o, lse = oracle.fwd(q, k, v, scale, True)
    np.testing.assert_array_equal(o[:, :, 0], _f64(v[:, :, 0]))
    dot0 = (_f64(q[:, :, 0]) * _f64(k[:, :, 0])).sum(-1)
    np.testing.assert_allclose(lse[:, :, 0], scale * dot0, rtol=1e-15, atol=1e-15)
    # a single key (N = 1) returns V[0] whatever the query, causal or not
    o1, _ = oracle.fwd(q[:, :, :1].contiguous(), k[:, :, :1].contiguous(),
                       v[:, :, :1].contiguous(), scale, False)
    np.testing.assert_array_equal(o1[:, :, 0], _f64(v[:, :, 0]))


# --------------------------------------------------------------------------
# The method: tile-by-tile online softmax equals three-pass, by brute force
# --------------------------------------------------------------------------

@pytest.mark.parametrize("d", [1, 4, 8])
@pytest.mark.parametrize("causal", [False, True])
def test_online_recurrence_equals_three_pass(oracle_lib, d, causal):
    worst = 0.0
    for seed in range(5):
        for n in range(1, 17):
            q, k, v = (_rand((1, 1, n, d), scale=2.0, seed=100 * seed + 10 * n + j)
                       for j in range(3))
            scale = 1.0 / math.sqrt(d)
            o_ref, lse_ref = oracle.fwd(q, k, v, scale, causal)
            qq, kk, vv = (_f64(t[0, 0]) for t in (q, k, v))
            sc = float(np.float32(scale))
            for bc in range(1, n + 1):
                for br in sorted({1, n}):
                    for form in (online_ref.deferred, online_ref.normalised):
                        o, lse = form(qq, kk, vv, sc, causal, br=br, bc=bc)
                        err = np.max(np.abs(o - o_ref[0, 0])) / max(1.0, np.max(np.abs(o_ref)))
                        err_l = np.max(np.abs(lse - lse_ref[0, 0]) / np.maximum(1.0, np.abs(lse_ref[0, 0])))
                        worst = max(worst, err, err_l)
    assert worst <= 1e-13, worst


# --------------------------------------------------------------------------
# Independent library routines on small shapes
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 8), (7, 8), (33, 64), (64, 16)])
def test_matches_torch_sdpa_fp64(oracle_lib, dtype, causal, N, d):
    B, H = 2, 3
    q, k, v = (_rand((B, H, N, d), dtype, scale=1.5, seed=s) for s in (11, 12, 13))
    scale = 1.0 / math.sqrt(d)
    sc = float(np.float32(scale))
    o, lse = oracle.fwd(q, k, v, scale, causal)
    q64, k64, v64 = (t.to(torch.float64) for t in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(
        q64, k64, v64, is_causal=causal, scale=sc).numpy()
    logits = sc * torch.matmul(q64, k64.transpose(-1, -2).contiguous())
    if causal:
        logits = logits.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    ref_lse = torch.logsumexp(logits, dim=-1).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_matches_scipy_softmax(oracle_lib):
    from scipy.special import softmax
    N, d = 40, 24
    q, k, v = (_rand((1, 1, N, d), seed=s) for s in (21, 22, 23))
    scale = 0.3
    o, _ = oracle.fwd(q, k, v, scale, False)
    s = float(np.float32(scale)) * (_f64(q[0, 0]) @ _f64(k[0, 0]).T)
    ref = softmax(s, axis=1) @ _f64(v[0, 0])
    np.testing.assert_allclose(o[0, 0], ref, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------
# Invariants
# --------------------------------------------------------------------------

def _int_valued(shape, seed, lo=-4, hi=5):
    g = np.random.default_rng(seed)
    return torch.from_numpy((g.integers(lo, hi, size=shape) / 4.0).astype(np.float32))


def test_joint_key_value_permutation_leaves_output(oracle_lib):
    B, H, N, d = 1, 2, 29, 8
    q, k, v = (_rand((B, H, N, d), seed=s) for s in (31, 32, 33))
    perm = torch.from_numpy(np.random.default_rng(34).permutation(N))
    o1, l1 = oracle.fwd(q, k, v, 0.4, False)
    o2, l2 = oracle.fwd(q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous(), 0.4, False)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-14, atol=1e-14)


def test_query_permutation_permutes_rows(oracle_lib):
    B, H, N, d = 2, 1, 23, 8
    q, k, v = (_rand((B, H, N, d), seed=s) for s in (41, 42, 43))
    perm = np.random.default_rng(44).permutation(N)
    o1, l1 = oracle.fwd(q, k, v, 0.4, False)
    o2, l2 = oracle.fwd(q[:, :, torch.from_numpy(perm)].contiguous(), k, v, 0.4, False)
    np.testing.assert_array_equal(o1[:, :, perm], o2)
    np.testing.assert_array_equal(l1[:, :, perm], l2)


@pytest.mark.parametrize("causal", [False, True])
def test_common_key_shift_moves_only_lse(oracle_lib, causal):
    # K' = K + w (exact: small multiples of 1/4) shifts row i's scores by
    # scale*q_i.w, so O is unchanged and LSE_i grows by exactly that.
    B, H, N, d = 1, 2, 31, 8
    q, k, v = _int_valued((B, H, N, d), 51), _int_valued((B, H, N, d), 52), _rand((B, H, N, d), seed=53)
    w = _int_valued((d,), 54)
    scale = 0.5
    o1, l1 = oracle.fwd(q, k, v, scale, causal)
    o2, l2 = oracle.fwd(q, (k + w).contiguous(), v, scale, causal)
    shift = scale * (_f64(q) @ _f64(w))
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l2, l1 + shift, rtol=1e-13, atol=1e-12)


def test_row_subset_equals_full_rows(oracle_lib):
    B, H, N, d = 2, 3, 45, 16
    q, k, v = (_rand((B, H, N, d), seed=s) for s in (61, 62, 63))
    o, l = oracle.fwd(q, k, v, 0.25, True)
    rows = np.array([0, 44, 45, 100, B * H * N - 1])
    os_, ls_ = oracle.fwd(q, k, v, 0.25, True, rows=rows)
    np.testing.assert_array_equal(os_, o.reshape(-1, d)[rows])
    np.testing.assert_array_equal(ls_, l.reshape(-1)[rows])


# --------------------------------------------------------------------------
# Grouped K/V heads, separate query/key lengths, merging key ranges
# --------------------------------------------------------------------------

@pytest.mark.parametrize("H,H_kv", [(4, 2), (6, 3), (4, 1), (3, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_grouped_heads_equal_repeated_kv_heads(oracle_lib, H, H_kv, causal):
    # Query head h reads K/V head h // (H / H_kv): the same as multi-head
    # attention on K/V whose heads are repeated H / H_kv times in place
    # (torch fp64 reference on the repeated tensors).
    B, N, d = 2, 13, 8
    q = _rand((B, H, N, d), seed=71)
    k, v = (_rand((B, H_kv, N, d), seed=s) for s in (72, 73))
    o, lse = oracle.fwd_gqa(q, k, v, 0.3, causal)
    g = H // H_kv
    kr, vr = (t.repeat_interleave(g, dim=1).contiguous() for t in (k, v))
    sc = float(np.float32(0.3))
    q64, k64, v64 = (t.to(torch.float64) for t in (q, kr, vr))
    logits = sc * torch.matmul(q64, k64.transpose(-1, -2).contiguous())
    if causal:
        logits = logits.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    ref = torch.matmul(torch.softmax(logits, -1), v64).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, torch.logsumexp(logits, -1).numpy(), rtol=1e-13, atol=1e-13)
    o2, l2 = oracle.fwd(q, kr, vr, 0.3, causal)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-15)


@pytest.mark.parametrize("n_q", [1, 2, 5, 17])
def test_causal_rows_stand_at_the_end_of_the_keys(oracle_lib, n_q):
    # With N_q < N_kv, causal query row i stands at key position
    # N_kv - N_q + i: the N_q rows equal the last N_q rows of square causal
    # attention over the same keys.  N_q = 1 (a decoding step) sees every key.
    B, H, N, d = 1, 2, 17, 8
    q, k, v = (_rand((B, H, N, d), seed=s) for s in (81, 82, 83))
    o_full, l_full = oracle.fwd(q, k, v, 0.4, True)
    qs = q[:, :, N - n_q:].contiguous()
    o, lse = oracle.fwd_gqa(qs, k, v, 0.4, True)
    np.testing.assert_array_equal(o, o_full[:, :, N - n_q:])
    np.testing.assert_array_equal(lse, l_full[:, :, N - n_q:])
    if n_q == 1:
        o_nc, l_nc = oracle.fwd_gqa(qs, k, v, 0.4, False)
        np.testing.assert_array_equal(o, o_nc)
        np.testing.assert_array_equal(lse, l_nc)


def test_more_queries_than_keys_leaves_early_rows_empty(oracle_lib):
    # N_q > N_kv, causal: rows i < N_q - N_kv see no key (O = 0, LSE = -inf);
    # the last N_kv rows are square causal attention over the keys.
    B, H, Nq, Nk, d = 1, 2, 11, 6, 8
    q = _rand((B, H, Nq, d), seed=91)
    k, v = (_rand((B, H, Nk, d), seed=s) for s in (92, 93))
    o, lse = oracle.fwd_gqa(q, k, v, 0.5, True)
    e = Nq - Nk
    assert np.all(o[:, :, :e] == 0.0) and np.all(np.isneginf(lse[:, :, :e]))
    o_sq, l_sq = oracle.fwd(q[:, :, e:].contiguous(), k, v, 0.5, True)
    np.testing.assert_array_equal(o[:, :, e:], o_sq)
    np.testing.assert_array_equal(lse[:, :, e:], l_sq)


@pytest.mark.parametrize("Nq,Nk", [(1, 40), (7, 33), (30, 9)])
def test_rectangular_non_causal_matches_library_softmax(oracle_lib, Nq, Nk):
    from scipy.special import logsumexp, softmax
    d = 16
    q = _rand((1, 1, Nq, d), seed=101)
    k, v = (_rand((1, 1, Nk, d), seed=s) for s in (102, 103))
    o, lse = oracle.fwd_gqa(q, k, v, 0.25, False)
    s = float(np.float32(0.25)) * (_f64(q[0, 0]) @ _f64(k[0, 0]).T)
    np.testing.assert_allclose(o[0, 0], softmax(s, axis=1) @ _f64(v[0, 0]), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], logsumexp(s, axis=1), rtol=1e-13, atol=1e-13)


def test_zero_keys_gives_empty_rows(oracle_lib):
    q = _rand((1, 2, 3, 8), seed=104)
    k = torch.zeros((1, 1, 0, 8))
    o, lse = oracle.fwd_gqa(q, k, k, 0.5, False)
    assert np.all(o == 0.0) and np.all(np.isneginf(lse))


def _range_partials(q, k, v, scale, cuts):
    """Oracle results of each key range [cuts[i], cuts[i+1]) (non-causal)."""
    os_, ls_ = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        o, l = oracle.fwd_gqa(q, k[:, :, a:b].contiguous(), v[:, :, a:b].contiguous(), scale, False)
        os_.append(o.reshape(-1, q.shape[-1]))
        ls_.append(l.reshape(-1))
    return np.stack(os_), np.stack(ls_)


@pytest.mark.parametrize("cuts", [[0, 40], [0, 1, 40], [0, 13, 14, 27, 40], [0, 0, 20, 20, 40],
                                  list(range(41))])
def test_combine_of_key_ranges_equals_full_attention(oracle_lib, cuts):
    # Splitting the keys into ranges, attending to each, and merging by
    # logsumexp gives attention over all keys (empty ranges included: they
    # carry LSE = -inf and must drop out).
    B, H, N, d = 2, 2, 40, 8
    q, k, v = (_rand((B, H, N, d), scale=1.5, seed=s) for s in (111, 112, 113))
    o_full, l_full = oracle.fwd(q, k, v, 0.3, False)
    op, lp = _range_partials(q, k, v, 0.3, cuts)
    o, lse = oracle.combine(op, lp)
    np.testing.assert_allclose(o, o_full.reshape(-1, d), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, l_full.reshape(-1), rtol=1e-13, atol=1e-13)
    # the order of the ranges does not matter
    perm = np.random.default_rng(114).permutation(len(cuts) - 1)
    o2, l2 = oracle.combine(op[perm], lp[perm])
    np.testing.assert_allclose(o2, o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l2, lse, rtol=1e-14, atol=1e-14)


def test_combine_closed_forms(oracle_lib):
    # Two ranges with equal LSE a: the plain average, LSE a + ln 2.  One
    # range: unchanged.  Only empty ranges: O = 0, LSE = -inf.
    g = np.random.default_rng(115)
    o1, o2 = g.standard_normal((2, 3, 4))
    a = np.array([0.5, -3.0, 40.0])
    o, lse = oracle.combine(np.stack([o1, o2]), np.stack([a, a]))
    np.testing.assert_allclose(o, (o1 + o2) / 2, rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(lse, a + math.log(2.0), rtol=1e-15)
    o, lse = oracle.combine(o1[None], a[None])
    np.testing.assert_allclose(o, o1, rtol=1e-15, atol=0)
    np.testing.assert_array_equal(lse, a)
    o, lse = oracle.combine(np.zeros((3, 3, 4)), np.full((3, 3), -np.inf))
    assert np.all(o == 0.0) and np.all(np.isneginf(lse))
    # weights e^(LSE_s - LSE): ranges with LSE 0 and ln 3 weigh 1/4 and 3/4
    o, lse = oracle.combine(np.stack([o1, o2]), np.stack([np.zeros(3), np.full(3, math.log(3.0))]))
    np.testing.assert_allclose(o, 0.25 * o1 + 0.75 * o2, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse, np.full(3, math.log(4.0)), rtol=1e-15)


# --------------------------------------------------------------------------
# Gradients (backward pass)
# --------------------------------------------------------------------------

def _eighths(shape, seed):
    # values k/8 with |k| <= 16: a +-2^-12 step is exact in fp32
    g = np.random.default_rng(seed)
    return torch.from_numpy((g.integers(-16, 17, size=shape) / 8.0).astype(np.float32))


@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_finite_differences_of_the_forward(oracle_lib, causal):
    # dL/dx for L = sum(dO * O(x)): central differences of the (separately
    # pinned) forward oracle with an exact step h = 2^-12.
    B, H, N, d = 1, 2, 5, 4
    q, k, v, g = (_eighths((B, H, N, d), s) for s in (121, 122, 123, 124))
    scale = 0.5
    dq, dk, dv = oracle.bwd(q, k, v, g, scale, causal)
    h = 2.0 ** -12
    gg = _f64(g)

    def loss(q_, k_, v_):
        o, _ = oracle.fwd(q_, k_, v_, scale, causal)
        return float((o * gg).sum())

    worst = 0.0
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for idx in np.ndindex(B, H, N, d):
            args_p = [q.clone(), k.clone(), v.clone()]
            args_m = [q.clone(), k.clone(), v.clone()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            worst = max(worst, abs(fd - grad[idx]))
    assert worst <= 1e-6, worst


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 8), (9, 16), (40, 8)])
def test_gradients_match_torch_autograd_fp64(oracle_lib, dtype, causal, N, d):
    B, H = 2, 2
    q, k, v, g = (_rand((B, H, N, d), dtype, seed=s) for s in (131, 132, 133, 134))
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = oracle.bwd(q, k, v, g, scale, causal)
    sc = float(np.float32(scale))
    q64, k64, v64 = (t.to(torch.float64).requires_grad_(True) for t in (q, k, v))
    logits = sc * torch.matmul(q64, k64.transpose(-1, -2))
    if causal:
        logits = logits.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    o = torch.matmul(torch.softmax(logits, -1), v64)
    o.backward(g.to(torch.float64))
    for got, ref in ((dq, q64.grad), (dk, k64.grad), (dv, v64.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_gradients_one_head_rows_split_over_threads(oracle_lib, causal):
    # One K/V head with fewer heads than threads: the oracle deals the query
    # rows of the head to its threads (each sums its own dK, dV share, the
    # shares are added in order).  Against fp64 autograd, and against the
    # one-thread result (same sums, another order).
    B, H, N, d = 1, 1, 300, 16
    q, k, v, g = (_rand((B, H, N, d), torch.bfloat16, seed=s) for s in (141, 142, 143, 144))
    scale = 0.25
    dq, dk, dv = oracle.bwd(q, k, v, g, scale, causal, threads=7)
    q64, k64, v64 = (t.to(torch.float64).requires_grad_(True) for t in (q, k, v))
    logits = scale * torch.matmul(q64, k64.transpose(-1, -2))
    if causal:
        logits = logits.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    o = torch.matmul(torch.softmax(logits, -1), v64)
    o.backward(g.to(torch.float64))
    for got, ref in ((dq, q64.grad), (dk, k64.grad), (dv, v64.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=1e-11, atol=1e-12)
    one = oracle.bwd(q, k, v, g, scale, causal, threads=1)
    for a, b in zip((dq, dk, dv), one):
        np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_invariants(oracle_lib, causal):
    # Softmax rows are shift-invariant, so every dS row sums to zero and the
    # key gradients of a head sum to zero; the weights of a row sum to one,
    # so the value gradients of a head sum to the sum of dO rows.
    B, H, N, d = 2, 3, 33, 8
    q, k, v, g = (_rand((B, H, N, d), seed=s) for s in (141, 142, 143, 144))
    dq, dk, dv = oracle.bwd(q, k, v, g, 0.4, causal)
    assert np.max(np.abs(dk.sum(axis=2))) <= 1e-12 * max(1.0, np.abs(dk).max())
    np.testing.assert_allclose(dv.sum(axis=2), _f64(g).sum(axis=2), rtol=1e-12, atol=1e-12)


def test_dq_rows_equal_full_gradient(oracle_lib):
    B, H, N, d = 2, 2, 30, 8
    q, k, v, g = (_rand((B, H, N, d), seed=s) for s in (151, 152, 153, 154))
    for causal in (False, True):
        dq, _, _ = oracle.bwd(q, k, v, g, 0.3, causal)
        rows = np.array([0, 7, 29, 30, 59, 100, B * H * N - 1])
        got = oracle.bwd_dq_rows(q, k, v, g, 0.3, causal, rows)
        np.testing.assert_allclose(got, dq.reshape(-1, d)[rows], rtol=1e-14, atol=1e-15)


# --------------------------------------------------------------------------
# Gradients with grouped K/V heads and N_q != N_kv
# --------------------------------------------------------------------------

def _autograd_gqa(q, k, v, g, scale, causal):
    # Independent fp64 reference: K/V heads repeated to the query heads
    # (repeat_interleave's backward sums each group), the end-aligned causal
    # mask written out, and rows without a visible key zeroed explicitly.
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    q64, k64, v64 = (t.to(torch.float64).requires_grad_(True) for t in (q, k, v))
    kk = k64.repeat_interleave(H // Hkv, dim=1)
    vv = v64.repeat_interleave(H // Hkv, dim=1)
    logits = float(np.float32(scale)) * torch.matmul(q64, kk.transpose(-1, -2))
    i = torch.arange(Nq).view(-1, 1)
    j = torch.arange(Nk).view(1, -1)
    masked = (j > i + (Nk - Nq)) if causal else torch.zeros(Nq, Nk, dtype=torch.bool)
    empty = masked.all(dim=1, keepdim=True)
    logits = logits.masked_fill(masked | empty, float("-inf")).masked_fill(empty, 0.0)
    w = torch.softmax(logits, -1) * (~empty).to(torch.float64)
    o = torch.matmul(w, vv)
    o.backward(g.to(torch.float64))
    return q64.grad.numpy(), k64.grad.numpy(), v64.grad.numpy()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H,Hkv,Nq,Nk", [(4, 2, 9, 9), (6, 2, 5, 13), (4, 1, 13, 5),
                                         (4, 4, 7, 11), (2, 1, 1, 17)])
def test_grouped_gradients_match_torch_autograd_fp64(oracle_lib, dtype, causal, H, Hkv, Nq, Nk):
    B, d = 2, 8
    q = _rand((B, H, Nq, d), dtype, seed=161)
    k = _rand((B, Hkv, Nk, d), dtype, seed=162)
    v = _rand((B, Hkv, Nk, d), dtype, seed=163)
    g = _rand((B, H, Nq, d), dtype, seed=164)
    dq, dk, dv = oracle.bwd(q, k, v, g, 0.35, causal)
    assert dq.shape == (B, H, Nq, d) and dk.shape == dv.shape == (B, Hkv, Nk, d)
    rq, rk, rv = _autograd_gqa(q, k, v, g, 0.35, causal)
    for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
        np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)
    if causal and Nq > Nk:  # the first Nq - Nk rows see no key
        assert np.all(dq[:, :, : Nq - Nk] == 0.0)


def test_grouped_gradients_match_finite_differences(oracle_lib):
    # Central differences (exact step 2^-12) of the pinned grouped forward
    # oracle, causal with N_q < N_kv and two query heads on one K/V head.
    B, H, Hkv, Nq, Nk, d = 1, 2, 1, 3, 5, 4
    q, g = (_eighths((B, H, Nq, d), s) for s in (171, 174))
    k, v = (_eighths((B, Hkv, Nk, d), s) for s in (172, 173))
    scale = 0.5
    dq, dk, dv = oracle.bwd(q, k, v, g, scale, True)
    h = 2.0 ** -12
    gg = _f64(g)

    def loss(q_, k_, v_):
        o, _ = oracle.fwd_gqa(q_, k_, v_, scale, True)
        return float((o * gg).sum())

    worst = 0.0
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        base = (q, k, v)[which]
        for idx in np.ndindex(*base.shape):
            args_p = [q.clone(), k.clone(), v.clone()]
            args_m = [q.clone(), k.clone(), v.clone()]
            args_p[which][idx] += h
            args_m[which][idx] -= h
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            worst = max(worst, abs(fd - grad[idx]))
    assert worst <= 1e-6, worst


@pytest.mark.parametrize("causal", [False, True])
def test_grouped_gradient_invariants(oracle_lib, causal):
    # Per K/V head: key gradients sum to zero; value gradients sum to the sum
    # of the dO rows of every query head in the group (every row sees a key).
    B, H, Hkv, Nq, Nk, d = 2, 6, 2, 11, 20, 8
    q, g = _rand((B, H, Nq, d), seed=181), _rand((B, H, Nq, d), seed=184)
    k, v = _rand((B, Hkv, Nk, d), seed=182), _rand((B, Hkv, Nk, d), seed=183)
    dq, dk, dv = oracle.bwd(q, k, v, g, 0.4, causal)
    assert np.max(np.abs(dk.sum(axis=2))) <= 1e-12 * max(1.0, np.abs(dk).max())
    gsum = _f64(g).sum(axis=2).reshape(B, Hkv, H // Hkv, d).sum(axis=2)
    np.testing.assert_allclose(dv.sum(axis=2), gsum, rtol=1e-12, atol=1e-12)


def test_grouped_dq_rows_equal_full_gradient(oracle_lib):
    B, H, Hkv, Nq, Nk, d = 2, 4, 2, 9, 14, 8
    q, g = _rand((B, H, Nq, d), seed=191), _rand((B, H, Nq, d), seed=194)
    k, v = _rand((B, Hkv, Nk, d), seed=192), _rand((B, Hkv, Nk, d), seed=193)
    for causal in (False, True):
        dq, _, _ = oracle.bwd(q, k, v, g, 0.3, causal)
        rows = np.array([0, 5, 8, 9, 20, 35, 40, B * H * Nq - 1])
        got = oracle.bwd_dq_rows(q, k, v, g, 0.3, causal, rows)
        np.testing.assert_allclose(got, dq.reshape(-1, d)[rows], rtol=1e-14, atol=1e-15)
