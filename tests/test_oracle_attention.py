"""Pins for the fp64 attention oracle (CPU only).

Each test checks the oracle against something other than itself: a closed form,
an invariant of softmax attention, brute force, or finite differences.  They
are chosen so that a dropped term, a wrong sign or index, a transposed operand
or a missing scale in the oracle fails at least one of them.
"""

import math

import numpy as np
import pytest

from oracle.attention import (attention_bwd, attention_fwd,
                              attention_fwd_loops, attention_fwd_online,
                              attention_fwd_rows)


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 1), (2, 3), (5, 4), (13, 8), (16, 5)])
def test_vectorised_equals_scalar_loops(N, d, causal):
    q, k, v = (rnd((2, 2, N, d), s) for s in (1, 2, 3))
    o1, l1 = attention_fwd(q, k, v, causal=causal, scale=0.7)
    o2, l2 = attention_fwd_loops(q, k, v, causal=causal, scale=0.7)
    assert np.max(np.abs(o1 - o2)) <= 1e-13
    assert np.max(np.abs(l1 - l2)) <= 1e-13


@pytest.mark.parametrize("row_block", [1, 7, 64])
def test_row_blocking_does_not_change_result(row_block):
    q, k, v = (rnd((1, 2, 50, 8), s) for s in (4, 5, 6))
    for causal in (False, True):
        o1, l1 = attention_fwd(q, k, v, causal=causal, row_block=row_block)
        o2, l2 = attention_fwd_loops(q, k, v, causal=causal)
        assert np.max(np.abs(o1 - o2)) <= 1e-12
        assert np.max(np.abs(l1 - l2)) <= 1e-12


def test_sampled_rows_match_full():
    q, k, v = (rnd((1, 1, 300, 16), s) for s in (7, 8, 9))
    rows = [0, 1, 17, 128, 299]
    for causal in (False, True):
        o, l = attention_fwd(q, k, v, causal=causal)
        o2, l2 = attention_fwd_rows(q[0, 0], k[0, 0], v[0, 0], rows,
                                    causal=causal)
        assert np.max(np.abs(o[0, 0, rows] - o2)) <= 1e-13
        assert np.max(np.abs(l[0, 0, rows] - l2)) <= 1e-13


# ------------------------------------------------------------- closed forms

def test_probabilities_rows_sum_to_one_and_nonnegative():
    # With V = identity (d = N) the output rows are the probability rows.
    N = 12
    q, k = rnd((1, 1, N, 4), 10), rnd((1, 1, N, 4), 11)
    q4 = np.concatenate([q, np.zeros((1, 1, N, N - 4))], axis=-1)
    k4 = np.concatenate([k, np.zeros((1, 1, N, N - 4))], axis=-1)
    v = np.eye(N)[None, None]
    for causal in (False, True):
        p, _ = attention_fwd(q4, k4, v, causal=causal, scale=0.9)
        assert np.all(p >= 0)
        assert np.max(np.abs(p.sum(axis=-1) - 1.0)) <= 1e-14
        if causal:
            assert np.all(np.triu(p[0, 0], 1) == 0)
        # softmax by hand for row 3
        s = 0.9 * (q4[0, 0, 3] @ k4[0, 0].T)
        if causal:
            s = s[:4]
        ref = np.exp(s - s.max())
        ref /= ref.sum()
        assert np.allclose(p[0, 0, 3, :len(ref)], ref, atol=1e-15, rtol=0)


def test_zero_queries_give_column_mean_noncausal():
    N, d = 37, 6
    q = np.zeros((1, 2, N, d))
    k, v = rnd((1, 2, N, d), 12), rnd((1, 2, N, d), 13)
    o, lse = attention_fwd(q, k, v)
    assert np.allclose(o, v.mean(axis=2, keepdims=True).repeat(N, axis=2),
                       atol=1e-14, rtol=0)
    assert np.allclose(lse, math.log(N), atol=1e-14, rtol=0)


def test_zero_queries_give_prefix_mean_causal():
    N, d = 37, 6
    q = np.zeros((1, 1, N, d))
    k, v = rnd((1, 1, N, d), 14), rnd((1, 1, N, d), 15)
    o, lse = attention_fwd(q, k, v, causal=True)
    prefix = np.cumsum(v[0, 0], axis=0) / np.arange(1, N + 1)[:, None]
    assert np.allclose(o[0, 0], prefix, atol=1e-14, rtol=0)
    assert np.allclose(lse[0, 0], np.log(np.arange(1, N + 1)), atol=1e-14,
                       rtol=0)


def test_causal_row_zero_is_first_value():
    q, k, v = (rnd((2, 3, 20, 8), s) for s in (16, 17, 18))
    o, lse = attention_fwd(q, k, v, causal=True, scale=0.5)
    assert np.array_equal(o[:, :, 0], v[:, :, 0])
    ref = 0.5 * np.einsum("bhc,bhc->bh", q[:, :, 0], k[:, :, 0])
    assert np.allclose(lse[:, :, 0], ref, atol=1e-14, rtol=0)


def test_single_key_and_two_key_closed_forms():
    q, k, v = (rnd((1, 1, 1, 5), s) for s in (19, 20, 21))
    o, lse = attention_fwd(q, k, v, scale=0.3)
    assert np.array_equal(o, v)
    assert abs(lse[0, 0, 0] - 0.3 * float(q[0, 0, 0] @ k[0, 0, 0])) <= 1e-15
    # N = 2: weights are the logistic function of the score difference.
    q, k, v = (rnd((1, 1, 2, 5), s) for s in (22, 23, 24))
    o, lse = attention_fwd(q, k, v, scale=0.3)
    for i in range(2):
        s1 = 0.3 * float(q[0, 0, i] @ k[0, 0, 0])
        s2 = 0.3 * float(q[0, 0, i] @ k[0, 0, 1])
        w1 = 1.0 / (1.0 + math.exp(s2 - s1))
        w2 = 1.0 / (1.0 + math.exp(s1 - s2))
        assert np.allclose(o[0, 0, i], w1 * v[0, 0, 0] + w2 * v[0, 0, 1],
                           atol=1e-14, rtol=0)
        assert abs(lse[0, 0, i] - math.log(math.exp(s1) + math.exp(s2))) <= 1e-14


# ------------------------------------------------------------- invariants

def test_constant_values_pass_through():
    q, k = rnd((1, 2, 30, 4), 25, 3.0), rnd((1, 2, 30, 4), 26, 3.0)
    c = rnd((4,), 27)
    v = np.broadcast_to(c, (1, 2, 30, 4)).copy()
    for causal in (False, True):
        o, _ = attention_fwd(q, k, v, causal=causal)
        assert np.allclose(o, v, atol=1e-14, rtol=0)


def test_permutation_equivariance_noncausal():
    N = 23
    q, k, v = (rnd((1, 1, N, 7), s) for s in (28, 29, 30))
    perm = np.random.default_rng(31).permutation(N)
    o, l = attention_fwd(q, k, v)
    o2, l2 = attention_fwd(q[:, :, perm], k, v)
    assert np.allclose(o2, o[:, :, perm], atol=1e-14, rtol=0)
    assert np.allclose(l2, l[:, :, perm], atol=1e-14, rtol=0)
    o3, l3 = attention_fwd(q, k[:, :, perm], v[:, :, perm])
    assert np.allclose(o3, o, atol=1e-14, rtol=0)
    assert np.allclose(l3, l, atol=1e-13, rtol=0)


def test_causal_is_not_permutation_invariant():
    # Guards against a causal mask that silently does nothing.
    N = 16
    q, k, v = (rnd((1, 1, N, 4), s) for s in (32, 33, 34))
    o, _ = attention_fwd(q, k, v, causal=True)
    o_nc, _ = attention_fwd(q, k, v, causal=False)
    assert np.max(np.abs(o - o_nc)) > 1e-3
    assert np.allclose(o[0, 0, -1], o_nc[0, 0, -1], atol=1e-14, rtol=0)


def test_linear_in_values_and_key_shift():
    q, k, v1, v2 = (rnd((1, 2, 19, 5), s) for s in (35, 36, 37, 38))
    for causal in (False, True):
        o1, _ = attention_fwd(q, k, v1, causal=causal)
        o2, _ = attention_fwd(q, k, v2, causal=causal)
        o12, _ = attention_fwd(q, k, 2.0 * v1 - 3.0 * v2, causal=causal)
        assert np.allclose(o12, 2.0 * o1 - 3.0 * o2, atol=1e-13, rtol=0)
        u = rnd((5,), 39)
        o, lse = attention_fwd(q, k, v1, causal=causal, scale=0.4)
        os_, lses = attention_fwd(q, k + u, v1, causal=causal, scale=0.4)
        assert np.allclose(os_, o, atol=1e-13, rtol=0)
        assert np.allclose(lses - lse, 0.4 * (q @ u), atol=1e-13, rtol=0)


def test_scale_matters():
    q, k, v = (rnd((1, 1, 9, 4), s) for s in (40, 41, 42))
    o1, _ = attention_fwd(q, k, v, scale=0.5)
    o2, _ = attention_fwd(2.0 * q, k, v, scale=0.25)
    o3, _ = attention_fwd(q, k, v, scale=0.25)
    assert np.allclose(o1, o2, atol=1e-14, rtol=0)
    assert np.max(np.abs(o1 - o3)) > 1e-3
    o4, _ = attention_fwd(q, k, v)  # default 1/sqrt(d) = 0.5 for d = 4
    assert np.allclose(o4, o1, atol=1e-15, rtol=0)


# ------------------------------------------------------ online recurrence

@pytest.mark.parametrize("tile", [1, 3, 16, 64, 200])
@pytest.mark.parametrize("N", [1, 17, 129])
@pytest.mark.parametrize("causal", [False, True])
def test_online_recurrence_reaches_materialised(tile, N, causal):
    q, k, v = (rnd((1, 2, N, 8), s, 2.0) for s in (43, 44, 45))
    o, lse = attention_fwd(q, k, v, causal=causal)
    for base2 in (False, True):
        o2, lse2 = attention_fwd_online(q, k, v, causal=causal, key_tile=tile,
                                        base2=base2)
        assert np.max(np.abs(o - o2)) <= 1e-12
        assert np.max(np.abs(lse - lse2)) <= 1e-12


def test_online_recurrence_with_huge_scores_no_overflow():
    q, k, v = (rnd((1, 1, 40, 4), s, 30.0) for s in (46, 47, 48))
    o, lse = attention_fwd(q, k, v, causal=True)
    o2, lse2 = attention_fwd_online(q, k, v, causal=True, key_tile=8)
    assert np.all(np.isfinite(o2)) and np.all(np.isfinite(lse2))
    assert np.max(np.abs(o - o2)) <= 1e-10
    assert np.max(np.abs(lse - lse2)) <= 1e-10 * np.max(np.abs(lse))


# --------------------------------------------------------------- backward

def _loss(q, k, v, do, causal, scale):
    o, _ = attention_fwd(q, k, v, causal=causal, scale=scale)
    return float(np.sum(o * do))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_finite_differences(causal):
    B, H, N, d = 1, 2, 9, 5
    q, k, v, do = (rnd((B, H, N, d), s) for s in (49, 50, 51, 52))
    scale = 0.6
    dq, dk, dv = attention_bwd(q, k, v, do, causal=causal, scale=scale)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy()
            xp[idx] += eps
            xm = x.copy()
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name] = xp
            args_m[name] = xm
            fp = _loss(args_p["q"], args_p["k"], args_p["v"], do, causal, scale)
            fm = _loss(args_m["q"], args_m["k"], args_m["v"], do, causal, scale)
            num[idx] = (fp - fm) / (2 * eps)
        rel = np.linalg.norm(num - g) / np.linalg.norm(num)
        assert rel <= 1e-6, (name, rel)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_identities(causal):
    q, k, v, do = (rnd((2, 2, 21, 6), s) for s in (53, 54, 55, 56))
    dq, dk, dv = attention_bwd(q, k, v, do, causal=causal, row_block=8)
    # Rows of dS sum to zero, so the key gradients sum to zero.
    assert np.max(np.abs(dk.sum(axis=2))) <= 1e-12
    # Rows of P sum to one, so dV sums to the sum of dO.
    assert np.allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12, rtol=0)
    # dO = 0 gives zero gradients.
    z = attention_bwd(q, k, v, np.zeros_like(do), causal=causal)
    assert all(np.all(g == 0) for g in z)


def test_backward_equal_keys_give_zero_dq():
    q, v, do = (rnd((1, 1, 15, 4), s) for s in (57, 58, 59))
    k = np.broadcast_to(rnd((4,), 60), (1, 1, 15, 4)).copy()
    dq, _, _ = attention_bwd(q, k, v, do)
    assert np.max(np.abs(dq)) <= 1e-13


def test_backward_row_block_independent():
    q, k, v, do = (rnd((1, 1, 33, 4), s) for s in (61, 62, 63, 64))
    a = attention_bwd(q, k, v, do, causal=True, row_block=5)
    b = attention_bwd(q, k, v, do, causal=True, row_block=1024)
    for x, y in zip(a, b):
        assert np.max(np.abs(x - y)) <= 1e-13
