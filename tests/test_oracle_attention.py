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


# ---------------------------------------------------------------- backward rounding bound

def _round16(x, dtype):
    import torch
    t = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    return torch.from_numpy(np.ascontiguousarray(x)).to(t).double().numpy()


def _simulated_rounded_backward(q, k, v, do, causal, scale, dtype):
    """The rounding model that grad_rounding_bound states, carried out
    literally: fp32 arithmetic (numpy float32) with P, the forward's O, dS,
    dK and dV rounded to the 16-bit type at the stated points."""
    B, H, N, d = q.shape
    out = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)]
    f = np.float32
    for b in range(B):
        for h in range(H):
            Q, K, V, dO = (x[b, h].astype(f) for x in (q, k, v, do))
            s = (Q @ K.T) * f(scale)
            if causal:
                s = np.where(np.arange(N)[None, :] > np.arange(N)[:, None], -np.inf, s).astype(f)
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m).astype(f)
            l = e.sum(axis=1, keepdims=True, dtype=f)
            lse = (m + np.log(l)).astype(f)
            o = _round16((_round16(e, dtype).astype(f) @ V) / l, dtype).astype(f)
            p = _round16(np.exp(s - lse).astype(f), dtype).astype(f)
            dd = (dO * o).sum(axis=1, keepdims=True, dtype=f)
            ds = _round16(p * (dO @ V.T - dd), dtype).astype(f)
            out[0][b, h] = (ds @ K) * f(scale)
            out[1][b, h] = _round16(f(scale) * (ds.T @ Q), dtype)
            out[2][b, h] = _round16(p.T @ dO, dtype)
    return out


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,scale", [(17, None), (129, None), (96, 0.2)])
def test_grad_rounding_bound_holds_and_is_attained(dtype, causal, N, scale):
    """The backward's elementwise rounding bound covers a literal simulation
    of the rounding model it states (fp32 sums; P, O, dS, dK, dV rounded to
    the 16-bit type, fp16 subnormals included), and is not vacuous: a
    single-term gradient (dV of the last keys under the causal mask) comes
    close to it."""
    from oracle.attention import attention_bwd, grad_rounding_bound
    rng = np.random.default_rng(21 + N)
    B, H, d = 1, 2, 64
    q, k, v, do = (_round16(rng.standard_normal((B, H, N, d)), dtype) for _ in range(4))
    sc = scale if scale is not None else 1.0 / np.sqrt(d)
    exact = attention_bwd(q, k, v, do, causal=causal, scale=sc)
    sim = _simulated_rounded_backward(q, k, v, do, causal, sc, dtype)
    bounds = grad_rounding_bound(q, k, v, do, causal=causal, scale=sc, dtype=dtype)
    ratios = []
    for g, r, bd in zip(sim, exact, bounds):
        err = np.abs(g - r)
        assert np.all(err <= bd)
        ratios.append(float(np.max(err / bd)))
    if causal and scale is None:
        assert ratios[2] >= 0.5, ratios


def test_grad_rounding_bound_needs_its_underflow_term():
    """With fp16 and a small softmax scale many probabilities underflow; a
    bound without the absolute subnormal term fails there (the relative
    model alone is not enough), the stated one holds."""
    from oracle.attention import _grad_rounding_bound, attention_bwd, grad_rounding_bound
    rng = np.random.default_rng(5)
    B, H, N, d = 1, 2, 256, 128
    q, k, v, do = (_round16(rng.standard_normal((B, H, N, d)), "fp16") for _ in range(4))
    exact = attention_bwd(q, k, v, do, causal=True, scale=0.2)
    sim = _simulated_rounded_backward(q, k, v, do, True, 0.2, "fp16")
    full = grad_rounding_bound(q, k, v, do, causal=True, scale=0.2, dtype="fp16")
    rel_only = _grad_rounding_bound(q, k, v, do, True, 0.2, 2.0 ** -11, 0.0)
    assert all(np.all(np.abs(g - r) <= b) for g, r, b in zip(sim, exact, full))
    assert np.any(np.abs(sim[2] - exact[2]) > rel_only[2])
