"""Pins of the split-KV oracle: attention at explicit positions and the
log-sum-exp merge of partial results (oracle/attention.py).

Each check ties the oracle to something other than itself: a scalar loop
written from the definition, the already-pinned ``attention_fwd``, invariants
of the mask (translation, decoding) and the merge identity (merging the
partial results over any split of the keys reproduces attention over all
keys).
"""

import math

import numpy as np
import pytest

from oracle.attention import (attention_fwd, attention_fwd_positions,
                              attention_fwd_positions_rows, merge_partials)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _loops(q, k, v, scale, causal, qp0, kp0):
    """Scalar triple loop: one (b, h) head, q [Nq, d], k, v [Nk, d]."""
    Nq, d = len(q), len(q[0])
    Nk = len(k)
    o = [[0.0] * d for _ in range(Nq)]
    lse = [0.0] * Nq
    for i in range(Nq):
        vis = [j for j in range(Nk) if not causal or kp0 + j <= qp0 + i]
        if not vis:
            lse[i] = -math.inf
            continue
        sc = {j: scale * sum(q[i][c] * k[j][c] for c in range(d)) for j in vis}
        m = max(sc.values())
        den = sum(math.exp(sc[j] - m) for j in vis)
        for c in range(d):
            o[i][c] = sum(math.exp(sc[j] - m) / den * v[j][c] for j in vis)
        lse[i] = m + math.log(den)
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("qp0,kp0", [(0, 0), (5, 2), (1, 6), (0, 9)])
def test_positions_match_scalar_loops(causal, qp0, kp0):
    rng = np.random.default_rng(11 + qp0 + 7 * kp0)
    q, k, v = _rand(rng, 1, 1, 6, 4), _rand(rng, 1, 1, 9, 4), _rand(rng, 1, 1, 9, 4)
    o, lse = attention_fwd_positions(q, k, v, causal=causal, scale=0.7,
                                     q_pos0=qp0, k_pos0=kp0)
    o_ref, lse_ref = _loops(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(),
                            0.7, causal, qp0, kp0)
    assert np.array_equal(np.isinf(lse[0, 0]), np.isinf(lse_ref))
    fin = np.isfinite(lse_ref)
    assert np.allclose(lse[0, 0][fin], lse_ref[fin], rtol=0, atol=1e-12)
    assert np.allclose(o[0, 0], o_ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_offsets_reduce_to_plain_forward(causal):
    rng = np.random.default_rng(3)
    q, k, v = (_rand(rng, 2, 2, 37, 16) for _ in range(3))
    o, lse = attention_fwd_positions(q, k, v, causal=causal)
    o_ref, lse_ref = attention_fwd(q, k, v, causal=causal)
    assert np.allclose(o, o_ref, atol=1e-13) and np.allclose(lse, lse_ref, atol=1e-13)


def test_translation_invariance_and_decoding():
    rng = np.random.default_rng(4)
    q, k, v = (_rand(rng, 1, 2, 21, 8) for _ in range(3))
    o0, l0 = attention_fwd_positions(q, k, v, causal=True)
    o1, l1 = attention_fwd_positions(q, k, v, causal=True, q_pos0=1000, k_pos0=1000)
    assert np.allclose(o0, o1, atol=1e-14) and np.allclose(l0, l1, atol=1e-14)
    # One query at the last position sees every key: causal = full.
    qd = _rand(rng, 1, 2, 1, 8)
    oc, lc = attention_fwd_positions(qd, k, v, causal=True, q_pos0=20)
    of, lf = attention_fwd_positions(qd, k, v, causal=False)
    assert np.allclose(oc, of, atol=1e-14) and np.allclose(lc, lf, atol=1e-14)


def test_rows_that_see_no_key():
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, 1, 1, 8, 4), _rand(rng, 1, 1, 5, 4), _rand(rng, 1, 1, 5, 4)
    o, lse = attention_fwd_positions(q, k, v, causal=True, q_pos0=0, k_pos0=3)
    assert np.all(np.isneginf(lse[0, 0, :3])) and np.all(o[0, 0, :3] == 0.0)
    assert np.all(np.isfinite(lse[0, 0, 3:]))
    # Row 3 (position 3) sees key 0 only: O = V[0], LSE = its score.
    assert np.allclose(o[0, 0, 3], v[0, 0, 0], atol=1e-14)
    assert math.isclose(lse[0, 0, 3], 0.5 * float(q[0, 0, 3] @ k[0, 0, 0]), abs_tol=1e-14)


def test_selected_rows_match_full():
    rng = np.random.default_rng(6)
    q, k, v = _rand(rng, 1, 1, 30, 8), _rand(rng, 1, 1, 19, 8), _rand(rng, 1, 1, 19, 8)
    o, lse = attention_fwd_positions(q, k, v, causal=True, q_pos0=3, k_pos0=10)
    rows = np.array([0, 6, 7, 29])
    o_r, l_r = attention_fwd_positions_rows(q[0, 0], k[0, 0], v[0, 0], rows, causal=True,
                                            q_pos0=3, k_pos0=10)
    assert np.allclose(o_r, o[0, 0, rows]) and np.array_equal(l_r, lse[0, 0, rows])


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("cuts", [(0, 40), (0, 1, 40), (0, 7, 8, 23, 40), (0, 13, 26, 39, 40)])
def test_merge_of_parts_is_attention_over_all_keys(causal, cuts):
    """Split the keys at `cuts`; each part at its own key positions; merge."""
    rng = np.random.default_rng(7 + len(cuts))
    q = _rand(rng, 2, 2, 17, 8)
    k, v = _rand(rng, 2, 2, 40, 8), _rand(rng, 2, 2, 40, 8)
    qp0 = 23  # queries at positions 23..39, so early rows miss late parts
    parts = [attention_fwd_positions(q, k[:, :, a:b], v[:, :, a:b], causal=causal,
                                     q_pos0=qp0, k_pos0=a)
             for a, b in zip(cuts[:-1], cuts[1:])]
    o, lse = merge_partials(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    o_ref, lse_ref = attention_fwd_positions(q, k, v, causal=causal, q_pos0=qp0)
    assert np.allclose(o, o_ref, atol=1e-13) and np.allclose(lse, lse_ref, atol=1e-13)


def test_merge_algebra():
    rng = np.random.default_rng(8)
    o1, l1 = _rand(rng, 3, 4), _rand(rng, 3)
    o, l = merge_partials(o1[None], l1[None])        # one part: identity
    assert np.allclose(o, o1) and np.allclose(l, l1)
    o, l = merge_partials(np.stack([o1, o1]), np.stack([l1, l1]))  # twice: L + ln 2
    assert np.allclose(o, o1) and np.allclose(l, l1 + math.log(2.0))
    bad = np.full_like(o1, np.nan)                   # empty part: O never read
    o, l = merge_partials(np.stack([o1, bad]), np.stack([l1, np.full(3, -np.inf)]))
    assert np.allclose(o, o1) and np.allclose(l, l1)
    o, l = merge_partials(np.stack([bad, bad]), np.full((2, 3), -np.inf))  # all empty
    assert np.all(o == 0.0) and np.all(np.isneginf(l))
    # Unequal weights: exp(L_p - L) by hand.
    o2, l2 = _rand(rng, 3, 4), l1 + 1.5
    o, l = merge_partials(np.stack([o1, o2]), np.stack([l1, l2]))
    w1 = 1.0 / (1.0 + math.exp(1.5))
    assert np.allclose(o, w1 * o1 + (1 - w1) * o2, atol=1e-14)
    assert np.allclose(l, l1 + math.log(1.0 + math.exp(1.5)), atol=1e-14)
