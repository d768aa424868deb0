"""Pins of the block-sparse oracle (attention_fwd_blockmask): the mask
reading against the plain forward (all-ones mask), independent diagonal
blocks, a scalar loop on a tiny input, empty rows and a key-block
permutation."""

import math

import numpy as np
import pytest

from oracle.attention import attention_fwd, attention_fwd_blockmask


def _qkv(rng, B, H, N, d):
    return (rng.standard_normal((B, H, N, d)) for _ in range(3))


@pytest.mark.parametrize("causal", [False, True])
def test_all_ones_mask_is_plain_attention(causal):
    rng = np.random.default_rng(1)
    q, k, v = _qkv(rng, 2, 3, 21, 8)
    mask = np.ones((3, 6, 6), np.uint8)
    o, lse = attention_fwd_blockmask(q, k, v, mask, block=4, causal=causal)
    o_ref, lse_ref = attention_fwd(q, k, v, causal=causal)
    assert np.allclose(o, o_ref, atol=1e-13) and np.allclose(lse, lse_ref, atol=1e-13)


def test_block_diagonal_mask_is_blockwise_attention():
    rng = np.random.default_rng(2)
    q, k, v = _qkv(rng, 1, 2, 16, 8)
    mask = np.eye(4, dtype=np.uint8)[None].repeat(2, axis=0)
    o, lse = attention_fwd_blockmask(q, k, v, mask, block=4)
    for i in range(4):
        sl = slice(4 * i, 4 * i + 4)
        o_ref, lse_ref = attention_fwd(q[:, :, sl], k[:, :, sl], v[:, :, sl])
        assert np.allclose(o[:, :, sl], o_ref, atol=1e-13)
        assert np.allclose(lse[:, :, sl], lse_ref, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_scalar_loop(causal):
    rng = np.random.default_rng(3)
    q, k, v = _qkv(rng, 1, 1, 7, 3)
    mask = np.array([[[1, 0, 1, 0], [0, 0, 0, 0], [1, 1, 0, 1], [0, 1, 1, 0]]], np.uint8)
    o, lse = attention_fwd_blockmask(q, k, v, mask, block=2, causal=causal, scale=0.9)
    for i in range(7):
        vis = [j for j in range(7) if mask[0, i // 2, j // 2] and (not causal or j <= i)]
        if not vis:
            assert math.isinf(lse[0, 0, i]) and lse[0, 0, i] < 0
            assert np.all(o[0, 0, i] == 0.0)
            continue
        sc = {j: 0.9 * sum(q[0, 0, i, c] * k[0, 0, j, c] for c in range(3)) for j in vis}
        m = max(sc.values())
        den = sum(math.exp(x - m) for x in sc.values())
        assert math.isclose(lse[0, 0, i], m + math.log(den), abs_tol=1e-12)
        for c in range(3):
            ref = sum(math.exp(sc[j] - m) / den * v[0, 0, j, c] for j in vis)
            assert math.isclose(o[0, 0, i, c], ref, abs_tol=1e-12)


def test_key_block_permutation_and_per_batch_masks():
    rng = np.random.default_rng(4)
    q, k, v = _qkv(rng, 2, 2, 12, 4)
    mask = (rng.random((2, 2, 3, 3)) < 0.6).astype(np.uint8)
    o, lse = attention_fwd_blockmask(q, k, v, mask, block=4)
    perm = [2, 0, 1]
    idx = np.concatenate([np.arange(4 * p, 4 * p + 4) for p in perm])
    o2, lse2 = attention_fwd_blockmask(q, k[:, :, idx], v[:, :, idx], mask[..., perm], block=4)
    assert np.allclose(o, o2, atol=1e-13) and np.array_equal(np.isinf(lse), np.isinf(lse2))
    fin = np.isfinite(lse)
    assert np.allclose(lse[fin], lse2[fin], atol=1e-13)
    # A per-batch mask equals running each batch with its own shared mask.
    for b in range(2):
        ob, lb = attention_fwd_blockmask(q[b:b + 1], k[b:b + 1], v[b:b + 1], mask[b], block=4)
        assert np.allclose(ob, o[b:b + 1], atol=1e-14)


def test_rows_selection_matches_full():
    rng = np.random.default_rng(5)
    q, k, v = _qkv(rng, 1, 2, 30, 8)
    mask = (rng.random((2, 4, 4)) < 0.5).astype(np.uint8)
    o, lse = attention_fwd_blockmask(q, k, v, mask, block=8, causal=True)
    rows = [0, 7, 8, 29]
    o_r, l_r = attention_fwd_blockmask(q, k, v, mask, block=8, causal=True, rows=rows)
    assert np.allclose(o_r, o[:, :, rows]) and np.array_equal(l_r, lse[:, :, rows])
