"""Split-KV parity: fa_fwd_partial, fa_merge and fa_fwd_splitkv (HIP, through
the C ABI) against the fp64 oracle (attention at explicit positions and the
log-sum-exp merge).

Bar: as the forward -- O max-abs <= 2e-2 and RMSE <= 2e-3, LSE max-abs <=
1e-3 -- for the 16-bit outputs and for the fp32 partial outputs alike (the
partials are more accurate: they skip the final rounding).  Rows that see no
key must come back as exactly O = 0 and LSE = -inf.  Small shapes are
compared in full, the full-size shapes (decoding over 16k keys; the bench
shape cut into four causal key chunks, as one ring-attention pass) on
sampled rows of sampled heads.
"""

import numpy as np
import pytest

from exact_tiled_attention_16_amd import inputs
from oracle.attention import (attention_fwd_positions, attention_fwd_positions_rows,
                              merge_partials)
from tests.helpers import host_round, max_abs, rmse, sample_rows, to_device

pytestmark = pytest.mark.gpu

O_MAX_ABS = 2e-2
O_RMSE = 2e-3
LSE_MAX_ABS = 1e-3


def _fa():
    from exact_tiled_attention_16_amd import fa
    return fa


def _banner(msg):
    print(f"\n[splitkv] {msg}", flush=True)


def _inputs(B, H, Nq, Nk, d, workload, dtype="bf16"):
    q = inputs.qkv(B, H, Nq, d, workload)[0]
    _, k, v = inputs.qkv(B, H, Nk, d, workload + 1)
    (qt, q64), (kt, k64), (vt, v64) = (host_round(x, dtype) for x in (q, k, v))
    return (qt, kt, vt), (q64, k64, v64)


def _np(t):
    import torch
    return t.to(torch.float64).cpu().numpy()


def _compare(o, lse, o_ref, lse_ref, what):
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), what
    assert np.all(o[empty] == 0.0), what
    assert np.all(np.isfinite(o)), what
    assert max_abs(o, o_ref) <= O_MAX_ABS, what
    assert rmse(o, o_ref) <= O_RMSE, what
    if (~empty).any():
        assert max_abs(lse[~empty], lse_ref[~empty]) <= LSE_MAX_ABS, what


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("Nq,Nk,qp0,kp0,causal", [
    (300, 257, 0, 0, False),     # ragged, more queries than keys
    (300, 257, 100, 37, True),   # diagonal inside the part
    (129, 500, 371, 0, True),    # queries at the end of the keys
    (200, 300, 0, 150, True),    # first 150 rows see no key of the part
    (1, 1000, 999, 0, True),     # one decoding query, every key visible
    (70, 64, 5000, 0, True),     # every key visible to every row
])
def test_partial_matches_oracle(d, Nq, Nk, qp0, kp0, causal):
    fa = _fa()
    _banner(f"partial d={d} Nq={Nq} Nk={Nk} q_pos0={qp0} k_pos0={kp0} causal={causal}")
    (qt, kt, vt), (q64, k64, v64) = _inputs(2, 3, Nq, Nk, d, 300 + d)
    o, lse = fa.fwd_partial(to_device(qt), to_device(kt), to_device(vt), causal=causal,
                            q_pos0=qp0, k_pos0=kp0)
    o_ref, lse_ref = attention_fwd_positions(q64, k64, v64, causal=causal, q_pos0=qp0,
                                             k_pos0=kp0)
    _compare(_np(o), _np(lse), o_ref, lse_ref, "partial")


@pytest.mark.parametrize("S", [1, 3, 6])
@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "fp16"), (256, "bf16")])
def test_merge_matches_oracle(S, d, dtype):
    """Random partials with some empty parts (LSE -inf, O NaN: never read)
    and some rows empty in every part."""
    import torch
    fa = _fa()
    _banner(f"merge S={S} d={d} {dtype}")
    rng = np.random.default_rng(S * 1000 + d)
    B, H, N = 2, 3, 77
    o_parts = rng.standard_normal((S, B, H, N, d)).astype(np.float32)
    lse_parts = (3.0 * rng.standard_normal((S, B, H, N))).astype(np.float32)
    empty = rng.random((S, B, H, N)) < 0.3
    empty[:, 0, 0, :5] = True                       # rows with no key at all
    lse_parts[empty] = -np.inf
    o_parts[empty] = np.nan
    dt = torch.bfloat16 if dtype == "bf16" else torch.float16
    o, lse = fa.merge(torch.from_numpy(o_parts).cuda(), torch.from_numpy(lse_parts).cuda(),
                      dtype=dt)
    torch.cuda.synchronize()
    o_ref, lse_ref = merge_partials(o_parts, lse_parts)
    o, lse = _np(o), _np(lse)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_ref))
    fin = np.isfinite(lse_ref)
    assert np.all(o[~fin] == 0.0) and np.all(np.isfinite(o))
    assert max_abs(o, o_ref) <= O_MAX_ABS
    assert max_abs(lse[fin], lse_ref[fin]) <= 1e-5 * max(1.0, np.abs(lse_ref[fin]).max())


@pytest.mark.parametrize("B,H,Nq,Nk,d,splits,causal", [
    (4, 8, 1, 4097, 128, 8, False),    # decoding, ragged key count
    (4, 8, 1, 4097, 128, 8, True),     # decoding at the last position
    (2, 4, 16, 2000, 64, 3, True),     # speculative block of 16 queries
    (1, 2, 1000, 1000, 256, 4, True),  # equal lengths: fa_fwd's causal mask
    (2, 2, 5, 130, 128, 50, False),    # more splits than 64-key tiles
    (1, 3, 33, 64, 64, 1, True),       # one split
])
def test_splitkv_matches_oracle(B, H, Nq, Nk, d, splits, causal):
    fa = _fa()
    _banner(f"splitkv B={B} H={H} Nq={Nq} Nk={Nk} d={d} splits={splits} causal={causal}")
    (qt, kt, vt), (q64, k64, v64) = _inputs(B, H, Nq, Nk, d, 400 + splits)
    o, lse = fa.fwd_splitkv(to_device(qt), to_device(kt), to_device(vt), splits,
                            causal=causal)
    o_ref, lse_ref = attention_fwd_positions(q64, k64, v64, causal=causal,
                                             q_pos0=Nk - Nq)
    _compare(_np(o), _np(lse), o_ref, lse_ref, "splitkv")


@pytest.mark.parametrize("Nq,splits", [(1, 8), (40, 3)])
def test_splitkv_fp16(Nq, splits):
    """fp16 inputs through both partial configurations (one-wave workgroups
    for Nq <= 32, the default tile otherwise) and the fp16 merge."""
    fa = _fa()
    _banner(f"splitkv fp16 Nq={Nq} splits={splits}")
    B, H, Nk, d = 2, 3, 777, 128
    (qt, kt, vt), (q64, k64, v64) = _inputs(B, H, Nq, Nk, d, 450 + Nq, dtype="fp16")
    o, lse = fa.fwd_splitkv(to_device(qt), to_device(kt), to_device(vt), splits, causal=True)
    o_ref, lse_ref = attention_fwd_positions(q64, k64, v64, causal=True, q_pos0=Nk - Nq)
    _compare(_np(o), _np(lse), o_ref, lse_ref, "splitkv fp16")


def test_splitkv_equal_lengths_matches_fa_fwd():
    """With Nq = Nk the split result equals the single-pass forward to within
    rounding (the parts change only the order of the fp32 sums)."""
    import torch
    fa = _fa()
    _banner("splitkv vs fa_fwd")
    (qt, kt, vt), _ = _inputs(2, 4, 1500, 1500, 128, 77)
    q, k, v = to_device(qt), to_device(kt), to_device(vt)
    for causal in (False, True):
        o1, l1 = fa.fwd(q, k, v, causal=causal)
        o2, l2 = fa.fwd_splitkv(q, k, v, 6, causal=causal)
        torch.cuda.synchronize()
        assert max_abs(_np(o1), _np(o2)) <= 2 * 2 ** -8 * 4
        assert max_abs(_np(l1), _np(l2)) <= 1e-4


def test_ring_pass_over_key_chunks_full_size_sampled():
    """B=2, H=16, N=8192, d=128 causal, keys in four chunks: one partial call
    per chunk at its key positions, then the merge -- the work of one
    ring-attention pass on one GPU.  Sampled rows against the oracle over all
    keys, and the whole output against fa_fwd."""
    import torch
    fa = _fa()
    _banner("ring pass B=2 H=16 N=8192 d=128, 4 chunks")
    B, H, N, d, G = 2, 16, 8192, 128, 4
    (qt, kt, vt), (q64, k64, v64) = _inputs(B, H, N, N, d, 500)
    q, k, v = to_device(qt), to_device(kt), to_device(vt)
    c = N // G
    o_parts = torch.empty((G, B, H, N, d), dtype=torch.float32, device="cuda")
    lse_parts = torch.empty((G, B, H, N), dtype=torch.float32, device="cuda")
    for g in range(G):
        kc, vc = k[:, :, g * c:(g + 1) * c].contiguous(), v[:, :, g * c:(g + 1) * c].contiguous()
        fa.fwd_partial(q, kc, vc, causal=True, q_pos0=0, k_pos0=g * c,
                       out=o_parts[g], lse=lse_parts[g])
    o, lse = fa.merge(o_parts, lse_parts, dtype=torch.bfloat16)
    o_ref1, lse_ref1 = fa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert max_abs(_np(o), _np(o_ref1)) <= 2 * 2 ** -8 * 4
    o, lse = _np(o), _np(lse)
    for b, h in ((0, 0), (B - 1, H - 1)):
        rows = sample_rows(N, seed=b * 17 + h)
        o_ref, lse_ref = attention_fwd_positions_rows(q64[b, h], k64[b, h], v64[b, h], rows,
                                                      causal=True)
        assert max_abs(o[b, h, rows], o_ref) <= O_MAX_ABS
        assert rmse(o[b, h, rows], o_ref) <= O_RMSE
        assert max_abs(lse[b, h, rows], lse_ref) <= LSE_MAX_ABS


def test_decode_full_size_sampled():
    """Decoding: B=16, H=16, one query over 16,384 keys, d=128, 16 splits."""
    import torch
    fa = _fa()
    _banner("decode B=16 H=16 Nq=1 Nk=16384 d=128")
    B, H, Nq, Nk, d = 16, 16, 1, 16384, 128
    (qt, kt, vt), (q64, k64, v64) = _inputs(B, H, Nq, Nk, d, 600)
    o, lse = fa.fwd_splitkv(to_device(qt), to_device(kt), to_device(vt), 16, causal=True)
    torch.cuda.synchronize()
    o, lse = _np(o), _np(lse)
    for b, h in ((0, 0), (7, 9), (B - 1, H - 1)):
        o_ref, lse_ref = attention_fwd_positions_rows(q64[b, h], k64[b, h], v64[b, h], [0],
                                                      causal=True, q_pos0=Nk - 1)
        assert max_abs(o[b, h], o_ref) <= O_MAX_ABS
        assert max_abs(lse[b, h], lse_ref) <= LSE_MAX_ABS
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
