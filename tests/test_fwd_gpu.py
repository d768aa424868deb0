"""Forward parity: fa_fwd (HIP, through the C ABI) against the fp64 oracle.

Bar (stated for bf16/fp16 forward): O max-abs error <= 2e-2 and RMSE <= 2e-3
against the oracle evaluated on the same rounded inputs; LSE max-abs error
<= 1e-3.  Small shapes are compared element by element over the whole output;
the full-size workloads (B*N = 16384 at H=16, d=128; N=16384 long context)
are compared on sampled rows of sampled heads, which the oracle computes one
by one.
"""

import math

import numpy as np
import pytest

from exact_tiled_attention_16_amd import inputs
from oracle.attention import attention_fwd, attention_fwd_rows
from tests.helpers import host_round, max_abs, rmse, sample_rows, to_device

pytestmark = pytest.mark.gpu

O_MAX_ABS = 2e-2
O_RMSE = 2e-3
LSE_MAX_ABS = 1e-3


def _fa():
    from exact_tiled_attention_16_amd import fa
    return fa


def _run(q, k, v, causal, scale=None):
    import torch
    fa = _fa()
    o, lse = fa.fwd(to_device(q), to_device(k), to_device(v), causal=causal,
                    scale=scale)
    torch.cuda.synchronize()
    return o.to(torch.float64).cpu().numpy(), lse.to(torch.float64).cpu().numpy()


def _case(B, H, N, d, workload, dtype):
    q, k, v = inputs.qkv(B, H, N, d, workload)
    (qt, q64), (kt, k64), (vt, v64) = (host_round(x, dtype) for x in (q, k, v))
    return (qt, kt, vt), (q64, k64, v64)


def _banner(msg):
    print(f"\n[fwd] {msg}", flush=True)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_tiny_workload_full_compare(dtype, causal):
    """B=1, H=2, N=256, d=64 from fp32 N(0,1) inputs."""
    _banner(f"tiny dtype={dtype} causal={causal}")
    (qt, kt, vt), (q64, k64, v64) = _case(1, 2, 256, 64, 1, dtype)
    o, lse = _run(qt, kt, vt, causal)
    o_ref, lse_ref = attention_fwd(q64, k64, v64, causal=causal)
    assert max_abs(o, o_ref) <= O_MAX_ABS
    assert rmse(o, o_ref) <= O_RMSE
    assert max_abs(lse, lse_ref) <= LSE_MAX_ABS
    # Context: the error of the same result against the unrounded fp32 inputs.
    q, k, v = inputs.qkv(1, 2, 256, 64, 1)
    o32, _ = attention_fwd(q, k, v, causal=causal)
    print(f"  rmse vs rounded-input oracle {rmse(o, o_ref):.3e}, "
          f"vs fp32-input oracle {rmse(o, o32):.3e}")


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("N", [1, 17, 129, 255, 300, 1000])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_and_multi_tile(d, N, causal):
    """Several tiles plus a ragged tail, every head dimension."""
    _banner(f"ragged d={d} N={N} causal={causal}")
    (qt, kt, vt), (q64, k64, v64) = _case(2, 3, N, d, 100 + d + N, "bf16")
    o, lse = _run(qt, kt, vt, causal)
    o_ref, lse_ref = attention_fwd(q64, k64, v64, causal=causal)
    assert max_abs(o, o_ref) <= O_MAX_ABS
    assert rmse(o, o_ref) <= O_RMSE
    assert max_abs(lse, lse_ref) <= LSE_MAX_ABS


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_nondefault_scale(dtype):
    _banner(f"scale=0.3 dtype={dtype}")
    (qt, kt, vt), (q64, k64, v64) = _case(1, 2, 384, 128, 7, dtype)
    for causal in (False, True):
        o, lse = _run(qt, kt, vt, causal, scale=0.3)
        o_ref, lse_ref = attention_fwd(q64, k64, v64, causal=causal, scale=0.3)
        assert max_abs(o, o_ref) <= O_MAX_ABS
        assert rmse(o, o_ref) <= O_RMSE
        assert max_abs(lse, lse_ref) <= LSE_MAX_ABS


def _sampled_check(B, H, N, d, workload, causal, dtype="bf16"):
    (qt, kt, vt), (q64, k64, v64) = _case(B, H, N, d, workload, dtype)
    o, lse = _run(qt, kt, vt, causal)
    heads = sorted({(0, 0), (B - 1, H - 1), (B // 2, H // 2)})
    for b, h in heads:
        rows = sample_rows(N, seed=b * 131 + h)
        o_ref, lse_ref = attention_fwd_rows(q64[b, h], k64[b, h], v64[b, h], rows,
                                            causal=causal)
        assert max_abs(o[b, h, rows], o_ref) <= O_MAX_ABS, (b, h)
        assert rmse(o[b, h, rows], o_ref) <= O_RMSE, (b, h)
        assert max_abs(lse[b, h, rows], lse_ref) <= LSE_MAX_ABS, (b, h)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


@pytest.mark.parametrize("B,N", [(8, 2048), (4, 4096), (2, 8192)])
@pytest.mark.parametrize("causal", [False, True])
def test_sweep_full_size_sampled(B, N, causal):
    """B*N = 16384 tokens, H=16, d=128 (the bench shapes)."""
    _banner(f"sweep B={B} N={N} causal={causal}")
    _sampled_check(B, 16, N, 128, 2, causal)


@pytest.mark.parametrize("H,d", [(16, 128), (32, 64), (8, 256)])
def test_long_context_sampled(H, d):
    """B=1, N=16384, causal, three head dimensions."""
    _banner(f"long context H={H} d={d}")
    _sampled_check(1, H, 16384, d, 3, True)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_persistent_grid_later_units_ragged(d, causal):
    """Launches run one workgroup per resident slot (256 on the MI355X), each
    taking several units (non-causal: w, w + G, ...; causal: the
    heaviest-first order) and fetching the next unit's Q rows and first key
    tiles during the current unit's epilogue.  B=1, H=33, N=2000 (ragged)
    gives 264 units of 256 rows at d <= 128 and 528 of 128 rows at d = 256,
    so some workgroups run second (and third) units; heads 4, 16 and 32 hold
    such units at d = 128 non-causal.  Whole heads against the oracle."""
    _banner(f"persistent later units d={d} causal={causal}")
    B, H, N = 1, 33, 2000
    (qt, kt, vt), (q64, k64, v64) = _case(B, H, N, d, 11, "bf16")
    o, lse = _run(qt, kt, vt, causal)
    for h in (0, 4, 16, 32):
        o_ref, lse_ref = attention_fwd(q64[:, h:h + 1], k64[:, h:h + 1], v64[:, h:h + 1],
                                       causal=causal)
        assert max_abs(o[:, h:h + 1], o_ref) <= O_MAX_ABS, h
        assert rmse(o[:, h:h + 1], o_ref) <= O_RMSE, h
        assert max_abs(lse[:, h:h + 1], lse_ref) <= LSE_MAX_ABS, h
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))


# ----------------------------------------------------------- invariants

@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_closed_form(causal):
    """Q = 0: rows are the (prefix) mean of V and LSE = ln(#visible keys)."""
    _banner(f"Q=0 causal={causal}")
    N, d = 777, 128
    _, _, v = inputs.qkv(1, 2, N, d, 11)
    vt, v64 = host_round(v, "bf16")
    qt, _ = host_round(np.zeros_like(v), "bf16")
    kt, _ = host_round(inputs.qkv(1, 2, N, d, 12)[1], "bf16")
    o, lse = _run(qt, kt, vt, causal)
    cnt = np.arange(1, N + 1) if causal else np.full(N, N)
    mean = (np.cumsum(v64, axis=2) / cnt[:, None]) if causal else \
        np.broadcast_to(v64.mean(axis=2, keepdims=True), v64.shape)
    assert max_abs(o, mean) <= 1e-2
    assert max_abs(lse, np.broadcast_to(np.log(cnt), lse.shape)) <= 1e-4


def test_causal_row_zero_is_first_value_row():
    _banner("causal row 0")
    (qt, kt, vt), (q64, k64, v64) = _case(2, 4, 513, 64, 13, "bf16")
    o, lse = _run(qt, kt, vt, True)
    assert max_abs(o[:, :, 0], v64[:, :, 0]) == 0.0
    ref = np.einsum("bhc,bhc->bh", q64[:, :, 0], k64[:, :, 0]) / 8.0
    assert max_abs(lse[:, :, 0], ref) <= 1e-4


def test_outputs_fully_overwritten_and_deterministic():
    """Outputs poisoned with NaN are fully overwritten; repeated launches are
    bitwise identical; the guard region after the outputs is untouched."""
    import torch
    fa = _fa()
    _banner("poison / determinism")
    B, H, N, d = 2, 4, 1000, 128
    (qt, kt, vt), _ = _case(B, H, N, d, 14, "bf16")
    q, k, v = to_device(qt), to_device(kt), to_device(vt)
    n = B * H * N * d
    obuf = torch.full((n + 4096,), float("nan"), dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((B * H * N + 1024,), float("nan"), dtype=torch.float32, device="cuda")
    o = obuf[:n].view(B, H, N, d)
    lse = lbuf[:B * H * N].view(B, H, N)
    first = None
    for causal in (False, True):
        for it in range(5):
            fa.fwd(q, k, v, causal=causal, out=o, lse=lse)
            torch.cuda.synchronize()
            assert not torch.isnan(o).any() and not torch.isnan(lse).any()
            snap = (o.clone(), lse.clone())
            if it == 0:
                first = snap
            else:
                assert torch.equal(snap[0], first[0]) and torch.equal(snap[1], first[1])
        assert torch.isnan(obuf[n:]).all() and torch.isnan(lbuf[B * H * N:]).all()


def test_two_streams_concurrently():
    import torch
    fa = _fa()
    _banner("two streams")
    (qt, kt, vt), (q64, k64, v64) = _case(2, 8, 1024, 128, 15, "bf16")
    q, k, v = to_device(qt), to_device(kt), to_device(vt)
    ref, _ = fa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for s, causal in ((s1, True), (s2, False)):
        with torch.cuda.stream(s):
            outs.append(fa.fwd(q, k, v, causal=causal)[0])
    torch.cuda.synchronize()
    assert torch.equal(outs[0], ref)
    o_ref, _ = attention_fwd(q64[:1, :2], k64[:1, :2], v64[:1, :2], causal=False)
    assert max_abs(outs[1][:1, :2].double().cpu().numpy(), o_ref) <= O_MAX_ABS


# ------------------------------------------------------------ causal schedule

@pytest.mark.parametrize("B,H,N,d", [(2, 16, 8192, 128),   # heads pinned to XCDs, 4 rounds
                                     (3, 7, 4096, 128),    # 21 heads: unpinned, 2 rounds
                                     (1, 5, 3000, 64),     # ragged, one partial round
                                     (2, 9, 2048, 256)])   # 128-row tiles, 18 heads
def test_causal_schedules_agree(B, H, N, d):
    """The persistent heaviest-first causal schedule (the default) and one
    workgroup per query tile (fa_testing_fwd_per_tile) run the same per-tile
    arithmetic, so they must agree bit for bit; every output element must be
    written (outputs start as NaN); sampled rows of the first and last heads
    match the oracle."""
    import torch
    fa = _fa()
    _banner(f"causal schedules B={B} H={H} N={N} d={d}")
    (qt, kt, vt), (q64, k64, v64) = _case(B, H, N, d, 60 + d, "bf16")
    q, k, v = to_device(qt), to_device(kt), to_device(vt)
    res = []
    for sched in (False, True):
        o = torch.full((B, H, N, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
        fa.fwd(q, k, v, causal=True, out=o, lse=lse, per_tile=sched)
        torch.cuda.synchronize()
        assert not torch.isnan(o).any() and not torch.isnan(lse).any(), sched
        res.append((o, lse))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])
    o = res[0][0].to(torch.float64).cpu().numpy()
    lse = res[0][1].to(torch.float64).cpu().numpy()
    for b, h in ((0, 0), (B - 1, H - 1)):
        rows = sample_rows(N, seed=7 * b + h)
        o_ref, lse_ref = attention_fwd_rows(q64[b, h], k64[b, h], v64[b, h], rows, causal=True)
        assert max_abs(o[b, h, rows], o_ref) <= O_MAX_ABS, (b, h)
        assert max_abs(lse[b, h, rows], lse_ref) <= LSE_MAX_ABS, (b, h)
