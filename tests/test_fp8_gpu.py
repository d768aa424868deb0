"""FP8 path parity: fa_quant_fp8 and fa_fwd_fp8 against the oracle.

* The quantiser is an encoding: codes and scales must be bit-exact against the
  oracle's fp32 emulation (same butterfly order, fp32 division, RNE e4m3).
* fa_fwd_fp8 runs on codes and scales produced by the *oracle's* quantiser and
  is compared with exact fp64 attention on the dequantised operands.  The
  device additionally rounds the probabilities to e4m3.  The gate is the RMS
  of the error: at most twice the expected RMS of that rounding
  (oracle.fp8.p_rounding_rms, plus the bf16 output rounding).  The
  elementwise worst-case bound (oracle.fp8.p_rounding_bound, widened by the
  score errors of oracle.fp8.score_error_bound) is checked too, but at long
  sequences it exceeds a typical |O| and discriminates little.  LSE is
  checked per row against oracle.fp8.lse_error_bound: the score errors of
  the e4m3 matrix instruction's accumulation plus fp32 sums, exp2 and log.
* On the outlier-injected workload (B=4, H=16, N=4096, d=128, 0.1 % of
  entries ~ N(0, 10^2)) the block-scaled + rotated path must have a lower
  RMSE than the per-tensor-scaled baseline, both measured end to end on the
  device against the fp64 oracle of the bf16 inputs.
"""

import math

import numpy as np
import pytest

from exact_tiled_attention_16_amd import inputs
from oracle.attention import attention_fwd
from oracle.fp8 import (attention_fwd_fp8, dequantize_fp8, lse_error_bound,
                        p_rounding_bound, p_rounding_rms, quantize_fp8,
                        score_error_bound)
from tests.helpers import host_round, max_abs, rmse, to_device

pytestmark = pytest.mark.gpu


def _fa():
    from exact_tiled_attention_16_amd import fa
    return fa


def _banner(msg):
    print(f"\n[fp8] {msg}", flush=True)


def _dev_quant(xt, signs, scale_mul, per_tensor, pow2=False):
    import torch
    fa = _fa()
    sd = None if signs is None else torch.from_numpy(signs).to("cuda")
    x8, sc = fa.quant_fp8(to_device(xt), signs=sd, scale_mul=scale_mul, per_tensor=per_tensor,
                          pow2=pow2)
    torch.cuda.synchronize()
    return x8.cpu().numpy(), sc.cpu().numpy()


MODES = [  # (label, rotate, scale_mul from d, per_tensor, power-of-two block scales)
    ("q_block_rot", True, True, False, False),
    ("k_block_rot", True, False, False, False),
    ("v_block", False, False, False, False),
    ("v_block_pow2", False, False, False, True),
    ("k_block_rot_pow2", True, False, False, True),
    ("per_tensor", False, False, True, False),
    ("per_tensor_rot", True, False, True, False),
]


@pytest.mark.parametrize("shape", [(2, 3, 300, 64), (1, 2, 1000, 128), (1, 2, 257, 256),
                                   (1, 1, 1, 128), (3, 2, 128, 64)])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_quantiser_bit_exact(shape, dtype):
    B, H, N, d = shape
    x = inputs.qkv_outliers(B, H, N, d, 40 + N)[0].copy()
    # Signed zeros: -0 / scale is -0, code 0x80; a row of zeros of both signs
    # also passes through the rotation's sums and differences.
    x[..., 0, :8] = np.array([-0.0, 0.0] * 4)
    if N > 1:
        x[0, 0, N - 1, :] = np.where(np.arange(d) % 3 == 0, -0.0, 0.0)
    xt, x64 = host_round(x, dtype)
    signs = inputs.signs(d, 40 + N)
    for label, rot, mul_d, pt, p2 in MODES:
        _banner(f"quant {shape} {dtype} {label}")
        sg = signs if rot else None
        mul = 1.0 / d if mul_d else 1.0
        codes, scales = _dev_quant(xt, sg, mul, pt, p2)
        rc, rs = quantize_fp8(x64.astype(np.float32), signs=sg, scale_mul=mul, per_tensor=pt,
                              pow2=p2)
        assert np.array_equal(scales.view(np.uint32), rs.view(np.uint32)), label
        mism = int(np.sum(codes != rc))
        assert mism == 0, (label, mism)


def test_quantiser_bit_exact_full_size():
    """The fp8 workload (B=4, H=16, N=4096, d=128): Q rotated with 1/d folded,
    V with power-of-two block scales."""
    _banner("quant full size")
    B, H, N, d = 4, 16, 4096, 128
    q, _, v = inputs.qkv_outliers(B, H, N, d, 4)
    s = inputs.signs(d, 4)
    for x, sg, mul, p2 in ((q, s, 1.0 / d, False), (v, None, 1.0, True)):
        xt, x64 = host_round(x, "bf16")
        codes, scales = _dev_quant(xt, sg, mul, False, p2)
        rc, rs = quantize_fp8(x64.astype(np.float32), signs=sg, scale_mul=mul, pow2=p2)
        assert np.array_equal(scales.view(np.uint32), rs.view(np.uint32))
        assert int(np.sum(codes != rc)) == 0


def _oracle_operands(B, H, N, d, workload, rotate=True, per_tensor=False, pow2_v=True):
    """Codes and scales from the oracle's quantiser.  V's block scales are
    powers of two by default (the fp8 forward then carries them as exponents
    of its products); pow2_v=False gives arbitrary fp32 block scales, which
    take the forward's rescaling path."""
    q, k, v = inputs.qkv_outliers(B, H, N, d, workload)
    s = inputs.signs(d, workload) if rotate else None
    q64, k64, v64 = (host_round(x, "bf16")[1].astype(np.float32) for x in (q, k, v))
    q8, qs = quantize_fp8(q64, signs=s, scale_mul=1.0 / d if rotate else 1.0,
                          per_tensor=per_tensor)
    k8, ks = quantize_fp8(k64, signs=s, per_tensor=per_tensor)
    v8, vs = quantize_fp8(v64, per_tensor=per_tensor, pow2=pow2_v and not per_tensor)
    return (q8, k8, v8, qs, ks, vs)


def _dev_fwd_fp8(ops, causal):
    import torch
    fa = _fa()
    q8, k8, v8, qs, ks, vs = (torch.from_numpy(np.ascontiguousarray(x)).to("cuda") for x in ops)
    o, lse = fa.fwd_fp8(q8, k8, v8, qs, ks, vs, causal=causal)
    torch.cuda.synchronize()
    return o.to(torch.float64).cpu().numpy(), lse.to(torch.float64).cpu().numpy()


# 1 .. 9 key tiles of 64: the kernel takes tiles in groups of four with one
# barrier per group, and these lengths end the last group after each of its
# positions (and ragged or whole).
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("N", [1, 65, 150, 200, 448, 513])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("pow2_v", [True, False])
def test_fwd_fp8_against_dequantised_oracle(d, N, causal, pow2_v):
    _banner(f"fwd_fp8 d={d} N={N} causal={causal} pow2_v={pow2_v}")
    ops = _oracle_operands(2, 2, N, d, 60 + N + d, pow2_v=pow2_v)
    o, lse = _dev_fwd_fp8(ops, causal)
    o_ref, lse_ref = attention_fwd_fp8(*ops, causal=causal)
    q, k, v = (dequantize_fp8(ops[i], ops[3 + i]) for i in range(3))
    delta = score_error_bound(q, k, causal=causal)
    bound = p_rounding_bound(q, k, v, causal=causal, score_error=delta)
    rms_bound = p_rounding_rms(q, k, v, causal=causal) + 2.0 ** -9 * np.sqrt(np.mean(o_ref ** 2))
    lse_err = np.abs(lse - lse_ref)
    lse_bound = lse_error_bound(q, k, causal=causal, score_error=delta)
    err = np.abs(o - o_ref)
    print(f"  rmse={rmse(o, o_ref):.3e} (RMS gate {2 * rms_bound:.3e}, "
          f"{rmse(o, o_ref) / (2 * rms_bound):.2f} of it) max err/bound="
          f"{float(np.max(err / bound)):.2f} lse_max={lse_err.max():.2e} "
          f"(max err/bound {float(np.max(lse_err / lse_bound)):.3f})")
    assert np.all(err <= bound)
    assert rmse(o, o_ref) <= 2 * rms_bound
    assert np.all(lse_err <= lse_bound)


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_fp8_per_tensor_operands(causal):
    """The per-tensor baseline's operands (one scale per tensor, no
    rotation) through the same kernel, against the oracle on those codes."""
    _banner(f"fwd_fp8 per-tensor operands causal={causal}")
    ops = _oracle_operands(2, 3, 700, 128, 77, rotate=False, per_tensor=True)
    o, lse = _dev_fwd_fp8(ops, causal)
    _check_fp8_heads(ops, o, lse, ((0, 0), (1, 2)), causal, "per-tensor N=700")


def _check_fp8_heads(ops, o, lse, heads, causal, label):
    """Whole heads of a device result against the oracle on the same codes:
    the RMS gate, the elementwise worst-case bound and the LSE."""
    for b, h in heads:
        sub = tuple(x[b:b + 1, h:h + 1] for x in ops)
        o_ref, lse_ref = attention_fwd_fp8(*sub, causal=causal)
        q, k, v = (dequantize_fp8(sub[i], sub[3 + i]) for i in range(3))
        rms_expected = (p_rounding_rms(q, k, v, causal=causal)
                        + 2.0 ** -9 * np.sqrt(np.mean(o_ref ** 2)))
        got = o[b:b + 1, h:h + 1]
        e = rmse(got, o_ref)
        delta = score_error_bound(q, k, causal=causal)
        lse_err = np.abs(lse[b:b + 1, h:h + 1] - lse_ref)
        lse_bound = lse_error_bound(q, k, causal=causal, score_error=delta)
        print(f"  {label} head ({b},{h}): rmse={e:.3e} (RMS gate {2 * rms_expected:.3e}, "
              f"{e / (2 * rms_expected):.2f} of it) "
              f"lse_max={lse_err.max():.2e} (max err/bound {float(np.max(lse_err / lse_bound)):.3f})")
        assert e <= 2 * rms_expected, ("RMS gate", b, h, e, rms_expected)
        assert np.all(np.abs(got - o_ref)
                      <= p_rounding_bound(q, k, v, causal=causal, score_error=delta)), (b, h)
        assert np.all(lse_err <= lse_bound), (b, h)


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_fp8_full_size_sampled_heads(causal):
    """The fp8 workload, B=4, H=16, N=4096, d=128 (outlier inputs), causal
    and not: whole heads against the oracle, with V's block scales powers of
    two (carried as exponents) and arbitrary (O rescaled per block)."""
    _banner(f"fwd_fp8 full size causal={causal}")
    B, H, N, d = 4, 16, 4096, 128
    for pow2_v in (True, False):
        ops = _oracle_operands(B, H, N, d, 4, pow2_v=pow2_v)
        o, lse = _dev_fwd_fp8(ops, causal)
        _check_fp8_heads(ops, o, lse, ((0, 0), (2, 9), (3, 15)), causal,
                         f"B=4 N=4096 pow2_v={pow2_v}")


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_fp8_persistent_grid_later_units_ragged(causal):
    """d = 128 launches run one workgroup per resident slot, each fetching
    its next unit's Q rows and first key tiles during the current unit's
    epilogue.  B=1, H=33, N=2000 (ragged) gives 264 units of 256 rows for
    256 slots, so some workgroups run second units (non-causal: heads 4, 16
    and 32 hold them).  Whole heads against the oracle on the same codes."""
    _banner(f"fwd_fp8 persistent later units causal={causal}")
    ops = _oracle_operands(1, 33, 2000, 128, 12)
    o, lse = _dev_fwd_fp8(ops, causal)
    _check_fp8_heads(ops, o, lse, ((0, 0), (0, 4), (0, 16), (0, 32)), causal, "H=33 N=2000")


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_fp8_bench_shape_sampled_heads(causal):
    """B=2, H=16, N=8192, d=128 (the shape the benchmark times), outlier
    inputs, causal and not: two whole heads against the oracle."""
    _banner(f"fwd_fp8 B=2 N=8192 causal={causal}")
    B, H, N, d = 2, 16, 8192, 128
    ops = _oracle_operands(B, H, N, d, 4)
    o, lse = _dev_fwd_fp8(ops, causal)
    _check_fp8_heads(ops, o, lse, ((0, 3), (1, 14)), causal, "B=2 N=8192")


def test_fp8_error_lower_than_per_tensor_baseline():
    """End to end on the device: block scales + rotation beat per-tensor."""
    import torch
    fa = _fa()
    _banner("fp8 error ordering (B=4, H=16, N=4096, d=128, outliers)")
    B, H, N, d = 4, 16, 4096, 128
    q, k, v = inputs.qkv_outliers(B, H, N, d, 4)
    (qt, q64), (kt, k64), (vt, v64) = (host_round(x, "bf16") for x in (q, k, v))
    qd, kd, vd = (to_device(t) for t in (qt, kt, vt))
    sg = torch.from_numpy(inputs.signs(d, 4)).to("cuda")

    def run(rotate, per_tensor, pow2_v=False):
        s = sg if rotate else None
        q8, qs = fa.quant_fp8(qd, signs=s, scale_mul=1.0 / d if rotate else 1.0,
                              per_tensor=per_tensor)
        k8, ks = fa.quant_fp8(kd, signs=s, per_tensor=per_tensor)
        v8, vs = fa.quant_fp8(vd, per_tensor=per_tensor, pow2=pow2_v)
        o, _ = fa.fwd_fp8(q8, k8, v8, qs, ks, vs)
        torch.cuda.synchronize()
        return o.to(torch.float64).cpu().numpy()

    o_blk = run(True, False, pow2_v=True)
    o_blk32 = run(True, False)
    o_pt = run(False, True)
    o_bf16, _ = fa.fwd(qd, kd, vd)
    o_bf16 = o_bf16.to(torch.float64).cpu().numpy()
    heads = [(0, 0), (1, 5), (2, 10), (3, 15)]
    err = {"block_rot": [], "block_rot_fp32_v": [], "per_tensor": [], "bf16": []}
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref, _ = attention_fwd(q64[sl], k64[sl], v64[sl])
        err["block_rot"].append(np.mean((o_blk[sl] - ref) ** 2))
        err["block_rot_fp32_v"].append(np.mean((o_blk32[sl] - ref) ** 2))
        err["per_tensor"].append(np.mean((o_pt[sl] - ref) ** 2))
        err["bf16"].append(np.mean((o_bf16[sl] - ref) ** 2))
    r = {k_: math.sqrt(np.mean(v_)) for k_, v_ in err.items()}
    print(f"  RMSE block+rotation {r['block_rot']:.3e} (fp32 V block scales "
          f"{r['block_rot_fp32_v']:.3e}), per-tensor {r['per_tensor']:.3e}, "
          f"ratio {r['per_tensor'] / r['block_rot']:.2f}x; bf16 path {r['bf16']:.3e}")
    assert r["block_rot"] < r["per_tensor"]
    assert r["block_rot_fp32_v"] < r["per_tensor"]


@pytest.mark.parametrize("B,H,N,d", [(2, 8, 2048, 128),   # 16 heads: pinned to XCDs
                                     (3, 7, 3000, 128),   # 21 heads: unpinned, ragged
                                     (1, 3, 700, 64),     # fewer units than slots
                                     (1, 5, 1500, 256)])  # one wave per SIMD
def test_causal_persistent_schedule_writes_every_unit(B, H, N, d):
    """The causal fp8 forward runs on a persistent grid that walks the units
    heaviest first; every output element must be written (O and LSE start
    as NaN) and the first and last heads must pass the parity gates."""
    import torch
    fa = _fa()
    _banner(f"fp8 causal persistent B={B} H={H} N={N} d={d}")
    ops = _oracle_operands(B, H, N, d, 90 + N)
    q8, k8, v8, qs, ks, vs = (torch.from_numpy(np.ascontiguousarray(x)).to("cuda") for x in ops)
    o = torch.full((B, H, N, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
    fa.fwd_fp8(q8, k8, v8, qs, ks, vs, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any() and not torch.isnan(lse).any()
    _check_fp8_heads(ops, o.to(torch.float64).cpu().numpy(), lse.to(torch.float64).cpu().numpy(),
                     ((0, 0), (B - 1, H - 1)), True, f"N={N} d={d}")
