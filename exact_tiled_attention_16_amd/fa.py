"""ctypes binding of libfa.so with the C ABI's entry-point names.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind ``include/fa.h``.  torch provides device memory (tensors) and
the stream (``torch.cuda.current_stream()``); there is no CPU or torch
fallback -- a missing library raises ``OSError``.

Raw entry points (``fa_fwd`` ...) take integers for pointers and streams and
return the status code; the tensor helpers (``fwd`` ...) allocate outputs with
torch, check shapes and raise ``FaError`` on a negative status.
"""

from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

FA_OK = 0
FA_ERR_INVALID = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_LAUNCH = -3
FA_ERR_TOO_LARGE = -4
BWD_NOALLOC_MAX_ROWS = 2097152
FA_BF16 = 0
FA_FP16 = 1
FP8_BLOCK = 128
FA_FP8_BLOCK_SCALES = 0
FA_FP8_TENSOR_SCALE = 1
FA_FP8_BLOCK_POW2 = 2

# Every symbol include/fa.h declares, with (restype, argtypes).
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
SIGNATURES = {
    "fa_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_quant_fp8": (_I, [_P, _I, _P, _P, _P, _F, _I, _I, _I, _I, _I, _P]),
    "fa_fwd_fp8": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F,
                        _I, _P]),
    "fa_bwd_workspace_size": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "fa_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I,
                    _I, _F, _I, _P]),
    "fa_bwd_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I,
                            _I, _I, _F, _I, _P]),
    "fa_fwd_partial": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I,
                            _I, _I, _P]),
    "fa_merge": (_I, [_P, _P, _I, _P, _P, _I, _I, _I, _I, _I, _P]),
    "fa_splitkv_workspace_size": (ctypes.c_size_t, [_I, _I, _I, _I, _I]),
    "fa_fwd_splitkv": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F,
                            _I, _I, _P]),
    "fa_blocksparse_workspace_size": (ctypes.c_size_t, [_I, _I, _I, _I, _I]),
    "fa_fwd_blocksparse": (_I, [_P, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I,
                                _F, _I, _P]),
    "fa_status_str": (ctypes.c_char_p, [_I]),
}
# Exported by libfa.so but not part of the C ABI (no declaration in
# include/): fa_fwd with the causal work dispatched as one workgroup per query
# tile instead of the persistent schedule, for comparing the two.
INTERNAL_SIGNATURES = {
    "fa_testing_fwd_per_tile": SIGNATURES["fa_fwd"],
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libfa.so once; raise if it is missing (build it first)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OSError(f"{LIB_PATH} is missing; run "
                          "`python -m exact_tiled_attention_16_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in {**SIGNATURES, **INTERNAL_SIGNATURES}.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


class FaError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"{status_str(code)} (status {code})")
        self.code = code


def status_str(code: int) -> str:
    return lib().fa_status_str(int(code)).decode()


def _check(code: int) -> None:
    if code != FA_OK:
        raise FaError(code)


# ------------------------------------------------------------ raw entry points

def fa_fwd(q, k, v, o, lse, B, H, N, d, dtype, scale, causal, stream) -> int:
    return lib().fa_fwd(q, k, v, o, lse, B, H, N, d, dtype, scale, causal,
                        stream)


def fa_testing_fwd_per_tile(q, k, v, o, lse, B, H, N, d, dtype, scale, causal,
                            stream) -> int:
    return lib().fa_testing_fwd_per_tile(q, k, v, o, lse, B, H, N, d, dtype,
                                         scale, causal, stream)


def fa_quant_fp8(x, dtype, x8, scales, signs, scale_mul, mode, B, H, N, d,
                 stream) -> int:
    return lib().fa_quant_fp8(x, dtype, x8, scales, signs, scale_mul, mode, B,
                              H, N, d, stream)


def fa_fwd_fp8(q8, k8, v8, qs, ks, vs, o, lse, B, H, N, d, scale, causal,
               stream) -> int:
    return lib().fa_fwd_fp8(q8, k8, v8, qs, ks, vs, o, lse, B, H, N, d,
                            scale, causal, stream)


def fa_bwd_workspace_size(B, H, N, d) -> int:
    return lib().fa_bwd_workspace_size(B, H, N, d)


def fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, B, H, N, d, dtype, scale,
           causal, stream) -> int:
    return lib().fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, B, H, N, d,
                        dtype, scale, causal, stream)


def fa_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, B, H, N, d, dtype, scale,
                   causal, stream) -> int:
    return lib().fa_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, B, H, N, d,
                                dtype, scale, causal, stream)


def fa_fwd_partial(q, k, v, o, lse, B, H, Nq, Nk, d, dtype, scale, causal,
                   q_pos0, k_pos0, stream) -> int:
    return lib().fa_fwd_partial(q, k, v, o, lse, B, H, Nq, Nk, d, dtype, scale,
                                causal, q_pos0, k_pos0, stream)


def fa_merge(o_parts, lse_parts, n_parts, o, lse, B, H, N, d, dtype,
             stream) -> int:
    return lib().fa_merge(o_parts, lse_parts, n_parts, o, lse, B, H, N, d,
                          dtype, stream)


def fa_splitkv_workspace_size(B, H, Nq, d, n_splits) -> int:
    return lib().fa_splitkv_workspace_size(B, H, Nq, d, n_splits)


def fa_fwd_splitkv(q, k, v, o, lse, ws, B, H, Nq, Nk, d, dtype, scale, causal,
                   n_splits, stream) -> int:
    return lib().fa_fwd_splitkv(q, k, v, o, lse, ws, B, H, Nq, Nk, d, dtype,
                                scale, causal, n_splits, stream)


def fa_blocksparse_workspace_size(B, H, N, d, mask_per_batch) -> int:
    return lib().fa_blocksparse_workspace_size(B, H, N, d, mask_per_batch)


def fa_fwd_blocksparse(q, k, v, o, lse, mask, per_batch, ws, B, H, N, d, dtype,
                       scale, causal, stream) -> int:
    return lib().fa_fwd_blocksparse(q, k, v, o, lse, mask, per_batch, ws, B, H,
                                    N, d, dtype, scale, causal, stream)


# ------------------------------------------------------------ tensor helpers

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float16:
        return FA_FP16
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float16")


def _check_tensor(t, name, shape=None, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _stream(t) -> int:
    return _torch().cuda.current_stream(t.device).cuda_stream


def fwd(q, k, v, causal: bool = False, scale: float | None = None,
        out=None, lse=None, per_tile: bool = False):
    """O, LSE = attention(q, k, v) for [B, H, N, d] bf16/fp16 device tensors.

    per_tile=True dispatches causal work as one workgroup per query tile
    (fa_testing_fwd_per_tile) instead of the persistent schedule; the outputs
    are the same bit for bit."""
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(t, name, (B, H, N, d), q.dtype)
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _check_tensor(out, "out", (B, H, N, d), q.dtype)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_tensor(lse, "lse", (B, H, N), torch.float32)
    entry = fa_testing_fwd_per_tile if per_tile else fa_fwd
    _check(entry(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                 lse.data_ptr(), B, H, N, d, dt, float(scale), int(bool(causal)),
                 _stream(q)))
    return out, lse


def bwd(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None,
        dq=None, dk=None, dv=None, workspace=None):
    """(dQ fp32, dK, dV) of <dout, attention(q, k, v)> given the forward's O and
    LSE; q, k, v, o, dout are [B, H, N, d] bf16/fp16 device tensors."""
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_tensor(t, name, (B, H, N, d), q.dtype)
    _check_tensor(lse, "lse", (B, H, N), torch.float32)
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if dq is None:
        dq = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
    if dk is None:
        dk = torch.empty_like(k)
    if dv is None:
        dv = torch.empty_like(v)
    _check_tensor(dq, "dq", (B, H, N, d), torch.float32)
    _check_tensor(dk, "dk", (B, H, N, d), q.dtype)
    _check_tensor(dv, "dv", (B, H, N, d), q.dtype)
    need = fa_bwd_workspace_size(B, H, N, d)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=q.device)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    _check(fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                  dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                  dv.data_ptr(), workspace.data_ptr(), B, H, N, d, dt, float(scale),
                  int(bool(causal)), _stream(q)))
    return dq, dk, dv


def quant_fp8(x, signs=None, scale_mul: float = 1.0, per_tensor: bool = False,
              out=None, scales=None, pow2: bool = False):
    """e4m3 codes (uint8 [B,H,N,d]) and block scales (float32 [B,H,ceil(N/128)])
    of a bf16/fp16 device tensor; ``signs`` (float32 device tensor of d +-1
    values) turns on the Hadamard rotation; ``per_tensor`` uses one scale for
    the tensor, ``pow2`` rounds the block scales up to powers of two."""
    if per_tensor and pow2:
        raise ValueError("pow2 is a block-scale option")
    mode = (FA_FP8_TENSOR_SCALE if per_tensor
            else FA_FP8_BLOCK_POW2 if pow2 else FA_FP8_BLOCK_SCALES)
    torch = _torch()
    if x.dim() != 4:
        raise ValueError("x must be [B, H, N, d]")
    B, H, N, d = x.shape
    _check_tensor(x, "x", (B, H, N, d), x.dtype)
    dt = _dtype_code(x)
    nblk = -(-N // FP8_BLOCK)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((B, H, nblk), dtype=torch.float32, device=x.device)
    _check_tensor(out, "out", (B, H, N, d), torch.uint8)
    _check_tensor(scales, "scales", (B, H, nblk), torch.float32)
    sp = None
    if signs is not None:
        _check_tensor(signs, "signs", (d,), torch.float32)
        sp = signs.data_ptr()
    _check(fa_quant_fp8(x.data_ptr(), dt, out.data_ptr(), scales.data_ptr(), sp,
                        float(scale_mul), mode, B, H, N, d, _stream(x)))
    return out, scales


def fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, causal: bool = False,
            scale: float | None = None, out=None, lse=None):
    """O (bf16) and LSE of attention on e4m3 operands from ``quant_fp8``."""
    torch = _torch()
    if q8.dim() != 4:
        raise ValueError("q8 must be [B, H, N, d]")
    B, H, N, d = q8.shape
    nblk = -(-N // FP8_BLOCK)
    for name, t in (("q8", q8), ("k8", k8), ("v8", v8)):
        _check_tensor(t, name, (B, H, N, d), torch.uint8)
    for name, t in (("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)):
        _check_tensor(t, name, (B, H, nblk), torch.float32)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    _check_tensor(out, "out", (B, H, N, d), torch.bfloat16)
    _check_tensor(lse, "lse", (B, H, N), torch.float32)
    _check(fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), q_scale.data_ptr(),
                      k_scale.data_ptr(), v_scale.data_ptr(), out.data_ptr(), lse.data_ptr(),
                      B, H, N, d, float(scale), int(bool(causal)), _stream(q8)))
    return out, lse


def _qkv_shapes(q, k, v):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    _check_tensor(q, "q", (B, H, Nq, d))
    for name, t in (("k", k), ("v", v)):
        _check_tensor(t, name, (B, H, Nk, d), q.dtype)
    return B, H, Nq, Nk, d


def fwd_partial(q, k, v, causal: bool = False, scale: float | None = None,
                q_pos0: int = 0, k_pos0: int = 0, out=None, lse=None):
    """Attention of q [B, H, Nq, d] over one key/value part k, v
    [B, H, Nk, d]: (O_p fp32 normalised over the part, L_p fp32 log-sum-exp,
    -inf where no key is visible).  Causal positions: query i at q_pos0 + i,
    key j at k_pos0 + j."""
    torch = _torch()
    B, H, Nq, Nk, d = _qkv_shapes(q, k, v)
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=torch.float32, device=q.device)
    _check_tensor(out, "out", (B, H, Nq, d), torch.float32)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check_tensor(lse, "lse", (B, H, Nq), torch.float32)
    _check(fa_fwd_partial(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                          out.data_ptr(), lse.data_ptr(), B, H, Nq, Nk, d, dt,
                          float(scale), int(bool(causal)), int(q_pos0),
                          int(k_pos0), _stream(q)))
    return out, lse


def merge(o_parts, lse_parts, dtype=None, out=None, lse=None):
    """Log-sum-exp merge of partial results: o_parts [S, B, H, N, d] fp32,
    lse_parts [S, B, H, N] fp32 -> (O [B, H, N, d] in `dtype` (bf16 by
    default), LSE [B, H, N] fp32)."""
    torch = _torch()
    if o_parts.dim() != 5:
        raise ValueError("o_parts must be [S, B, H, N, d]")
    S, B, H, N, d = o_parts.shape
    _check_tensor(o_parts, "o_parts", (S, B, H, N, d), torch.float32)
    _check_tensor(lse_parts, "lse_parts", (S, B, H, N), torch.float32)
    dtype = dtype or (out.dtype if out is not None else torch.bfloat16)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=dtype, device=o_parts.device)
    _check_tensor(out, "out", (B, H, N, d), dtype)
    dt = _dtype_code(out)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=o_parts.device)
    _check_tensor(lse, "lse", (B, H, N), torch.float32)
    _check(fa_merge(o_parts.data_ptr(), lse_parts.data_ptr(), S, out.data_ptr(),
                    lse.data_ptr(), B, H, N, d, dt, _stream(o_parts)))
    return out, lse


def fwd_splitkv(q, k, v, n_splits: int, causal: bool = False,
                scale: float | None = None, out=None, lse=None, workspace=None):
    """Attention of q [B, H, Nq, d] over k, v [B, H, Nk, d] with the keys in
    up to n_splits parts run in parallel and merged.  Causal aligns the
    queries with the last Nq keys."""
    torch = _torch()
    B, H, Nq, Nk, d = _qkv_shapes(q, k, v)
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=q.dtype, device=q.device)
    _check_tensor(out, "out", (B, H, Nq, d), q.dtype)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check_tensor(lse, "lse", (B, H, Nq), torch.float32)
    need = fa_splitkv_workspace_size(B, H, Nq, d, n_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    _check(fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                          out.data_ptr(), lse.data_ptr(), workspace.data_ptr(),
                          B, H, Nq, Nk, d, dt, float(scale), int(bool(causal)),
                          int(n_splits), _stream(q)))
    return out, lse


SPARSE_BLOCK = 128


def fwd_blocksparse(q, k, v, block_mask, causal: bool = False,
                    scale: float | None = None, out=None, lse=None,
                    workspace=None):
    """Block-sparse attention of [B, H, N, d] bf16/fp16 device tensors:
    block_mask is a uint8 (or bool) device tensor [H, nb, nb] (shared by the
    batch) or [B, H, nb, nb], nb = ceil(N / 128); nonzero = the 128-row
    query block attends to the 128-key block."""
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(t, name, (B, H, N, d), q.dtype)
    nb = -(-N // SPARSE_BLOCK)
    if block_mask.dtype == torch.bool:
        block_mask = block_mask.to(torch.uint8)
    per_batch = 1 if block_mask.dim() == 4 else 0
    shape = (B, H, nb, nb) if per_batch else (H, nb, nb)
    _check_tensor(block_mask, "block_mask", shape, torch.uint8)
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _check_tensor(out, "out", (B, H, N, d), q.dtype)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_tensor(lse, "lse", (B, H, N), torch.float32)
    need = fa_blocksparse_workspace_size(B, H, N, d, per_batch)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace needs {need} bytes")
    _check(fa_fwd_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                              out.data_ptr(), lse.data_ptr(), block_mask.data_ptr(),
                              per_batch, workspace.data_ptr(), B, H, N, d, dt,
                              float(scale), int(bool(causal)), _stream(q)))
    return out, lse
