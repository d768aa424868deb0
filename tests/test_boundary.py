"""C-ABI boundary checks that need no GPU.

* libfa.so loads and exports every function include/fa.h declares;
* the binding's names and argument counts match the header;
* invalid arguments are rejected synchronously with the documented status
  codes (no pointer is dereferenced and nothing is enqueued on these paths,
  so the fake non-null addresses below are never touched).
"""

import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

# A 16-byte-aligned address that is never dereferenced on the error paths.
FAKE = 0x10000


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    decls = {}
    for m in re.finditer(r"\b(?:int|size_t|const char\*)\s+(fa_\w+)\s*\(([^)]*)\)\s*;",
                         text):
        args = [a for a in m.group(2).split(",") if a.strip() and a.strip() != "void"]
        decls[m.group(1)] = len(args)
    return decls


@pytest.fixture(scope="module")
def fa():
    from exact_tiled_attention_16_amd import fa as mod
    if not os.path.exists(mod.LIB_PATH):
        pytest.fail("libfa.so is not built; run `python -m exact_tiled_attention_16_amd.build`")
    mod.lib()
    return mod


def test_header_declares_expected_entry_points():
    d = _declared()
    assert {"fa_fwd", "fa_quant_fp8", "fa_fwd_fp8", "fa_bwd", "fa_bwd_noalloc",
            "fa_bwd_workspace_size", "fa_status_str", "fa_fwd_partial", "fa_merge",
            "fa_splitkv_workspace_size", "fa_fwd_splitkv", "fa_fwd_blocksparse",
            "fa_blocksparse_workspace_size"} <= set(d)


def test_library_exports_every_declared_symbol(fa):
    lib = fa.lib()
    for name, nargs in _declared().items():
        assert hasattr(lib, name), name
        assert name in fa.SIGNATURES, name
        assert len(fa.SIGNATURES[name][1]) == nargs, name


def test_status_strings(fa):
    for code in (fa.FA_OK, fa.FA_ERR_INVALID, fa.FA_ERR_UNSUPPORTED, fa.FA_ERR_LAUNCH,
                 fa.FA_ERR_TOO_LARGE):
        assert fa.status_str(code) and fa.status_str(code) != "unknown status"
    assert fa.status_str(12345) == "unknown status"


def _fwd(fa, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, N=16, d=64,
                dtype=fa.FA_BF16, scale=0.125, causal=0, stream=None)
    args.update(kw)
    return fa.fa_fwd(**args)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(o=None), -1),
    (dict(q=FAKE + 8), -1), (dict(o=FAKE + 2), -1), (dict(lse=FAKE + 2), -1),
    (dict(B=0), -1), (dict(H=-1), -1), (dict(N=0), -1),
    (dict(dtype=2), -1), (dict(scale=0.0), -1), (dict(scale=float("inf")), -1),
    (dict(scale=float("nan")), -1), (dict(scale=-1.0), -1), (dict(causal=2), -1),
    (dict(d=32), -2), (dict(d=96), -2), (dict(d=512), -2),
])
def test_fwd_rejects(fa, kw, code):
    assert _fwd(fa, **kw) == code


def test_quant_fp8_rejects(fa):
    base = dict(x=FAKE, dtype=0, x8=FAKE, scales=FAKE, signs=None, scale_mul=1.0,
                mode=0, B=1, H=1, N=16, d=128, stream=None)
    for kw, code in ((dict(x=None), -1), (dict(x8=None), -1), (dict(scales=None), -1),
                     (dict(N=0), -1), (dict(dtype=5), -1), (dict(mode=3), -1),
                     (dict(mode=-1), -1),
                     (dict(d=100), -2), (dict(x=FAKE + 4), -1), (dict(x8=FAKE + 8), -1),
                     (dict(scale_mul=0.0), -1), (dict(scales=FAKE + 2), -1)):
        a = dict(base)
        a.update(kw)
        assert fa.fa_quant_fp8(**a) == code, kw


def test_fwd_fp8_rejects(fa):
    base = dict(q8=FAKE, k8=FAKE, v8=FAKE, qs=FAKE, ks=FAKE, vs=FAKE, o=FAKE, lse=None,
                B=1, H=1, N=16, d=128, scale=0.1, causal=0, stream=None)
    for kw, code in ((dict(q8=None), -1), (dict(vs=None), -1), (dict(o=None), -1),
                     (dict(H=0), -1), (dict(scale=0.0), -1), (dict(causal=-1), -1),
                     (dict(d=48), -2), (dict(k8=FAKE + 1), -1), (dict(o=FAKE + 8), -1)):
        a = dict(base)
        a.update(kw)
        assert fa.fa_fwd_fp8(**a) == code, kw


def test_bwd_rejects_and_workspace(fa):
    assert fa.fa_bwd_workspace_size(4, 16, 4096, 128) >= 4 * 16 * 4096 * 4
    assert fa.fa_bwd_workspace_size(0, 16, 4096, 128) == 0
    assert fa.fa_bwd_workspace_size(1, 1, 16, 80) == 0
    base = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE,
                dv=FAKE, ws=FAKE, B=1, H=1, N=16, d=128, dtype=0, scale=0.1, causal=1,
                stream=None)
    for kw, code in ((dict(do=None), -1), (dict(lse=None), -1), (dict(ws=None), -1),
                     (dict(dq=None), -1), (dict(N=-5), -1), (dict(dtype=7), -1),
                     (dict(scale=float("nan")), -1), (dict(d=16), -2),
                     (dict(dk=FAKE + 2), -1), (dict(dq=FAKE + 4), -1)):
        a = dict(base)
        a.update(kw)
        assert fa.fa_bwd(**a) == code, kw


def test_bwd_refuses_d256(fa):
    """The backward is built for d = 64 and 128: d = 256 is refused before
    anything is enqueued, and its workspace size is 0 (as include/fa.h
    documents)."""
    assert fa.fa_bwd_workspace_size(1, 1, 256, 256) == 0
    assert fa.fa_bwd_workspace_size(1, 1, 256, 128) > 0
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE,
                dv=FAKE, ws=FAKE, B=1, H=1, N=256, d=256, dtype=0, scale=0.0625, causal=0,
                stream=None)
    assert fa.fa_bwd(**args) == fa.FA_ERR_UNSUPPORTED


def test_internal_per_tile_hook_validates_like_fwd(fa):
    """The per-tile schedule hook (exported, not in the header) shares
    fa_fwd's argument checks."""
    lib = fa.lib()
    assert hasattr(lib, "fa_testing_fwd_per_tile")
    assert "fa_testing_fwd_per_tile" not in _declared()
    base = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, N=16, d=64,
                dtype=fa.FA_BF16, scale=0.125, causal=1, stream=None)
    for kw, code in ((dict(q=None), -1), (dict(N=0), -1), (dict(d=96), -2),
                     (dict(scale=0.0), -1), (dict(causal=3), -1)):
        a = dict(base)
        a.update(kw)
        assert fa.fa_testing_fwd_per_tile(**a) == code, kw


def test_splitkv_entry_points_reject(fa):
    base = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, Nq=4, Nk=100, d=128,
                dtype=0, scale=0.1, causal=1, q_pos0=96, k_pos0=0, stream=None)
    for kw, code in ((dict(q=None), -1), (dict(lse=None), -1), (dict(o=FAKE + 4), -1),
                     (dict(Nq=0), -1), (dict(Nk=-1), -1), (dict(Nk=(1 << 29) + 1), -1),
                     (dict(q_pos0=-1), -1), (dict(k_pos0=(1 << 29) + 1), -1),
                     (dict(causal=3), -1), (dict(scale=0.0), -1), (dict(dtype=4), -1),
                     (dict(d=80), -2)):
        a = dict(base)
        a.update(kw)
        assert fa.fa_fwd_partial(**a) == code, kw
    base = dict(o_parts=FAKE, lse_parts=FAKE, n_parts=3, o=FAKE, lse=None, B=1, H=2, N=16,
                d=64, dtype=0, stream=None)
    for kw, code in ((dict(o_parts=None), -1), (dict(lse_parts=None), -1), (dict(o=None), -1),
                     (dict(n_parts=0), -1), (dict(N=0), -1), (dict(o_parts=FAKE + 4), -1),
                     (dict(lse=FAKE + 1), -1), (dict(dtype=9), -1), (dict(d=100), -2)):
        a = dict(base)
        a.update(kw)
        assert fa.fa_merge(**a) == code, kw
    assert fa.fa_splitkv_workspace_size(2, 4, 1, 128, 8) == 2 * 4 * 1 * 8 * 129 * 4
    assert fa.fa_splitkv_workspace_size(2, 4, 1, 128, 0) == 0
    assert fa.fa_splitkv_workspace_size(2, 4, 1, 96, 8) == 0
    base = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, ws=FAKE, B=1, H=1, Nq=1, Nk=100,
                d=64, dtype=1, scale=0.1, causal=0, n_splits=4, stream=None)
    for kw, code in ((dict(ws=None), -1), (dict(ws=FAKE + 8), -1), (dict(n_splits=0), -1),
                     (dict(Nq=-2), -1), (dict(k=None), -1), (dict(causal=5), -1),
                     (dict(d=512), -2)):
        a = dict(base)
        a.update(kw)
        assert fa.fa_fwd_splitkv(**a) == code, kw


def test_blocksparse_rejects_and_workspace(fa):
    # d=128: 128-row query tiles, 64-key tiles; list = 2 counts + tiles + 6 pad.
    n_qt, stride = 8192 // 128, 8192 // 64 + 8
    assert fa.fa_blocksparse_workspace_size(2, 16, 8192, 128, 0) == 16 * n_qt * stride * 4
    assert fa.fa_blocksparse_workspace_size(2, 16, 8192, 128, 1) == 32 * n_qt * stride * 4
    assert fa.fa_blocksparse_workspace_size(2, 16, 8192, 100, 0) == 0
    assert fa.fa_blocksparse_workspace_size(2, 16, 8192, 128, 2) == 0
    base = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, mask=FAKE, per_batch=0, ws=FAKE,
                B=1, H=2, N=300, d=64, dtype=0, scale=0.1, causal=0, stream=None)
    for kw, code in ((dict(mask=None), -1), (dict(ws=None), -1), (dict(ws=FAKE + 2), -1),
                     (dict(per_batch=2), -1), (dict(N=0), -1), (dict(q=FAKE + 4), -1),
                     (dict(scale=-1.0), -1), (dict(d=96), -2)):
        a = dict(base)
        a.update(kw)
        assert fa.fa_fwd_blocksparse(**a) == code, kw


def test_python_helpers_reject_bad_tensors(fa):
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fwd(q, q, q)  # host tensors are refused before any call
    with pytest.raises(ValueError):
        fa.fwd(torch.zeros(8, 64, dtype=torch.bfloat16), q, q)


def test_clock_probe_library_exports():
    """The bench's clock probe is its own small library (not the C ABI of the
    attention library); it must be built and export its two entry points."""
    import ctypes
    path = os.path.join(ROOT, "exact_tiled_attention_16_amd", "libfa_probe.so")
    if not os.path.exists(path):
        pytest.fail("libfa_probe.so is not built; run `python -m exact_tiled_attention_16_amd.build`")
    lib = ctypes.CDLL(path)
    assert hasattr(lib, "fa_probe_clock") and hasattr(lib, "fa_probe_wall_rate_khz")
    lib.fa_probe_clock.restype = ctypes.c_int
    lib.fa_probe_clock.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p]
    assert lib.fa_probe_clock(None, 100, None) == -1  # rejected before any launch


def test_bwd_noalloc_rejects(fa):
    """The allocation-free backward checks its arguments like fa_bwd and
    refuses problems beyond its fixed scratch, all before touching the
    device."""
    base = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, dq=FAKE, dk=FAKE,
                dv=FAKE, B=1, H=1, N=16, d=128, dtype=0, scale=0.1, causal=1, stream=None)
    rows = fa.BWD_NOALLOC_MAX_ROWS
    for kw, code in ((dict(do=None), -1), (dict(lse=None), -1), (dict(dq=FAKE + 4), -1),
                     (dict(N=0), -1), (dict(dtype=7), -1), (dict(scale=0.0), -1),
                     (dict(d=256), -2), (dict(d=80), -2),
                     (dict(B=1, H=1, N=rows + 1), fa.FA_ERR_TOO_LARGE),
                     (dict(B=16, H=32, N=4097), fa.FA_ERR_TOO_LARGE),
                     (dict(B=rows, H=2, N=1), fa.FA_ERR_TOO_LARGE)):
        a = dict(base)
        a.update(kw)
        assert fa.fa_bwd_noalloc(**a) == code, kw
    assert "fa_bwd_noalloc" in fa.status_str(fa.FA_ERR_TOO_LARGE)
