"""Exact tiled attention (FlashAttention forward, backward and FP8 forward)
for AMD Instinct MI355X (gfx950).

The compute lives in ``libfa.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/fa.h``).  ``exact_tiled_attention_16_amd.fa`` is a thin
ctypes binding with the same entry-point names; torch supplies device memory
and streams only.  The library is loaded on first use and a missing or
unloadable library raises -- there is no fallback path.

Submodules are imported explicitly: ``from exact_tiled_attention_16_amd import
fa`` (the binding) or ``... import inputs`` (seeded synthetic workloads).
"""
