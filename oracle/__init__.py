"""fp64 CPU oracle for exact tiled attention -- TEST INFRASTRUCTURE ONLY.

This package is the correctness reference that the HIP path is checked against.
It is plain, slow and materialises the full score matrix.  It shares no code,
header, table or constant with the HIP library and imports nothing from it.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call anything in here.  The product path never does.

Sources (the pages this follows):
  * "FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness",
    abstract (citation-hub page): attention is computed *exactly*; tiling only
    changes where intermediates live, not the result.
  * "FlashAttention-3: Fast and Accurate Attention with Asynchrony and
    Low-precision", abstract (pith.science review page): block quantization and
    incoherent processing for FP8.
  * FlashAttention-4 related-papers page, online-softmax snippet: a running
    row maximum and normaliser make the tiled computation exact.

Modules:
  attention  -- materialising forward/backward, a scalar loop version and the
                online-softmax recurrence written out in fp64.
  fp8        -- OCP e4m3 codec, Sylvester Hadamard matrix, fast Walsh-Hadamard
                transform in fp32, block/per-tensor quantiser, fp8 attention
                semantics.
"""

from . import attention, fp8  # noqa: F401
