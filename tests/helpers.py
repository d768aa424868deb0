"""Shared helpers for the parity tests: seeded inputs in the kernel's dtype
(rounded on the host, so the oracle sees exactly the values the device reads)
and error metrics."""

from __future__ import annotations

import numpy as np

TORCH_DTYPES = {}


def torch_dtype(name: str):
    import torch
    return {"bf16": torch.bfloat16, "fp16": torch.float16}[name]


def host_round(x: np.ndarray, dtype: str):
    """fp32 numpy -> CPU torch tensor of the kernel dtype (round to nearest
    even), plus its fp64 numpy widening for the oracle."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch_dtype(dtype))
    return t, t.to(torch.float64).numpy()


def to_device(t):
    return t.to("cuda").contiguous()


def rmse(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.sqrt(np.mean((a - b) ** 2)))


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def sample_rows(N: int, seed: int, extra: int = 24) -> np.ndarray:
    """Tile edges, the ends, the middle and some random rows of [0, N)."""
    fixed = [0, 1, 2, 31, 32, 33, 63, 64, 127, 128, 255, 256, 511, 512,
             N // 2, N - 2, N - 1]
    rnd = np.random.default_rng(seed).integers(0, N, extra)
    rows = np.unique(np.array([r for r in fixed if 0 <= r < N] + list(rnd)))
    return rows.astype(np.int64)
