"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers; it holds no attention arithmetic.  Both
the HIP path (through tests and the bench) and the fp64 oracle consume what it
returns, so the two sides always see the same values.

Recipe (numpy ``default_rng`` = PCG64):
  * every tensor is ``standard_normal`` in float32 with seed
    ``1000 * workload + index``; index 0 = Q, 1 = K, 2 = V, 3 = dO,
    4 = outlier mask, 5 = outlier values, 6 = rotation signs;
  * outlier injection replaces each entry independently with probability
    ``prob`` by a draw of standard deviation ``std`` (default 0.1 % and 10);
  * rotation signs are +-1 with equal probability.

Workload ids name the five synthetic shapes the library is exercised on:
  1 tiny forward (B=1, H=2, N=256, d=64), 2 bf16 forward sweep (B*N = 16384,
  H=16, d=128), 3 long-context forward (B=1, N=16384, H*d = 2048), 4 fp8
  forward with outliers (B=4, H=16, N=4096, d=128), 5 bf16 backward (B=4,
  H=16, N=4096, d=128, causal).
"""

from __future__ import annotations

import numpy as np

Q, K, V, DO, OUTLIER_MASK, OUTLIER_VALUES, SIGNS = range(7)


def seed_for(workload: int, index: int) -> int:
    return 1000 * int(workload) + int(index)


def normal(shape, seed: int) -> np.ndarray:
    """i.i.d. N(0, 1) float32 array."""
    return np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)


def qkv(B: int, H: int, N: int, d: int, workload: int):
    """(Q, K, V) float32 [B, H, N, d]."""
    shape = (B, H, N, d)
    return tuple(normal(shape, seed_for(workload, i)) for i in (Q, K, V))


def dout(B: int, H: int, N: int, d: int, workload: int) -> np.ndarray:
    """Upstream gradient dO, float32 [B, H, N, d]."""
    return normal((B, H, N, d), seed_for(workload, DO))


def inject_outliers(x: np.ndarray, workload: int, slot: int,
                    prob: float = 1e-3, std: float = 10.0) -> np.ndarray:
    """Copy of ``x`` with a random fraction ``prob`` of entries replaced by
    N(0, std^2) draws.  ``slot`` separates the streams of Q, K and V."""
    rm = np.random.default_rng(seed_for(workload, OUTLIER_MASK) * 16 + slot)
    rv = np.random.default_rng(seed_for(workload, OUTLIER_VALUES) * 16 + slot)
    mask = rm.random(x.shape, dtype=np.float32) < prob
    vals = rv.standard_normal(x.shape, dtype=np.float32) * np.float32(std)
    return np.where(mask, vals, x).astype(np.float32)


def qkv_outliers(B: int, H: int, N: int, d: int, workload: int,
                 prob: float = 1e-3, std: float = 10.0):
    """(Q, K, V) float32 with outliers injected independently in each."""
    q, k, v = qkv(B, H, N, d, workload)
    return (inject_outliers(q, workload, 0, prob, std),
            inject_outliers(k, workload, 1, prob, std),
            inject_outliers(v, workload, 2, prob, std))


def signs(d: int, workload: int) -> np.ndarray:
    """Seeded +-1 float32 vector of length d."""
    r = np.random.default_rng(seed_for(workload, SIGNS))
    return np.where(r.random(d) < 0.5, -1.0, 1.0).astype(np.float32)
