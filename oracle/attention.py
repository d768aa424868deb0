"""Exact softmax attention in fp64 -- oracle, TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module.  It shares nothing with the HIP library.

What is computed (the plain definition the tiled method reaches exactly):

    S = scale * Q K^T                 (N x N per batch b and head h)
    causal: S[i, j] = -inf for j > i  (top-left aligned, N_q = N_k)
    m_i = max_j S[i, j];  E = exp(S - m);  l_i = sum_j E[i, j];  P = E / l
    O = P V;   LSE_i = m_i + ln l_i

FlashAttention (IO-Awareness paper, abstract on the citation-hub page) is an
*exact* attention algorithm: tiling moves data between HBM and on-chip memory
but does not change the result, so the oracle is the definition itself.  The
log-sum-exp output and the backward by recomputation are not spelled out on the
pages; LSE is the natural log of the softmax normaliser (scale included), and
the gradients below are the derivative of <dO, O> (softmax Jacobian):

    D_i = sum_c dO[i, c] O[i, c]
    dV = P^T dO;  dP = dO V^T;  dS = P * (dP - D 1^T)
    dQ = scale * dS K;  dK = scale * dS^T Q

The online-softmax recurrence (``attention_fwd_online``) follows the running
maximum / running normaliser description on the FlashAttention-4
related-papers page (online-softmax snippet) and the rescaling of the output
accumulator named in the FlashAttention-3 Appendix B fragment (exp2, row_sum
and O rescaling).  It is written out here only so that tests can check that
the recurrence reaches the materialising result; the GPU does not use it.

Split-KV (``attention_fwd_positions``, ``merge_partials``): attention of
N_q queries over N_k keys at explicit positions -- query i at q_pos0 + i, key
j at k_pos0 + j, the key visible under the causal mask iff its position is
not after the query's -- is the same definition with that mask; a row that
sees no key has no softmax, and is given O = 0 and LSE = -inf (the identity
element of the merge below).  Partial results over parts of the keys combine
as L = ln sum_p exp(L_p), O = sum_p exp(L_p - L) O_p: the online softmax's
rescaling (FlashAttention-4 related-papers page, online-softmax snippet)
applied across parts, which Ring Attention and Lean Attention (reference list
of the FlashAttention-3 page) use to combine per-device and per-split
results.  The merge is checked against the definition over all keys.

Block-sparse (``attention_fwd_blockmask``): FlashAttention extends to
block-sparse attention (IO-Awareness paper, abstract on the citation-hub
page).  The pages give no block size or mask format; the reading taken here:
the N x N scores are cut into blocks of `block` query rows by `block` keys and
query i may attend to key j only where the block mask is nonzero at
(i // block, j // block) (and j <= i when causal).  That is the same
definition with that mask; rows that see no key get O = 0, LSE = -inf.

All arrays are [B, H, N, d]; inputs of any float dtype are widened to fp64.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "attention_fwd",
    "attention_fwd_blockmask",
    "attention_fwd_positions",
    "attention_fwd_positions_rows",
    "merge_partials",
    "attention_bwd",
    "attention_fwd_loops",
    "attention_fwd_online",
    "attention_fwd_rows",
    "default_scale",
    "grad_rounding_bound",
]


def default_scale(d: int) -> float:
    """Softmax scale 1/sqrt(d), the standard scaled dot-product choice."""
    return 1.0 / math.sqrt(d)


def _as64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _scores(qb: np.ndarray, k: np.ndarray, scale: float, row0: int,
            causal: bool) -> np.ndarray:
    """Scaled scores of query rows [row0, row0+len(qb)) against all keys."""
    s = (qb @ k.T) * scale
    if causal:
        rows = np.arange(row0, row0 + qb.shape[0])[:, None]
        cols = np.arange(k.shape[0])[None, :]
        s = np.where(cols > rows, -np.inf, s)
    return s


def _softmax_rows(s: np.ndarray):
    """Row softmax of a score block; returns (P, m, l)."""
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    return e / l[:, None], m, l


def attention_fwd(q, k, v, causal: bool = False, scale: float | None = None,
                  row_block: int = 1024):
    """Materialising forward.  Returns (O [B,H,N,d] fp64, LSE [B,H,N] fp64).

    Scores are built ``row_block`` query rows at a time to bound memory; each
    block holds the complete rows of S, so this is still the plain definition.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, N, d = q.shape
    if scale is None:
        scale = default_scale(d)
    o = np.empty_like(q)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, row_block):
                r1 = min(N, r0 + row_block)
                s = _scores(q[b, h, r0:r1], k[b, h], scale, r0, causal)
                p, m, l = _softmax_rows(s)
                o[b, h, r0:r1] = p @ v[b, h]
                lse[b, h, r0:r1] = m + np.log(l)
    return o, lse


def attention_fwd_rows(q, k, v, rows, causal: bool = False,
                       scale: float | None = None):
    """Forward for selected query rows of one head: q,k,v are [N, d].

    Used to check full-size outputs at sampled rows.  Returns (O [len(rows), d],
    LSE [len(rows)]) in fp64.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    d = q.shape[1]
    if scale is None:
        scale = default_scale(d)
    rows = np.asarray(rows, dtype=np.int64)
    s = (q[rows] @ k.T) * scale
    if causal:
        cols = np.arange(k.shape[0])[None, :]
        s = np.where(cols > rows[:, None], -np.inf, s)
    p, m, l = _softmax_rows(s)
    return p @ v, m + np.log(l)


def attention_bwd(q, k, v, do, causal: bool = False,
                  scale: float | None = None, row_block: int = 1024):
    """Materialising backward.  Returns (dQ, dK, dV), each [B,H,N,d] fp64.

    Recomputes P from the definition (not from any saved tiled state) and
    applies the softmax-Jacobian formulas in the module docstring.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    B, H, N, d = q.shape
    if scale is None:
        scale = default_scale(d)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            kb, vb = k[b, h], v[b, h]
            for r0 in range(0, N, row_block):
                r1 = min(N, r0 + row_block)
                qb, dob = q[b, h, r0:r1], do[b, h, r0:r1]
                s = _scores(qb, kb, scale, r0, causal)
                p, _, _ = _softmax_rows(s)
                ob = p @ vb
                dd = (dob * ob).sum(axis=1)
                dv[b, h] += p.T @ dob
                dp = dob @ vb.T
                ds = p * (dp - dd[:, None])
                dq[b, h, r0:r1] = scale * (ds @ kb)
                dk[b, h] += scale * (ds.T @ qb)
    return dq, dk, dv


def attention_fwd_loops(q, k, v, causal: bool = False,
                        scale: float | None = None):
    """Scalar triple loop over (query, key, channel); for N <= 16 only.

    Written with no vector operations so that a reader can check it against the
    definition term by term.  Used to pin the vectorised ``attention_fwd``.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, N, d = q.shape
    if scale is None:
        scale = default_scale(d)
    o = np.zeros_like(q)
    lse = np.zeros((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for i in range(N):
                scores = []
                for j in range(N):
                    if causal and j > i:
                        continue
                    dot = 0.0
                    for c in range(d):
                        dot += q[b, h, i, c] * k[b, h, j, c]
                    scores.append((j, scale * dot))
                mx = max(s for _, s in scores)
                total = 0.0
                for _, s in scores:
                    total += math.exp(s - mx)
                for j, s in scores:
                    w = math.exp(s - mx) / total
                    for c in range(d):
                        o[b, h, i, c] += w * v[b, h, j, c]
                lse[b, h, i] = mx + math.log(total)
    return o, lse


def attention_fwd_online(q, k, v, causal: bool = False,
                         scale: float | None = None, key_tile: int = 64,
                         base2: bool = False):
    """The online-softmax recurrence over key tiles, in fp64.

    Keeps, per query row, a running maximum m, a running normaliser l and an
    unnormalised output accumulator A; each key tile raises m if needed,
    rescales l and A by exp(m_old - m_new), and adds its own exponentials.
    ``base2`` runs the same recurrence with exp2 on scores pre-multiplied by
    log2(e) (the exp2 form named in the FlashAttention-3 Appendix B fragment);
    LSE is then ln2 * m2 + ln l.  A tile whose visible scores are all -inf
    leaves the state untouched, so no NaN can arise.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, N, d = q.shape
    if scale is None:
        scale = default_scale(d)
    mult = scale * (1.0 / math.log(2.0) if base2 else 1.0)
    expf = np.exp2 if base2 else np.exp
    o = np.empty_like(q)
    lse = np.empty((B, H, N), dtype=np.float64)
    rows = np.arange(N)[:, None]
    for b in range(B):
        for h in range(H):
            m = np.full(N, -np.inf)
            l = np.zeros(N)
            acc = np.zeros((N, d))
            for j0 in range(0, N, key_tile):
                j1 = min(N, j0 + key_tile)
                s = (q[b, h] @ k[b, h, j0:j1].T) * mult
                if causal:
                    cols = np.arange(j0, j1)[None, :]
                    s = np.where(cols > rows, -np.inf, s)
                m_new = np.maximum(m, s.max(axis=1))
                live = np.isfinite(m_new)
                alpha = np.zeros(N)
                alpha[live] = expf(m[live] - m_new[live])
                p = np.zeros_like(s)
                p[live] = expf(s[live] - m_new[live, None])
                l = alpha * l + p.sum(axis=1)
                acc = alpha[:, None] * acc + p @ v[b, h, j0:j1]
                m = m_new
            o[b, h] = acc / l[:, None]
            lse[b, h] = (m * math.log(2.0) if base2 else m) + np.log(l)
    return o, lse


def _positions_block(qb, k, v, scale, qpos, kpos, causal):
    """(O, LSE) of query rows at positions qpos against all keys k, v."""
    s = (qb @ k.T) * scale
    if causal:
        s = np.where(kpos[None, :] > qpos[:, None], -np.inf, s)
    m = s.max(axis=1)
    empty = ~np.isfinite(m)          # every key masked (or no key at all)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(s - m_safe[:, None])  # exp(-inf) = 0 for masked keys
    l = e.sum(axis=1)
    l_safe = np.where(empty, 1.0, l)
    o = (e / l_safe[:, None]) @ v
    o[empty] = 0.0
    lse = np.where(empty, -np.inf, m_safe + np.log(l_safe))
    return o, lse


def attention_fwd_positions(q, k, v, causal: bool = False,
                            scale: float | None = None, q_pos0: int = 0,
                            k_pos0: int = 0, row_block: int = 1024):
    """Attention of q [B,H,Nq,d] over k, v [B,H,Nk,d] with query i at
    position q_pos0 + i and key j at k_pos0 + j (causal: visible iff
    k_pos0 + j <= q_pos0 + i).  Rows that see no key: O = 0, LSE = -inf.
    Returns (O [B,H,Nq,d], LSE [B,H,Nq]) in fp64."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = default_scale(d)
    kpos = k_pos0 + np.arange(Nk)
    o = np.empty_like(q)
    lse = np.empty((B, H, Nq), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, Nq, row_block):
                r1 = min(Nq, r0 + row_block)
                qpos = q_pos0 + np.arange(r0, r1)
                o[b, h, r0:r1], lse[b, h, r0:r1] = _positions_block(
                    q[b, h, r0:r1], k[b, h], v[b, h], scale, qpos, kpos, causal)
    return o, lse


def attention_fwd_positions_rows(q, k, v, rows, causal: bool = False,
                                 scale: float | None = None, q_pos0: int = 0,
                                 k_pos0: int = 0):
    """``attention_fwd_positions`` for selected query rows of one head
    (q [Nq, d], k, v [Nk, d]).  Returns (O [len(rows), d], LSE [len(rows)])."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    if scale is None:
        scale = default_scale(q.shape[1])
    rows = np.asarray(rows, dtype=np.int64)
    kpos = k_pos0 + np.arange(k.shape[0])
    return _positions_block(q[rows], k, v, scale, q_pos0 + rows, kpos, causal)


def merge_partials(o_parts, lse_parts):
    """Combine partial attention results over parts of the keys.

    o_parts [S, ..., d] (each part's O, normalised over its keys), lse_parts
    [S, ...] (each part's LSE, -inf for a part that row cannot see):
        L = ln sum_p exp(L_p),   O = sum_p exp(L_p - L) O_p.
    Parts with L_p = -inf get weight 0 and their O_p is not read; a row with
    every L_p = -inf gets O = 0, L = -inf.  Returns (O, L) in fp64."""
    o_parts, lse_parts = _as64(o_parts), _as64(lse_parts)
    m = lse_parts.max(axis=0)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(lse_parts - m_safe[None])            # 0 for empty parts
    wsum = w.sum(axis=0)
    contrib = np.where((w > 0)[..., None], o_parts, 0.0) * w[..., None]
    o = contrib.sum(axis=0) / np.where(empty, 1.0, wsum)[..., None]
    o[empty] = 0.0
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, wsum)))
    return o, lse


def attention_fwd_blockmask(q, k, v, block_mask, block: int = 128,
                            causal: bool = False, scale: float | None = None,
                            rows=None):
    """Block-sparse attention: q, k, v [B,H,N,d]; block_mask [H,nb,nb]
    (shared by the batch) or [B,H,nb,nb], nb = ceil(N / block), nonzero =
    the query block attends to the key block.  Rows that see no key: O = 0,
    LSE = -inf.  `rows` (optional) restricts the output to those query rows
    of every head.  Returns (O [B,H,R,d], LSE [B,H,R]) in fp64."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, H, N, d = q.shape
    if scale is None:
        scale = default_scale(d)
    bm = np.asarray(block_mask) != 0
    if bm.ndim == 3:
        bm = np.broadcast_to(bm[None], (B,) + bm.shape)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    cols = np.arange(N)
    o = np.empty((B, H, len(rows), d))
    lse = np.empty((B, H, len(rows)))
    for b in range(B):
        for h in range(H):
            allowed = bm[b, h][rows[:, None] // block, cols[None, :] // block]
            if causal:
                allowed = allowed & (cols[None, :] <= rows[:, None])
            s = (q[b, h, rows] @ k[b, h].T) * scale
            s = np.where(allowed, s, -np.inf)
            m = s.max(axis=1)
            empty = ~np.isfinite(m)
            m_safe = np.where(empty, 0.0, m)
            e = np.exp(s - m_safe[:, None])
            l = e.sum(axis=1)
            l_safe = np.where(empty, 1.0, l)
            o[b, h] = (e / l_safe[:, None]) @ v[b, h]
            o[b, h][empty] = 0.0
            lse[b, h] = np.where(empty, -np.inf, m_safe + np.log(l_safe))
    return o, lse


def grad_rounding_bound(q, k, v, do, causal: bool = False,
                        scale: float | None = None, dtype: str = "bf16"):
    """Elementwise bound on |gradient_device - gradient_exact| for a backward
    by recomputation that rounds as follows (the device's arithmetic; the
    pages do not describe the backward, so this is the reading it is held
    to): scores, the log-sum-exp, D and all products accumulate in fp32 over
    inputs of the 16-bit type; the rebuilt probabilities P and the products
    dS = P o (dP - D) are rounded to the 16-bit type before they enter
    matrix products; D is formed from the forward's stored O (itself the
    result of a forward that rounds P and O to the 16-bit type); dK and dV
    are rounded to the 16-bit type at the end, dQ stays fp32.

    Rounding x to the 16-bit type errs by at most u |x| + eta: u = 2^-8
    (bf16) or 2^-11 (fp16) for normal values, and eta = half the smallest
    subnormal, 2^-134 (bf16) or 2^-25 (fp16), where the value falls into the
    subnormal range or flushes to zero (small probabilities in fp16 do).

    Arguments as for ``attention_bwd`` (the 16-bit values, widened).
    Returns (bound_dQ, bound_dK, bound_dV), each [B,H,N,d] fp64.  First-order
    worst case: every rounding error takes its largest magnitude and the
    same sign, so at long sequences the bound is far above the typical
    error (the relative Frobenius error is the sharper test).  A sum of n
    fp32 terms is charged n 2^-24 times the sum of their magnitudes.
    """
    u, eta = {"bf16": (2.0 ** -8, 2.0 ** -134), "fp16": (2.0 ** -11, 2.0 ** -25)}[dtype]
    return _grad_rounding_bound(q, k, v, do, causal, scale, u, eta)


def _grad_rounding_bound(q, k, v, do, causal, scale, u, eta):
    """grad_rounding_bound with the rounding constants given: relative
    error u for normal values, absolute error eta where values underflow."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    B, H, N, d = q.shape
    if scale is None:
        scale = default_scale(d)
    f32 = 2.0 ** -24
    g_d = d * f32          # sums over the head dimension
    g_n = (N + 2) * f32    # sums over queries or keys
    bq, bk, bv = (np.zeros_like(x) for x in (q, k, v))
    for b in range(B):
        for h in range(H):
            Q, K, V, dO = q[b, h], k[b, h], v[b, h], do[b, h]
            s = _scores(Q, K, scale, 0, causal)
            p, _, _ = _softmax_rows(s)
            vis = np.isfinite(s)
            o = p @ V
            # Absolute error of the rounded probability: fp32 scores and
            # log-sum-exp (a relative error), then the rounding.
            e_s = g_d * scale * (np.abs(Q) @ np.abs(K).T)
            e_lse = g_n + np.max(np.where(vis, e_s, 0.0), axis=1, keepdims=True)
            a = np.expm1(e_s + e_lse)
            e_p = np.where(vis, (a + u + a * u) * p + eta, 0.0)
            # The forward's stored O: rounded P, fp32 sums, O rounded.
            e_o = (np.where(vis, u * p + eta, 0.0) + g_n * p) @ np.abs(V) \
                + u * np.abs(o) + eta
            dd = (dO * o).sum(axis=1, keepdims=True)
            e_dd = (np.abs(dO) * e_o).sum(axis=1, keepdims=True) \
                + g_d * (np.abs(dO) * np.abs(o)).sum(axis=1, keepdims=True)
            dp = dO @ V.T
            e_dp = g_d * (np.abs(dO) @ np.abs(V).T)
            ds = p * (dp - dd)
            e_ds = e_p * np.abs(dp - dd) + (p + e_p) * (e_dd + e_dp)
            e_ds = np.where(vis, e_ds + u * (np.abs(ds) + e_ds) + eta, 0.0)  # dS rounded
            ads = np.abs(ds) + e_ds
            dv = p.T @ dO
            ev = e_p.T @ np.abs(dO) + g_n * (p + e_p).T @ np.abs(dO)
            bv[b, h] = ev + u * (np.abs(dv) + ev) + eta
            dk = scale * (ds.T @ Q)
            ek = scale * (e_ds.T @ np.abs(Q)) + g_n * scale * (ads.T @ np.abs(Q))
            bk[b, h] = ek + u * (np.abs(dk) + ek) + eta
            dq = scale * (ds @ K)
            eq = scale * (e_ds @ np.abs(K)) + g_n * scale * (ads @ np.abs(K))
            bq[b, h] = eq + 2 * f32 * (np.abs(dq) + eq)
    return bq, bk, bv
