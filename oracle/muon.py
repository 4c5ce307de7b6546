"""CPU oracle of per-head Newton-Schulz on fused QKV weights (NumPy, fp64).

TEST INFRASTRUCTURE ONLY, under the same rules as ``oracle.reference``: only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; it shares no code with the HIP library or with the
Python layer that drives it.

What is computed (DeepSpeed page "[muon] Per-head Newton-Schulz for fused QKV
projections", "What this PR does"): a fused q|k|v weight is a stack of head
blocks of head_dim rows each, in either the sectioned or the interleaved
order; the update orthogonalises every block on its own with Newton-Schulz and
scales it by max(1, rows/cols)**0.5 of the block, so the result does not depend
on the order of the blocks.  A weight is split only when its row count is the
exact fused total (n_q + 2 n_kv) * head_dim; anything else is declined to the
full-matrix path (the page's Conv1D and Falcon examples).  The full-matrix path
orthogonalises the whole weight and scales by max(1, rows/cols)**0.5 of the
whole (the review comment on the same page: up to sqrt(3) for [3h, h]).

Readings (the page names Newton-Schulz and the scale, not the iteration): the
quintic iteration of the Muon optimizer, with coefficients (3.4445, -4.7750,
2.0315) and 5 steps, on X0 = G / (||G||_F + 1e-7), working on the wide
orientation (a block with more rows than columns is transposed first and the
result transposed back): A = X X^T, X <- a X + (b A + c A A) X.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

QUINTIC = (3.4445, -4.7750, 2.0315)
NS_STEPS = 5
NS_EPS = 1e-7


def newton_schulz(G: np.ndarray, steps: int = NS_STEPS, eps: float = NS_EPS) -> np.ndarray:
    """Approximate orthogonalisation U V^T of G (fp64), by the quintic iteration."""
    X = np.asarray(G, dtype=np.float64)
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T
    X = X / (np.sqrt(np.sum(X * X)) + eps)
    a, b, c = QUINTIC
    for _ in range(steps):
        A = X @ X.T
        X = a * X + (b * A + c * (A @ A)) @ X
    return X.T if tall else X


def scale(rows: int, cols: int) -> float:
    return max(1.0, rows / cols) ** 0.5


def head_block_count(rows: int, n_q: int, n_kv: int, head_dim: int) -> Optional[int]:
    """Head blocks of a fused weight with `rows` rows, or None when it is not the exact fused total."""
    blocks = n_q + 2 * n_kv
    return blocks if rows == blocks * head_dim else None


def per_head_update(W: np.ndarray, n_q: int, n_kv: int, head_dim: int, steps: int = NS_STEPS) -> np.ndarray:
    """Newton-Schulz on every head_dim-row block of a fused weight, each scaled on its own."""
    W = np.asarray(W, dtype=np.float64)
    nb = head_block_count(W.shape[0], n_q, n_kv, head_dim)
    if nb is None:
        raise ValueError("not the exact fused total: declined to the full-matrix path")
    cols = W.shape[1]
    out = np.empty_like(W)
    for blk in range(nb):
        rows = slice(blk * head_dim, (blk + 1) * head_dim)
        out[rows] = newton_schulz(W[rows], steps) * scale(head_dim, cols)
    return out


def full_matrix_update(W: np.ndarray, steps: int = NS_STEPS) -> np.ndarray:
    """Newton-Schulz on the whole weight, scaled by its own shape."""
    W = np.asarray(W, dtype=np.float64)
    return newton_schulz(W, steps) * scale(W.shape[0], W.shape[1])
