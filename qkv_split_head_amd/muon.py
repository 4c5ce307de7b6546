"""Per-head Newton-Schulz (the Muon update's orthogonalisation) on fused QKV weights.

DeepSpeed page "[muon] Per-head Newton-Schulz for fused QKV projections":
every head of a fused q|k|v weight is head_dim contiguous rows in both the
sectioned and the interleaved order, so the per-head update is a batched
update over a zero-copy ``[blocks, head_dim, in]`` view, and it does not depend
on which order the weight uses.  The weight is split only when its row count
is the exact fused total (``qkvnr_fused_head_blocks``); otherwise it is
declined to the full-matrix path.

Each Newton-Schulz step on the blocks' wide orientation X is X <- P X with
P = a I + b X X^T + c (X X^T)^2, a polynomial in G G^T; so the iterate after
any number of steps is M G with M a polynomial in G G^T.  For bf16 blocks of
side 64 or 128 the iteration is taken that way, in three launches:
``qkvnr_gram_partials`` (G G^T with MFMA, reading both factors as rows of G),
``qkvnr_ns_collapse`` (the steps on d x d matrices, one workgroup per block,
products from operands split into two bf16 terms) and ``qkvnr_ns_apply``
(Y = M G, M in two bf16 terms): G is read twice and Y written once, instead of
two reads and a write a step.  Other bf16 blocks of side 32..128 take the steps
one by one: ``qkvnr_gram_partials``, ``qkvnr_ns_poly`` (P, with the first
step's Frobenius normalisation and the last step's block scale folded in) and
a batched library GEMM for P X; fp32 and other sides take library GEMMs for
both products.  The blocks never leave the ``[blocks, d, in]`` layout.

``compute_dtype`` bf16 is Muon's usual precision (GEMMs in bf16 with fp32
accumulation); fp32 runs the same steps in fp32.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _binding as b

STEPS = 5
EPS = 1e-7


def fused_head_blocks(n_q: int, n_kv: int, head_dim: int, weight_rows: int) -> int:
    """Head blocks of a fused weight, or QkvnrError when the exact-total guard declines it."""
    return b.qkvnr_fused_head_blocks(n_q, n_kv, head_dim, weight_rows)


def _gram_parts(nb: int, cols: int) -> int:
    """Column slices for the Gram kernel (one workgroup per block and slice): about one
    workgroup per CU, slices of >= 512 columns."""
    return max(1, min(256 // nb, cols // 512))


def _newton_schulz_blocks(X: torch.Tensor, scale: float, steps: int, eps: float) -> torch.Tensor:
    """X: [blocks, d, cols] wide blocks (d <= cols), contiguous; returns the orthogonalised blocks."""
    nb, d, cols = X.shape
    dtype = b.DTYPES[X.dtype]
    own_gram = X.dtype == torch.bfloat16 and d in (32, 64, 96, 128) and cols % 8 == 0
    parts = _gram_parts(nb, cols) if own_gram else 1
    gram = torch.empty((nb, parts, d, d), dtype=torch.float32, device=X.device)
    if own_gram and d in (64, 128):
        # collapsed: G's Gram matrices, the whole iteration as M per block, then M G
        b.qkvnr_gram_partials(nb, d, cols, X, parts, gram)
        M = torch.empty((nb, 2, d, d), dtype=X.dtype, device=X.device)
        b.qkvnr_ns_collapse(nb, d, gram, parts, steps, scale, eps, M)
        Y = torch.empty_like(X)
        b.qkvnr_ns_apply(nb, d, cols, M, X, Y, parts)
        return Y
    P = torch.empty((nb, d, d), dtype=X.dtype, device=X.device)
    for i in range(steps):
        if own_gram:   # the library kernel reads both factors as rows of X
            b.qkvnr_gram_partials(nb, d, cols, X, parts, gram)
        else:          # fp32 and other block sides: a library GEMM (right operand made contiguous)
            gram.view(nb, d, d).copy_(torch.bmm(X, X.transpose(1, 2).contiguous()))
        b.qkvnr_ns_poly(dtype, nb, d, gram, parts, i == 0, scale if i == steps - 1 else 1.0, eps, P)
        X = torch.bmm(P, X)
    return X


def per_head_newton_schulz(G: torch.Tensor, n_q: int, n_kv: int, head_dim: int, *, steps: int = STEPS,
                           compute_dtype: Optional[torch.dtype] = None, eps: float = EPS) -> torch.Tensor:
    """Per-head orthogonalised update of a fused q|k|v weight (or its gradient / momentum).

    G is ``[(n_q + 2 n_kv) * head_dim, in_features]`` in either block order; the
    result has G's shape and block order and ``compute_dtype`` (default: G's).
    Each block is scaled by max(1, head_dim / in_features) ** 0.5.  Every sum is
    taken in a fixed order: the result does not change from run to run.
    """
    if steps < 1:   # the first step carries the Frobenius normalisation
        raise ValueError(f"steps must be >= 1, got {steps}")
    if G.dim() != 2:
        raise ValueError("G must be a 2-D weight")
    b._need(G, "G", contiguous=False)   # the kernels take device addresses: a host weight is refused here
    rows, cols = G.shape
    nb = fused_head_blocks(n_q, n_kv, head_dim, rows)
    dt = G.dtype if compute_dtype is None else compute_dtype
    if dt not in (torch.bfloat16, torch.float32):
        raise ValueError(f"unsupported compute dtype {dt}")
    X = G.to(dt).contiguous()
    if X.data_ptr() % 16:   # the kernels read 16 bytes at a time: an offset view gets an aligned copy
        X = X.clone()
    X = X.view(nb, head_dim, cols)
    scale = max(1.0, head_dim / cols) ** 0.5
    if head_dim <= cols:
        return _newton_schulz_blocks(X, scale, steps, eps).view(rows, cols)
    # tall blocks: iterate on the transposes
    Y = _newton_schulz_blocks(X.transpose(1, 2).contiguous(), scale, steps, eps)
    return Y.transpose(1, 2).contiguous().view(rows, cols)
