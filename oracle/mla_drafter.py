"""CPU oracle of one MLA drafter layer's q path and kv path (NumPy, fp64).

TEST INFRASTRUCTURE ONLY, under the same rules as ``oracle.reference``: only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; it shares no code with the HIP library or with the
Python layer that drives it.

What is computed (TensorRT-LLM page "MLA DSpark: run each drafter layer's kv
path beside its q path", Description): after the layer's input norm,

* the kv path: the kv_a projection gives a latent row [c (kv_lora_rank) ||
  k_pe (rope)]; c is RMSNormed with the kv_a norm weight, k_pe is rotated
  (rotate-half RoPE at the token's position), and the row goes to the pool at
  the block-table slot of that position;
* the q path: q_a projection -> RMSNorm with the q_a norm weight -> q_b
  projection, viewed as heads of [nope || rope]; the rope part is rotated like
  k_pe; the nope part is multiplied by the head's W_UK ("k absorption"), so
  that its dot product with a latent c equals the nope part's dot product with
  the head's up-projected key W_UK c.

Running the two paths on two streams changes no value: this module has one
order of evaluation and is the reference for every switch setting.

Readings (the page names the steps only): DeepSeek-V3-style MLA; every norm
is ``x * w / sqrt(mean(x^2) + eps)`` over the whole vector; the rope part of
each q head and the latent row's k_pe use the same rotate-half RoPE and theta;
projections are ``x @ W`` with ``W`` stored ``[in, out]``.

Rounding.  The layer's tensors are bf16, so with ``storage="bf16"`` the
oracle rounds (nearest-even) where the layer stores a tensor: after the input
norm, after each projection, after the q_a norm, after the q rotation and
after the absorption; everything between two storage points is exact fp64.
With ``storage=None`` nothing is rounded (the exact chain, for the library
pins).  The latent row itself is returned unrounded, from the stored kv_a
output, like ``latent_forward``.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from .reference import latent_forward, rmsnorm, rope_angles, rope_rotate_half, round_to_storage, to_f64


def _store(x: np.ndarray, storage: Optional[str]) -> np.ndarray:
    """Value of x after the layer stores it in ``storage`` (or x itself)."""
    if storage is None:
        return x
    return to_f64(round_to_storage(x, storage), storage)


def absorb(q_nope: np.ndarray, w_uk: np.ndarray) -> np.ndarray:
    """q_abs[n, h, :] = q_nope[n, h, :] @ W_UK[h]  ([N, H, nope] x [H, nope, L] -> [N, H, L])."""
    return np.einsum("nhd,hdl->nhl", q_nope, w_uk)


def drafter_layer(x, w_input_ln, w_q_a, w_q_a_ln, w_q_b, w_uk, w_kv_a, w_kv_a_ln, pos, *,
                  heads: int, qk_nope_head_dim: int, qk_rope_head_dim: int, kv_lora_rank: int,
                  eps: float, theta: float, dtype: str = "bf16",
                  storage: Optional[str] = "bf16") -> Dict[str, np.ndarray]:
    """One decode step of the layer on stored inputs (``dtype`` bit patterns).

    Returns fp64 arrays: ``xn`` [N, hidden]; ``q_nope`` [N, H, nope]; ``q_pe``
    [N, H, rope]; ``q_abs`` [N, H, kv_lora]; ``kv`` [N, kv_lora + rope] (the kv_a
    output); ``rows`` [N, kv_lora + rope] (the latent rows, unrounded).
    """
    X = to_f64(x, dtype)
    N = X.shape[0]
    xn = _store(rmsnorm(X, to_f64(w_input_ln, dtype), eps), storage)
    # q path
    q_a = _store(xn @ to_f64(w_q_a, dtype), storage)
    q_a = _store(rmsnorm(q_a, to_f64(w_q_a_ln, dtype), eps), storage)
    q = _store(q_a @ to_f64(w_q_b, dtype), storage).reshape(N, heads, qk_nope_head_dim + qk_rope_head_dim)
    q_nope = q[..., :qk_nope_head_dim]
    q_pe = _store(rope_rotate_half(q[..., qk_nope_head_dim:], rope_angles(pos, theta, qk_rope_head_dim)), storage)
    q_abs = _store(absorb(q_nope, to_f64(w_uk, dtype)), storage)
    # kv path
    kv = _store(xn @ to_f64(w_kv_a, dtype), storage)
    rows = latent_forward(kv, "fp64", pos, to_f64(w_kv_a_ln, dtype), eps, theta, kv_lora_rank, qk_rope_head_dim)
    return {"xn": xn, "q_nope": q_nope, "q_pe": q_pe, "q_abs": q_abs, "kv": kv, "rows": rows}
