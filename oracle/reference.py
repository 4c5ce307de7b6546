"""CPU oracle for the packed-QKV split + per-head RMSNorm + RoPE path (NumPy, fp64).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or run
this module: it is used by ``tests/``, by ``__graft_entry__.smoke()`` and by the
``cpu_baseline`` leg of ``bench.py``, and by nothing else.  It shares no code
with the HIP library (no kernels, headers, helpers or tables); the two meet only
in the seeded input generators of ``qkv_inputs``, which hold no arithmetic of
the method.

What is computed, and where the pages define it
------------------------------------------------
* torchtitan page "[muse_spark][perf] Split the packed qkv inside the q/k
  region" (P1):
    - Problem, item 1: the projection returns q, k and v packed as
      ``[T, 16 kv heads, 10, 64]``: per kv group, 8 q heads, then 1 k, then 1 v.
    - Problem, item 2: q, k and v are split out into contiguous tensors.
    - Problem, item 3 and Solution, item 3: per-head norms of q and k, then
      RoPE; the before/after diagram orders the region as split -> norm -> RoPE,
      with v copied.
    - Results, Numerics: RoPE layers and NoPE layers (no rotation).
    - Problem, item 4 and Solution, item 3: the backward writes one packed grad
      (no concatenation of three grads).
* DeepSpeed page "[muon] Per-head Newton-Schulz for fused QKV projections" (P2),
  "What this PR does": the two fused layouts (sectioned ``cat([q, k, v])`` and
  interleaved per KV group), both a partition into ``n_q + 2 n_kv`` head blocks
  of ``head_dim`` rows in a different order, and the exact-total guard.
* TensorRT-LLM page "MLA DSpark: run each drafter layer's kv path beside its q
  path" (P3), Description: the latent kv path's RMSNorm/RoPE stores the latent
  rows straight into the paged context pool at block-table pages/offsets, which
  must be bitwise what a staged buffer plus scatter writes (Test Coverage).

Readings where the pages are silent (each one is listed in the design notes):
rotate-half RoPE on pairs (i, i + R/2) with angle ``pos * theta**(-2i/R)`` taken
as the exact real angle; RMSNorm mean over one head's D values with eps inside
the square root and a plain multiplicative weight shared by all heads of a kind;
norm before RoPE; one rounding at the end; q head h belongs to kv group
h // q_per_kv; the latent row is RMSNorm over its first ``norm_dim`` values and
RoPE (no norm) over its last ``rope_dim``; NoPE is RoPE at position 0.

Every function here is pinned by a ``-m "not gpu"`` test against something other
than itself (library routines in fp64, closed forms, invariants, finite
differences, brute force, the page's printed layout examples).
"""
from __future__ import annotations

import math

import numpy as np

# --------------------------------------------------------------------------- #
# Decoding and rounding of the storage dtypes
# --------------------------------------------------------------------------- #


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of a stored tensor: bf16 bit patterns (uint16), fp32 or fp64."""
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "fp32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "fp64":
        return np.asarray(a, dtype=np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 values once, to nearest-even, into the storage dtype.

    bf16 results are returned as uint16 bit patterns.  The fp64 -> bf16 rounding
    is done directly on the fp64 significand (no intermediate fp32 rounding),
    valid for the normal range of bf16, which every value here lies in.
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    if dtype == "fp32":
        return x.astype(np.float32)
    if dtype != "bf16":
        raise ValueError(dtype)
    u = x.view(np.uint64)
    # keep sign, 11 exponent bits and the top 7 fraction bits: drop 45 bits, ties to even
    keep_lsb = (u >> np.uint64(45)) & np.uint64(1)
    r = (u + np.uint64((1 << 44) - 1) + keep_lsb) >> np.uint64(45)
    rounded = (r << np.uint64(45)).view(np.float64)          # exactly a bf16 value
    return (rounded.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# --------------------------------------------------------------------------- #
# Layouts: split, unsplit, head blocks (P2 "What this PR does"; P1 Problem.1-2)
# --------------------------------------------------------------------------- #


def head_blocks(n_q: int, n_kv: int) -> int:
    """Number of head_dim-row blocks a fused q|k|v holds: n_q query + n_kv key + n_kv value."""
    return n_q + 2 * n_kv


def exact_total_ok(width: int, n_q: int, n_kv: int, head_dim: int) -> bool:
    """The fused width must be exactly (n_q + 2 n_kv) * head_dim, else the layout is declined."""
    return width == head_blocks(n_q, n_kv) * head_dim


def split(X: np.ndarray, kind: str, n_kv: int, q_per_kv: int, head_dim: int):
    """Split a packed q|k|v into contiguous q [T, n_q, D], k [T, n_kv, D], v [T, n_kv, D].

    interleaved: X is [T, n_kv, q_per_kv + 2, D]; in group g, slots 0..q_per_kv-1
    are q heads g*q_per_kv + s, slot q_per_kv is k head g, the last slot is v head g.
    sectioned:   X is [T, (n_q + 2 n_kv) * D]: n_q q heads, n_kv k heads, n_kv v heads.
    Pure indexing: works on any element type, bits are moved unchanged.
    """
    T = X.shape[0]
    n_q = n_kv * q_per_kv
    D = head_dim
    if kind == "interleaved":
        X = X.reshape(T, n_kv, q_per_kv + 2, D)
        q = np.empty((T, n_q, D), dtype=X.dtype)
        k = np.empty((T, n_kv, D), dtype=X.dtype)
        v = np.empty((T, n_kv, D), dtype=X.dtype)
        for g in range(n_kv):
            for s in range(q_per_kv):
                q[:, g * q_per_kv + s, :] = X[:, g, s, :]
            k[:, g, :] = X[:, g, q_per_kv, :]
            v[:, g, :] = X[:, g, q_per_kv + 1, :]
        return q, k, v
    if kind == "sectioned":
        X = X.reshape(T, head_blocks(n_q, n_kv), D)
        q = X[:, :n_q, :].copy()
        k = X[:, n_q:n_q + n_kv, :].copy()
        v = X[:, n_q + n_kv:, :].copy()
        return q, k, v
    raise ValueError(kind)


def unsplit(q: np.ndarray, k: np.ndarray, v: np.ndarray, kind: str, q_per_kv: int):
    """Inverse of :func:`split`: pack q, k, v back into the given layout."""
    T, n_q, D = q.shape
    n_kv = k.shape[1]
    if kind == "interleaved":
        X = np.empty((T, n_kv, q_per_kv + 2, D), dtype=q.dtype)
        for g in range(n_kv):
            for s in range(q_per_kv):
                X[:, g, s, :] = q[:, g * q_per_kv + s, :]
            X[:, g, q_per_kv, :] = k[:, g, :]
            X[:, g, q_per_kv + 1, :] = v[:, g, :]
        return X
    if kind == "sectioned":
        return np.concatenate([q, k, v], axis=1).reshape(T, head_blocks(n_q, n_kv) * D)
    raise ValueError(kind)


# --------------------------------------------------------------------------- #
# The per-head math
# --------------------------------------------------------------------------- #


def rope_angles(pos: np.ndarray, theta: float, R: int) -> np.ndarray:
    """phi[t, i] = pos[t] * theta ** (-2 i / R), i < R/2, as fp64 real angles [T, R/2]."""
    i = np.arange(R // 2, dtype=np.float64)
    inv_freq = np.float64(theta) ** (-2.0 * i / R)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]


def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x * w / sqrt(mean(x**2 over the last axis) + eps)."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * w


def rope_rotate_half(x: np.ndarray, phi: np.ndarray) -> np.ndarray:
    """Rotate pairs (i, i + R/2) of the last axis by phi (broadcast over middle axes).

    y_i = x_i cos - x_{i+R/2} sin,   y_{i+R/2} = x_{i+R/2} cos + x_i sin.
    x is [T, ..., R], phi is [T, R/2].
    """
    R = x.shape[-1]
    h = R // 2
    shape = (phi.shape[0],) + (1,) * (x.ndim - 2) + (h,)
    c = np.cos(phi).reshape(shape)
    s = np.sin(phi).reshape(shape)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def rope_rotate_half_inverse(g: np.ndarray, phi: np.ndarray) -> np.ndarray:
    """Transpose of :func:`rope_rotate_half` (rotation by -phi)."""
    return rope_rotate_half(g, -phi)


# --------------------------------------------------------------------------- #
# GQA forward / backward (P1 diagram "after": split -> norm -> RoPE, copy v;
# backward writes the packed grad)
# --------------------------------------------------------------------------- #


def forward_gqa(qkv, dtype, kind, n_kv, q_per_kv, head_dim, pos, q_norm_w, k_norm_w,
                eps, theta, rope=True):
    """Forward of the region on a packed input; returns exact-valued results.

    Returns ``(q64, k64, v_bits)``: q and k as unrounded fp64 [T, heads, D] and v
    as the input's own stored values, unchanged.  NoPE layers (``rope=False``)
    skip the rotation.
    """
    q_raw, k_raw, v_raw = split(np.asarray(qkv), kind, n_kv, q_per_kv, head_dim)
    wq = to_f64(q_norm_w, dtype)
    wk = to_f64(k_norm_w, dtype)
    qn = rmsnorm(to_f64(q_raw, dtype), wq, eps)
    kn = rmsnorm(to_f64(k_raw, dtype), wk, eps)
    if rope:
        phi = rope_angles(pos, theta, head_dim)
        qn = rope_rotate_half(qn, phi)
        kn = rope_rotate_half(kn, phi)
    return qn, kn, v_raw


def _norm_rope_backward(x, g, w, eps, phi):
    """Backward of y = RoPE(RMSNorm(x) * w) for heads along the last axis.

    Returns dx, the per-element weight-grad terms u*xhat, with u = R(-phi) g.
    """
    u = g if phi is None else rope_rotate_half_inverse(g, phi)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    r = 1.0 / np.sqrt(ms + eps)
    xhat = x * r
    a = w * u
    dx = r * (a - xhat * np.mean(a * xhat, axis=-1, keepdims=True))
    return dx, u * xhat


def backward_gqa(qkv, dtype, kind, n_kv, q_per_kv, head_dim, pos, q_norm_w, k_norm_w,
                 eps, theta, dq, dk, dv, rope=True, chunk=1024):
    """Backward of :func:`forward_gqa`; the packed grad is written in the input layout.

    Returns a dict:
      ``dx_q``, ``dx_k``  fp64 grads of the q and k slots, [T, heads, D];
      ``dv_bits``         dv moved unchanged (it lands in the v slots);
      ``dqkv64``          fp64 packed grad in the input layout (v slots hold dv's values);
      ``dw_q``, ``dw_k``  fp64 norm-weight grads [D] (sum over tokens and heads);
      ``dw_q_l2``, ``dw_k_l2``  sqrt of the sum of squared terms of each weight grad
                          (how well conditioned each sum is).
    Tokens are processed in chunks of ``chunk`` to bound host memory; the sums
    over chunks are plain fp64 additions.
    """
    T = np.asarray(qkv).shape[0]
    wq = to_f64(q_norm_w, dtype)
    wk = to_f64(k_norm_w, dtype)
    n_q = n_kv * q_per_kv
    D = head_dim
    dx_q = np.empty((T, n_q, D))
    dx_k = np.empty((T, n_kv, D))
    dw_q = np.zeros(D)
    dw_k = np.zeros(D)
    sq_q = np.zeros(D)
    sq_k = np.zeros(D)
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        q_raw, k_raw, _ = split(np.asarray(qkv)[t0:t1], kind, n_kv, q_per_kv, D)
        phi = rope_angles(np.asarray(pos)[t0:t1], theta, D) if rope else None
        gq = to_f64(np.asarray(dq)[t0:t1], dtype)
        gk = to_f64(np.asarray(dk)[t0:t1], dtype)
        dxq, tq = _norm_rope_backward(to_f64(q_raw, dtype), gq, wq, eps, phi)
        dxk, tk = _norm_rope_backward(to_f64(k_raw, dtype), gk, wk, eps, phi)
        dx_q[t0:t1] = dxq
        dx_k[t0:t1] = dxk
        dw_q += tq.sum(axis=(0, 1))
        dw_k += tk.sum(axis=(0, 1))
        sq_q += (tq * tq).sum(axis=(0, 1))
        sq_k += (tk * tk).sum(axis=(0, 1))
    dv_bits = np.asarray(dv)
    dqkv64 = unsplit(dx_q, dx_k, to_f64(dv_bits, dtype), kind, q_per_kv)
    return {
        "dx_q": dx_q, "dx_k": dx_k, "dv_bits": dv_bits, "dqkv64": dqkv64,
        "dw_q": dw_q, "dw_k": dw_k, "dw_q_l2": np.sqrt(sq_q), "dw_k_l2": np.sqrt(sq_k),
    }


# --------------------------------------------------------------------------- #
# Latent rows and the paged pool (P3 Description and Test Coverage)
# --------------------------------------------------------------------------- #


def latent_forward(rows, dtype, pos, norm_w, eps, theta, norm_dim, rope_dim):
    """One latent row per token: [RMSNorm(c[:norm_dim]) * w  ||  RoPE(c[norm_dim:])].

    Returns unrounded fp64 rows [T, norm_dim + rope_dim].
    """
    x = to_f64(rows, dtype)
    c, kpe = x[:, :norm_dim], x[:, norm_dim:norm_dim + rope_dim]
    cn = rmsnorm(c, to_f64(norm_w, dtype), eps)
    kr = rope_rotate_half(kpe, rope_angles(pos, theta, rope_dim))
    return np.concatenate([cn, kr], axis=1)


def paged_slots(pos, block_table, tokens_per_req, page_size):
    """Pool slot of each token: request b = t // tokens_per_req, page = table[b][pos // P].

    Returns ``(page, offset)`` int64 arrays; the flat slot is page * P + offset.
    """
    pos = np.asarray(pos, dtype=np.int64)
    b = np.arange(pos.shape[0]) // tokens_per_req
    page = np.asarray(block_table, dtype=np.int64)[b, pos // page_size]
    return page, pos % page_size


def staged_then_scatter(pool, staged_rows, page, offset):
    """The pre-change path: rows computed into a staging buffer, then scattered.

    ``pool`` is [num_pages, P, ...]; returns a new pool with the rows written.
    """
    out = np.array(pool, copy=True)
    for r in range(staged_rows.shape[0]):
        out[page[r], offset[r]] = staged_rows[r]
    return out
