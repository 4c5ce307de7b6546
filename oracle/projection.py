"""CPU oracle for the QKV projection with the region fused into its epilogue (NumPy, fp64).

TEST INFRASTRUCTURE ONLY: used by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``; the product path never imports it, and it
shares no code with the HIP library.

torchtitan page "[muse_spark][perf] Split the packed qkv inside the q/k region":
the region's input is the packed output of the attention's QKV projection
(Problem, item 1), and the page times the region with the GEMMs excluded (its
Results).  Fusing the region into the projection's epilogue removes the packed
tensor altogether: the projection's output never reaches memory, so it is never
rounded to the storage dtype.  The plain definition of the fused result is
therefore the exact product followed by the region:

    Y = x w_qkv^T                      (exact, fp64 from the stored bf16 values)
    q, k, v = split(Y)                 (the layout's head-block order)
    q, k = RoPE(RMSNorm(q) * w_q), RoPE(RMSNorm(k) * w_k)
    v = Y's v heads

each rounded once to the output dtype by the caller.  The split, RMSNorm and
RoPE are the region oracle's own steps (``oracle.reference``).
"""
from __future__ import annotations

import numpy as np

from .reference import rmsnorm, rope_angles, rope_rotate_half, split, to_f64


def project(x, w_qkv, dtype: str = "bf16") -> np.ndarray:
    """The packed projection output x w_qkv^T, exact in fp64: x [T, hidden], w_qkv [width, hidden]."""
    return to_f64(x, dtype) @ to_f64(w_qkv, dtype).T


def projected_forward_gqa(x, w_qkv, kind, n_kv, q_per_kv, head_dim, pos, q_norm_w, k_norm_w, eps, theta,
                          rope=True, dtype="bf16", chunk=1024):
    """The fused projection + region; returns unrounded fp64 ``(q [T, n_q, D], k [T, n_kv, D], v [T, n_kv, D])``.

    Tokens are processed in chunks of ``chunk`` rows to bound host memory.
    """
    x = np.asarray(x)
    T = x.shape[0]
    n_q = n_kv * q_per_kv
    D = head_dim
    wq = to_f64(q_norm_w, dtype)
    wk = to_f64(k_norm_w, dtype)
    q = np.empty((T, n_q, D))
    k = np.empty((T, n_kv, D))
    v = np.empty((T, n_kv, D))
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        Y = project(x[t0:t1], w_qkv, dtype)
        q_raw, k_raw, v_raw = split(Y, kind, n_kv, q_per_kv, D)
        qn = rmsnorm(q_raw, wq, eps)
        kn = rmsnorm(k_raw, wk, eps)
        if rope:
            phi = rope_angles(np.asarray(pos)[t0:t1], theta, D)
            qn = rope_rotate_half(qn, phi)
            kn = rope_rotate_half(kn, phi)
        q[t0:t1], k[t0:t1], v[t0:t1] = qn, kn, v_raw
    return q, k, v
