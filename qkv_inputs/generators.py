"""Seeded generators for the five workloads and for ad-hoc parity cases.

Every array is drawn with ``numpy.random.Generator(PCG64(seed))`` in a fixed
order: packed input, norm weights (q, then k), positions, cotangents, block
table.  bf16 tensors are fp32 draws rounded to nearest-even and kept as their
16-bit patterns (``uint16``); the same bits go to the GPU and to the oracle.

Shapes follow the workloads of the torchtitan page "[muse_spark][perf] Split the
packed qkv inside the q/k region" (Problem, item 1: a packed ``[T, 16, 10, 64]``
output, per kv group 8 q heads + 1 k + 1 v), the DeepSpeed page "[muon] Per-head
Newton-Schulz for fused QKV projections" (the sectioned and interleaved fused
layouts) and the TensorRT-LLM page "MLA DSpark: run each drafter layer's kv path
beside its q path" (latent rows written straight into a paged pool).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# Seeds of the five named workloads (decode uses 1000 + T).
SEEDS = {"tiny": 0, "decode_base": 1000, "prefill": 2, "train": 3, "latent": 4}


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bit patterns.

    Input preparation only: turns fp32 random draws into bf16 test tensors.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if not np.all(np.isfinite(x)):
        raise ValueError("only finite values are rounded here")
    # finite patterns are at most 0xFF7FFFFF, so adding < 0x8001 cannot wrap
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    """One synthetic batch for the path, plus the layout it is packed in.

    ``kind`` is ``"interleaved"`` (``qkv`` is ``[T, n_kv, q_per_kv + 2, D]``),
    ``"sectioned"`` (``qkv`` is ``[T, (n_q + 2 n_kv) * D]``, heads ordered
    q..., k..., v...) or ``"latent"`` (``qkv`` is ``[T, norm_dim + rope_dim]``).
    bf16 arrays are ``uint16`` bit patterns; fp32 arrays are ``float32``.
    """

    name: str
    kind: str
    dtype: str
    T: int
    n_kv: int
    q_per_kv: int
    head_dim: int
    rope_dim: int
    eps: float
    theta: float
    qkv: np.ndarray
    positions: np.ndarray
    q_norm_w: Optional[np.ndarray]
    k_norm_w: np.ndarray
    norm_dim: int = 0
    dq: Optional[np.ndarray] = None
    dk: Optional[np.ndarray] = None
    dv: Optional[np.ndarray] = None
    # paged store (latent rows, or GQA k/v)
    block_table: Optional[np.ndarray] = None
    tokens_per_req: int = 0
    page_size: int = 0
    num_pages: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def n_q(self) -> int:
        return self.n_kv * self.q_per_kv

    @property
    def width(self) -> int:
        """Elements per token of the packed row."""
        if self.kind == "latent":
            return self.norm_dim + self.rope_dim
        return (self.n_q + 2 * self.n_kv) * self.head_dim

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4


def _draw(rng: np.random.Generator, shape, dtype: str, mean: float = 0.0, std: float = 1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if mean != 0.0 or std != 1.0:
        x = (np.float32(mean) + np.float32(std) * x).astype(np.float32)
    if dtype == "bf16":
        return bf16_bits_from_f32(x).reshape(shape)
    if dtype == "fp32":
        return x.reshape(shape)
    raise ValueError(dtype)


def _packed_shape(kind, T, n_kv, q_per_kv, D):
    if kind == "interleaved":
        return (T, n_kv, q_per_kv + 2, D)
    if kind == "sectioned":
        return (T, (n_kv * q_per_kv + 2 * n_kv) * D)
    raise ValueError(kind)


def custom_gqa(
    kind: str,
    dtype: str,
    T: int,
    n_kv: int,
    q_per_kv: int,
    head_dim: int,
    *,
    rope: bool = True,
    theta: float = 10000.0,
    eps: float = 1e-6,
    seed: int = 0,
    positions: str = "arange",
    max_pos: int = 131072,
    grads: bool = False,
    name: str = "custom",
) -> Workload:
    """A GQA workload of any shape: packed input ~N(0,1), weights ~N(1,0.1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    qkv = _draw(rng, _packed_shape(kind, T, n_kv, q_per_kv, head_dim), dtype)
    wq = _draw(rng, (head_dim,), dtype, 1.0, 0.1)
    wk = _draw(rng, (head_dim,), dtype, 1.0, 0.1)
    if positions == "arange":
        pos = np.arange(T, dtype=np.int32)
    elif positions == "random":
        pos = rng.integers(0, max_pos, size=T, dtype=np.int64).astype(np.int32)
    elif positions == "zeros":
        pos = np.zeros(T, dtype=np.int32)
    else:
        raise ValueError(positions)
    w = Workload(
        name=name, kind=kind, dtype=dtype, T=T, n_kv=n_kv, q_per_kv=q_per_kv,
        head_dim=head_dim, rope_dim=head_dim if rope else 0, eps=eps, theta=theta,
        qkv=qkv, positions=pos, q_norm_w=wq, k_norm_w=wk,
    )
    if grads:
        w.dq = _draw(rng, (T, w.n_q, head_dim), dtype)
        w.dk = _draw(rng, (T, n_kv, head_dim), dtype)
        w.dv = _draw(rng, (T, n_kv, head_dim), dtype)
    return w


def tiny_interleaved() -> Workload:
    """T=16, interleaved [16, 2, 4+2, 64] fp32, weights fp32, theta 1e4, positions 0..15."""
    return custom_gqa("interleaved", "fp32", 16, 2, 4, 64, rope=True, theta=1e4,
                      eps=1e-6, seed=SEEDS["tiny"], positions="arange", name="tiny_interleaved_fp32")


def decode_interleaved(T: int) -> Workload:
    """Muse-Spark-shaped decode: bf16 [T, 16, 8+2, 64], random positions < 131072, theta 5e5."""
    return custom_gqa("interleaved", "bf16", T, 16, 8, 64, rope=True, theta=5e5, eps=1e-6,
                      seed=SEEDS["decode_base"] + T, positions="random", max_pos=131072,
                      name=f"muse_decode_T{T}")


def prefill_interleaved(T: int = 16384, rope: bool = True) -> Workload:
    """Muse-Spark-shaped prefill: bf16 [T, 16, 10, 64], positions 0..T-1; RoPE or NoPE layer."""
    return custom_gqa("interleaved", "bf16", T, 16, 8, 64, rope=rope, theta=5e5, eps=1e-6,
                      seed=SEEDS["prefill"], positions="arange",
                      name=f"muse_prefill_T{T}_{'rope' if rope else 'nope'}")


def train_sectioned(T: int = 16384, grads: bool = True) -> Workload:
    """Qwen3-8B-like training: sectioned bf16 [T, (32+8+8)*128], theta 1e6, with cotangents."""
    return custom_gqa("sectioned", "bf16", T, 8, 4, 128, rope=True, theta=1e6, eps=1e-6,
                      seed=SEEDS["train"], positions="arange", grads=grads,
                      name=f"qwen3_8b_train_T{T}")


def token_positions(T: int, seed: int, high: int = 2**31 - 1) -> np.ndarray:
    """T int32 positions drawn uniformly from [0, high).

    For batches too large to draw row by row: their packed rows are a smaller
    draw repeated, and each token still gets a position of its own, so no two
    tokens see the same rotation.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, high, size=T, dtype=np.int64).astype(np.int32)


def _block_table(rng, B, T_req, num_pages, page_size, ctx_lo, ctx_hi):
    """Context lengths, draft-token positions and a non-overlapping block table.

    Draft token i of request b sits at position ``ctx_b + i``.  Request b owns
    ``ceil((ctx_b + T_req) / page_size)`` distinct pages taken in order from one
    seeded permutation of all pages; unused table entries are -1.  Context
    lengths are redrawn (same generator) until the pages fit in the pool.
    """
    bt_stride = -(-(ctx_hi + T_req) // page_size)
    while True:
        ctx = rng.integers(ctx_lo, ctx_hi, size=B, endpoint=True, dtype=np.int64)
        need = -(-(ctx + T_req) // page_size)
        if int(need.sum()) <= num_pages:
            break
    pos = (ctx[:, None] + np.arange(T_req, dtype=np.int64)[None, :]).reshape(-1).astype(np.int32)
    perm = rng.permutation(num_pages).astype(np.int32)
    table = np.full((B, bt_stride), -1, dtype=np.int32)
    at = 0
    for b in range(B):
        n = int(need[b])
        table[b, :n] = perm[at:at + n]
        at += n
    return ctx, pos, table


def latent_paged(
    B: int = 4,
    T_req: int = 16,
    num_pages: int = 8192,
    page_size: int = 64,
    norm_dim: int = 512,
    rope_dim: int = 64,
    ctx_lo: int = 2048,
    ctx_hi: int = 131072,
    seed: int = SEEDS["latent"],
) -> Workload:
    """MLA-style latent rows [B*T_req, 512+64] bf16 and a random non-overlapping block table."""
    rng = np.random.Generator(np.random.PCG64(seed))
    T = B * T_req
    rows = _draw(rng, (T, norm_dim + rope_dim), "bf16")
    w = _draw(rng, (norm_dim,), "bf16", 1.0, 0.1)
    ctx, pos, table = _block_table(rng, B, T_req, num_pages, page_size, ctx_lo, ctx_hi)
    return Workload(
        name=f"mla_latent_paged_B{B}_T{T_req}", kind="latent", dtype="bf16", T=T,
        n_kv=1, q_per_kv=0, head_dim=norm_dim + rope_dim, rope_dim=rope_dim,
        eps=1e-6, theta=1e4, qkv=rows, positions=pos, q_norm_w=None, k_norm_w=w,
        norm_dim=norm_dim, block_table=table, tokens_per_req=T_req,
        page_size=page_size, num_pages=num_pages, extra={"ctx": ctx},
    )


def gqa_paged(
    kind: str,
    dtype: str,
    B: int,
    T_req: int,
    n_kv: int,
    q_per_kv: int,
    head_dim: int,
    *,
    num_pages: int = 256,
    page_size: int = 16,
    ctx_lo: int = 0,
    ctx_hi: int = 2000,
    rope: bool = True,
    theta: float = 1e4,
    seed: int = 0,
) -> Workload:
    """GQA batch whose k/v go to paged pools: B requests of T_req tokens after random contexts."""
    rng = np.random.Generator(np.random.PCG64(seed))
    T = B * T_req
    qkv = _draw(rng, _packed_shape(kind, T, n_kv, q_per_kv, head_dim), dtype)
    wq = _draw(rng, (head_dim,), dtype, 1.0, 0.1)
    wk = _draw(rng, (head_dim,), dtype, 1.0, 0.1)
    ctx, pos, table = _block_table(rng, B, T_req, num_pages, page_size, ctx_lo, ctx_hi)
    return Workload(
        name=f"gqa_paged_{kind}_{dtype}_B{B}_T{T_req}", kind=kind, dtype=dtype, T=T, n_kv=n_kv,
        q_per_kv=q_per_kv, head_dim=head_dim, rope_dim=head_dim if rope else 0, eps=1e-6, theta=theta,
        qkv=qkv, positions=pos, q_norm_w=wq, k_norm_w=wk, block_table=table, tokens_per_req=T_req,
        page_size=page_size, num_pages=num_pages, extra={"ctx": ctx},
    )


@dataclass
class MlaDrafterInputs:
    """One MLA drafter layer's decode-step inputs and random-init weights.

    Matrices are stored ``[in, out]`` (a projection is ``x @ W``).  bf16 arrays
    are ``uint16`` bit patterns.  Projection weights are N(0, 1/fan_in), so
    every projection output is O(1); norm weights are N(1, 0.1).
    """

    name: str
    B: int
    T_req: int
    hidden: int
    q_lora_rank: int
    kv_lora_rank: int
    qk_nope_head_dim: int
    qk_rope_head_dim: int
    heads: int
    eps: float
    theta: float
    x: np.ndarray             # [B*T_req, hidden], the layer input
    w_input_ln: np.ndarray    # [hidden]
    w_q_a: np.ndarray         # [hidden, q_lora_rank]
    w_q_a_ln: np.ndarray      # [q_lora_rank]
    w_q_b: np.ndarray         # [q_lora_rank, heads * (nope + rope)]
    w_uk: np.ndarray          # [heads, nope, kv_lora_rank]
    w_kv_a: np.ndarray        # [hidden, kv_lora_rank + rope]
    w_kv_a_ln: np.ndarray     # [kv_lora_rank]
    positions: np.ndarray     # [B*T_req] int32
    block_table: np.ndarray   # [B, bt_stride] int32, -1 = unused
    tokens_per_req: int
    page_size: int
    num_pages: int
    extra: dict = field(default_factory=dict)


def mla_drafter_layer(
    B: int = 4,
    T_req: int = 16,
    *,
    hidden: int = 7168,
    q_lora_rank: int = 1536,
    kv_lora_rank: int = 512,
    qk_nope_head_dim: int = 128,
    qk_rope_head_dim: int = 64,
    heads: int = 16,
    num_pages: int = 8192,
    page_size: int = 64,
    ctx_lo: int = 2048,
    ctx_hi: int = 131072,
    seed: Optional[int] = None,
) -> MlaDrafterInputs:
    """A DeepSeek-V3-style MLA layer at one rank's share of tensor parallelism 8
    (128 heads / 8 = 16), B requests of T_req draft tokens after random contexts.

    Draw order: layer input, input-norm weight, q_a, q_a norm weight, q_b, W_UK,
    kv_a, kv_a norm weight, then the block table (as for the latent workload).
    """
    if seed is None:
        seed = 50 + B
    rng = np.random.Generator(np.random.PCG64(seed))
    N = B * T_req
    qh = qk_nope_head_dim + qk_rope_head_dim
    x = _draw(rng, (N, hidden), "bf16")
    w_in = _draw(rng, (hidden,), "bf16", 1.0, 0.1)
    w_qa = _draw(rng, (hidden, q_lora_rank), "bf16", 0.0, float(hidden) ** -0.5)
    w_qa_ln = _draw(rng, (q_lora_rank,), "bf16", 1.0, 0.1)
    w_qb = _draw(rng, (q_lora_rank, heads * qh), "bf16", 0.0, float(q_lora_rank) ** -0.5)
    w_uk = _draw(rng, (heads, qk_nope_head_dim, kv_lora_rank), "bf16", 0.0, float(qk_nope_head_dim) ** -0.5)
    w_kva = _draw(rng, (hidden, kv_lora_rank + qk_rope_head_dim), "bf16", 0.0, float(hidden) ** -0.5)
    w_kva_ln = _draw(rng, (kv_lora_rank,), "bf16", 1.0, 0.1)
    ctx, pos, table = _block_table(rng, B, T_req, num_pages, page_size, ctx_lo, ctx_hi)
    return MlaDrafterInputs(
        name=f"mla_drafter_B{B}_T{T_req}", B=B, T_req=T_req, hidden=hidden, q_lora_rank=q_lora_rank,
        kv_lora_rank=kv_lora_rank, qk_nope_head_dim=qk_nope_head_dim, qk_rope_head_dim=qk_rope_head_dim,
        heads=heads, eps=1e-6, theta=1e4, x=x, w_input_ln=w_in, w_q_a=w_qa, w_q_a_ln=w_qa_ln, w_q_b=w_qb,
        w_uk=w_uk, w_kv_a=w_kva, w_kv_a_ln=w_kva_ln, positions=pos, block_table=table, tokens_per_req=T_req,
        page_size=page_size, num_pages=num_pages, extra={"ctx": ctx},
    )


@dataclass
class ProjectionInputs:
    """The QKV projection's input and weight, plus the region's own parameters.

    ``x`` is ``[T, hidden]``; ``w_qkv`` is ``[(n_q + 2 n_kv) * head_dim, hidden]``
    (``[out, in]``: the packed output is ``x @ w_qkv^T``), its head blocks of
    ``head_dim`` rows in the layout's order (``kind``).  bf16 arrays are ``uint16``
    bit patterns.  The weight is N(0, 1/hidden), so the packed values are O(1);
    norm weights are N(1, 0.1).
    """

    name: str
    kind: str
    T: int
    hidden: int
    n_kv: int
    q_per_kv: int
    head_dim: int
    rope: bool
    eps: float
    theta: float
    x: np.ndarray
    w_qkv: np.ndarray
    q_norm_w: np.ndarray
    k_norm_w: np.ndarray
    positions: np.ndarray

    @property
    def n_q(self) -> int:
        return self.n_kv * self.q_per_kv

    @property
    def width(self) -> int:
        return (self.n_q + 2 * self.n_kv) * self.head_dim


def projection(
    kind: str,
    T: int,
    hidden: int,
    n_kv: int,
    q_per_kv: int,
    head_dim: int,
    *,
    rope: bool = True,
    theta: float = 1e6,
    eps: float = 1e-6,
    seed: int = 60,
    positions: str = "arange",
    max_pos: int = 131072,
    name: str = "projection",
) -> ProjectionInputs:
    """bf16 projection inputs.  Draw order: x, w_qkv, q norm weight, k norm weight, positions."""
    rng = np.random.Generator(np.random.PCG64(seed))
    width = (n_kv * q_per_kv + 2 * n_kv) * head_dim
    x = _draw(rng, (T, hidden), "bf16")
    w = _draw(rng, (width, hidden), "bf16", 0.0, float(hidden) ** -0.5)
    wq = _draw(rng, (head_dim,), "bf16", 1.0, 0.1)
    wk = _draw(rng, (head_dim,), "bf16", 1.0, 0.1)
    if positions == "arange":
        pos = np.arange(T, dtype=np.int32)
    elif positions == "random":
        pos = rng.integers(0, max_pos, size=T, dtype=np.int64).astype(np.int32)
    else:
        raise ValueError(positions)
    return ProjectionInputs(name=name, kind=kind, T=T, hidden=hidden, n_kv=n_kv, q_per_kv=q_per_kv,
                            head_dim=head_dim, rope=rope, eps=eps, theta=theta, x=x, w_qkv=w,
                            q_norm_w=wq, k_norm_w=wk, positions=pos)
