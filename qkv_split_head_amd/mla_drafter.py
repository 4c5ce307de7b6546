"""One MLA drafter layer's q path and kv path, side by side on two HIP streams.

TensorRT-LLM page "MLA DSpark: run each drafter layer's kv path beside its q
path", Description: after the layer's input norm, the kv path (kv_a
projection -> RMSNorm/RoPE of the latent row -> block write into the context
pool) and the q path (q_a projection -> q_a norm -> q_b projection -> RoPE of
each head's rope part -> k absorption) are independent until attention.  With
the split switch on, the layer forks the kv path to an auxiliary stream after
the input norm and joins it before returning (where attention would start):

* everything the auxiliary stream reads (the normed input, the positions, the
  block table, the weights) is written before the fork, and everything it
  writes (the pool rows) is read only after the join;
* the fork/join are events, so the layer can be captured in a HIP graph, where
  they become graph edges;
* the switch is read per call (argument, else the ``QKVNR_MLA_SPLIT_STREAMS``
  environment variable), as the page's own switch is.

The latent row's RMSNorm/RoPE and its pool store run in this library's kernel
(``qkvnr_forward_paged`` on a LATENT layout).  With ``direct_pool_write`` off,
the kernel writes a contiguous staging buffer instead and a scatter moves the
rows into the pool (the page's "staged write"; the two are bitwise equal).
The q path's rotation of each head's rope part ("rope_into") is this
library's ``qkvnr_rope_inplace``; the projections are plain library GEMMs
(torch -> hipBLASLt) and the two RMSNorms of the layer's input and of q_a are
torch's: the q path is the work the kv path hides behind.

Shapes follow DeepSeek-V3-style MLA at one rank's share of 8-way tensor
parallelism (the page measures a Kimi drafter at per-rank shapes it does not
print): hidden 7168, q_lora_rank 1536, kv_lora_rank 512, per-head nope 128 and
rope 64, 16 heads.
"""
from __future__ import annotations

import os
from dataclasses import dataclass
from typing import Dict, Optional, Tuple

import torch
import torch.nn.functional as F

from . import _binding as b

ENV_SPLIT = "QKVNR_MLA_SPLIT_STREAMS"


@dataclass(frozen=True)
class MlaDims:
    hidden: int = 7168
    q_lora_rank: int = 1536
    kv_lora_rank: int = 512
    qk_nope_head_dim: int = 128
    qk_rope_head_dim: int = 64
    heads: int = 16
    eps: float = 1e-6
    theta: float = 1e4

    @property
    def q_head_dim(self) -> int:
        return self.qk_nope_head_dim + self.qk_rope_head_dim


def split_streams_requested(split: Optional[bool]) -> bool:
    """The per-call switch: an explicit argument wins, else the environment variable."""
    if split is not None:
        return bool(split)
    return os.environ.get(ENV_SPLIT, "0").strip().lower() in ("1", "true", "yes", "on")


class MlaDrafterLayer:
    """Weights of one layer (bf16, projections stored ``[in, out]``) and its forward.

    ``forward`` returns ``(q_absorbed [heads, N, kv_lora_rank], q_pe [N, heads,
    rope])`` (q_pe a view into the q projection's output) and leaves the N latent rows in ``pool [num_pages, page, kv_lora +
    rope]`` at the block-table slots of their positions (tokens the table does
    not map are not stored).  All work is enqueued on the current stream (and,
    split, on the layer's auxiliary stream, joined back before return).
    """

    def __init__(self, weights: Dict[str, torch.Tensor], dims: MlaDims = MlaDims()):
        self.dims = dims
        need = ("w_input_ln", "w_q_a", "w_q_a_ln", "w_q_b", "w_uk", "w_kv_a", "w_kv_a_ln")
        for k in need:
            t = weights[k]
            if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"{k} must be a contiguous bf16 device tensor")
        d = dims
        shapes = {
            "w_input_ln": (d.hidden,), "w_q_a": (d.hidden, d.q_lora_rank), "w_q_a_ln": (d.q_lora_rank,),
            "w_q_b": (d.q_lora_rank, d.heads * d.q_head_dim),
            "w_uk": (d.heads, d.qk_nope_head_dim, d.kv_lora_rank),
            "w_kv_a": (d.hidden, d.kv_lora_rank + d.qk_rope_head_dim), "w_kv_a_ln": (d.kv_lora_rank,),
        }
        for k, s in shapes.items():
            if tuple(weights[k].shape) != s:
                raise ValueError(f"{k} has shape {tuple(weights[k].shape)}, expected {s}")
        self.w = {k: weights[k] for k in need}
        # projections kept [out, in] for F.linear: the library GEMMs are 2-4x
        # faster on these skinny products in that layout than on x @ W
        self.wt = {k: weights[k].t().contiguous() for k in ("w_q_a", "w_q_b", "w_kv_a")}
        # the merged schedule's one projection: [q_a rows; kv_a rows] of [out, in]
        self.wt["w_qkv_a"] = torch.cat([self.wt["w_q_a"], self.wt["w_kv_a"]], dim=0)
        self._aux: Optional[torch.cuda.Stream] = None
        self._fork = torch.cuda.Event()
        self._join = torch.cuda.Event()

    # ------------------------------------------------------------------ streams

    def aux_stream(self) -> torch.cuda.Stream:
        """The auxiliary stream, created on first use (default priority)."""
        if self._aux is None:
            self._aux = torch.cuda.Stream(device=self.w["w_q_a"].device)
        return self._aux

    # ------------------------------------------------------------------ paths

    def input_norm(self, x: torch.Tensor) -> torch.Tensor:
        d = self.dims
        return F.rms_norm(x, (d.hidden,), self.w["w_input_ln"], d.eps)

    def q_path(self, xn: torch.Tensor, positions: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
        return self.q_from_q_a(F.linear(xn, self.wt["w_q_a"]), positions)

    def q_from_q_a(self, q_a: torch.Tensor, positions: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
        """The q path after its projection: q_a norm -> q_b -> RoPE of the rope parts -> k absorption."""
        d = self.dims
        N = q_a.shape[0]
        q_a = F.rms_norm(q_a, (d.q_lora_rank,), self.w["w_q_a_ln"], d.eps)
        q = F.linear(q_a, self.wt["w_q_b"]).view(N, d.heads, d.q_head_dim)
        # "rope_into": the library kernel rotates each head's rope part in place
        b.rope_inplace(q, positions, rope_offset=d.qk_nope_head_dim, rope_dim=d.qk_rope_head_dim, theta=d.theta)
        # k absorption: each head's nope part times that head's W_UK
        q_abs = torch.bmm(q[..., : d.qk_nope_head_dim].transpose(0, 1).contiguous(), self.w["w_uk"])
        return q_abs, q[..., d.qk_nope_head_dim:]

    def kv_a(self, xn: torch.Tensor) -> torch.Tensor:
        """The kv_a projection: latent rows [N, kv_lora_rank + rope] before their norm/RoPE."""
        return F.linear(xn, self.wt["w_kv_a"])

    def qkv_a(self, xn: torch.Tensor) -> torch.Tensor:
        """The merged schedule's projection: [q_a (q_lora_rank) || kv_a (kv_lora_rank + rope)] per token."""
        return F.linear(xn, self.wt["w_qkv_a"])

    def kv_path(self, xn: torch.Tensor, positions: torch.Tensor, block_table: torch.Tensor,
                pool: torch.Tensor, tokens_per_req: int, direct_pool_write: bool,
                slots: Optional[torch.Tensor] = None) -> None:
        self.kv_store(self.kv_a(xn), positions, block_table, pool, tokens_per_req, direct_pool_write, slots)

    def kv_store(self, kv: torch.Tensor, positions: torch.Tensor, block_table: torch.Tensor, pool: torch.Tensor,
                 tokens_per_req: int, direct_pool_write: bool, slots: Optional[torch.Tensor] = None) -> None:
        """RMSNorm/RoPE of the latent rows kv (dense rows, any row stride) and their pool write."""
        d = self.dims
        if direct_pool_write:
            b.forward_latent_paged(kv, positions, self.w["w_kv_a_ln"], block_table, pool,
                                   tokens_per_req=tokens_per_req, eps=d.eps, theta=d.theta,
                                   norm_dim=d.kv_lora_rank, rope_dim=d.qk_rope_head_dim)
            return
        rows = b.forward_latent(kv, positions, self.w["w_kv_a_ln"], eps=d.eps, theta=d.theta,
                                norm_dim=d.kv_lora_rank, rope_dim=d.qk_rope_head_dim)
        if slots is None:
            slots = staged_slots(positions, block_table, tokens_per_req, pool.shape[1], pool.shape[0] * pool.shape[1])
        flat = pool.view(-1, pool.shape[-1])
        flat.index_copy_(0, slots, rows)

    # ------------------------------------------------------------------ layer

    def forward(self, x: torch.Tensor, positions: torch.Tensor, block_table: torch.Tensor,
                pool: torch.Tensor, tokens_per_req: int, *, split_streams: Optional[bool] = None,
                direct_pool_write: bool = True, merge_kv_a: bool = False, slots: Optional[torch.Tensor] = None,
                aux_delay_cycles: int = 0, main_delay_cycles: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
        """One decode step of the layer.

        Three schedules of the same arithmetic:
        * serial (default): kv path, then q path, on the current stream;
        * split (``split_streams``, or the environment switch): the kv path on
          the auxiliary stream between a fork and a join, as the page does;
        * merged (``merge_kv_a``; the switch is then not read): the q_a and
          kv_a projections as one GEMM over both weights (they read the same
          normed input), then the latent rows' norm/RoPE/pool write and the
          rest of the q path, on the current stream.  On this GPU a fork/join
          inside a HIP graph costs more than the kv path it would hide (see the
          design notes), and the merged projection removes most of that path.
        ``slots`` (the staged write only) are the tokens' flat pool slots from
        :func:`staged_slots`, computed once per step; ``aux_delay_cycles`` /
        ``main_delay_cycles`` enqueue a spin kernel at the head of the kv path /
        q path: with the fork and join in place, delaying either stream must
        not change a bit (the page's delay controls).
        """
        d = self.dims
        N = x.shape[0]
        if x.shape != (N, d.hidden) or positions.shape != (N,):
            raise ValueError("x must be [N, hidden] and positions [N]")
        if pool.shape[-1] != d.kv_lora_rank + d.qk_rope_head_dim:
            raise ValueError("pool rows must hold kv_lora_rank + rope values")
        if not direct_pool_write and slots is None and not torch.cuda.is_current_stream_capturing():
            _, ok = pool_slots(positions, block_table, tokens_per_req, pool.shape[1], pool.shape[0])
            if not bool(ok.all()):
                raise ValueError("the staged pool write needs every token mapped by the block table")
        xn = self.input_norm(x)
        if merge_kv_a:
            qkv_a = self.qkv_a(xn)
            self.kv_store(qkv_a[:, d.q_lora_rank:], positions, block_table, pool, tokens_per_req,
                          direct_pool_write, slots)
            return self.q_from_q_a(qkv_a[:, : d.q_lora_rank], positions)
        if not split_streams_requested(split_streams):
            if aux_delay_cycles:
                torch.cuda._sleep(aux_delay_cycles)
            self.kv_path(xn, positions, block_table, pool, tokens_per_req, direct_pool_write, slots)
            if main_delay_cycles:
                torch.cuda._sleep(main_delay_cycles)
            return self.q_path(xn, positions)
        main = torch.cuda.current_stream()
        aux = self.aux_stream()
        self._fork.record(main)
        aux.wait_event(self._fork)
        with torch.cuda.stream(aux):
            if aux_delay_cycles:
                torch.cuda._sleep(aux_delay_cycles)
            self.kv_path(xn, positions, block_table, pool, tokens_per_req, direct_pool_write, slots)
            self._join.record(aux)
        # tensors made on the main stream and read on the auxiliary one stay
        # allocated until the auxiliary stream's work is done
        for t in (xn, positions, block_table) + ((slots,) if slots is not None else ()):
            t.record_stream(aux)
        if main_delay_cycles:
            torch.cuda._sleep(main_delay_cycles)
        out = self.q_path(xn, positions)
        main.wait_event(self._join)
        return out


def staged_slots(positions: torch.Tensor, block_table: torch.Tensor, tokens_per_req: int, page_size: int,
                 num_slots: int) -> torch.Tensor:
    """Flat pool slots for the staged write (every token must be mapped; see :func:`pool_slots`),
    clamped into [0, num_slots) so that the scatter stays in bounds whatever the table holds."""
    slot, _ = pool_slots(positions, block_table, tokens_per_req, page_size, num_slots // page_size)
    return slot.clamp(0, num_slots - 1)


def pool_slots(positions: torch.Tensor, block_table: torch.Tensor, tokens_per_req: int,
               page_size: int, num_pages: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """Flat pool slot of each token and whether the table maps it (for the staged write,
    whose scatter needs every token mapped, as a drafter's tokens always are).  A token is
    mapped when its position is >= 0, its page index is inside the table's row and the
    page id is in [0, num_pages): the rule of the direct pool write, which skips any other
    token."""
    N = positions.shape[0]
    pos = positions.to(torch.int64)
    req = torch.arange(N, device=positions.device) // tokens_per_req
    pi = pos // page_size
    ok = (pos >= 0) & (pi < block_table.shape[1])
    page = block_table[req, pi.clamp(0, block_table.shape[1] - 1)].to(torch.int64)
    ok = ok & (page >= 0) & (page < num_pages)
    return page * page_size + pos % page_size, ok
