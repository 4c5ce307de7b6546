"""qkvnr: packed-QKV split + per-head RMSNorm + RoPE on MI355X (gfx950).

Python face of ``libqkvnr.so`` (C ABI in ``include/qkvnr.h``).  The functions
named like the C entry points (``qkvnr_forward``, ``qkvnr_backward``,
``qkvnr_forward_paged``) pass tensors straight through; ``forward``,
``backward``, ``forward_paged``, ``forward_latent`` and
``forward_latent_paged`` also allocate the outputs; ``rope_inplace`` rotates a
tensor's rope parts in place.  ``mla_drafter`` runs an MLA drafter layer's kv
path beside its q path on two streams; ``muon`` runs per-head Newton-Schulz
on fused QKV weights; ``proj_forward`` (``qkvnr_proj_forward``) runs the
QKV projection with the split, norms and RoPE in its epilogue.
"""
from ._binding import (  # noqa: F401
    BF16,
    EALIGN,
    EHIP,
    EINVAL,
    EUNSUPPORTED,
    FP32,
    INTERLEAVED,
    LATENT,
    OK,
    SECTIONED,
    Layout,
    QkvnrError,
    backward,
    backward_workspace,
    forward,
    forward_latent,
    forward_latent_paged,
    forward_paged,
    gqa_layout,
    header_functions,
    latent_layout,
    lib,
    proj_forward,
    qkvnr_backward,
    qkvnr_backward_noalloc,
    qkvnr_backward_workspace_bytes,
    qkvnr_forward,
    qkvnr_forward_paged,
    qkvnr_fused_head_blocks,
    qkvnr_gram_partials,
    qkvnr_ns_apply,
    qkvnr_ns_collapse,
    qkvnr_ns_poly,
    qkvnr_ns_update,
    qkvnr_proj_forward,
    qkvnr_rope_inplace,
    rope_inplace,
    qkvnr_version,
)
