"""ctypes binding of libqkvnr.so.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  torch is used for device memory (allocating outputs) and to name the
current HIP stream; there is no other code path, and loading fails loudly when
the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqkvnr.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "qkvnr.h")

# Mirrors of the header's constants.
OK, EINVAL, EALIGN, EUNSUPPORTED, EHIP = 0, -1, -2, -3, -4
INTERLEAVED, SECTIONED, LATENT = 0, 1, 2
BF16, FP32 = 0, 1
KINDS = {"interleaved": INTERLEAVED, "sectioned": SECTIONED, "latent": LATENT}
DTYPES = {torch.bfloat16: BF16, torch.float32: FP32}


class Layout(ctypes.Structure):
    """``qkvnr_layout`` of the header."""

    _fields_ = [
        ("kind", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("T", ctypes.c_int64),
        ("n_kv", ctypes.c_int32),
        ("q_per_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("rope_dim", ctypes.c_int32),
        ("norm_dim", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("width", ctypes.c_int64),
        ("in_row_stride", ctypes.c_int64),
    ]


class QkvnrError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"qkvnr error {code}: {message}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first (python -m qkv_split_head_amd.build); "
                "there is no fallback implementation")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32p, f32p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
        lp = ctypes.POINTER(Layout)
        L.qkvnr_forward.argtypes = [lp, vp, i32p, vp, vp, ctypes.c_float, ctypes.c_double, vp, vp, vp, vp]
        L.qkvnr_forward.restype = ctypes.c_int
        L.qkvnr_backward.argtypes = [lp, vp, i32p, vp, vp, ctypes.c_float, ctypes.c_double, vp, vp, vp, vp,
                                     f32p, f32p, vp, ctypes.c_int64, vp]
        L.qkvnr_backward.restype = ctypes.c_int
        L.qkvnr_backward_noalloc.argtypes = [lp, vp, i32p, vp, vp, ctypes.c_float, ctypes.c_double, vp, vp, vp,
                                             vp, f32p, f32p, vp]
        L.qkvnr_backward_noalloc.restype = ctypes.c_int
        L.qkvnr_backward_workspace_bytes.argtypes = [lp]
        L.qkvnr_backward_workspace_bytes.restype = ctypes.c_int64
        L.qkvnr_forward_paged.argtypes = [lp, vp, i32p, vp, vp, ctypes.c_float, ctypes.c_double, i32p,
                                          ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                          vp, vp, vp, vp]
        L.qkvnr_forward_paged.restype = ctypes.c_int
        L.qkvnr_rope_inplace.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int64,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, i32p, ctypes.c_double,
                                         vp, vp]
        L.qkvnr_rope_inplace.restype = ctypes.c_int
        L.qkvnr_fused_head_blocks.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                              ctypes.POINTER(ctypes.c_int64)]
        L.qkvnr_fused_head_blocks.restype = ctypes.c_int
        L.qkvnr_gram_partials.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int64, vp, ctypes.c_int32,
                                          vp, vp]
        L.qkvnr_gram_partials.restype = ctypes.c_int
        L.qkvnr_ns_poly.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, vp, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_float, ctypes.c_float, vp, vp]
        L.qkvnr_ns_poly.restype = ctypes.c_int
        L.qkvnr_ns_update.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int64, vp, vp, vp, ctypes.c_int32,
                                      vp, vp]
        L.qkvnr_ns_update.restype = ctypes.c_int
        L.qkvnr_ns_collapse.argtypes = [ctypes.c_int64, ctypes.c_int32, vp, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_float, ctypes.c_float, vp, vp]
        L.qkvnr_ns_collapse.restype = ctypes.c_int
        L.qkvnr_ns_apply.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int64, vp, vp, vp, ctypes.c_int32, vp]
        L.qkvnr_ns_apply.restype = ctypes.c_int
        L.qkvnr_proj_forward.argtypes = [lp, ctypes.c_int64, vp, vp, i32p, vp, vp, ctypes.c_float, ctypes.c_double,
                                         vp, vp, vp, vp]
        L.qkvnr_proj_forward.restype = ctypes.c_int
        L.qkvnr_strerror.argtypes = [ctypes.c_int]
        L.qkvnr_strerror.restype = ctypes.c_char_p
        L.qkvnr_version.argtypes = []
        L.qkvnr_version.restype = ctypes.c_int
        _lib = L
    return _lib


def header_functions() -> list:
    """Names of the functions ``include/qkvnr.h`` declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(qkvnr_\w+)\s*\(", text, re.M)))


def _check(rc: int) -> None:
    if rc != OK:
        raise QkvnrError(rc, lib().qkvnr_strerror(rc).decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _need(t, name: str, *, device: Optional[torch.device] = None, dtype=None, shape=None,
          contiguous: bool = True) -> None:
    """Checks a tensor argument of the tensor-level wrappers before its address reaches a kernel.

    The C ABI sees plain pointers and cannot tell a host address, a wrong
    element type or a buffer too small for the sizes it is given; these
    wrappers know the shapes, so they reject such arguments here.  ``device``
    None means the current GPU.
    """
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor, not {type(t).__name__}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} is on {t.device}; the library's kernels need GPU tensors")
    want = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    if t.device != want:
        raise ValueError(f"{name} is on {t.device}; it must be on {want} (the current GPU)")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_inputs(x: torch.Tensor, positions, q_norm_w, k_norm_w, head_dim: int, need_pos: bool) -> None:
    """positions int32 [T] and norm weights [head_dim] of x's dtype, all on x's (current) device."""
    _need(x, "the packed input", contiguous=False)
    T = x.shape[0]
    if positions is not None or need_pos:
        _need(positions, "positions", device=x.device, dtype=torch.int32, shape=(T,))
    for w, nm in ((q_norm_w, "q_norm_w"), (k_norm_w, "k_norm_w")):
        if w is not None:
            _need(w, nm, device=x.device, dtype=x.dtype, shape=(head_dim,))


# ------------------------------------------------------------------ raw entry points


def qkvnr_forward(layout: Layout, qkv, positions, q_norm_w, k_norm_w, eps: float, theta: float, q, k, v,
                  stream=None) -> None:
    """Call ``qkvnr_forward``: tensors (or raw device addresses) in, outputs written in place."""
    _check(lib().qkvnr_forward(ctypes.byref(layout), _ptr(qkv), _ptr(positions), _ptr(q_norm_w), _ptr(k_norm_w),
                               eps, theta, _ptr(q), _ptr(k), _ptr(v), _stream(stream)))


def qkvnr_backward(layout: Layout, qkv, positions, q_norm_w, k_norm_w, eps: float, theta: float, dq, dk, dv,
                   dqkv, dq_norm_w, dk_norm_w, workspace, workspace_bytes: int, stream=None) -> None:
    """Call ``qkvnr_backward``."""
    _check(lib().qkvnr_backward(ctypes.byref(layout), _ptr(qkv), _ptr(positions), _ptr(q_norm_w), _ptr(k_norm_w),
                                eps, theta, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dqkv), _ptr(dq_norm_w),
                                _ptr(dk_norm_w), _ptr(workspace), workspace_bytes, _stream(stream)))


def qkvnr_backward_noalloc(layout: Layout, qkv, positions, q_norm_w, k_norm_w, eps: float, theta: float, dq, dk,
                           dv, dqkv, dq_norm_w, dk_norm_w, stream=None) -> None:
    """Call ``qkvnr_backward_noalloc`` (the weight-grad slots live inside the library)."""
    _check(lib().qkvnr_backward_noalloc(ctypes.byref(layout), _ptr(qkv), _ptr(positions), _ptr(q_norm_w),
                                        _ptr(k_norm_w), eps, theta, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dqkv),
                                        _ptr(dq_norm_w), _ptr(dk_norm_w), _stream(stream)))


def qkvnr_backward_workspace_bytes(layout: Layout) -> int:
    return lib().qkvnr_backward_workspace_bytes(ctypes.byref(layout))


_workspaces = {}


def backward_workspace(device=None) -> torch.Tensor:
    """The zero-filled backward workspace this module keeps for a device.

    Every completed backward call leaves it zero again, so calls issued in
    sequence can share it.  Calls that may overlap (different streams) must
    pass workspaces of their own.  Allocated on first use, which must not
    happen during HIP-graph capture.
    """
    dev = torch.device("cuda", torch.cuda.current_device() if device is None else torch.device(device).index)
    ws = _workspaces.get(dev.index)
    if ws is None:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError("the backward workspace is allocated on first use: run one backward call "
                               "before capturing it in a graph, or pass workspace=")
        size = lib().qkvnr_backward_workspace_bytes(None)
        ws = torch.zeros(size, dtype=torch.uint8, device=dev)
        _workspaces[dev.index] = ws
    return ws


def _keep_workspace_clean(call, ws, device_index) -> None:
    """Runs a backward call on workspace ``ws``.  A call that fails with QKVNR_EHIP
    may have enqueued kernels whose partial sums stay in the workspace (the
    library still enqueues the fold that zeroes them, but that launch may have
    failed too), so this module's cached workspace of that device is dropped and
    the next call allocates a zero-filled one.  Validation errors enqueue nothing
    and keep it."""
    try:
        call()
    except QkvnrError as e:
        if e.code == EHIP and _workspaces.get(device_index) is ws:
            del _workspaces[device_index]
        raise


def qkvnr_forward_paged(layout: Layout, qkv, positions, q_norm_w, k_norm_w, eps: float, theta: float,
                        block_table, bt_stride: int, tokens_per_req: int, page_size: int, num_pages: int,
                        q, k_pool, v_pool, stream=None) -> None:
    """Call ``qkvnr_forward_paged``."""
    _check(lib().qkvnr_forward_paged(ctypes.byref(layout), _ptr(qkv), _ptr(positions), _ptr(q_norm_w),
                                     _ptr(k_norm_w), eps, theta, _ptr(block_table), bt_stride, tokens_per_req,
                                     page_size, num_pages, _ptr(q), _ptr(k_pool), _ptr(v_pool), _stream(stream)))


def qkvnr_rope_inplace(dtype: int, T: int, heads: int, token_stride: int, head_stride: int, rope_offset: int,
                       rope_dim: int, positions, theta: float, x, stream=None) -> None:
    """Call ``qkvnr_rope_inplace``."""
    _check(lib().qkvnr_rope_inplace(dtype, T, heads, token_stride, head_stride, rope_offset, rope_dim,
                                    _ptr(positions), theta, _ptr(x), _stream(stream)))


def qkvnr_fused_head_blocks(n_q: int, n_kv: int, head_dim: int, weight_rows: int) -> int:
    """Head blocks of a fused q|k|v weight (the exact-total guard); raises QkvnrError when declined."""
    out = ctypes.c_int64(0)
    _check(lib().qkvnr_fused_head_blocks(n_q, n_kv, head_dim, weight_rows, ctypes.byref(out)))
    return out.value


def qkvnr_gram_partials(blocks: int, d: int, cols: int, x, parts: int, out, stream=None) -> None:
    """Call ``qkvnr_gram_partials``."""
    _check(lib().qkvnr_gram_partials(blocks, d, cols, _ptr(x), parts, _ptr(out), _stream(stream)))


def qkvnr_ns_poly(dtype: int, blocks: int, d: int, gram, parts: int, first: bool, scale: float, eps: float, p,
                  stream=None) -> None:
    """Call ``qkvnr_ns_poly``."""
    _check(lib().qkvnr_ns_poly(dtype, blocks, d, _ptr(gram), parts, 1 if first else 0, scale, eps, _ptr(p),
                               _stream(stream)))


def qkvnr_ns_update(blocks: int, d: int, cols: int, p, x, y, parts: int, gram=None, stream=None) -> None:
    """Call ``qkvnr_ns_update`` (``gram`` None: no Gram partials)."""
    _check(lib().qkvnr_ns_update(blocks, d, cols, _ptr(p), _ptr(x), _ptr(y), parts, _ptr(gram), _stream(stream)))


def qkvnr_ns_collapse(blocks: int, d: int, gram, parts: int, steps: int, scale: float, eps: float, m,
                      stream=None) -> None:
    """Call ``qkvnr_ns_collapse`` (the whole iteration as M, from the Gram partials of G)."""
    _check(lib().qkvnr_ns_collapse(blocks, d, _ptr(gram), parts, steps, scale, eps, _ptr(m), _stream(stream)))


def qkvnr_ns_apply(blocks: int, d: int, cols: int, m, x, y, parts: int, stream=None) -> None:
    """Call ``qkvnr_ns_apply`` (Y = (M hi + M lo) X)."""
    _check(lib().qkvnr_ns_apply(blocks, d, cols, _ptr(m), _ptr(x), _ptr(y), parts, _stream(stream)))


def qkvnr_proj_forward(layout: Layout, hidden: int, x, w_qkv, positions, q_norm_w, k_norm_w, eps: float,
                       theta: float, q, k, v, stream=None) -> None:
    """Call ``qkvnr_proj_forward``."""
    _check(lib().qkvnr_proj_forward(ctypes.byref(layout), hidden, _ptr(x), _ptr(w_qkv), _ptr(positions),
                                    _ptr(q_norm_w), _ptr(k_norm_w), eps, theta, _ptr(q), _ptr(k), _ptr(v),
                                    _stream(stream)))


def qkvnr_version() -> int:
    return lib().qkvnr_version()


# ------------------------------------------------------------------ tensor-level wrappers


def gqa_layout(qkv: torch.Tensor, kind: str, n_kv: int, q_per_kv: int, head_dim: int, rope: bool) -> Layout:
    """Describe a packed GQA tensor whose rows may be strided but whose row contents are dense."""
    if qkv.dtype not in DTYPES:
        raise TypeError(f"qkv dtype {qkv.dtype} is not bf16 or fp32")
    T = qkv.shape[0]
    width = (n_kv * q_per_kv + 2 * n_kv) * head_dim
    if T > 0:
        if qkv[0].numel() != width:
            raise ValueError(f"packed row holds {qkv[0].numel()} values, not (n_q + 2 n_kv) * head_dim = {width}")
        if not qkv[0].is_contiguous():
            raise ValueError("the values of a packed row must be dense")
    row_stride = qkv.stride(0) if T > 1 else width
    return Layout(kind=KINDS[kind], dtype=DTYPES[qkv.dtype], T=T, n_kv=n_kv, q_per_kv=q_per_kv, head_dim=head_dim,
                  rope_dim=head_dim if rope else 0, norm_dim=0, reserved=0, width=width, in_row_stride=row_stride)


def latent_layout(rows: torch.Tensor, norm_dim: int = 512, rope_dim: int = 64) -> Layout:
    if rows.dim() != 2 or rows.stride(1) != 1:
        raise ValueError("latent rows must be a 2-D tensor with dense rows")
    T = rows.shape[0]
    width = norm_dim + rope_dim
    return Layout(kind=LATENT, dtype=DTYPES[rows.dtype], T=T, n_kv=1, q_per_kv=0, head_dim=0, rope_dim=rope_dim,
                  norm_dim=norm_dim, reserved=0, width=width, in_row_stride=rows.stride(0) if T > 1 else width)


def forward(qkv: torch.Tensor, positions: Optional[torch.Tensor], q_norm_w: torch.Tensor, k_norm_w: torch.Tensor,
            *, kind: str, n_kv: int, q_per_kv: int, head_dim: int, rope: bool = True, eps: float = 1e-6,
            theta: float = 10000.0, out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
            stream=None):
    """Split + q/k RMSNorm + RoPE + v copy; returns contiguous (q [T,n_q,D], k [T,n_kv,D], v [T,n_kv,D])."""
    L = gqa_layout(qkv, kind, n_kv, q_per_kv, head_dim, rope)
    _need_inputs(qkv, positions, q_norm_w, k_norm_w, head_dim, rope)
    T = qkv.shape[0]
    if out is None:
        q = torch.empty((T, n_kv * q_per_kv, head_dim), dtype=qkv.dtype, device=qkv.device)
        k = torch.empty((T, n_kv, head_dim), dtype=qkv.dtype, device=qkv.device)
        v = torch.empty((T, n_kv, head_dim), dtype=qkv.dtype, device=qkv.device)
    else:
        q, k, v = out
        _need(q, "q", device=qkv.device, dtype=qkv.dtype, shape=(T, n_kv * q_per_kv, head_dim))
        _need(k, "k", device=qkv.device, dtype=qkv.dtype, shape=(T, n_kv, head_dim))
        _need(v, "v", device=qkv.device, dtype=qkv.dtype, shape=(T, n_kv, head_dim))
    qkvnr_forward(L, qkv, positions, q_norm_w, k_norm_w, eps, theta, q, k, v, stream)
    return q, k, v


def backward(qkv: torch.Tensor, positions: Optional[torch.Tensor], q_norm_w: torch.Tensor, k_norm_w: torch.Tensor,
             dq: torch.Tensor, dk: torch.Tensor, dv: torch.Tensor, *, kind: str, n_kv: int, q_per_kv: int,
             head_dim: int, rope: bool = True, eps: float = 1e-6, theta: float = 10000.0, out=None,
             workspace: Optional[torch.Tensor] = None, stream=None):
    """Packed dqkv (input layout) and fp32 norm-weight grads (dq_norm_w, dk_norm_w)."""
    L = gqa_layout(qkv, kind, n_kv, q_per_kv, head_dim, rope)
    _need_inputs(qkv, positions, q_norm_w, k_norm_w, head_dim, rope)
    T, n_q = qkv.shape[0], n_kv * q_per_kv
    _need(dq, "dq", device=qkv.device, dtype=qkv.dtype, shape=(T, n_q, head_dim))
    _need(dk, "dk", device=qkv.device, dtype=qkv.dtype, shape=(T, n_kv, head_dim))
    _need(dv, "dv", device=qkv.device, dtype=qkv.dtype, shape=(T, n_kv, head_dim))
    if out is None:
        dqkv = torch.empty_strided(qkv.shape, qkv.stride(), dtype=qkv.dtype, device=qkv.device)
        dwq = torch.empty(head_dim, dtype=torch.float32, device=qkv.device)
        dwk = torch.empty(head_dim, dtype=torch.float32, device=qkv.device)
    else:
        dqkv, dwq, dwk = out
        _need(dqkv, "dqkv", device=qkv.device, dtype=qkv.dtype, shape=qkv.shape, contiguous=False)
        if T > 1 and dqkv.stride(0) != qkv.stride(0):   # written with the input's row stride
            raise ValueError(f"dqkv has row stride {dqkv.stride(0)}, the packed input {qkv.stride(0)}")
        if T > 0 and not dqkv[0].is_contiguous():
            raise ValueError("the values of a dqkv row must be dense")
        _need(dwq, "dq_norm_w", device=qkv.device, dtype=torch.float32, shape=(head_dim,))
        _need(dwk, "dk_norm_w", device=qkv.device, dtype=torch.float32, shape=(head_dim,))
    ws = backward_workspace(qkv.device) if workspace is None else workspace
    _need(ws, "workspace", device=qkv.device)
    _keep_workspace_clean(
        lambda: qkvnr_backward(L, qkv, positions, q_norm_w, k_norm_w, eps, theta, dq, dk, dv, dqkv, dwq, dwk, ws,
                               ws.numel() * ws.element_size(), stream),
        ws, qkv.device.index)
    return dqkv, dwq, dwk


def _need_table(block_table, device: torch.device, T: int, tokens_per_req: int) -> None:
    """int32 block table with a row for every request of the batch (T / tokens_per_req, rounded up)."""
    _need(block_table, "block_table", device=device, dtype=torch.int32)
    if block_table.dim() != 2:
        raise ValueError("block_table must be [requests, pages per request]")
    if tokens_per_req < 1:
        raise ValueError("tokens_per_req must be >= 1")
    if block_table.shape[0] < -(-T // tokens_per_req):
        raise ValueError(f"block_table has {block_table.shape[0]} rows; {T} tokens of {tokens_per_req} per "
                         f"request need {-(-T // tokens_per_req)}")


def forward_paged(qkv, positions, q_norm_w, k_norm_w, block_table: torch.Tensor, k_pool: torch.Tensor,
                  v_pool: torch.Tensor, *, kind: str, n_kv: int, q_per_kv: int, head_dim: int,
                  tokens_per_req: int, rope: bool = True, eps: float = 1e-6, theta: float = 10000.0,
                  q: Optional[torch.Tensor] = None, stream=None):
    """GQA forward with k/v stored into pools [num_pages, page_size, n_kv, D]; returns q."""
    L = gqa_layout(qkv, kind, n_kv, q_per_kv, head_dim, rope)
    _need_inputs(qkv, positions, q_norm_w, k_norm_w, head_dim, rope)
    T = qkv.shape[0]
    _need_table(block_table, qkv.device, T, tokens_per_req)
    if k_pool.dim() != 4:
        raise ValueError("k_pool must be [num_pages, page_size, n_kv, head_dim]")
    num_pages, page_size = k_pool.shape[0], k_pool.shape[1]
    _need(k_pool, "k_pool", device=qkv.device, dtype=qkv.dtype, shape=(num_pages, page_size, n_kv, head_dim))
    _need(v_pool, "v_pool", device=qkv.device, dtype=qkv.dtype, shape=(num_pages, page_size, n_kv, head_dim))
    if q is None:
        q = torch.empty((T, n_kv * q_per_kv, head_dim), dtype=qkv.dtype, device=qkv.device)
    else:
        _need(q, "q", device=qkv.device, dtype=qkv.dtype, shape=(T, n_kv * q_per_kv, head_dim))
    qkvnr_forward_paged(L, qkv, positions, q_norm_w, k_norm_w, eps, theta, block_table, block_table.shape[1],
                        tokens_per_req, page_size, num_pages, q, k_pool, v_pool, stream)
    return q


def _need_latent(rows: torch.Tensor, positions, norm_w, norm_dim: int) -> None:
    _need(rows, "rows", contiguous=False)
    if rows.dtype not in DTYPES:
        raise TypeError(f"rows dtype {rows.dtype} is not bf16 or fp32")
    _need(positions, "positions", device=rows.device, dtype=torch.int32, shape=(rows.shape[0],))
    _need(norm_w, "norm_w", device=rows.device, dtype=rows.dtype, shape=(norm_dim,))


def forward_latent(rows: torch.Tensor, positions: torch.Tensor, norm_w: torch.Tensor, *, eps: float = 1e-6,
                   theta: float = 10000.0, norm_dim: int = 512, rope_dim: int = 64,
                   out: Optional[torch.Tensor] = None, stream=None):
    """Latent rows [T, norm_dim + rope_dim] -> [RMSNorm(head) || RoPE(tail)], contiguous."""
    L = latent_layout(rows, norm_dim, rope_dim)
    _need_latent(rows, positions, norm_w, norm_dim)
    if out is None:
        out = torch.empty((rows.shape[0], norm_dim + rope_dim), dtype=rows.dtype, device=rows.device)
    else:
        _need(out, "out", device=rows.device, dtype=rows.dtype, shape=(rows.shape[0], norm_dim + rope_dim))
    qkvnr_forward(L, rows, positions, None, norm_w, eps, theta, None, out, None, stream)
    return out


def forward_latent_paged(rows: torch.Tensor, positions: torch.Tensor, norm_w: torch.Tensor,
                         block_table: torch.Tensor, pool: torch.Tensor, *, tokens_per_req: int,
                         eps: float = 1e-6, theta: float = 10000.0, norm_dim: int = 512, rope_dim: int = 64,
                         stream=None) -> None:
    """Latent rows stored straight into pool [num_pages, page_size, norm_dim + rope_dim]."""
    L = latent_layout(rows, norm_dim, rope_dim)
    _need_latent(rows, positions, norm_w, norm_dim)
    _need_table(block_table, rows.device, rows.shape[0], tokens_per_req)
    if pool.dim() != 3:
        raise ValueError("pool must be [num_pages, page_size, norm_dim + rope_dim]")
    _need(pool, "pool", device=rows.device, dtype=rows.dtype, shape=(pool.shape[0], pool.shape[1], norm_dim + rope_dim))
    qkvnr_forward_paged(L, rows, positions, None, norm_w, eps, theta, block_table, block_table.shape[1],
                        tokens_per_req, pool.shape[1], pool.shape[0], None, pool, None, stream)


def rope_inplace(x: torch.Tensor, positions: torch.Tensor, *, rope_offset: int, rope_dim: int = 64,
                 theta: float = 10000.0, stream=None) -> torch.Tensor:
    """Rotate x[..., rope_offset:rope_offset + rope_dim] in place; x is [T, heads, head_stride]
    with a contiguous last dimension (token and head strides taken from the tensor)."""
    if x.dim() != 3 or x.stride(2) != 1:
        raise ValueError("x must be [T, heads, head_stride] with a contiguous last dimension")
    if x.dtype not in DTYPES:
        raise ValueError(f"unsupported dtype {x.dtype}")
    _need(x, "x", contiguous=False)
    _need(positions, "positions", device=x.device, dtype=torch.int32, shape=(x.shape[0],))
    if rope_offset < 0 or rope_dim < 0 or rope_offset + rope_dim > x.shape[2]:
        raise ValueError(f"rotated span [{rope_offset}, {rope_offset + rope_dim}) is outside the {x.shape[2]} "
                         "values of a head")
    qkvnr_rope_inplace(DTYPES[x.dtype], x.shape[0], x.shape[1], x.stride(0), x.stride(1), rope_offset, rope_dim,
                       positions, theta, x, stream)
    return x


def proj_forward(x: torch.Tensor, w_qkv: torch.Tensor, positions: Optional[torch.Tensor], q_norm_w: torch.Tensor,
                 k_norm_w: torch.Tensor, *, kind: str, n_kv: int, q_per_kv: int, head_dim: int, rope: bool = True,
                 eps: float = 1e-6, theta: float = 10000.0,
                 out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None, stream=None):
    """The QKV projection x w_qkv^T with split + q/k RMSNorm + RoPE in its epilogue (bf16).

    x [T, hidden] and w_qkv [(n_q + 2 n_kv) * head_dim, hidden] are contiguous;
    the weight's head blocks are in the ``kind`` order.  Returns contiguous
    (q [T, n_q, D], k [T, n_kv, D], v [T, n_kv, D]).

    The packed product is never rounded, so q, k and v differ from a library
    GEMM followed by ``forward`` by at most a rounding.  It is not the faster
    route on MI355X: at 16384 x 4096 -> 6144 it takes about 700 us against
    about 594 us for ``torch.matmul`` then ``forward``, whose GEMM alone takes
    about 526 us.
    """
    if x.dim() != 2 or w_qkv.dim() != 2 or not x.is_contiguous() or not w_qkv.is_contiguous():
        raise ValueError("x and w_qkv must be contiguous 2-D tensors")
    T, hidden = x.shape
    width = (n_kv * q_per_kv + 2 * n_kv) * head_dim
    if w_qkv.shape[1] != hidden:
        raise ValueError(f"w_qkv has {w_qkv.shape[1]} columns, x has {hidden}")
    _need(x, "x")
    _need(w_qkv, "w_qkv", device=x.device, dtype=x.dtype)
    _need_inputs(x, positions, q_norm_w, k_norm_w, head_dim, rope)
    L = Layout(kind=KINDS[kind], dtype=DTYPES[x.dtype], T=T, n_kv=n_kv, q_per_kv=q_per_kv, head_dim=head_dim,
               rope_dim=head_dim if rope else 0, norm_dim=0, reserved=0, width=w_qkv.shape[0], in_row_stride=width)
    if out is None:
        q = torch.empty((T, n_kv * q_per_kv, head_dim), dtype=x.dtype, device=x.device)
        k = torch.empty((T, n_kv, head_dim), dtype=x.dtype, device=x.device)
        v = torch.empty((T, n_kv, head_dim), dtype=x.dtype, device=x.device)
    else:
        q, k, v = out
        _need(q, "q", device=x.device, dtype=x.dtype, shape=(T, n_kv * q_per_kv, head_dim))
        _need(k, "k", device=x.device, dtype=x.dtype, shape=(T, n_kv, head_dim))
        _need(v, "v", device=x.device, dtype=x.dtype, shape=(T, n_kv, head_dim))
    qkvnr_proj_forward(L, hidden, x, w_qkv, positions, q_norm_w, k_norm_w, eps, theta, q, k, v, stream)
    return q, k, v
