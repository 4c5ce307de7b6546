"""C-ABI library: loading, exported symbols and host-side validation (CPU only).

Every call here is rejected by the host checks before the library makes any
HIP call (or is a T = 0 forward, which enqueues nothing), so the fake device
addresses below are never dereferenced and no kernel is ever launched.
"""
import ctypes
import os
import re

import pytest

import qkv_split_head_amd as qk
from qkv_split_head_amd import Layout

A = 0x7F0000000000  # a 16-byte aligned fake device address, never dereferenced
B = A + (1 << 30)
C = A + (2 << 30)
Dp = A + (3 << 30)
E = A + (4 << 30)
F = A + (5 << 30)


def _lay(kind=qk.INTERLEAVED, dtype=qk.BF16, T=4, n_kv=16, q_per_kv=8, head_dim=64, rope_dim=64, width=None,
         stride=None, norm_dim=0):
    w = (n_kv * q_per_kv + 2 * n_kv) * head_dim if width is None else width
    return Layout(kind=kind, dtype=dtype, T=T, n_kv=n_kv, q_per_kv=q_per_kv, head_dim=head_dim,
                  rope_dim=rope_dim, norm_dim=norm_dim, reserved=0, width=w,
                  in_row_stride=w if stride is None else stride)


def _fwd(L, qkv=A, pos=B, wq=C, wk=C + 4096, q=Dp, k=E, v=F, eps=1e-6, theta=1e4):
    return qk.lib().qkvnr_forward(ctypes.byref(L), qkv, pos, wq, wk, eps, theta, q, k, v, None)


def test_library_exports_every_header_function():
    lib = qk.lib()
    names = qk.header_functions()
    assert {"qkvnr_forward", "qkvnr_backward", "qkvnr_forward_paged", "qkvnr_strerror",
            "qkvnr_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_version_matches_header():
    text = open(os.path.join(os.path.dirname(qk.__file__), "..", "include", "qkvnr.h")).read()
    v = int(re.search(r"#define QKVNR_VERSION (\d+)", text).group(1))
    assert qk.qkvnr_version() == v


def test_layout_struct_matches_c_size():
    # int32 kind, dtype; int64 T; 6 x int32; int64 width, in_row_stride
    assert ctypes.sizeof(Layout) == 56
    assert Layout.width.offset == 40 and Layout.in_row_stride.offset == 48 and Layout.T.offset == 8


def test_null_layout():
    assert qk.lib().qkvnr_forward(None, A, B, C, C, 1e-6, 1e4, Dp, E, F, None) == qk.EINVAL


@pytest.mark.parametrize("field,value", [("kind", 7), ("dtype", 5), ("T", -1), ("n_kv", 0), ("q_per_kv", 0)])
def test_bad_descriptor_fields(field, value):
    L = _lay()
    setattr(L, field, value)
    assert _fwd(L) == qk.EINVAL


def test_exact_total_guard_declines_wrong_width():
    # a descriptor claiming 8 kv heads for a row built with 1 (the multi-query case):
    # (8 + 2*8) * 64 = 1536 described, (8 + 2*1) * 64 = 640 present
    L = _lay(n_kv=8, q_per_kv=1, width=640)
    assert _fwd(L) == qk.EINVAL
    assert "exact total" in qk.lib().qkvnr_strerror(qk.EINVAL).decode()


def test_unsupported_head_dim_and_partial_rope():
    assert _fwd(_lay(head_dim=96, rope_dim=96)) == qk.EUNSUPPORTED
    assert _fwd(_lay(head_dim=64, rope_dim=32)) == qk.EUNSUPPORTED
    assert _fwd(_lay(head_dim=64, rope_dim=33)) == qk.EINVAL
    assert _fwd(_lay(head_dim=64, rope_dim=128)) == qk.EINVAL


def test_row_stride_checks():
    w = (16 * 8 + 32) * 64
    assert _fwd(_lay(stride=w - 8)) == qk.EINVAL
    assert _fwd(_lay(stride=w + 1)) == qk.EALIGN  # 2 bytes past a 16-byte multiple


def test_pointer_checks():
    assert _fwd(_lay(), qkv=0) == qk.EINVAL
    assert _fwd(_lay(), qkv=A + 8) == qk.EALIGN
    assert _fwd(_lay(), pos=0) == qk.EINVAL          # RoPE layer needs positions
    assert _fwd(_lay(), pos=B + 2) == qk.EALIGN
    assert _fwd(_lay(), q=0) == qk.EINVAL
    assert _fwd(_lay(), wk=C + 8) == qk.EALIGN


def test_scalar_checks():
    assert _fwd(_lay(), eps=-1.0) == qk.EINVAL
    assert _fwd(_lay(), eps=float("nan")) == qk.EINVAL
    assert _fwd(_lay(), theta=0.0) == qk.EINVAL
    assert _fwd(_lay(), theta=float("inf")) == qk.EINVAL


def test_outputs_must_not_overlap_inputs():
    assert _fwd(_lay(), q=A + 1024) == qk.EINVAL  # q inside qkv
    assert _fwd(_lay(), k=Dp + 16) == qk.EINVAL   # k inside q


def test_empty_batch_forward_enqueues_nothing():
    # T = 0 passes validation and returns before any HIP call
    assert _fwd(_lay(T=0)) == qk.OK
    # NoPE layers do not need positions
    assert _fwd(_lay(T=0, rope_dim=0), pos=0) == qk.OK


def test_latent_descriptor_checks():
    lat = _lay(kind=qk.LATENT, n_kv=1, q_per_kv=0, head_dim=0, rope_dim=64, norm_dim=512, width=576)
    assert qk.lib().qkvnr_forward(ctypes.byref(lat), A, B, C, C, 1e-6, 1e4, None, Dp, None, None) == qk.EINVAL
    assert qk.lib().qkvnr_forward(ctypes.byref(lat), A, B, None, C, 1e-6, 1e4, Dp, Dp, None, None) == qk.EINVAL
    bad_w = _lay(kind=qk.LATENT, n_kv=1, q_per_kv=0, head_dim=0, rope_dim=64, norm_dim=512, width=512)
    assert qk.lib().qkvnr_forward(ctypes.byref(bad_w), A, B, None, C, 1e-6, 1e4, None, Dp, None, None) == qk.EINVAL
    f32 = _lay(kind=qk.LATENT, dtype=qk.FP32, n_kv=1, q_per_kv=0, head_dim=0, rope_dim=64, norm_dim=512, width=576)
    assert qk.lib().qkvnr_forward(ctypes.byref(f32), A, B, None, C, 1e-6, 1e4, None, Dp, None, None) == qk.EUNSUPPORTED
    n256 = _lay(kind=qk.LATENT, n_kv=1, q_per_kv=0, head_dim=0, rope_dim=64, norm_dim=256, width=320)
    assert qk.lib().qkvnr_forward(ctypes.byref(n256), A, B, None, C, 1e-6, 1e4, None, Dp, None, None) == qk.EUNSUPPORTED
    assert qk.lib().qkvnr_backward(ctypes.byref(lat), A, B, None, C, 1e-6, 1e4, A, A, A, Dp, E, F, A + (8 << 30),
                                   1 << 20, None) == qk.EUNSUPPORTED


def test_latent_empty_batch():
    lat = _lay(kind=qk.LATENT, T=0, n_kv=1, q_per_kv=0, head_dim=0, rope_dim=64, norm_dim=512, width=576)
    assert qk.lib().qkvnr_forward(ctypes.byref(lat), A, B, None, C, 1e-6, 1e4, None, Dp, None, None) == qk.OK


def test_paged_argument_checks():
    L = _lay()
    f = qk.lib().qkvnr_forward_paged
    assert f(ctypes.byref(L), A, B, C, C + 4096, 1e-6, 1e4, None, 4, 4, 64, 16, Dp, E, F, None) == qk.EINVAL
    assert f(ctypes.byref(L), A, B, C, C + 4096, 1e-6, 1e4, A + (6 << 30), 4, 4, 0, 16, Dp, E, F, None) == qk.EINVAL
    assert f(ctypes.byref(L), A, B, C, C + 4096, 1e-6, 1e4, A + (6 << 30) + 2, 4, 4, 64, 16, Dp, E, F,
             None) == qk.EALIGN
    L0 = _lay(T=0)
    assert f(ctypes.byref(L0), A, B, C, C + 4096, 1e-6, 1e4, A + (6 << 30), 4, 4, 64, 16, Dp, E, F, None) == qk.OK


def test_backward_argument_checks():
    L = _lay()
    f = qk.lib().qkvnr_backward
    WS = A + (8 << 30)
    need = qk.qkvnr_backward_workspace_bytes(L)
    args = [A, B, C, C + 4096, 1e-6, 1e4, Dp, E, F, A + (6 << 30), A + (7 << 30), A + (7 << 30) + 4096, WS, need]

    def call(**change):
        a = list(args)
        for i, v in change.items():
            a[int(i[1:])] = v
        return f(ctypes.byref(L), *a, None)

    assert call(i9=0) == qk.EINVAL                       # dqkv NULL
    assert call(i10=A + (7 << 30) + 2) == qk.EALIGN      # dq_norm_w misaligned
    assert call(i9=A + 64) == qk.EINVAL                  # dqkv overlaps qkv
    assert call(i12=0) == qk.EINVAL                      # workspace NULL
    assert call(i12=WS + 8) == qk.EALIGN                 # workspace misaligned
    assert call(i13=need - 4) == qk.EINVAL               # workspace too small
    assert "workspace" in qk.lib().qkvnr_strerror(qk.EINVAL).decode()
    assert call(i12=A + 4096) == qk.EINVAL               # workspace overlaps qkv


def test_backward_noalloc_argument_checks():
    """The no-alloc backward validates like qkvnr_backward (less the workspace) before any HIP call."""
    L = _lay()
    f = qk.lib().qkvnr_backward_noalloc
    args = [A, B, C, C + 4096, 1e-6, 1e4, Dp, E, F, A + (6 << 30), A + (7 << 30), A + (7 << 30) + 4096]

    def call(layout=L, **change):
        a = list(args)
        for i, v in change.items():
            a[int(i[1:])] = v
        return f(ctypes.byref(layout), *a, None)

    assert f(None, *args, None) == qk.EINVAL             # no layout
    assert call(i9=0) == qk.EINVAL                       # dqkv NULL
    assert call(i10=A + (7 << 30) + 2) == qk.EALIGN      # dq_norm_w misaligned
    assert call(i9=A + 64) == qk.EINVAL                  # dqkv overlaps qkv
    assert call(i11=A + (7 << 30) + 8) == qk.EINVAL      # the two weight grads overlap
    assert call(i4=-1.0) == qk.EINVAL                    # eps
    assert call(layout=_lay(width=100)) == qk.EINVAL     # not the exact total
    assert call(layout=_lay(head_dim=96, width=(16 * 8 + 32) * 96, rope_dim=96)) == qk.EUNSUPPORTED
    lat = _lay(kind=qk.LATENT, n_kv=1, q_per_kv=0, head_dim=0, rope_dim=64, width=576, norm_dim=512)
    assert call(layout=lat) == qk.EUNSUPPORTED           # no latent backward


def test_noalloc_scratch_size_in_header():
    text = open(qk._binding.HEADER).read()
    cap = int(re.search(r"#define QKVNR_NOALLOC_SCRATCH_BYTES (\d+)", text).group(1))
    assert cap >= qk.lib().qkvnr_backward_workspace_bytes(None)


def test_backward_workspace_size():
    L128 = _lay(n_kv=8, q_per_kv=4, head_dim=128, rope_dim=128)
    L64 = _lay()
    text = open(qk._binding.HEADER).read()
    cap = int(re.search(r"#define QKVNR_BACKWARD_WORKSPACE_MAX (\d+)", text).group(1))
    assert qk.qkvnr_backward_workspace_bytes(L64) <= qk.qkvnr_backward_workspace_bytes(L128) == cap
    assert qk.lib().qkvnr_backward_workspace_bytes(None) == cap


def test_rope_inplace_argument_checks():
    f = qk.lib().qkvnr_rope_inplace
    # dtype, T, heads, token_stride, head_stride, rope_offset, rope_dim, positions, theta, x
    ok = [qk.BF16, 16, 16, 16 * 192, 192, 128, 64, B, 1e4, A]

    def call(**change):
        a = list(ok)
        for i, v in change.items():
            a[int(i[1:])] = v
        return f(*a, None)

    assert call(i0=7) == qk.EINVAL                       # unknown dtype
    assert call(i0=qk.FP32) == qk.EUNSUPPORTED           # fp32 has no kernel
    assert call(i1=-1) == qk.EINVAL                      # T < 0
    assert call(i2=0) == qk.EINVAL                       # no heads
    assert call(i6=32) == qk.EUNSUPPORTED                # rope_dim without a kernel
    assert call(i5=160) == qk.EINVAL                     # rope part past the head
    assert call(i3=15 * 192) == qk.EINVAL                # heads do not fit the token stride
    assert call(i5=124) == qk.EALIGN                     # rope offset not a multiple of 8 values
    assert call(i4=196, i3=16 * 196) == qk.EALIGN        # head stride not a multiple of 8 values
    assert call(i8=0.0) == qk.EINVAL                     # theta
    assert call(i9=0) == qk.EINVAL                       # x NULL
    assert call(i9=A + 2) == qk.EALIGN                   # x misaligned
    assert call(i7=0) == qk.EINVAL                       # positions NULL
    assert call(i7=A + 64) == qk.EINVAL                  # positions inside x
    assert call(i1=0, i7=0, i9=0) == qk.OK               # empty batch: nothing is touched


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU driver is present; this case is for GPU-less hosts")
def test_valid_call_without_gpu_is_unsupported_not_a_crash():
    # every argument valid: the library reaches its device query, finds no gfx950, and says so
    assert _fwd(_lay()) == qk.EUNSUPPORTED
    assert "gfx950" in qk.lib().qkvnr_strerror(qk.EUNSUPPORTED).decode() or \
        "device" in qk.lib().qkvnr_strerror(qk.EUNSUPPORTED).decode()


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU driver is present; this case is for GPU-less hosts")
def test_strided_rows_are_counted_to_their_last_value():
    # latent rows as the last 576 columns of [T, 2112] rows (a merged projection's
    # output): an output that starts right after the last row's last value does
    # not overlap the input, although it lies within T * row_stride of its start
    T, stride = 4, 2112
    L = Layout(kind=qk.LATENT, dtype=qk.BF16, T=T, n_kv=1, q_per_kv=0, head_dim=0, rope_dim=64, norm_dim=512,
               reserved=0, width=576, in_row_stride=stride)
    rows = A + 1536 * 2
    end = rows + ((T - 1) * stride + 576) * 2
    f = qk.lib().qkvnr_forward
    assert f(ctypes.byref(L), rows, B, None, C, 1e-6, 1e4, None, end, None, None) == qk.EUNSUPPORTED  # no GPU here
    assert f(ctypes.byref(L), rows, B, None, C, 1e-6, 1e4, None, end - 16, None, None) == qk.EINVAL


def test_fused_head_block_guard():
    import json
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_layout_examples.json")))
    hb = g["head_block_count"]
    assert qk.qkvnr_fused_head_blocks(hb["n_q"], hb["n_kv"], 64, hb["blocks"] * 64) == hb["blocks"]
    f = g["falcon_exact_total"]
    assert qk.qkvnr_fused_head_blocks(8, 8, 8, f["config_rows"]) == 24
    with pytest.raises(qk.QkvnrError):
        qk.qkvnr_fused_head_blocks(8, 8, 8, f["weight_rows"])        # declined
    with pytest.raises(qk.QkvnrError):
        qk.qkvnr_fused_head_blocks(12, 12, 64, 768)                  # transposed Conv1D [hidden, 3 hidden]
    with pytest.raises(qk.QkvnrError):
        qk.qkvnr_fused_head_blocks(0, 0, 64, 0)
    out = ctypes.c_int64(5)
    assert qk.lib().qkvnr_fused_head_blocks(8, 2, 16, 100, ctypes.byref(out)) == qk.EINVAL and out.value == 0
    assert qk.lib().qkvnr_fused_head_blocks(8, 2, 16, 192, None) == qk.EINVAL


def test_ns_poly_argument_checks():
    f = qk.lib().qkvnr_ns_poly
    # dtype, blocks, d, gram, parts, first, scale, eps, p
    ok = [qk.BF16, 48, 128, A, 11, 1, 1.0, 1e-7, B]

    def call(**change):
        a = list(ok)
        for i, v in change.items():
            a[int(i[1:])] = v
        return f(*a, None)

    assert call(i0=9) == qk.EINVAL
    assert call(i1=-1) == qk.EINVAL
    assert call(i1=(1 << 22) + 1) == qk.EINVAL   # more blocks than one launch holds
    assert call(i2=129) == qk.EUNSUPPORTED
    assert call(i2=0) == qk.EUNSUPPORTED
    assert call(i4=0) == qk.EINVAL               # parts
    assert call(i6=0.0) == qk.EINVAL             # scale
    assert call(i7=-1.0) == qk.EINVAL            # eps
    assert call(i3=A + 2) == qk.EALIGN
    assert call(i3=A + 4) == qk.EALIGN
    assert call(i8=0) == qk.EINVAL
    assert call(i8=B + 1) == qk.EALIGN
    assert call(i8=A + 64) == qk.EINVAL          # p overlaps gram
    assert call(i1=0, i3=0, i8=0) == qk.OK         # no blocks: nothing is touched


def test_gram_partials_argument_checks():
    f = qk.lib().qkvnr_gram_partials
    # blocks, d, cols, x, parts, out
    ok = [48, 128, 4096, A, 11, B]

    def call(**change):
        a = list(ok)
        for i, v in change.items():
            a[int(i[1:])] = v
        return f(*a, None)

    assert call(i0=-1) == qk.EINVAL
    assert call(i1=48) == qk.EUNSUPPORTED
    assert call(i2=4100) == qk.EALIGN            # cols not a multiple of 8
    assert call(i2=0) == qk.EALIGN
    assert call(i4=0) == qk.EINVAL
    assert call(i2=(1 << 30) + 8) == qk.EINVAL
    assert call(i0=1 << 31) == qk.EINVAL
    assert call(i0=(1 << 22) + 1) == qk.EINVAL   # more blocks than one launch holds
    assert call(i3=A + 8) == qk.EALIGN
    assert call(i5=B + 2) == qk.EALIGN
    assert call(i5=A + 4096) == qk.EINVAL         # out overlaps x
    assert call(i0=(1 << 31) - 1, i2=1 << 30) == qk.EINVAL   # byte counts past 2^63
    assert call(i0=0, i3=0, i5=0) == qk.OK


def test_ns_update_argument_checks():
    f = qk.lib().qkvnr_ns_update
    # blocks, d, cols, p, x, y, parts, gram
    ok = [48, 128, 4096, A, B, C, 11, Dp]

    def call(**change):
        a = list(ok)
        for i, v in change.items():
            a[int(i[1:])] = v
        return f(*a, None)

    assert call(i0=-1) == qk.EINVAL
    assert call(i0=1 << 31) == qk.EINVAL
    assert call(i0=(1 << 22) + 1) == qk.EINVAL   # more blocks than one launch holds
    assert call(i1=96) == qk.EUNSUPPORTED
    assert call(i1=32) == qk.EUNSUPPORTED
    assert call(i2=4100) == qk.EALIGN            # cols not a multiple of 8
    assert call(i2=0) == qk.EALIGN
    assert call(i2=(1 << 30) + 8) == qk.EINVAL
    assert call(i6=0) == qk.EINVAL               # parts
    assert call(i6=65536) == qk.EINVAL
    assert call(i0=(1 << 31) - 1, i2=1 << 30) == qk.EINVAL   # byte counts past 2^63
    assert call(i3=A + 8) == qk.EALIGN           # p
    assert call(i4=B + 8) == qk.EALIGN           # x
    assert call(i5=C + 8) == qk.EALIGN           # y
    assert call(i7=Dp + 2) == qk.EALIGN          # gram
    assert call(i5=B + 4096) == qk.EINVAL        # y overlaps x
    assert call(i5=A + 64) == qk.EINVAL          # y overlaps p
    assert call(i7=B + 4096) == qk.EINVAL        # gram overlaps x
    assert call(i7=C + 16) == qk.EINVAL          # gram overlaps y
    assert call(i7=A + 16) == qk.EINVAL          # gram overlaps p
    assert call(i0=0, i3=0, i4=0, i5=0, i7=0) == qk.OK   # no blocks: nothing is touched


def test_ns_collapse_argument_checks():
    f = qk.lib().qkvnr_ns_collapse
    # blocks, d, gram, parts, steps, scale, eps, m
    ok = [48, 128, A, 5, 5, 1.0, 1e-7, B]

    def call(**change):
        a = list(ok)
        for i, v in change.items():
            a[int(i[1:])] = v
        return f(*a, None)

    assert call(i0=-1) == qk.EINVAL
    assert call(i0=(1 << 22) + 1) == qk.EINVAL   # more blocks than one launch holds
    assert call(i1=32) == qk.EUNSUPPORTED         # sides 64 and 128
    assert call(i1=96) == qk.EUNSUPPORTED
    assert call(i3=0) == qk.EINVAL                # parts
    assert call(i3=65536) == qk.EINVAL
    assert call(i4=0) == qk.EINVAL                # steps
    assert call(i4=65) == qk.EINVAL
    assert call(i5=0.0) == qk.EINVAL              # scale
    assert call(i5=float("inf")) == qk.EINVAL
    assert call(i6=-1.0) == qk.EINVAL             # eps
    assert call(i2=0) == qk.EINVAL                # gram
    assert call(i2=A + 4) == qk.EALIGN
    assert call(i7=0) == qk.EINVAL                # m
    assert call(i7=B + 8) == qk.EALIGN
    assert call(i7=A + 4096) == qk.EINVAL         # m overlaps gram
    assert call(i0=0, i2=0, i7=0) == qk.OK        # no blocks: nothing is touched


def test_ns_apply_argument_checks():
    f = qk.lib().qkvnr_ns_apply
    # blocks, d, cols, m, x, y, parts
    ok = [48, 128, 4096, A, B, C, 5]

    def call(**change):
        a = list(ok)
        for i, v in change.items():
            a[int(i[1:])] = v
        return f(*a, None)

    assert call(i0=-1) == qk.EINVAL
    assert call(i0=(1 << 22) + 1) == qk.EINVAL
    assert call(i1=96) == qk.EUNSUPPORTED
    assert call(i2=0) == qk.EALIGN
    assert call(i2=4100) == qk.EALIGN
    assert call(i2=(1 << 30) + 8) == qk.EINVAL
    assert call(i6=0) == qk.EINVAL                # parts
    assert call(i0=(1 << 31) - 1, i2=1 << 30) == qk.EINVAL   # byte counts past 2^63
    assert call(i3=A + 8) == qk.EALIGN            # m
    assert call(i4=B + 8) == qk.EALIGN            # x
    assert call(i5=C + 8) == qk.EALIGN            # y
    assert call(i5=B + 4096) == qk.EINVAL         # y overlaps x
    assert call(i5=A + 64) == qk.EINVAL           # y overlaps m
    assert call(i0=0, i3=0, i4=0, i5=0) == qk.OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import qkv_split_head_amd._binding as b
    monkeypatch.setattr(b, "_lib", None)
    monkeypatch.setattr(b, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        b.lib()


def test_proj_forward_argument_checks():
    f = qk.lib().qkvnr_proj_forward

    def call(L=None, hidden=4096, x=A, w=B, pos=C, wq=C + 4096, wk=C + 8192, q=Dp, k=E, v=F, eps=1e-6, theta=1e6):
        L = _lay(qk.SECTIONED, T=300, n_kv=8, q_per_kv=4, head_dim=128, rope_dim=128) if L is None else L
        return f(ctypes.byref(L), hidden, x, w, pos, wq, wk, eps, theta, q, k, v, None)

    assert call(hidden=4100) == qk.EINVAL                     # not a multiple of 64
    assert call(hidden=0) == qk.EINVAL
    assert call(hidden=32) == qk.EINVAL
    assert call(hidden=(1 << 30) + 64) == qk.EINVAL
    assert call(L=_lay(qk.LATENT, T=4, width=576, norm_dim=512, rope_dim=64)) == qk.EUNSUPPORTED
    assert call(L=_lay(qk.SECTIONED, dtype=qk.FP32, T=4, n_kv=8, q_per_kv=4, head_dim=128, rope_dim=128)) \
        == qk.EUNSUPPORTED
    assert call(L=_lay(qk.SECTIONED, T=4, n_kv=8, q_per_kv=4, head_dim=128, rope_dim=128, width=6016)) == qk.EINVAL
    assert call(L=_lay(qk.SECTIONED, T=4, n_kv=8, q_per_kv=4, head_dim=96, rope_dim=96)) == qk.EUNSUPPORTED
    assert call(x=A + 8) == qk.EALIGN
    assert call(w=B + 2) == qk.EALIGN
    assert call(pos=C + 2) == qk.EALIGN
    assert call(q=None) == qk.EINVAL
    assert call(v=A + 64) == qk.EINVAL                          # an output overlaps x
    assert call(k=B + 4096) == qk.EINVAL                        # an output overlaps the weight
    assert call(eps=-1.0) == qk.EINVAL
    assert call(theta=0.0) == qk.EINVAL
    # NoPE: positions may be NULL (the call then fails only for want of a device here)
    nope = _lay(qk.INTERLEAVED, T=0, n_kv=2, q_per_kv=4, head_dim=64, rope_dim=0)
    assert call(L=nope, pos=None, x=0, w=0, q=0, k=0, v=0) == qk.OK   # T == 0 enqueues nothing


def test_tensor_wrappers_reject_host_tensors_before_any_call():
    """The tensor-level wrappers refuse host tensors themselves: their addresses never reach the C ABI."""
    import torch
    T, n_kv, Q, D = 4, 2, 2, 64
    qkv = torch.zeros((T, n_kv, Q + 2, D), dtype=torch.bfloat16)
    pos = torch.zeros(T, dtype=torch.int32)
    w = torch.ones(D, dtype=torch.bfloat16)
    kw = dict(kind="interleaved", n_kv=n_kv, q_per_kv=Q, head_dim=D)
    with pytest.raises(ValueError, match="need GPU tensors"):
        qk.forward(qkv, pos, w, w, **kw)
    g = torch.zeros((T, n_kv * Q, D), dtype=torch.bfloat16)
    gk = torch.zeros((T, n_kv, D), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="need GPU tensors"):
        qk.backward(qkv, pos, w, w, g, gk, gk, **kw)
    rows = torch.zeros((T, 576), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="need GPU tensors"):
        qk.forward_latent(rows, pos, torch.ones(512, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="need GPU tensors"):
        qk.rope_inplace(torch.zeros((T, 2, 64), dtype=torch.bfloat16), pos, rope_offset=0)
    from qkv_split_head_amd.muon import per_head_newton_schulz
    with pytest.raises(ValueError, match="need GPU tensors"):
        per_head_newton_schulz(torch.zeros((12 * 64, 256), dtype=torch.bfloat16), 8, 2, 64)
    with pytest.raises(TypeError, match="must be a torch tensor"):
        qk._binding._need(None, "positions")
