"""GPU parity: the HIP library (through its C ABI) against the fp64 CPU oracle.

Rules (see tests/helpers.py): bf16 within 2 bf16 ulps with an rms floor, fp32
within 1e-5 relative, v / dv / store locations / untouched memory bit-exact.
Inputs are the seeded generators of ``qkv_inputs``; the oracle and the library
see the same bits.
"""
import numpy as np
import pytest
import torch

import oracle
import qkv_split_head_amd as qk
from qkv_inputs import (custom_gqa, decode_interleaved, gqa_paged, latent_paged, prefill_interleaved, token_positions,
                        tiny_interleaved, train_sectioned)
from tests.helpers import (announce, assert_bits_equal, assert_close, assert_values_close, gpu_available,
                           host_value, to_dev, to_host_bits)

pytestmark = pytest.mark.gpu

SENT16 = 0x7FC1  # a NaN pattern no kernel result can equal
SENT32 = 0x7FC00001


@pytest.fixture(autouse=True)
def _gpu(request):
    if not gpu_available():
        pytest.skip("no GPU")
    qk.lib()  # fails loudly when the library is missing
    announce(request.node.nodeid)
    yield
    torch.cuda.synchronize()


# ------------------------------------------------------------------ helpers


def _sentinel_buffer(n_elems: int, dtype: str, pad: int):
    """Device buffer of n_elems + 2*pad elements filled with a NaN sentinel; returns (buf, middle view)."""
    if dtype == "bf16":
        buf = torch.full((n_elems + 2 * pad,), SENT16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    else:
        buf = torch.full((n_elems + 2 * pad,), SENT32, dtype=torch.int32, device="cuda").view(torch.float32)
    return buf, buf[pad:pad + n_elems]


def _pads_untouched(buf: torch.Tensor, pad: int, what: str):
    raw = buf.view(torch.int16) if buf.dtype == torch.bfloat16 else buf.view(torch.int32)
    sent = SENT16 if buf.dtype == torch.bfloat16 else SENT32
    assert bool((raw[:pad] == sent).all()) and bool((raw[raw.numel() - pad:] == sent).all()), \
        f"{what}: guard band overwritten"


def _dev_inputs(w):
    return (to_dev(w.qkv, w.dtype), to_dev(w.positions, "int32"), to_dev(w.q_norm_w, w.dtype),
            to_dev(w.k_norm_w, w.dtype))


def _gpu_forward(w, pad=64, stream=None):
    """Run the forward into guard-banded outputs; returns host bits of q, k, v."""
    qkv, pos, wq, wk = _dev_inputs(w)
    T, D = w.T, w.head_dim
    bq, q = _sentinel_buffer(T * w.n_q * D, w.dtype, pad)
    bk, k = _sentinel_buffer(T * w.n_kv * D, w.dtype, pad)
    bv, v = _sentinel_buffer(T * w.n_kv * D, w.dtype, pad)
    out = (q.view(T, w.n_q, D), k.view(T, w.n_kv, D), v.view(T, w.n_kv, D))
    qk.forward(qkv, pos, wq, wk, kind=w.kind, n_kv=w.n_kv, q_per_kv=w.q_per_kv, head_dim=D,
               rope=w.rope_dim > 0, eps=w.eps, theta=w.theta, out=out, stream=stream)
    torch.cuda.synchronize()
    for b, n in [(bq, "q"), (bk, "k"), (bv, "v")]:
        _pads_untouched(b, pad, n)
    return tuple(to_host_bits(t) for t in out)


def _check_forward(w, got, tokens=None):
    sel = slice(None) if tokens is None else tokens
    q64, k64, vbits = oracle.forward_gqa(w.qkv[sel], w.dtype, w.kind, w.n_kv, w.q_per_kv, w.head_dim,
                                         w.positions[sel], w.q_norm_w, w.k_norm_w, w.eps, w.theta,
                                         rope=w.rope_dim > 0)
    gq, gk, gv = (g[sel] for g in got)
    assert_close(gq, q64, w.dtype, f"{w.name} q")
    assert_close(gk, k64, w.dtype, f"{w.name} k")
    assert_bits_equal(gv, vbits, f"{w.name} v")


def _gpu_backward(w, stream=None):
    qkv, pos, wq, wk = _dev_inputs(w)
    dq, dk, dv = to_dev(w.dq, w.dtype), to_dev(w.dk, w.dtype), to_dev(w.dv, w.dtype)
    dqkv, dwq, dwk = qk.backward(qkv, pos, wq, wk, dq, dk, dv, kind=w.kind, n_kv=w.n_kv, q_per_kv=w.q_per_kv,
                                 head_dim=w.head_dim, rope=w.rope_dim > 0, eps=w.eps, theta=w.theta,
                                 stream=stream)
    torch.cuda.synchronize()
    return to_host_bits(dqkv), dwq.cpu().numpy().astype(np.float64), dwk.cpu().numpy().astype(np.float64)


def _check_backward(w, dqkv_bits, dwq, dwk, tokens=None, ref=None):
    sel = slice(None) if tokens is None else tokens
    if ref is None:
        ref = oracle.backward_gqa(w.qkv, w.dtype, w.kind, w.n_kv, w.q_per_kv, w.head_dim, w.positions,
                                  w.q_norm_w, w.k_norm_w, w.eps, w.theta, w.dq, w.dk, w.dv,
                                  rope=w.rope_dim > 0)
    gq, gk, gv = oracle.split(dqkv_bits[sel], w.kind, w.n_kv, w.q_per_kv, w.head_dim)
    assert_close(gq, ref["dx_q"][sel], w.dtype, f"{w.name} dq slots")
    assert_close(gk, ref["dx_k"][sel], w.dtype, f"{w.name} dk slots")
    assert_bits_equal(gv, w.dv[sel], f"{w.name} dv slots")
    assert_values_close(dwq, ref["dw_q"], w.dtype, f"{w.name} dq_norm_w", scale=ref["dw_q_l2"])
    assert_values_close(dwk, ref["dw_k"], w.dtype, f"{w.name} dk_norm_w", scale=ref["dw_k_l2"])


# ------------------------------------------------------------------ named workloads (small)


def test_tiny_fp32_interleaved():
    w = tiny_interleaved()
    _check_forward(w, _gpu_forward(w))


@pytest.mark.parametrize("T", [1, 8, 64, 256])
def test_muse_decode(T):
    w = decode_interleaved(T)
    _check_forward(w, _gpu_forward(w))


# ------------------------------------------------------------------ forward, shapes and edge cases

FWD_CASES = [
    # kind, dtype, T, n_kv, q_per_kv, D, rope, positions
    ("interleaved", "bf16", 300, 16, 8, 64, True, "random"),
    ("interleaved", "bf16", 777, 3, 5, 64, True, "random"),    # 21 heads: ragged last iteration
    ("interleaved", "bf16", 129, 2, 3, 128, True, "random"),
    ("interleaved", "fp32", 95, 2, 4, 64, True, "random"),
    ("interleaved", "fp32", 70, 3, 2, 128, True, "random"),    # 32 lanes per head
    ("sectioned", "bf16", 257, 8, 4, 128, True, "arange"),
    ("sectioned", "bf16", 333, 1, 1, 64, True, "random"),      # 3 heads per token
    ("sectioned", "fp32", 64, 2, 7, 128, True, "random"),
    ("sectioned", "bf16", 100, 4, 2, 64, False, "random"),     # NoPE
    ("interleaved", "fp32", 50, 2, 2, 64, False, "random"),    # NoPE fp32
    ("interleaved", "bf16", 5000, 4, 4, 64, True, "arange"),   # many units per wave
    # enough work units for the streaming schedule (4 iterations per wave, 3 loads in flight);
    # the cases above with fewer units take the one-iteration-per-wave schedule
    ("interleaved", "bf16", 3000, 3, 5, 64, True, "random"),   # 21 heads: ragged last iteration
    ("sectioned", "bf16", 2100, 8, 4, 128, True, "random"),    # 12 iterations: 3 full units per token
    ("interleaved", "fp32", 2500, 2, 3, 128, True, "random"),  # 5 iterations: a unit of 4 and a unit of 1
    ("sectioned", "bf16", 2200, 2, 5, 64, True, "random"),     # 2 iterations in a unit of 4
    ("interleaved", "bf16", 4096, 16, 8, 64, False, "random"), # NoPE
]


@pytest.mark.parametrize("kind,dtype,n_kv,Q,D", [("interleaved", "bf16", 16, 8, 64), ("sectioned", "bf16", 8, 4, 128),
                                                  ("interleaved", "fp32", 3, 2, 128)])
def test_small_and_streaming_schedules_agree_bitwise(kind, dtype, n_kv, Q, D):
    # the same tokens through the streaming schedule (a large batch) and the
    # one-iteration schedule (a small prefix of it): bitwise the same outputs
    w = custom_gqa(kind, dtype, 12000, n_kv, Q, D, theta=1e4, seed=31, positions="random")
    big = _gpu_forward(w)
    n = 40
    w.qkv, w.positions, w.T = w.qkv[:n], w.positions[:n], n
    small = _gpu_forward(w)
    for a, b, name in zip(big, small, "qkv"):
        assert_bits_equal(a[:n], b, f"{name}: streaming vs small-batch schedule")


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: "-".join(map(str, c)))
def test_forward_shapes(case):
    kind, dtype, T, n_kv, Q, D, rope, posmode = case
    w = custom_gqa(kind, dtype, T, n_kv, Q, D, rope=rope, theta=5e5, seed=T + D, positions=posmode)
    _check_forward(w, _gpu_forward(w))


def test_forward_positions_near_int32_max():
    w = custom_gqa("interleaved", "fp32", 40, 2, 2, 64, theta=1e4, seed=9, positions="random",
                   max_pos=2 ** 31 - 1)
    w.positions[:4] = [2 ** 31 - 1, 2 ** 31 - 2, 2 ** 30, 0]
    _check_forward(w, _gpu_forward(w))


def test_forward_zero_heads_stay_zero():
    w = custom_gqa("interleaved", "bf16", 9, 2, 2, 64, seed=3, positions="random")
    w.qkv[2] = 0  # a token whose every head is zero: normed and rotated value is 0 with eps > 0
    got = _gpu_forward(w)
    _check_forward(w, got)
    assert (host_value(got[0][2], "bf16") == 0).all() and (host_value(got[1][2], "bf16") == 0).all()


def test_forward_padded_row_stride():
    w = custom_gqa("sectioned", "bf16", 123, 2, 3, 128, seed=4, positions="random")
    width = w.width
    big = np.full((w.T, width + 24), SENT16, dtype=np.uint16)  # 48 extra bytes per row
    big[:, :width] = w.qkv
    qkv = to_dev(big, "bf16")[:, :width]
    pos = to_dev(w.positions, "int32")
    q, k, v = qk.forward(qkv, pos, to_dev(w.q_norm_w, "bf16"), to_dev(w.k_norm_w, "bf16"), kind="sectioned",
                         n_kv=2, q_per_kv=3, head_dim=128, eps=w.eps, theta=w.theta)
    torch.cuda.synchronize()
    _check_forward(w, (to_host_bits(q), to_host_bits(k), to_host_bits(v)))


def test_forward_empty_batch():
    w = custom_gqa("interleaved", "bf16", 0, 2, 2, 64, seed=1)
    q, k, v = qk.forward(to_dev(w.qkv, "bf16"), to_dev(w.positions, "int32"), to_dev(w.q_norm_w, "bf16"),
                         to_dev(w.k_norm_w, "bf16"), kind="interleaved", n_kv=2, q_per_kv=2, head_dim=64)
    torch.cuda.synchronize()
    assert q.shape == (0, 4, 64) and k.shape == (0, 2, 64)


def test_forward_rejects_misaligned_device_pointer():
    w = custom_gqa("interleaved", "bf16", 4, 2, 2, 64, seed=1)
    big = to_dev(np.concatenate([np.zeros(1, np.uint16), w.qkv.reshape(-1)]), "bf16")
    qkv = big[1:].view(4, 2, 4, 64)  # 2 bytes off a 16-byte boundary
    with pytest.raises(qk.QkvnrError) as ei:
        qk.forward(qkv, to_dev(w.positions, "int32"), to_dev(w.q_norm_w, "bf16"), to_dev(w.k_norm_w, "bf16"),
                   kind="interleaved", n_kv=2, q_per_kv=2, head_dim=64)
    assert ei.value.code == qk.EALIGN



def test_wrappers_refuse_mismatched_tensors():
    """Outputs of the wrong shape, positions of the wrong type and a block table with too few rows are
    refused by the tensor-level wrappers, before any kernel could write past a buffer."""
    w = custom_gqa("interleaved", "bf16", 8, 2, 2, 64, seed=3, grads=True)
    qkv, pos = to_dev(w.qkv, "bf16"), to_dev(w.positions, "int32")
    wq, wk = to_dev(w.q_norm_w, "bf16"), to_dev(w.k_norm_w, "bf16")
    kw = dict(kind="interleaved", n_kv=2, q_per_kv=2, head_dim=64, eps=w.eps, theta=w.theta)
    q, k, v = qk.forward(qkv, pos, wq, wk, **kw)
    with pytest.raises(ValueError, match="shape"):
        qk.forward(qkv, pos, wq, wk, out=(q[:4], k, v), **kw)
    with pytest.raises(TypeError, match="dtype"):
        qk.forward(qkv, pos.long(), wq, wk, **kw)
    with pytest.raises(TypeError, match="dtype"):
        qk.forward(qkv, pos, wq.float(), wk, **kw)
    dq, dk, dv = to_dev(w.dq, "bf16"), to_dev(w.dk, "bf16"), to_dev(w.dv, "bf16")
    with pytest.raises(ValueError, match="shape"):
        qk.backward(qkv, pos, wq, wk, dq[:2], dk, dv, **kw)
    dqkv, dwq, dwk = qk.backward(qkv, pos, wq, wk, dq, dk, dv, **kw)
    with pytest.raises(ValueError, match="shape"):
        qk.backward(qkv, pos, wq, wk, dq, dk, dv, out=(dqkv, dwq[:32], dwk), **kw)
    kp = torch.zeros((4, 16, 2, 64), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((1, 4), dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="block_table has 1 rows"):
        qk.forward_paged(qkv, pos, wq, wk, bt, kp, kp.clone(), tokens_per_req=4, **kw)
    with pytest.raises(ValueError, match="shape"):
        qk.forward_paged(qkv, pos, wq, wk, bt, kp, kp[:, :8], tokens_per_req=8, **kw)
    torch.cuda.synchronize()


# ------------------------------------------------------------------ GPU-vs-GPU bitwise equivalences


def test_nope_layer_equals_rope_at_position_zero_bitwise():
    w = custom_gqa("interleaved", "bf16", 200, 16, 8, 64, seed=5, positions="random")
    w.rope_dim = 0
    nope = _gpu_forward(w)
    w.rope_dim = 64
    w.positions = np.zeros_like(w.positions)
    rope0 = _gpu_forward(w)
    for a, b, n in zip(nope, rope0, "qkv"):
        assert_bits_equal(a, b, f"NoPE vs RoPE@0 {n}")


def _interleaved_to_sectioned_blocks(n_kv, Q):
    n_q = n_kv * Q
    return np.array([g * Q + s if s < Q else (n_q + g if s == Q else n_q + n_kv + g)
                     for g in range(n_kv) for s in range(Q + 2)])


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128), ("fp32", 64)])
def test_layouts_give_the_same_heads_bitwise(dtype, D):
    T, n_kv, Q = 150, 4, 3
    wi = custom_gqa("interleaved", dtype, T, n_kv, Q, D, seed=6, positions="random", grads=True)
    perm = _interleaved_to_sectioned_blocks(n_kv, Q)
    H = n_kv * (Q + 2)
    xs = np.empty_like(wi.qkv.reshape(T, H, D))
    xs[:, perm] = wi.qkv.reshape(T, H, D)
    ws = custom_gqa("sectioned", dtype, T, n_kv, Q, D, seed=6, positions="random", grads=True)
    ws.qkv = xs.reshape(T, H * D)
    ws.q_norm_w, ws.k_norm_w, ws.positions = wi.q_norm_w, wi.k_norm_w, wi.positions
    ws.dq, ws.dk, ws.dv = wi.dq, wi.dk, wi.dv
    for a, b, n in zip(_gpu_forward(wi), _gpu_forward(ws), "qkv"):
        assert_bits_equal(a, b, f"interleaved vs sectioned {n}")
    di, dwqi, dwki = _gpu_backward(wi)
    ds, dwqs, dwks = _gpu_backward(ws)
    assert_bits_equal(di.reshape(T, H, D), ds.reshape(T, H, D)[:, perm], "dqkv block permutation")
    # weight grads are summed with atomics: same values up to summation order
    assert np.allclose(dwqi, dwqs, rtol=1e-5, atol=1e-5 * np.abs(dwqi).max())
    assert np.allclose(dwki, dwks, rtol=1e-5, atol=1e-5 * np.abs(dwki).max())


def test_forward_is_deterministic_and_honours_the_stream():
    w = custom_gqa("interleaved", "bf16", 1000, 16, 8, 64, seed=7, positions="random")
    a = _gpu_forward(w)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = _gpu_forward(w, stream=s)
    for x, y, n in zip(a, b, "qkv"):
        assert_bits_equal(x, y, f"rerun {n}")


# ------------------------------------------------------------------ backward

BWD_CASES = [
    ("interleaved", "bf16", 300, 16, 8, 64, True),
    ("interleaved", "bf16", 211, 3, 5, 64, True),
    ("sectioned", "bf16", 257, 8, 4, 128, True),
    ("sectioned", "bf16", 97, 2, 3, 128, False),
    ("interleaved", "fp32", 80, 2, 4, 64, True),
    ("sectioned", "fp32", 66, 3, 2, 128, True),
    ("interleaved", "fp32", 40, 1, 1, 64, False),
    ("interleaved", "bf16", 3000, 4, 4, 128, True),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "-".join(map(str, c)))
def test_backward_shapes(case):
    kind, dtype, T, n_kv, Q, D, rope = case
    w = custom_gqa(kind, dtype, T, n_kv, Q, D, rope=rope, theta=1e6, seed=T * 3 + D, positions="random",
                   grads=True)
    _check_backward(w, *_gpu_backward(w))


def test_backward_with_eps_zero():
    # eps = 0 is allowed: v heads (never normed) must not leak NaN into the weight grads
    w = custom_gqa("interleaved", "bf16", 150, 4, 3, 64, eps=0.0, seed=31, positions="random", grads=True)
    dqkv, dwq, dwk = _gpu_backward(w)
    assert np.isfinite(dwq).all() and np.isfinite(dwk).all()
    _check_backward(w, dqkv, dwq, dwk)


def test_backward_workspace_is_left_zero():
    w = custom_gqa("sectioned", "bf16", 500, 8, 4, 128, seed=32, positions="random", grads=True)
    ws = torch.zeros(qk.qkvnr_backward_workspace_bytes(qk.gqa_layout(to_dev(w.qkv, "bf16"), "sectioned", 8, 4,
                                                                        128, True)),
                     dtype=torch.uint8, device="cuda")
    qkv, pos, wq, wk = _dev_inputs(w)
    dq, dk, dv = to_dev(w.dq, "bf16"), to_dev(w.dk, "bf16"), to_dev(w.dv, "bf16")
    for _ in range(3):
        dqkv, dwq, dwk = qk.backward(qkv, pos, wq, wk, dq, dk, dv, kind="sectioned", n_kv=8, q_per_kv=4,
                                     head_dim=128, eps=w.eps, theta=w.theta, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero()) == 0
    _check_backward(w, to_host_bits(dqkv), dwq.cpu().numpy().astype(np.float64),
                    dwk.cpu().numpy().astype(np.float64))


def test_backward_calls_of_changing_size_share_one_workspace():
    # grid sizes change call to call; the last block of each call must fold the
    # slots and leave the shared workspace zero for the next
    ws = qk.backward_workspace()
    for i, (kind, T, n_kv, Q, D) in enumerate([("sectioned", 700, 8, 4, 128), ("interleaved", 5, 16, 8, 64),
                                               ("interleaved", 1, 2, 2, 64), ("sectioned", 3001, 2, 3, 128),
                                               ("interleaved", 64, 3, 5, 64)]):
        w = custom_gqa(kind, "bf16", T, n_kv, Q, D, theta=1e6, seed=40 + i, positions="random", grads=True)
        _check_backward(w, *_gpu_backward(w))
        assert int(ws.count_nonzero()) == 0, f"workspace not left zero after call {i}"


def test_backward_padded_row_stride_leaves_padding():
    w = custom_gqa("interleaved", "bf16", 77, 2, 4, 64, seed=8, positions="random", grads=True)
    width = w.width
    big = np.full((w.T, width + 8), SENT16, dtype=np.uint16)
    big[:, :width] = w.qkv.reshape(w.T, width)
    qkv = to_dev(big, "bf16")[:, :width]
    dqkv_big = torch.full((w.T, width + 8), SENT16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    dqkv = dqkv_big[:, :width]
    dwq = torch.full((64,), float("nan"), device="cuda")
    dwk = torch.full((64,), float("nan"), device="cuda")
    qk.backward(qkv, to_dev(w.positions, "int32"), to_dev(w.q_norm_w, "bf16"), to_dev(w.k_norm_w, "bf16"),
                to_dev(w.dq, "bf16"), to_dev(w.dk, "bf16"), to_dev(w.dv, "bf16"), kind="interleaved", n_kv=2,
                q_per_kv=4, head_dim=64, eps=w.eps, theta=w.theta, out=(dqkv, dwq, dwk))
    torch.cuda.synchronize()
    pad = to_host_bits(dqkv_big)[:, width:]
    assert (pad == SENT16).all()
    got = to_host_bits(dqkv_big)[:, :width].reshape(w.qkv.shape)
    _check_backward(w, got, dwq.cpu().numpy().astype(np.float64), dwk.cpu().numpy().astype(np.float64))


def test_backward_empty_batch_zeroes_weight_grads():
    w = custom_gqa("sectioned", "bf16", 0, 2, 2, 128, seed=1, grads=True)
    dwq = torch.full((128,), float("nan"), device="cuda")
    dwk = torch.full((128,), float("nan"), device="cuda")
    dqkv = torch.empty((0, w.width), dtype=torch.bfloat16, device="cuda")
    qk.backward(to_dev(w.qkv, "bf16"), to_dev(w.positions, "int32"), to_dev(w.q_norm_w, "bf16"),
                to_dev(w.k_norm_w, "bf16"), to_dev(w.dq, "bf16"), to_dev(w.dk, "bf16"), to_dev(w.dv, "bf16"),
                kind="sectioned", n_kv=2, q_per_kv=2, head_dim=128, out=(dqkv, dwq, dwk))
    torch.cuda.synchronize()
    assert bool((dwq == 0).all()) and bool((dwk == 0).all())


def test_backward_weight_grads_are_overwritten_not_accumulated():
    w = custom_gqa("interleaved", "bf16", 64, 2, 2, 64, seed=10, positions="random", grads=True)
    a = _gpu_backward(w)
    b = _gpu_backward(w)
    # atomics: the same sums up to summation order
    for x, y in [(a[1], b[1]), (a[2], b[2])]:
        assert np.allclose(x, y, rtol=1e-5, atol=1e-5 * np.abs(x).max())
    assert_bits_equal(a[0], b[0], "dqkv rerun")


# ------------------------------------------------------------------ paged store


@pytest.mark.parametrize("kind,dtype,D", [("interleaved", "bf16", 64), ("sectioned", "bf16", 128),
                                          ("interleaved", "fp32", 64)])
def test_gqa_paged_direct_equals_staged_scatter(kind, dtype, D):
    w = gqa_paged(kind, dtype, B=3, T_req=7, n_kv=2, q_per_kv=4, head_dim=D, num_pages=300, page_size=16,
                  ctx_hi=1500, seed=11)
    qkv, pos, wq, wk = _dev_inputs(w)
    shape = (w.num_pages, w.page_size, w.n_kv, D)
    pools = [_sentinel_buffer(int(np.prod(shape)), dtype, 0)[1].view(shape) for _ in range(4)]
    kp, vp, ks, vs = pools
    bt = to_dev(w.block_table, "int32")
    q_direct = qk.forward_paged(qkv, pos, wq, wk, bt, kp, vp, kind=kind, n_kv=2, q_per_kv=4, head_dim=D,
                                tokens_per_req=w.tokens_per_req, eps=w.eps, theta=w.theta)
    q_c, k_c, v_c = qk.forward(qkv, pos, wq, wk, kind=kind, n_kv=2, q_per_kv=4, head_dim=D, eps=w.eps,
                               theta=w.theta)
    page, off = oracle.paged_slots(w.positions, w.block_table, w.tokens_per_req, w.page_size)
    slot = torch.from_numpy(page * w.page_size + off).cuda()
    ks.view(-1, w.n_kv, D)[slot] = k_c
    vs.view(-1, w.n_kv, D)[slot] = v_c
    torch.cuda.synchronize()
    assert_bits_equal(to_host_bits(q_direct), to_host_bits(q_c), "paged q")
    assert_bits_equal(to_host_bits(kp), to_host_bits(ks), "k pool direct vs staged")
    assert_bits_equal(to_host_bits(vp), to_host_bits(vs), "v pool direct vs staged")
    # written rows against the oracle, and every other row untouched
    kh = to_host_bits(kp)
    written = np.zeros(shape[:2], dtype=bool)
    written[page, off] = True
    q64, k64, vbits = oracle.forward_gqa(w.qkv, dtype, kind, 2, 4, D, w.positions, w.q_norm_w, w.k_norm_w,
                                         w.eps, w.theta)
    assert_close(kh[page, off], k64, dtype, "paged k rows")
    assert_bits_equal(to_host_bits(vp)[page, off], vbits, "paged v rows")
    rest = kh[~written]
    if dtype == "bf16":
        assert (rest.view(np.uint16) == SENT16).all()
    else:
        assert (rest.view(np.uint32) == SENT32).all()


def test_gqa_paged_skips_unmapped_tokens():
    w = gqa_paged("interleaved", "bf16", B=2, T_req=4, n_kv=1, q_per_kv=2, head_dim=64, num_pages=64,
                  page_size=16, ctx_hi=300, seed=12)
    page, off = oracle.paged_slots(w.positions, w.block_table, w.tokens_per_req, w.page_size)
    bad_tbl = w.block_table.copy()
    bad_tbl[1, :] = -1  # request 1 unmapped
    qkv, pos, wq, wk = _dev_inputs(w)
    shape = (w.num_pages, w.page_size, 1, 64)
    kp = _sentinel_buffer(int(np.prod(shape)), "bf16", 0)[1].view(shape)
    vp = _sentinel_buffer(int(np.prod(shape)), "bf16", 0)[1].view(shape)
    qk.forward_paged(qkv, pos, wq, wk, to_dev(bad_tbl, "int32"), kp, vp, kind="interleaved", n_kv=1,
                     q_per_kv=2, head_dim=64, tokens_per_req=4, eps=w.eps, theta=w.theta)
    torch.cuda.synchronize()
    kh = to_host_bits(kp)
    assert (kh[page[4:], off[4:]] == SENT16).all()  # request 1 not stored
    assert not (kh[page[:4], off[:4]] == SENT16).any()  # request 0 stored


def test_latent_rows_contiguous():
    w = latent_paged(B=8, T_req=37, num_pages=32768, ctx_lo=0, ctx_hi=131072, seed=13)
    rows = to_dev(w.qkv, "bf16")
    out = qk.forward_latent(rows, to_dev(w.positions, "int32"), to_dev(w.k_norm_w, "bf16"), eps=w.eps,
                            theta=w.theta)
    torch.cuda.synchronize()
    ref = oracle.latent_forward(w.qkv, "bf16", w.positions, w.k_norm_w, w.eps, w.theta, 512, 64)
    got = to_host_bits(out)
    assert_close(got[:, :512], ref[:, :512], "bf16", "latent normed part")
    assert_close(got[:, 512:], ref[:, 512:], "bf16", "latent rotated part")


def test_mla_latent_paged_store_full_pool():
    # B = 4 requests x 16 draft tokens into a [8192, 64, 576] bf16 pool
    w = latent_paged()
    rows, pos, wk = to_dev(w.qkv, "bf16"), to_dev(w.positions, "int32"), to_dev(w.k_norm_w, "bf16")
    shape = (w.num_pages, w.page_size, 576)
    pool = _sentinel_buffer(int(np.prod(shape)), "bf16", 0)[1].view(shape)
    qk.forward_latent_paged(rows, pos, wk, to_dev(w.block_table, "int32"), pool,
                            tokens_per_req=w.tokens_per_req, eps=w.eps, theta=w.theta)
    staged = qk.forward_latent(rows, pos, wk, eps=w.eps, theta=w.theta)
    page, off = oracle.paged_slots(w.positions, w.block_table, w.tokens_per_req, w.page_size)
    pt, ot = torch.from_numpy(page).cuda(), torch.from_numpy(off).cuda()
    torch.cuda.synchronize()
    assert_bits_equal(to_host_bits(pool[pt, ot]), to_host_bits(staged), "latent pool rows vs staged")
    raw = pool.view(torch.int16)
    touched_rows = int((raw != SENT16).any(dim=-1).sum())
    assert touched_rows == w.T, f"{touched_rows} pool rows changed, expected {w.T}"
    ref = oracle.latent_forward(w.qkv, "bf16", w.positions, w.k_norm_w, w.eps, w.theta, 512, 64)
    got = to_host_bits(pool[pt, ot])
    assert_close(got[:, :512], ref[:, :512], "bf16", "pool normed part")
    assert_close(got[:, 512:], ref[:, 512:], "bf16", "pool rotated part")


@pytest.mark.parametrize("T,heads,head_stride,rope_offset,rope_dim,token_pad", [
    (16, 16, 192, 128, 64, 0),      # the MLA drafter's q heads: [nope 128 | rope 64]
    (64, 16, 192, 128, 64, 0),
    (37, 5, 136, 8, 128, 24),       # ragged heads per wave, rope part in the middle, padded token stride
    (1, 1, 64, 0, 64, 0),
    (300, 9, 72, 8, 64, 8),
])
def test_rope_inplace_matches_oracle(T, heads, head_stride, rope_offset, rope_dim, token_pad):
    rng = np.random.default_rng(T * 7 + heads)
    from qkv_inputs import bf16_bits_from_f32
    token_stride = heads * head_stride + token_pad
    bits = bf16_bits_from_f32(rng.standard_normal((T, token_stride)).astype(np.float32))
    pos = rng.integers(0, 131072, size=T).astype(np.int32)
    x = to_dev(bits, "bf16")
    view = x.view(T, token_stride)[:, :heads * head_stride].view(T, heads, head_stride)
    qk.rope_inplace(view, to_dev(pos, "int32"), rope_offset=rope_offset, rope_dim=rope_dim, theta=1e4)
    got = to_host_bits(x)
    torch.cuda.synchronize()
    heads_h = bits[:, :heads * head_stride].reshape(T, heads, head_stride)
    got_h = got[:, :heads * head_stride].reshape(T, heads, head_stride)
    part = slice(rope_offset, rope_offset + rope_dim)
    ref = oracle.rope_rotate_half(oracle.to_f64(heads_h[..., part], "bf16"), oracle.rope_angles(pos, 1e4, rope_dim))
    assert_close(got_h[..., part], ref, "bf16", "rope part")
    keep = np.ones(head_stride, bool)
    keep[part] = False
    assert_bits_equal(got_h[..., keep], heads_h[..., keep], "rest of each head")
    assert_bits_equal(got[:, heads * head_stride:], bits[:, heads * head_stride:], "token padding")


def test_rope_inplace_empty_batch_is_a_no_op():
    qk.qkvnr_rope_inplace(qk.BF16, 0, 4, 4 * 64, 64, 0, 64, None, 1e4, None)


# ------------------------------------------------------------------ full-size workloads (every token)


def _check_forward_all_tokens(w, got, chunk=2048):
    """q and k of every token against the oracle, chunk by chunk (the rms floor of the bf16 rule is taken
    over each chunk of `chunk` tokens); v of every token bit-exact."""
    for t0 in range(0, w.T, chunk):
        _check_forward(w, got, tokens=slice(t0, min(w.T, t0 + chunk)))


@pytest.mark.parametrize("rope", [True, False], ids=["rope", "nope"])
def test_muse_prefill_16k_all_tokens(rope):
    w = prefill_interleaved(16384, rope=rope)
    _check_forward_all_tokens(w, _gpu_forward(w, pad=256))


def test_qwen3_train_16k_fwd_bwd():
    w = train_sectioned(16384)
    _check_forward_all_tokens(w, _gpu_forward(w, pad=256))
    dqkv, dwq, dwk = _gpu_backward(w)
    ref = oracle.backward_gqa(w.qkv, w.dtype, w.kind, w.n_kv, w.q_per_kv, w.head_dim, w.positions, w.q_norm_w,
                              w.k_norm_w, w.eps, w.theta, w.dq, w.dk, w.dv, chunk=2048)
    # every token's dq/dk slots (the rms floor over each 2048-token chunk), dv slots bit-exact, weight grads
    for t0 in range(0, w.T, 2048):
        sel = slice(t0, t0 + 2048)
        gq, gk, gv = oracle.split(dqkv[sel], w.kind, w.n_kv, w.q_per_kv, w.head_dim)
        assert_close(gq, ref["dx_q"][sel], w.dtype, f"{w.name} dq slots, tokens {t0}..")
        assert_close(gk, ref["dx_k"][sel], w.dtype, f"{w.name} dk slots, tokens {t0}..")
        assert_bits_equal(gv, w.dv[sel], f"{w.name} dv slots, tokens {t0}..")
    assert_values_close(dwq, ref["dw_q"], w.dtype, f"{w.name} dq_norm_w", scale=ref["dw_q_l2"])
    assert_values_close(dwk, ref["dw_k"], w.dtype, f"{w.name} dk_norm_w", scale=ref["dw_k_l2"])


def test_batches_past_one_launch():
    """2^24 + 2^23 tokens of 3 heads (D = 64): the forward, the backward and the in-place RoPE each take two
    launches (a dispatch holds fewer than 2^32 work-items; pieces of 2^24 work units or tokens). Sampled rows on
    both sides of the piece boundary match the oracle, and the weight grads of the whole batch equal the sums of
    its two halves taken in one launch each, so a piece dropped or run twice would show."""
    T, P, h = (1 << 24) + (1 << 23), 4096, 1 << 24
    w = custom_gqa("sectioned", "bf16", P, 1, 1, 64, seed=41, positions="random", grads=True)
    pos_h = token_positions(T, seed=42)

    def tiled(bits, row_shape):  # the P drawn rows repeated over the batch, on the device
        return to_dev(bits, "bf16").reshape(P, -1).repeat(T // P, 1).reshape((T,) + row_shape)

    qkv, pos = tiled(w.qkv, (192,)), to_dev(pos_h, "int32")
    wq, wk = to_dev(w.q_norm_w, "bf16"), to_dev(w.k_norm_w, "bf16")
    kw = dict(kind="sectioned", n_kv=1, q_per_kv=1, head_dim=64, eps=w.eps, theta=w.theta)
    rng = np.random.Generator(np.random.PCG64(43))
    toks = np.unique(np.concatenate([np.arange(3), np.arange(h - 3, h + 3), np.arange(T - 3, T),
                                     rng.choice(T, size=40, replace=False)]))
    sel = torch.from_numpy(toks).cuda()
    rows = w.qkv[toks % P]

    q, k, v = qk.forward(qkv, pos, wq, wk, **kw)
    got = [to_host_bits(t.index_select(0, sel)) for t in (q, k, v)]
    del q, k, v
    q64, k64, vbits = oracle.forward_gqa(rows, "bf16", "sectioned", 1, 1, 64, pos_h[toks], w.q_norm_w,
                                         w.k_norm_w, w.eps, w.theta)
    assert_close(got[0], q64, "bf16", "q past one launch")
    assert_close(got[1], k64, "bf16", "k past one launch")
    assert_bits_equal(got[2], vbits, "v past one launch")

    dq, dk, dv = tiled(w.dq, (1, 64)), tiled(w.dk, (1, 64)), tiled(w.dv, (1, 64))
    dqkv, dwq, dwk = qk.backward(qkv, pos, wq, wk, dq, dk, dv, **kw)
    got = to_host_bits(dqkv.index_select(0, sel))
    del dqkv
    ref = oracle.backward_gqa(rows, "bf16", "sectioned", 1, 1, 64, pos_h[toks], w.q_norm_w, w.k_norm_w,
                              w.eps, w.theta, w.dq[toks % P], w.dk[toks % P], w.dv[toks % P])
    gq, gk, gv = oracle.split(got, "sectioned", 1, 1, 64)
    assert_close(gq, ref["dx_q"], "bf16", "dq slots past one launch")
    assert_close(gk, ref["dx_k"], "bf16", "dk slots past one launch")
    assert_bits_equal(gv, w.dv[toks % P], "dv slots past one launch")
    halves = []
    for a, b in ((0, h), (h, T)):
        _, hq, hk = qk.backward(qkv[a:b], pos[a:b], wq, wk, dq[a:b], dk[a:b], dv[a:b], **kw)
        halves.append((hq.cpu().numpy().astype(np.float64), hk.cpu().numpy().astype(np.float64)))
    for i, (full, name) in enumerate(((dwq, "dq_norm_w"), (dwk, "dk_norm_w"))):
        full = full.cpu().numpy().astype(np.float64)
        a, b = halves[0][i], halves[1][i]
        err = np.linalg.norm(full - (a + b))
        assert err <= 1e-3 * (np.linalg.norm(a) + np.linalg.norm(b)), f"{name}: whole batch vs halves {err}"
    del qkv, dq, dk, dv

    x = tiled(w.qkv[:, :64], (1, 64))   # one head of 64 values per token, rotated in place
    qk.rope_inplace(x, pos, rope_offset=0, rope_dim=64, theta=1e4)
    got = to_host_bits(x.index_select(0, sel))
    ref = oracle.rope_rotate_half(oracle.to_f64(w.qkv[toks % P, :64][:, None, :], "bf16"),
                                  oracle.rope_angles(pos_h[toks], 1e4, 64))
    assert_close(got, ref, "bf16", "rope in place past one launch")
    torch.cuda.synchronize()


# ------------------------------------------------------------------ HIP graphs


def test_graph_replays_match_eager():
    # forward + backward captured once, replayed several times with eager work and
    # synchronisations in between; each replay must reproduce the eager results
    w = custom_gqa("sectioned", "bf16", 512, 8, 4, 128, seed=21, positions="random", grads=True)
    qkv, pos, wq, wk = _dev_inputs(w)
    dq, dk, dv = to_dev(w.dq, "bf16"), to_dev(w.dk, "bf16"), to_dev(w.dv, "bf16")
    kw = dict(kind="sectioned", n_kv=8, q_per_kv=4, head_dim=128, eps=w.eps, theta=w.theta)
    outs = (torch.empty((512, 32, 128), dtype=torch.bfloat16, device="cuda"),
            torch.empty((512, 8, 128), dtype=torch.bfloat16, device="cuda"),
            torch.empty((512, 8, 128), dtype=torch.bfloat16, device="cuda"))
    bouts = (torch.empty_like(qkv), torch.empty(128, device="cuda"), torch.empty(128, device="cuda"))
    qk.forward(qkv, pos, wq, wk, out=outs, **kw)
    qk.backward(qkv, pos, wq, wk, dq, dk, dv, out=bouts, **kw)
    torch.cuda.synchronize()
    ref = [to_host_bits(t) for t in outs + bouts[:1]]
    ref_dw = [t.cpu().numpy() for t in bouts[1:]]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        qk.forward(qkv, pos, wq, wk, out=outs, **kw)
        qk.backward(qkv, pos, wq, wk, dq, dk, dv, out=bouts, **kw)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qk.forward(qkv, pos, wq, wk, out=outs, **kw)
        qk.backward(qkv, pos, wq, wk, dq, dk, dv, out=bouts, **kw)
    for r in range(4):
        for t in outs + bouts:
            t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, exp, n in zip([to_host_bits(t) for t in outs + bouts[:1]], ref, ["q", "k", "v", "dqkv"]):
            assert_bits_equal(got, exp, f"replay {r} {n}")
        for got, exp in zip([t.cpu().numpy() for t in bouts[1:]], ref_dw):
            assert np.allclose(got, exp, rtol=1e-5, atol=1e-5 * np.abs(exp).max())
