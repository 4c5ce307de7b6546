"""qkvnr_backward_noalloc (the backward whose weight-grad slots live in the
library's own static device array) against qkvnr_backward with a caller's
workspace, through the C ABI, and both against the fp64 oracle.

Two calls in a row, the second with a smaller input of a different head size:
the first call must leave the shared array zero for the second.  dqkv comes
from the same kernel on both paths, so it must be bitwise equal; the weight
grads are fp32 atomic sums, equal up to summation order, and each meets the
weight-grad rule against the oracle.  The last test captures the no-alloc call
in a HIP graph and replays it with eager work in between.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import qkv_split_head_amd as qk
from qkv_inputs import custom_gqa
from tests.helpers import (announce, assert_bits_equal, assert_close, assert_values_close, gpu_available, to_dev,
                           to_host_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu(request):
    if not gpu_available():
        pytest.skip("no GPU")
    qk.lib()
    announce(request.node.nodeid)
    yield
    torch.cuda.synchronize()


def _inputs(w):
    d = w.dtype
    return dict(qkv=to_dev(w.qkv, d), pos=to_dev(w.positions, "int32"), wq=to_dev(w.q_norm_w, d),
                wk=to_dev(w.k_norm_w, d), dq=to_dev(w.dq, d), dk=to_dev(w.dk, d), dv=to_dev(w.dv, d))


def _outputs(x):
    return (torch.full_like(x["qkv"], float("nan")), torch.full((x["wq"].numel(),), float("nan"), device="cuda"),
            torch.full((x["wq"].numel(),), float("nan"), device="cuda"))


def _layout(w, x):
    return qk.gqa_layout(x["qkv"], w.kind, w.n_kv, w.q_per_kv, w.head_dim, w.rope_dim > 0)


def _noalloc(w, x, out, stream=None):
    L = _layout(w, x)
    qk.qkvnr_backward_noalloc(L, x["qkv"], x["pos"], x["wq"], x["wk"], w.eps, w.theta, x["dq"], x["dk"], x["dv"],
                              out[0], out[1], out[2], stream)


def _with_workspace(w, x, out):
    L = _layout(w, x)
    ws = torch.zeros(qk.qkvnr_backward_workspace_bytes(L), dtype=torch.uint8, device="cuda")
    qk.qkvnr_backward(L, x["qkv"], x["pos"], x["wq"], x["wk"], w.eps, w.theta, x["dq"], x["dk"], x["dv"],
                      out[0], out[1], out[2], ws, ws.numel())
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0


def _check(w, out, ref, tag):
    gq, gk, gv = oracle.split(to_host_bits(out[0]), w.kind, w.n_kv, w.q_per_kv, w.head_dim)
    assert_close(gq, ref["dx_q"], w.dtype, f"{tag} dq slots")
    assert_close(gk, ref["dx_k"], w.dtype, f"{tag} dk slots")
    assert_bits_equal(gv, w.dv, f"{tag} dv slots")
    assert_values_close(out[1].cpu().numpy(), ref["dw_q"], w.dtype, f"{tag} dq_norm_w", scale=ref["dw_q_l2"])
    assert_values_close(out[2].cpu().numpy(), ref["dw_k"], w.dtype, f"{tag} dk_norm_w", scale=ref["dw_k_l2"])


CASES = [("sectioned", "bf16", 3001, 8, 4, 128, True, 61),   # many blocks: every slot takes atomics
         ("interleaved", "bf16", 37, 3, 5, 64, True, 62),    # smaller, other head size, ragged iterations
         ("interleaved", "fp32", 5, 2, 2, 64, False, 63)]    # smaller still, fp32 NoPE


def test_noalloc_matches_workspace_backward_on_calls_in_a_row():
    for kind, dtype, T, n_kv, Q, D, rope, seed in CASES:
        w = custom_gqa(kind, dtype, T, n_kv, Q, D, rope=rope, theta=1e6, seed=seed, positions="random", grads=True)
        x = _inputs(w)
        a, b = _outputs(x), _outputs(x)
        _noalloc(w, x, a)
        _with_workspace(w, x, b)
        torch.cuda.synchronize()
        tag = f"{kind} {dtype} T={T} D={D}"
        assert_bits_equal(to_host_bits(a[0]), to_host_bits(b[0]), f"{tag}: dqkv no-alloc vs workspace")
        for i, nm in ((1, "dq_norm_w"), (2, "dk_norm_w")):
            x1, x2 = a[i].cpu().numpy().astype(np.float64), b[i].cpu().numpy().astype(np.float64)
            assert np.allclose(x1, x2, rtol=1e-5, atol=1e-5 * np.abs(x2).max()), f"{tag}: {nm} differ"
        ref = oracle.backward_gqa(w.qkv, dtype, kind, n_kv, Q, D, w.positions, w.q_norm_w, w.k_norm_w, w.eps,
                                  w.theta, w.dq, w.dk, w.dv, rope=rope)
        _check(w, a, ref, f"no-alloc {tag}")


def test_noalloc_rejects_what_the_workspace_backward_rejects():
    w = custom_gqa("interleaved", "bf16", 8, 2, 2, 64, seed=64, positions="random", grads=True)
    x = _inputs(w)
    out = _outputs(x)
    L = _layout(w, x)
    rc = qk.lib().qkvnr_backward_noalloc(ctypes.byref(L), x["qkv"].data_ptr(), x["pos"].data_ptr(),
                                         x["wq"].data_ptr(), x["wk"].data_ptr(), w.eps, w.theta, x["dq"].data_ptr(),
                                         x["dk"].data_ptr(), x["dv"].data_ptr(), x["qkv"].data_ptr(),
                                         out[1].data_ptr(), out[2].data_ptr(), None)
    assert rc == qk.EINVAL  # dqkv overlaps qkv: refused before any launch
    # the array was not touched: the next call is still exact
    _noalloc(w, x, out)
    torch.cuda.synchronize()
    ref = oracle.backward_gqa(w.qkv, "bf16", "interleaved", 2, 2, 64, w.positions, w.q_norm_w, w.k_norm_w, w.eps,
                              w.theta, w.dq, w.dk, w.dv)
    _check(w, out, ref, "no-alloc after a refused call")


def test_noalloc_graph_replays_match_eager():
    w = custom_gqa("sectioned", "bf16", 700, 8, 4, 128, theta=1e6, seed=65, positions="random", grads=True)
    x = _inputs(w)
    out = _outputs(x)
    _noalloc(w, x, out)
    torch.cuda.synchronize()
    ref_dqkv = to_host_bits(out[0])
    ref_dw = [t.cpu().numpy().astype(np.float64) for t in out[1:]]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _noalloc(w, x, out, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _noalloc(w, x, out)
    small = custom_gqa("interleaved", "bf16", 50, 2, 3, 64, seed=66, positions="random", grads=True)
    xs = _inputs(small)
    for r in range(4):
        for t in out:
            t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_bits_equal(to_host_bits(out[0]), ref_dqkv, f"replay {r} dqkv")
        for got, exp in zip(out[1:], ref_dw):
            got = got.cpu().numpy().astype(np.float64)
            assert np.allclose(got, exp, rtol=1e-5, atol=1e-5 * np.abs(exp).max()), f"replay {r} weight grads"
        # eager no-alloc work on the same array between replays
        so = _outputs(xs)
        _noalloc(small, xs, so)
        torch.cuda.synchronize()
        ref = oracle.backward_gqa(small.qkv, "bf16", "interleaved", 2, 3, 64, small.positions, small.q_norm_w,
                                  small.k_norm_w, small.eps, small.theta, small.dq, small.dk, small.dv)
        _check(small, so, ref, f"eager no-alloc between replays {r}")
