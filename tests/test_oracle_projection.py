"""Pins of the fused projection + region oracle (CPU only).

``oracle.projection`` is checked against things other than its own formulas:
a one-hot weight makes the projection an exact column selection, so the fused
result must equal the region oracle on the selected columns, bit for bit (this
fixes the product's orientation and the weight's row order); brute-force sums
for the product; doubling the weight doubles v exactly and leaves the eps-free
norm unchanged; and the DeepSpeed page's layout fact that the sectioned and the
interleaved packings of the same heads give the same heads.
"""
import math

import numpy as np
import pytest

from oracle import forward_gqa, project, projected_forward_gqa, to_f64
from qkv_inputs.generators import bf16_bits_from_f32, projection

ONE_BF16 = np.uint16(0x3F80)


def _one_hot_weight(rng, width, hidden):
    cols = rng.choice(hidden, size=width, replace=False)
    w = np.zeros((width, hidden), dtype=np.uint16)
    w[np.arange(width), cols] = ONE_BF16
    return w, cols


@pytest.mark.parametrize("kind", ["interleaved", "sectioned"])
@pytest.mark.parametrize("rope", [True, False])
def test_one_hot_weight_reduces_to_the_region_exactly(kind, rope):
    n_kv, Q, D = 2, 3, 16
    inp = projection(kind, 7, 5 * 16 * 2 + 3, n_kv, Q, D, rope=rope, theta=1e4, positions="random", seed=61)
    rng = np.random.default_rng(5)
    w, cols = _one_hot_weight(rng, inp.width, inp.hidden)
    got = projected_forward_gqa(inp.x, w, kind, n_kv, Q, D, inp.positions, inp.q_norm_w, inp.k_norm_w,
                                inp.eps, inp.theta, rope=rope)
    packed = inp.x[:, cols]
    if kind == "interleaved":
        packed = packed.reshape(inp.T, n_kv, Q + 2, D)
    q64, k64, v_bits = forward_gqa(packed, "bf16", kind, n_kv, Q, D, inp.positions, inp.q_norm_w, inp.k_norm_w,
                                   inp.eps, inp.theta, rope=rope)
    np.testing.assert_array_equal(got[0], q64)
    np.testing.assert_array_equal(got[1], k64)
    np.testing.assert_array_equal(got[2], to_f64(v_bits, "bf16"))


def test_product_equals_brute_force_sums():
    rng = np.random.default_rng(6)
    x = bf16_bits_from_f32(rng.standard_normal((3, 5)).astype(np.float32))
    w = bf16_bits_from_f32(rng.standard_normal((4, 5)).astype(np.float32))
    xf, wf = to_f64(x, "bf16"), to_f64(w, "bf16")
    want = np.array([[math.fsum(xf[t, c] * wf[j, c] for c in range(5)) for j in range(4)] for t in range(3)])
    np.testing.assert_allclose(project(x, w), want, rtol=1e-15, atol=1e-15)


def test_doubling_the_weight():
    inp = projection("sectioned", 6, 64, 2, 2, 16, theta=1e4, seed=62)
    w2 = bf16_bits_from_f32(2.0 * to_f64(inp.w_qkv, "bf16").astype(np.float32))   # exact: a power of two
    args = (inp.kind, inp.n_kv, inp.q_per_kv, inp.head_dim, inp.positions, inp.q_norm_w, inp.k_norm_w)
    a = projected_forward_gqa(inp.x, inp.w_qkv, *args, 0.0, inp.theta)
    b = projected_forward_gqa(inp.x, w2, *args, 0.0, inp.theta)
    np.testing.assert_array_equal(b[2], 2.0 * a[2])                  # v is linear in the weight
    np.testing.assert_allclose(b[0], a[0], rtol=1e-13, atol=1e-13)    # RMSNorm without eps is scale-free
    np.testing.assert_allclose(b[1], a[1], rtol=1e-13, atol=1e-13)


def test_sectioned_and_interleaved_weights_give_the_same_heads():
    n_kv, Q, D, hidden = 2, 3, 16, 48
    inp = projection("sectioned", 5, hidden, n_kv, Q, D, theta=1e4, positions="random", seed=63)
    n_q = n_kv * Q
    blocks = inp.w_qkv.reshape(n_q + 2 * n_kv, D, hidden)
    order = []   # sectioned block of each interleaved block
    for g in range(n_kv):
        order += [g * Q + s for s in range(Q)] + [n_q + g, n_q + n_kv + g]
    w_inter = blocks[order].reshape(-1, hidden)
    args = (n_kv, Q, D, inp.positions, inp.q_norm_w, inp.k_norm_w, inp.eps, inp.theta)
    s = projected_forward_gqa(inp.x, inp.w_qkv, "sectioned", *args)
    i = projected_forward_gqa(inp.x, w_inter, "interleaved", *args)
    for a, b in zip(s, i):
        np.testing.assert_array_equal(a, b)


def test_chunks_do_not_change_the_result():
    inp = projection("interleaved", 37, 32, 1, 2, 16, theta=1e4, seed=64)
    args = (inp.kind, inp.n_kv, inp.q_per_kv, inp.head_dim, inp.positions, inp.q_norm_w, inp.k_norm_w,
            inp.eps, inp.theta)
    whole = projected_forward_gqa(inp.x, inp.w_qkv, *args, chunk=1024)
    pieces = projected_forward_gqa(inp.x, inp.w_qkv, *args, chunk=8)
    for a, b in zip(whole, pieces):
        np.testing.assert_array_equal(a, b)
