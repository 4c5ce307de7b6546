"""Pins of the per-head Newton-Schulz oracle (CPU only).

``oracle.muon`` is checked against things other than its own formulas: the
singular value decomposition (a matrix polynomial in X X^T applied to X keeps
the singular vectors and maps each singular value through the scalar
iteration; the same fact lets the library collapse the steps into one matrix
polynomial in G G^T), the DeepSpeed page's layout facts (sectioned and interleaved fused
weights give the same update up to the block permutation; 8 query heads over 2
kv heads are 12 blocks; the Falcon and Conv1D shapes are declined), the scale
rule's closed forms, and the rank-one case.
"""
import json
import os

import numpy as np
import pytest

from oracle import muon

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_layout_examples.json")


def _scalar_iterate(s, steps=5):
    # the quintic acting on one singular value
    a, b, c = 3.4445, -4.7750, 2.0315
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


@pytest.mark.parametrize("shape", [(16, 40), (40, 16), (8, 8), (1, 33)])
def test_newton_schulz_equals_its_spectral_form(shape):
    rng = np.random.default_rng(sum(shape))
    G = rng.standard_normal(shape)
    U, S, Vt = np.linalg.svd(G, full_matrices=False)
    want = U @ np.diag(_scalar_iterate(S / (np.linalg.norm(G) + 1e-7))) @ Vt
    np.testing.assert_allclose(muon.newton_schulz(G), want, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("shape,steps", [((16, 40), 5), ((8, 64), 1), ((32, 32), 3), ((12, 200), 7)])
def test_iteration_collapses_to_a_polynomial_in_the_gram_matrix(shape, steps):
    # every step multiplies X by a polynomial in G G^T, so the iterate is M G with M from the recurrence
    # P_k = a I + b A_k + c A_k^2, A_{k+1} = P_k A_k P_k, M_{k+1} = P_k M_k on the normalised Gram matrix:
    # the reformulation the library's collapsed iteration takes, against the steps as the oracle takes them
    a, b, c = 3.4445, -4.7750, 2.0315
    G = np.random.default_rng(sum(shape) + steps).standard_normal(shape)
    n = np.linalg.norm(G) + 1e-7
    A, M = G @ G.T / n ** 2, np.eye(shape[0])
    for _ in range(steps):
        P = a * np.eye(shape[0]) + b * A + c * A @ A
        A, M = P @ A @ P, P @ M
    np.testing.assert_allclose(M @ G / n, muon.newton_schulz(G, steps=steps), rtol=1e-9, atol=1e-12)


def test_rank_one_block_has_a_closed_form():
    g = np.random.default_rng(1).standard_normal(50)
    G = g[None, :]
    s = _scalar_iterate(np.linalg.norm(g) / (np.linalg.norm(g) + 1e-7))
    np.testing.assert_allclose(muon.newton_schulz(G)[0], s * g / np.linalg.norm(g), rtol=1e-12)


def test_output_is_nearly_orthogonal_and_scale_free():
    rng = np.random.default_rng(2)
    G = rng.standard_normal((32, 256))
    X = muon.newton_schulz(G)
    sv = np.linalg.svd(X, compute_uv=False)
    assert sv.min() > 0.6 and sv.max() < 1.25, sv  # the quintic's band after 5 steps
    # equal up to the 1e-7 guard in the normalisation (relative 1e-9 here)
    np.testing.assert_allclose(muon.newton_schulz(1e3 * G), X, rtol=0, atol=1e-8)


def _heads(rng, n, D, cols):
    return [rng.standard_normal((D, cols)) for _ in range(n)]


def test_sectioned_and_interleaved_updates_are_the_same_block_permutation():
    rng = np.random.default_rng(3)
    n_kv, Q, D, cols = 2, 4, 8, 24
    n_q = n_kv * Q
    q, k, v = _heads(rng, n_q, D, cols), _heads(rng, n_kv, D, cols), _heads(rng, n_kv, D, cols)
    sectioned = np.concatenate(q + k + v)
    inter_blocks = []
    order = []   # sectioned block index of each interleaved block
    for g in range(n_kv):
        for s in range(Q):
            inter_blocks.append(q[g * Q + s]); order.append(g * Q + s)
        inter_blocks.append(k[g]); order.append(n_q + g)
        inter_blocks.append(v[g]); order.append(n_q + n_kv + g)
    interleaved = np.concatenate(inter_blocks)
    us = muon.per_head_update(sectioned, n_q, n_kv, D).reshape(-1, D, cols)
    ui = muon.per_head_update(interleaved, n_q, n_kv, D).reshape(-1, D, cols)
    np.testing.assert_array_equal(ui, us[order])


def test_fused_and_separately_stored_weights_get_the_same_per_head_update():
    rng = np.random.default_rng(4)
    n_q, n_kv, D, cols = 6, 2, 8, 16
    q, k, v = (np.concatenate(_heads(rng, n, D, cols)) for n in (n_q, n_kv, n_kv))
    fused = muon.per_head_update(np.concatenate([q, k, v]), n_q, n_kv, D)
    separate = np.concatenate([muon.per_head_update(part, n, 0, D) for part, n in ((q, n_q), (k, n_kv), (v, n_kv))])
    np.testing.assert_array_equal(fused, separate)


def test_full_matrix_scale_of_a_fused_square_projection_is_sqrt3():
    # [3h, h]: the full-matrix path scales by sqrt(3); per head (head_dim < h) by 1
    rng = np.random.default_rng(5)
    h = 12
    W = rng.standard_normal((3 * h, h))
    np.testing.assert_allclose(muon.full_matrix_update(W), np.sqrt(3.0) * muon.newton_schulz(W), rtol=1e-12)
    per = muon.per_head_update(W, 3, 0, h)   # three h x h blocks: scale 1
    np.testing.assert_allclose(per[:h], muon.newton_schulz(W[:h]), rtol=1e-12)
    assert muon.scale(4, 2) == pytest.approx(np.sqrt(2.0)) and muon.scale(2, 4) == 1.0


def test_head_block_count_and_exact_total_guard():
    g = json.load(open(GOLDEN))
    hb = g["head_block_count"]
    assert muon.head_block_count(hb["blocks"] * 16, hb["n_q"], hb["n_kv"], 16) == hb["blocks"]
    f = g["falcon_exact_total"]
    # the config's fused total describes 3 n_q heads of head_dim 8; the weight holds 80 rows
    assert muon.head_block_count(f["weight_rows"], 8, 8, 8) is None
    assert muon.head_block_count(f["config_rows"], 8, 8, 8) == 24
    # a transposed Conv1D weight [hidden, 3 hidden] (12 heads of 64): dim 0 is the input axis
    assert muon.head_block_count(768, 12, 12, 64) is None
    with pytest.raises(ValueError):
        muon.per_head_update(np.zeros((80, 4)), 8, 8, 8)
