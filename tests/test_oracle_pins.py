"""Pins of the CPU oracle against things other than itself (CPU only).

Each test checks the oracle against a library routine evaluated in fp64 (or in
fp32 where that library only works in fp32), a closed form, an invariant of the
definition, fp64 finite differences, brute force on tiny inputs, or a layout
example printed on the pages (``tests/golden/``).  Together they are chosen so
that a dropped term, a wrong sign, a wrong index or a transposed operand
anywhere in the oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from qkv_inputs import bf16_bits_from_f32, custom_gqa, latent_paged

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# --------------------------------------------------------------------------- #
# Layouts
# --------------------------------------------------------------------------- #


@pytest.mark.parametrize("kind", ["interleaved", "sectioned"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("shape", [(5, 2, 3, 64), (3, 16, 8, 64), (4, 8, 4, 128), (2, 1, 1, 8)])
def test_split_unsplit_roundtrip_bit_exact(kind, dtype, shape):
    T, n_kv, Q, D = shape
    w = custom_gqa(kind, dtype, T, n_kv, Q, D, seed=11)
    q, k, v = oracle.split(w.qkv, kind, n_kv, Q, D)
    assert q.shape == (T, n_kv * Q, D) and k.shape == (T, n_kv, D) and v.shape == (T, n_kv, D)
    back = oracle.unsplit(q, k, v, kind, Q)
    assert back.dtype == w.qkv.dtype
    assert np.array_equal(back.reshape(-1).view(np.uint8), w.qkv.reshape(-1).view(np.uint8))


def _labelled(T, H, D):
    # element value encodes (token, block, d) so every move can be traced
    t = np.arange(T)[:, None, None]
    b = np.arange(H)[None, :, None]
    d = np.arange(D)[None, None, :]
    return (t * 1_000_000 + b * 1_000 + d).astype(np.int64)


def test_split_labels_interleaved():
    # Muse-style grouping: per kv group, q_per_kv q heads, then one k, then one v
    T, n_kv, Q, D = 3, 4, 3, 8
    X = _labelled(T, n_kv * (Q + 2), D)
    q, k, v = oracle.split(X, "interleaved", n_kv, Q, D)
    for t in range(T):
        for h in range(n_kv * Q):
            g, s = divmod(h, Q)
            assert np.array_equal(q[t, h], X[t, g * (Q + 2) + s])
        for g in range(n_kv):
            assert np.array_equal(k[t, g], X[t, g * (Q + 2) + Q])
            assert np.array_equal(v[t, g], X[t, g * (Q + 2) + Q + 1])


def test_split_labels_sectioned():
    T, n_kv, Q, D = 2, 2, 4, 8
    n_q = n_kv * Q
    X = _labelled(T, n_q + 2 * n_kv, D)
    q, k, v = oracle.split(X.reshape(T, -1), "sectioned", n_kv, Q, D)
    assert np.array_equal(q, X[:, :n_q])
    assert np.array_equal(k, X[:, n_q:n_q + n_kv])
    assert np.array_equal(v, X[:, n_q + n_kv:])


def test_page_layout_examples():
    ex = json.load(open(os.path.join(GOLDEN, "page_layout_examples.json")))
    hb = ex["head_block_count"]
    assert oracle.head_blocks(hb["n_q"], hb["n_kv"]) == hb["blocks"]
    assert oracle.head_blocks(hb["n_q"], hb["n_kv"]) not in hb["not_blocks"]

    m = ex["muse_spark_packed"]
    G, S, D = m["packed_shape_per_token"]
    assert oracle.head_blocks(m["q_heads"], m["n_kv"]) == m["blocks_per_token"] == G * S
    assert oracle.exact_total_ok(m["width"], m["q_heads"], m["n_kv"], D)
    X = np.zeros((2, G, S, D), dtype=np.uint16)
    q, k, v = oracle.split(X, "interleaved", m["n_kv"], m["q_per_kv"], D)
    assert q.shape == (2, m["q_heads"], D) and k.shape == (2, G, D) and v.shape == (2, G, D)

    f = ex["falcon_exact_total"]
    n_q, D = f["n_q"], f["head_dim"]
    assert oracle.head_blocks(n_q, f["config_n_kv"]) * D == f["config_rows"]
    assert oracle.head_blocks(n_q, f["built_n_kv"]) * D == f["weight_rows"]
    # the config's description is declined for the weight that was actually built
    assert not oracle.exact_total_ok(f["weight_rows"], n_q, f["config_n_kv"], D)
    assert oracle.exact_total_ok(f["weight_rows"], n_q, f["built_n_kv"], D)


def _interleaved_to_sectioned_block(n_kv, Q):
    """Block j of the interleaved row -> its block index in the sectioned row."""
    n_q = n_kv * Q
    m = []
    for g in range(n_kv):
        for s in range(Q + 2):
            m.append(g * Q + s if s < Q else (n_q + g if s == Q else n_q + n_kv + g))
    return np.array(m)


@pytest.mark.parametrize("rope", [True, False])
def test_layouts_are_one_permutation_fwd_and_bwd(rope):
    # the same logical heads packed both ways give the same per-head results, and
    # the packed grads are the same block permutation of each other
    T, n_kv, Q, D = 6, 2, 3, 16
    w = custom_gqa("interleaved", "fp32", T, n_kv, Q, D, rope=rope, seed=5, grads=True,
                   positions="random", max_pos=1000)
    perm = _interleaved_to_sectioned_block(n_kv, Q)
    H = n_kv * (Q + 2)
    Xi = w.qkv.reshape(T, H, D)
    Xs = np.empty_like(Xi)
    Xs[:, perm] = Xi
    Xs = Xs.reshape(T, H * D)
    args = dict(dtype="fp32", n_kv=n_kv, q_per_kv=Q, head_dim=D, pos=w.positions,
                q_norm_w=w.q_norm_w, k_norm_w=w.k_norm_w, eps=w.eps, theta=w.theta, rope=rope)
    qi, ki, vi = oracle.forward_gqa(w.qkv, kind="interleaved", **args)
    qs, ks, vs = oracle.forward_gqa(Xs, kind="sectioned", **args)
    assert np.array_equal(qi, qs) and np.array_equal(ki, ks) and np.array_equal(vi, vs)
    bi = oracle.backward_gqa(w.qkv, kind="interleaved", dq=w.dq, dk=w.dk, dv=w.dv, **args)
    bs = oracle.backward_gqa(Xs, kind="sectioned", dq=w.dq, dk=w.dk, dv=w.dv, **args)
    assert np.array_equal(bi["dqkv64"].reshape(T, H, D), bs["dqkv64"].reshape(T, H, D)[:, perm])
    assert np.array_equal(bi["dw_q"], bs["dw_q"]) and np.array_equal(bi["dw_k"], bs["dw_k"])


# --------------------------------------------------------------------------- #
# RoPE
# --------------------------------------------------------------------------- #


def test_rope_hand_worked_head():
    # D = R = 4, theta = 1e4: inv_freq = (1, 1e4**(-1/2)) = (1, 0.01); at position
    # 100 the angles are (100 rad, 1 rad).  x = (3, 4, 0, 0) has rms 2.5, so with
    # w = 1 and eps = 0 the normed head is (1.2, 1.6, 0, 0) and the rotated head is
    # (1.2 cos 100, 1.6 cos 1, 1.2 sin 100, 1.6 sin 1).
    phi = oracle.rope_angles(np.array([100]), 1e4, 4)
    assert phi[0, 0] == 100.0 and abs(phi[0, 1] - 1.0) < 1e-15
    n = oracle.rmsnorm(np.array([[3.0, 4.0, 0.0, 0.0]]), np.ones(4), 0.0)
    assert np.allclose(n, [[1.2, 1.6, 0.0, 0.0]], rtol=0, atol=1e-15)
    y = oracle.rope_rotate_half(n, phi)
    want = [1.2 * math.cos(100), 1.6 * math.cos(1), 1.2 * math.sin(100), 1.6 * math.sin(1)]
    assert np.allclose(y[0], want, rtol=0, atol=1e-14)


def test_rope_matches_complex_multiplication():
    # pair (x_i, x_{i+R/2}) as the complex number x_i + 1j x_{i+R/2}, times e^{j phi_i}
    rng = _rng(1)
    T, H, R = 7, 3, 64
    x = rng.standard_normal((T, H, R))
    pos = rng.integers(0, 131072, size=T)
    phi = oracle.rope_angles(pos, 5e5, R)
    y = oracle.rope_rotate_half(x, phi)
    z = (x[..., :R // 2] + 1j * x[..., R // 2:]) * np.exp(1j * phi)[:, None, :]
    assert np.allclose(y[..., :R // 2], z.real, rtol=0, atol=1e-13)
    assert np.allclose(y[..., R // 2:], z.imag, rtol=0, atol=1e-13)


def test_rope_position_zero_is_identity():
    x = _rng(2).standard_normal((4, 5, 128))
    y = oracle.rope_rotate_half(x, oracle.rope_angles(np.zeros(4, dtype=np.int32), 1e6, 128))
    assert np.array_equal(x, y)


def test_rope_preserves_each_pair_norm():
    rng = _rng(3)
    x = rng.standard_normal((9, 2, 64))
    phi = oracle.rope_angles(rng.integers(0, 131072, size=9), 5e5, 64)
    y = oracle.rope_rotate_half(x, phi)
    nx = x[..., :32] ** 2 + x[..., 32:] ** 2
    ny = y[..., :32] ** 2 + y[..., 32:] ** 2
    assert np.allclose(nx, ny, rtol=1e-12, atol=0)


@pytest.mark.parametrize("theta,R", [(1e4, 64), (5e5, 64), (1e6, 128)])
def test_rope_scores_depend_only_on_relative_position(theta, R):
    rng = _rng(4)
    q = rng.standard_normal(R)
    k = rng.standard_normal(R)
    for m, n in [(0, 0), (5, 3), (131000, 130990), (16383, 0)]:
        base = None
        for shift in [0, 1, 777, 100000 - max(m, n) % 1000]:
            pm = oracle.rope_rotate_half(q[None, None], oracle.rope_angles(np.array([m + shift]), theta, R))
            pn = oracle.rope_rotate_half(k[None, None], oracle.rope_angles(np.array([n + shift]), theta, R))
            s = float(np.dot(pm.ravel(), pn.ravel()))
            if base is None:
                base = s
            assert abs(s - base) <= 1e-9 * max(1.0, abs(base))


def test_rope_inverse_undoes_rotation():
    rng = _rng(5)
    x = rng.standard_normal((6, 4, 64))
    phi = oracle.rope_angles(rng.integers(0, 131072, size=6), 5e5, 64)
    back = oracle.rope_rotate_half_inverse(oracle.rope_rotate_half(x, phi), phi)
    assert np.allclose(back, x, rtol=0, atol=1e-13)


@pytest.mark.parametrize("theta,D", [(1e6, 128), (5e5, 64), (1e4, 64)])
def test_rope_matches_transformers_qwen3(theta, D):
    # library pin: transformers' Qwen3 rotary embedding + apply_rotary_pos_emb (fp32
    # angles inside the library, so small positions and an fp32-level tolerance)
    from transformers import Qwen3Config
    from transformers.models.qwen3 import modeling_qwen3 as mq

    cfg = Qwen3Config(head_dim=D, num_attention_heads=4, num_key_value_heads=2, hidden_size=4 * D,
                      rope_parameters={"rope_type": "default", "rope_theta": theta})
    emb = mq.Qwen3RotaryEmbedding(cfg)
    T = 40
    pos = np.arange(T) * 3 % 47
    cos, sin = emb(torch.zeros(1, T, 4 * D), torch.from_numpy(pos)[None])
    x = _rng(6).standard_normal((T, 4, D))
    xt = torch.from_numpy(x).float().transpose(0, 1)[None]  # [1, H, T, D]
    yq, _ = mq.apply_rotary_pos_emb(xt, xt, cos, sin, unsqueeze_dim=1)
    lib = yq[0].transpose(0, 1).double().numpy()
    ours = oracle.rope_rotate_half(x, oracle.rope_angles(pos, theta, D))
    assert np.allclose(ours, lib, rtol=0, atol=3e-5)


# --------------------------------------------------------------------------- #
# RMSNorm
# --------------------------------------------------------------------------- #


@pytest.mark.parametrize("eps", [1e-6, 0.3])
def test_rmsnorm_matches_torch_fp64(eps):
    rng = _rng(7)
    x = rng.standard_normal((5, 3, 64)) * 3
    w = 1 + 0.1 * rng.standard_normal(64)
    lib = torch.nn.functional.rms_norm(torch.from_numpy(x), (64,), weight=torch.from_numpy(w), eps=eps)
    assert np.allclose(oracle.rmsnorm(x, w, eps), lib.numpy(), rtol=1e-14, atol=1e-14)


def test_rmsnorm_closed_form_rms():
    # with w = 1 the output's rms is sqrt(ms / (ms + eps)) exactly
    rng = _rng(8)
    x = rng.standard_normal((50, 64)) * rng.uniform(0.1, 3, size=(50, 1))
    eps = 0.25
    y = oracle.rmsnorm(x, np.ones(64), eps)
    ms = np.mean(x * x, axis=1)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=1)), np.sqrt(ms / (ms + eps)), rtol=1e-13)


def test_rmsnorm_is_per_head_not_per_row():
    # scaling one head leaves the other heads' outputs untouched and its own unchanged (eps = 0)
    rng = _rng(9)
    x = rng.standard_normal((2, 4, 16))
    w = rng.standard_normal(16)
    y0 = oracle.rmsnorm(x, w, 0.0)
    x2 = x.copy()
    x2[:, 1] *= 7.0
    y1 = oracle.rmsnorm(x2, w, 0.0)
    assert np.allclose(y0, y1, rtol=1e-14, atol=1e-14)


# --------------------------------------------------------------------------- #
# Whole forward against a library model's q/k preparation
# --------------------------------------------------------------------------- #


def test_forward_matches_transformers_qwen3_qk_prep():
    # Qwen3's attention applies a per-head RMSNorm to q and k, then rotate-half RoPE.
    from transformers import Qwen3Config
    from transformers.models.qwen3 import modeling_qwen3 as mq

    T, n_kv, Q, D = 12, 2, 2, 128
    n_q = n_kv * Q
    w = custom_gqa("sectioned", "fp32", T, n_kv, Q, D, theta=1e6, seed=12, positions="arange")
    cfg = Qwen3Config(head_dim=D, num_attention_heads=n_q, num_key_value_heads=n_kv,
                      hidden_size=n_q * D, rope_parameters={"rope_type": "default", "rope_theta": 1e6},
                      rms_norm_eps=w.eps)
    qn = mq.Qwen3RMSNorm(D, eps=w.eps)
    kn = mq.Qwen3RMSNorm(D, eps=w.eps)
    with torch.no_grad():
        qn.weight.copy_(torch.from_numpy(w.q_norm_w))
        kn.weight.copy_(torch.from_numpy(w.k_norm_w))
        X = torch.from_numpy(w.qkv).reshape(T, n_q + 2 * n_kv, D)
        q = qn(X[:, :n_q]).transpose(0, 1)[None]
        k = kn(X[:, n_q:n_q + n_kv]).transpose(0, 1)[None]
        cos, sin = mq.Qwen3RotaryEmbedding(cfg)(X[None], torch.from_numpy(w.positions.astype(np.int64))[None])
        ql, kl = mq.apply_rotary_pos_emb(q, k, cos, sin, unsqueeze_dim=1)
    q64, k64, v = oracle.forward_gqa(w.qkv, "fp32", "sectioned", n_kv, Q, D, w.positions,
                                     w.q_norm_w, w.k_norm_w, w.eps, w.theta)
    assert np.allclose(q64, ql[0].transpose(0, 1).double().numpy(), rtol=0, atol=2e-5)
    assert np.allclose(k64, kl[0].transpose(0, 1).double().numpy(), rtol=0, atol=2e-5)
    assert np.array_equal(v, X[:, n_q + n_kv:].numpy())


def test_nope_equals_rope_at_position_zero():
    w = custom_gqa("interleaved", "bf16", 5, 2, 4, 64, seed=13, positions="random")
    a = dict(dtype="bf16", kind="interleaved", n_kv=2, q_per_kv=4, head_dim=64,
             q_norm_w=w.q_norm_w, k_norm_w=w.k_norm_w, eps=w.eps, theta=w.theta)
    qn, kn, _ = oracle.forward_gqa(w.qkv, pos=w.positions, rope=False, **a)
    qr, kr, _ = oracle.forward_gqa(w.qkv, pos=np.zeros(5, np.int32), rope=True, **a)
    assert np.array_equal(qn, qr) and np.array_equal(kn, kr)


# --------------------------------------------------------------------------- #
# Backward
# --------------------------------------------------------------------------- #


def _tiny_fp64_case(seed, kind="interleaved", rope=True):
    rng = _rng(seed)
    T, n_kv, Q, D = 3, 2, 2, 8
    n_q = n_kv * Q
    shape = (T, n_kv, Q + 2, D) if kind == "interleaved" else (T, (n_q + 2 * n_kv) * D)
    return dict(
        qkv=rng.standard_normal(shape), dtype="fp64", kind=kind, n_kv=n_kv, q_per_kv=Q,
        head_dim=D, pos=np.array([0, 5, 130000]), q_norm_w=1 + 0.1 * rng.standard_normal(D),
        k_norm_w=1 + 0.1 * rng.standard_normal(D), eps=0.05, theta=1e4, rope=rope,
    ), rng.standard_normal((T, n_q, D)), rng.standard_normal((T, n_kv, D)), rng.standard_normal((T, n_kv, D))


def _loss(args, gq, gk, gv):
    q, k, v = oracle.forward_gqa(**args)
    return float(np.sum(q * gq) + np.sum(k * gk) + np.sum(v * gv))


@pytest.mark.parametrize("kind", ["interleaved", "sectioned"])
@pytest.mark.parametrize("rope", [True, False])
def test_backward_matches_central_finite_differences(kind, rope):
    args, gq, gk, gv = _tiny_fp64_case(21, kind, rope)
    out = oracle.backward_gqa(dq=gq, dk=gk, dv=gv, **args)
    h = 1e-6
    X = args["qkv"]
    fd = np.empty(X.size)
    flat = X.reshape(-1)
    for i in range(flat.size):
        old = flat[i]
        flat[i] = old + h
        lp = _loss(args, gq, gk, gv)
        flat[i] = old - h
        lm = _loss(args, gq, gk, gv)
        flat[i] = old
        fd[i] = (lp - lm) / (2 * h)
    got = out["dqkv64"].reshape(-1)
    assert np.allclose(got, fd, rtol=1e-7, atol=1e-7 * np.abs(fd).max())
    for key, wkey in [("dw_q", "q_norm_w"), ("dw_k", "k_norm_w")]:
        wv = args[wkey]
        fdw = np.empty_like(wv)
        for i in range(wv.size):
            old = wv[i]
            wv[i] = old + h
            lp = _loss(args, gq, gk, gv)
            wv[i] = old - h
            lm = _loss(args, gq, gk, gv)
            wv[i] = old
            fdw[i] = (lp - lm) / (2 * h)
        assert np.allclose(out[key], fdw, rtol=1e-7, atol=1e-7 * np.abs(fdw).max())


def test_backward_matches_torch_autograd_fp64():
    # composed from library pieces: F.rms_norm and transformers' rotate-half apply
    from transformers.models.qwen3 import modeling_qwen3 as mq

    args, gq, gk, gv = _tiny_fp64_case(22, "sectioned", True)
    T, D, n_kv, Q = 3, 8, 2, 2
    n_q = n_kv * Q
    X = torch.tensor(args["qkv"], requires_grad=True)
    wq = torch.tensor(args["q_norm_w"], requires_grad=True)
    wk = torch.tensor(args["k_norm_w"], requires_grad=True)
    H = X.reshape(T, n_q + 2 * n_kv, D)
    q = torch.nn.functional.rms_norm(H[:, :n_q], (D,), weight=wq, eps=args["eps"])
    k = torch.nn.functional.rms_norm(H[:, n_q:n_q + n_kv], (D,), weight=wk, eps=args["eps"])
    pos = torch.tensor(args["pos"], dtype=torch.float64)
    inv = args["theta"] ** (-torch.arange(0, D, 2, dtype=torch.float64) / D)
    ang = pos[:, None] * inv[None]
    emb = torch.cat([ang, ang], dim=-1)
    cos, sin = emb.cos()[:, None], emb.sin()[:, None]
    qr, kr = mq.apply_rotary_pos_emb(q, k, cos, sin, unsqueeze_dim=0)
    v = H[:, n_q + n_kv:]
    L = (qr * torch.from_numpy(gq)).sum() + (kr * torch.from_numpy(gk)).sum() + (v * torch.from_numpy(gv)).sum()
    L.backward()
    out = oracle.backward_gqa(dq=gq, dk=gk, dv=gv, **args)
    assert np.allclose(out["dqkv64"], X.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(out["dw_q"], wq.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(out["dw_k"], wk.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_backward_closed_form_input_projection():
    # per head: <x, dx> = eps / (ms + eps) * <xhat, w * u>, with u = R(-phi) g
    args, gq, gk, gv = _tiny_fp64_case(23, "interleaved", True)
    out = oracle.backward_gqa(dq=gq, dk=gk, dv=gv, **args)
    q_raw, _, _ = oracle.split(args["qkv"], "interleaved", 2, 2, 8)
    phi = oracle.rope_angles(args["pos"], args["theta"], 8)
    u = oracle.rope_rotate_half_inverse(gq, phi)
    ms = np.mean(q_raw ** 2, axis=-1)
    xhat = q_raw / np.sqrt(ms + args["eps"])[..., None]
    lhs = np.sum(q_raw * out["dx_q"], axis=-1)
    rhs = args["eps"] / (ms + args["eps"]) * np.sum(xhat * args["q_norm_w"] * u, axis=-1)
    assert np.allclose(lhs, rhs, rtol=1e-11, atol=1e-13)


def test_backward_v_slots_carry_dv_bits():
    w = custom_gqa("interleaved", "bf16", 4, 2, 3, 64, seed=14, grads=True)
    out = oracle.backward_gqa(w.qkv, "bf16", "interleaved", 2, 3, 64, w.positions, w.q_norm_w,
                              w.k_norm_w, w.eps, w.theta, w.dq, w.dk, w.dv)
    assert np.array_equal(out["dv_bits"], w.dv)
    _, _, vslots = oracle.split(out["dqkv64"], "interleaved", 2, 3, 64)
    assert np.array_equal(oracle.round_to_storage(vslots, "bf16"), w.dv)


# --------------------------------------------------------------------------- #
# Latent rows and the paged pool
# --------------------------------------------------------------------------- #


def test_latent_row_is_norm_then_rope_on_separate_parts():
    w = latent_paged(B=2, T_req=3, num_pages=64, ctx_lo=10, ctx_hi=1000)
    out = oracle.latent_forward(w.qkv, "bf16", w.positions, w.k_norm_w, w.eps, w.theta, 512, 64)
    x = oracle.to_f64(w.qkv, "bf16")
    lib = torch.nn.functional.rms_norm(torch.from_numpy(x[:, :512]), (512,),
                                       weight=torch.from_numpy(oracle.to_f64(w.k_norm_w, "bf16")), eps=w.eps)
    assert np.allclose(out[:, :512], lib.numpy(), rtol=1e-14, atol=1e-14)
    # rope part: no norm, pairwise norms preserved, complex form
    kpe = x[:, 512:]
    phi = oracle.rope_angles(w.positions, w.theta, 64)
    z = (kpe[:, :32] + 1j * kpe[:, 32:]) * np.exp(1j * phi)
    assert np.allclose(out[:, 512:544], z.real, atol=1e-13, rtol=0)
    assert np.allclose(out[:, 544:], z.imag, atol=1e-13, rtol=0)


def test_paged_slots_brute_force():
    # two requests of 3 tokens, pages of 4 rows; positions follow each context
    table = np.array([[7, 2, 9, -1], [0, 5, -1, -1]], dtype=np.int32)
    pos = np.array([5, 6, 7, 3, 4, 5], dtype=np.int32)
    page, off = oracle.paged_slots(pos, table, 3, 4)
    # request 0: pos 5,6,7 -> table[0][1] = 2, offsets 1,2,3; request 1: pos 3 -> page 0 off 3,
    # pos 4,5 -> table[1][1] = 5, offsets 0,1
    assert page.tolist() == [2, 2, 2, 0, 5, 5]
    assert off.tolist() == [1, 2, 3, 3, 0, 1]


def test_staged_scatter_touches_only_its_rows():
    w = latent_paged(B=4, T_req=16, num_pages=1024, ctx_lo=100, ctx_hi=10000)
    pool = np.full((1024, 64, 576), 0x7FC1, dtype=np.uint16)
    rows = oracle.round_to_storage(
        oracle.latent_forward(w.qkv, "bf16", w.positions, w.k_norm_w, w.eps, w.theta, 512, 64), "bf16")
    page, off = oracle.paged_slots(w.positions, w.block_table, w.tokens_per_req, w.page_size)
    out = oracle.staged_then_scatter(pool, rows, page, off)
    written = np.zeros((1024, 64), dtype=bool)
    written[page, off] = True
    assert written.sum() == 64  # all slots distinct
    assert np.array_equal(out[page, off], rows)
    assert np.all(out[~written] == 0x7FC1)


# --------------------------------------------------------------------------- #
# Storage rounding and the generators
# --------------------------------------------------------------------------- #


def test_round_to_storage_bf16_nearest_even_without_double_rounding():
    one = 1.0
    cases = {
        one + 2.0 ** -8: 0x3F80,                   # tie -> even (1.0)
        one + 3 * 2.0 ** -8: 0x3F82,               # tie -> even (1 + 2**-6)
        one + 2.0 ** -8 + 2.0 ** -30: 0x3F81,      # just above the tie: up (an fp32 detour would tie)
        -(one + 2.0 ** -8 + 2.0 ** -30): 0xBF81,
        2.0 ** -126: 0x0080,
        0.0: 0x0000,
    }
    xs = np.array(list(cases.keys()))
    assert oracle.round_to_storage(xs, "bf16").tolist() == list(cases.values())


def test_round_to_storage_matches_torch_on_fp32_values():
    x = _rng(15).standard_normal(100000).astype(np.float32)
    lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.round_to_storage(x.astype(np.float64), "bf16"), lib)
    assert np.array_equal(bf16_bits_from_f32(x), lib)


def test_generators_are_deterministic():
    a = custom_gqa("sectioned", "bf16", 8, 2, 4, 128, seed=99, grads=True, positions="random")
    b = custom_gqa("sectioned", "bf16", 8, 2, 4, 128, seed=99, grads=True, positions="random")
    for x, y in [(a.qkv, b.qkv), (a.dq, b.dq), (a.positions, b.positions), (a.q_norm_w, b.q_norm_w)]:
        assert np.array_equal(x, y)
    c = latent_paged()
    d = latent_paged()
    assert np.array_equal(c.block_table, d.block_table) and np.array_equal(c.positions, d.positions)
    used = c.block_table[c.block_table >= 0]
    assert used.size == np.unique(used).size  # pages never shared between requests
