"""Pins of the MLA drafter layer oracle (CPU only).

The oracle (``oracle.mla_drafter``) is checked against things other than
itself: transformers' DeepSeek-V3 attention modules in fp64 (an independent
implementation of the same q/kv preparation), the defining property of the k
absorption (scores against latents equal scores against up-projected keys),
and the storage rule (bf16 intermediates are representable and within half an
ulp of the exact chain at the first storage point).
"""
import numpy as np
import pytest
import torch

import oracle
from qkv_inputs import bf16_bits_from_f32, mla_drafter_layer

SMALL = dict(hidden=64, q_lora_rank=48, kv_lora_rank=32, qk_nope_head_dim=16, qk_rope_head_dim=8, heads=4)


def _small(B=1, T_req=5, seed=7):
    return mla_drafter_layer(B, T_req, num_pages=64, page_size=16, ctx_lo=0, ctx_hi=40, seed=seed, **SMALL)


def _run(m, storage):
    return oracle.drafter_layer(m.x, m.w_input_ln, m.w_q_a, m.w_q_a_ln, m.w_q_b, m.w_uk, m.w_kv_a, m.w_kv_a_ln,
                                m.positions, heads=m.heads, qk_nope_head_dim=m.qk_nope_head_dim,
                                qk_rope_head_dim=m.qk_rope_head_dim, kv_lora_rank=m.kv_lora_rank, eps=m.eps,
                                theta=m.theta, storage=storage)


def _f64(bits):
    return oracle.to_f64(bits, "bf16")


def test_absorption_equals_scores_against_up_projected_keys():
    rng = np.random.default_rng(3)
    N, H, d, L, M = 6, 3, 5, 7, 4
    q_nope = rng.standard_normal((N, H, d))
    w_uk = rng.standard_normal((H, d, L))
    c = rng.standard_normal((M, L))
    q_abs = oracle.absorb(q_nope, w_uk)
    for h in range(H):
        k_nope = c @ w_uk[h].T                   # [M, d]: head h's keys W_UK[h] c
        want = q_nope[:, h, :] @ k_nope.T         # [N, M]
        got = q_abs[:, h, :] @ c.T
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_drafter_matches_transformers_deepseek_v3():
    from transformers import DeepseekV3Config
    from transformers.models.deepseek_v3 import modeling_deepseek_v3 as md

    m = _small()
    ref = _run(m, storage=None)
    N, H = m.x.shape[0], m.heads
    nope, rope, L = m.qk_nope_head_dim, m.qk_rope_head_dim, m.kv_lora_rank
    v_dim = 8
    cfg = DeepseekV3Config(hidden_size=m.hidden, num_attention_heads=H, num_key_value_heads=H,
                           q_lora_rank=m.q_lora_rank, kv_lora_rank=L, qk_nope_head_dim=nope,
                           qk_rope_head_dim=rope, v_head_dim=v_dim, rope_interleave=False,
                           rms_norm_eps=m.eps, attention_bias=False,
                           rope_parameters={"rope_type": "default", "rope_theta": m.theta})
    att = md.DeepseekV3Attention(cfg, layer_idx=0).double()
    in_ln = md.DeepseekV3RMSNorm(m.hidden, eps=m.eps).double()
    rot = md.DeepseekV3RotaryEmbedding(cfg)
    t = lambda a: torch.from_numpy(_f64(a))  # noqa: E731
    with torch.no_grad():
        in_ln.weight.copy_(t(m.w_input_ln))
        att.q_a_proj.weight.copy_(t(m.w_q_a).T)
        att.q_a_layernorm.weight.copy_(t(m.w_q_a_ln))
        att.q_b_proj.weight.copy_(t(m.w_q_b).T)
        att.kv_a_proj_with_mqa.weight.copy_(t(m.w_kv_a).T)
        att.kv_a_layernorm.weight.copy_(t(m.w_kv_a_ln))
        kvb = torch.zeros(H * (nope + v_dim), L, dtype=torch.float64)
        for h in range(H):   # head h's key up-projection is W_UK[h]; its value part stays zero
            kvb[h * (nope + v_dim):h * (nope + v_dim) + nope] = t(m.w_uk)[h]
        att.kv_b_proj.weight.copy_(kvb)

        x = t(m.x)[None]                                            # [1, N, hidden]
        xn = in_ln(x)
        pos = torch.from_numpy(m.positions.astype(np.int64))[None]
        cos, sin = rot(xn, pos)
        q = att.q_b_proj(att.q_a_layernorm(att.q_a_proj(xn))).view(1, N, H, nope + rope).transpose(1, 2)
        q_pass, q_rot = q[..., :nope], q[..., nope:]
        ckv = att.kv_a_proj_with_mqa(xn)
        kv_nope, k_rot = ckv[..., :L], ckv[..., L:]
        kv_nope = att.kv_a_layernorm(kv_nope)
        q_rot, k_rot = md.apply_rotary_pos_emb(q_rot, k_rot.view(1, 1, N, rope), cos, sin)
        k_nope = att.kv_b_proj(kv_nope).view(1, N, H, nope + v_dim)[..., :nope]   # [1, N, H, nope]

    rel = lambda a, b: float(np.max(np.abs(a - b)) / np.sqrt(np.mean(b * b)))  # noqa: E731
    # the library's norm computes in fp32 and its rotary angles are fp32: fp32-level agreement
    assert rel(ref["xn"], xn[0].numpy()) < 1e-6
    assert rel(ref["q_nope"], q_pass[0].transpose(0, 1).numpy()) < 1e-6
    assert rel(ref["q_pe"], q_rot[0].transpose(0, 1).numpy()) < 1e-5
    assert rel(ref["rows"][:, :L], kv_nope[0].numpy()) < 1e-6
    assert rel(ref["rows"][:, L:], k_rot[0, 0].numpy()) < 1e-5
    # the absorbed q against the normed latents gives the library's nope scores
    c = ref["rows"][:, :L]
    for h in range(H):
        want = q_pass[0, h].numpy() @ k_nope[0, :, h, :].numpy().T
        got = ref["q_abs"][:, h, :] @ c.T
        assert rel(got, want) < 1e-6


def test_storage_points_hold_bf16_values():
    m = _small(seed=8)
    exact = _run(m, storage=None)
    stored = _run(m, storage="bf16")
    for k in ("xn", "q_nope", "q_pe", "q_abs", "kv"):
        v = stored[k]
        back = oracle.to_f64(bf16_bits_from_f32(v.astype(np.float32)), "bf16")
        np.testing.assert_array_equal(back, v, err_msg=k)
    # the first storage point sees the exact value: rounding moves it by at most half an ulp
    ulp = 2.0 ** (np.floor(np.log2(np.abs(exact["xn"]))) - 7)
    assert np.all(np.abs(stored["xn"] - exact["xn"]) <= 0.5 * ulp)


@pytest.mark.parametrize("B", [1, 4])
def test_generator_shapes_and_mapping(B):
    m = mla_drafter_layer(B, 16)
    N = B * 16
    assert m.x.shape == (N, 7168) and m.w_uk.shape == (16, 128, 512) and m.w_kv_a.shape == (7168, 576)
    page, off = oracle.paged_slots(m.positions, m.block_table, m.tokens_per_req, m.page_size)
    assert np.all(page >= 0) and np.all(page < m.num_pages)
    slots = page * m.page_size + off
    assert len(np.unique(slots)) == N
