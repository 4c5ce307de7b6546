"""GPU: per-head Newton-Schulz on fused QKV weights against the fp64 oracle.

DeepSpeed page "[muon] Per-head Newton-Schulz for fused QKV projections":
the sectioned and interleaved orders of one fused weight give the same update
up to the block permutation (here bitwise: every block goes through the same
launches, and every sum is taken in a fixed order), and a weight whose rows are
not the exact fused total is declined.  Values: fp32 compute within 1e-4 *
max(|ref|, rms) of the fp64 oracle, element by element and in Frobenius norm
(five steps of products over rows up to 4096 long, in fp32).  bf16 compute of
the step-by-step path (blocks of side 8, 16 or 32 here) rounds X and P to bf16
at every step (each a 2**-8 relative rounding, five times over), which the
quintic does not damp for the smallest singular values: within 2**-5 of the
oracle in Frobenius norm and 2**-3 * max(|ref|, rms) element by element
(observed over 8 seeds: at most 7.5e-2 element-wise and 1.4e-2 Frobenius).
The collapsed path (blocks of side 64 and 128) rounds only its output: within
2**-8 in Frobenius norm and 2**-5 * max(|ref|, rms) element by element.  Each
launch is also checked against its own definition.
"""
import numpy as np
import pytest
import torch

import qkv_split_head_amd as qk
from oracle import muon as oracle_muon
from qkv_split_head_amd.muon import per_head_newton_schulz
from tests.helpers import announce, gpu_available

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu(request):
    if not gpu_available():
        pytest.skip("no GPU")
    qk.lib()
    announce(request.node.nodeid)
    yield
    torch.cuda.synchronize()


def _rel_err(got, ref):
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), rms)))


# blocks of 128 x 4096 (the Qwen3-8B-like weight) and of 64 x 1024, tall blocks of 128 x 64 (iterated as
# 64 x 128): the collapsed iteration; tall blocks of 128 x 72 and 64 x 32 and small sides: steps one by one
@pytest.mark.parametrize("n_q,n_kv,D,cols", [(32, 8, 128, 4096), (8, 2, 64, 1024), (2, 1, 128, 72), (2, 1, 128, 64),
                                             (8, 2, 16, 64), (4, 1, 64, 32), (3, 0, 8, 40)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_per_head_matches_oracle(n_q, n_kv, D, cols, dtype):
    d, wide = min(D, cols), max(D, cols)   # the blocks' short and long sides
    if dtype == torch.float32:
        tol, normwise_tol = 1e-4, 1e-4
    elif d in (64, 128) and wide % 8 == 0:   # the collapsed iteration: only its output is rounded to bf16
        tol, normwise_tol = 2.0 ** -4, 2.0 ** -6
    else:                                    # bf16 steps one by one
        tol, normwise_tol = 2.0 ** -3, 2.0 ** -5
    rng = np.random.default_rng(n_q * 100 + D + cols)
    rows = (n_q + 2 * n_kv) * D
    G = rng.standard_normal((rows, cols)).astype(np.float32)
    g = torch.from_numpy(G).cuda().to(dtype)
    got = per_head_newton_schulz(g, n_q, n_kv, D).float().cpu().numpy()
    ref = oracle_muon.per_head_update(g.float().cpu().numpy().astype(np.float64), n_q, n_kv, D)
    err = _rel_err(got, ref)
    nerr = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    print(f"[muon] {rows}x{cols} blocks of {D} {dtype}: max err / max(|ref|, rms) = {err:.2e},"
          f" Frobenius-relative {nerr:.2e}", flush=True)
    assert err <= tol and nerr <= normwise_tol


def test_rank_deficient_blocks_through_the_collapsed_path():
    # blocks of rank 8 (plus a little noise): M is large on the near-null space, M G is not
    rng = np.random.default_rng(21)
    n_q, n_kv, D, cols = 4, 2, 128, 1024
    blocks = [(rng.standard_normal((D, 8)) @ rng.standard_normal((8, cols)) + 1e-3 * rng.standard_normal((D, cols)))
              for _ in range(n_q + 2 * n_kv)]
    g = torch.from_numpy(np.concatenate(blocks).astype(np.float32)).cuda().to(torch.bfloat16)
    got = per_head_newton_schulz(g, n_q, n_kv, D).float().cpu().numpy()
    ref = oracle_muon.per_head_update(g.float().cpu().numpy().astype(np.float64), n_q, n_kv, D)
    nerr = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    print(f"[muon] rank-8 blocks of 128 x 1024: Frobenius-relative {nerr:.2e}", flush=True)
    assert nerr <= 2.0 ** -5


@pytest.mark.parametrize("D,cols,steps", [(128, 1024, 1), (128, 1024, 3), (64, 512, 7), (32, 256, 3)])
def test_other_step_counts_match_the_oracle(D, cols, steps):
    rng = np.random.default_rng(D + cols + steps)
    n_q, n_kv = 4, 2
    g = torch.from_numpy(rng.standard_normal(((n_q + 2 * n_kv) * D, cols)).astype(np.float32)).cuda()
    g = g.to(torch.bfloat16)
    got = per_head_newton_schulz(g, n_q, n_kv, D, steps=steps).float().cpu().numpy()
    ref = oracle_muon.per_head_update(g.float().cpu().numpy().astype(np.float64), n_q, n_kv, D, steps=steps)
    nerr = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    print(f"[muon] blocks of {D} x {cols}, {steps} steps: Frobenius-relative {nerr:.2e}", flush=True)
    assert nerr <= (2.0 ** -6 if D in (64, 128) else 2.0 ** -5)


@pytest.mark.parametrize("D,dtype", [(128, torch.bfloat16), (32, torch.bfloat16), (128, torch.float32)])
def test_an_all_zero_head_block_stays_zero(D, dtype):
    # ||G||_F = 0 for that block: the first step divides by eps, the block stays exactly zero (no NaN), and the
    # other blocks are updated as they would be alone
    rng = np.random.default_rng(D)
    n_q, n_kv, cols = 2, 1, 512
    w = rng.standard_normal(((n_q + 2 * n_kv) * D, cols)).astype(np.float32)
    w[D:2 * D] = 0.0
    g = torch.from_numpy(w).cuda().to(dtype)
    got = per_head_newton_schulz(g, n_q, n_kv, D).float().cpu().numpy()
    assert np.all(got[D:2 * D] == 0.0) and np.all(np.isfinite(got))
    ref = oracle_muon.per_head_update(g.float().cpu().numpy().astype(np.float64), n_q, n_kv, D)
    assert np.all(ref[D:2 * D] == 0.0)
    nerr = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    assert nerr <= (1e-4 if dtype == torch.float32 else 2.0 ** -5)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_sectioned_and_interleaved_give_the_same_blocks_bitwise(dtype):
    rng = np.random.default_rng(9)
    n_kv, Q, D, cols = 8, 4, 128, 1024
    n_q = n_kv * Q
    blocks = rng.standard_normal((n_q + 2 * n_kv, D, cols)).astype(np.float32)
    sect = torch.from_numpy(blocks.reshape(-1, cols)).cuda().to(dtype)
    order = []   # sectioned block of each interleaved block
    for gi in range(n_kv):
        order += [gi * Q + s for s in range(Q)] + [n_q + gi, n_q + n_kv + gi]
    inter = torch.from_numpy(blocks[order].reshape(-1, cols)).cuda().to(dtype)
    us = per_head_newton_schulz(sect, n_q, n_kv, D).view(-1, D, cols)
    ui = per_head_newton_schulz(inter, n_q, n_kv, D).view(-1, D, cols)
    torch.cuda.synchronize()
    assert torch.equal(ui.view(torch.int16) if dtype == torch.bfloat16 else ui,
                       us[order].view(torch.int16) if dtype == torch.bfloat16 else us[order])


@pytest.mark.parametrize("D,cols", [(128, 4096), (64, 1024)])
def test_repeated_updates_are_bitwise_equal(D, cols):
    # every sum is taken in a fixed order: the same input gives the same bits
    rng = np.random.default_rng(D + cols)
    g = torch.from_numpy(rng.standard_normal((48 * D, cols)).astype(np.float32)).cuda().to(torch.bfloat16)
    first = per_head_newton_schulz(g, 32, 8, D)
    for _ in range(4):
        again = per_head_newton_schulz(g, 32, 8, D)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int16), first.view(torch.int16))


# the 4 waves of a tile take runs of 64 columns in turn; 1320 and 1064 columns end a wave's runs
# with an odd and an even count of whole runs before a partial one
@pytest.mark.parametrize("blocks,d,cols,parts", [(3, 32, 200, 3), (2, 64, 4096, 11), (5, 96, 72, 1),
                                                  (48, 128, 4096, 11), (1, 128, 24, 4), (48, 128, 4096, 1),
                                                  (2, 128, 1320, 1), (3, 64, 1064, 1), (7, 96, 3000, 2)])
def test_gram_partials_match_the_products(blocks, d, cols, parts):
    # each slice's Gram matrix, and their sum, against fp64 products of the same bf16 values
    rng = np.random.default_rng(blocks * d + cols)
    x = torch.from_numpy(rng.standard_normal((blocks, d, cols)).astype(np.float32)).cuda().to(torch.bfloat16)
    out = torch.full((blocks, parts, d, d), float("nan"), device="cuda")
    qk.qkvnr_gram_partials(blocks, d, cols, x, parts, out)
    torch.cuda.synchronize()
    xs = x.float().cpu().numpy().astype(np.float64)
    S = ((cols + parts - 1) // parts + 15) // 16 * 16
    got = out.cpu().numpy().astype(np.float64)
    for p in range(parts):
        sl = xs[:, :, p * S:min(cols, (p + 1) * S)]
        want = np.einsum("bik,bjk->bij", sl, sl)
        np.testing.assert_allclose(got[:, p], want, rtol=1e-5, atol=1e-5 * max(1.0, np.abs(want).max()))
    full = np.einsum("bik,bjk->bij", xs, xs)
    np.testing.assert_allclose(got.sum(axis=1), full, rtol=1e-5, atol=1e-5 * np.abs(full).max())


# ragged chunk tails (1000, 1064, 40 and 24 columns), an empty slice (40 columns in 4 slices of 16),
# both block sides, with and without the Gram matrices
@pytest.mark.parametrize("blocks,d,cols,parts", [(3, 128, 1000, 3), (48, 128, 4096, 5), (2, 64, 1064, 2),
                                                  (1, 128, 40, 4), (5, 64, 24, 1)])
@pytest.mark.parametrize("with_gram", [True, False])
def test_ns_update_matches_the_products(blocks, d, cols, parts, with_gram):
    rng = np.random.default_rng(blocks * d + cols + parts)
    x = torch.from_numpy(rng.standard_normal((blocks, d, cols)).astype(np.float32)).cuda().to(torch.bfloat16)
    p = torch.from_numpy((rng.standard_normal((blocks, d, d)) / np.sqrt(d)).astype(np.float32)).cuda()
    p = p.to(torch.bfloat16)
    y = torch.full_like(x, float("nan"))
    gram = torch.full((blocks, parts, d, d), float("nan"), device="cuda") if with_gram else None
    qk.qkvnr_ns_update(blocks, d, cols, p, x, y, parts, gram)
    torch.cuda.synchronize()
    xs = x.float().cpu().numpy().astype(np.float64)
    ps = p.float().cpu().numpy().astype(np.float64)
    got = y.float().cpu().numpy().astype(np.float64)
    want = np.matmul(ps, xs)
    # one rounding to bf16 (at most 2^-8 relative) of an fp32 sum of d products (within
    # d 2^-24 sum |p x| of the exact sum)
    acc_err = d * 2.0 ** -24 * np.matmul(np.abs(ps), np.abs(xs))
    assert np.all(np.abs(got - want) <= 2.0 ** -8 * np.abs(want) + 2 * acc_err + 1e-30)
    if with_gram:
        S = ((cols + parts - 1) // parts + 15) // 16 * 16
        g = gram.cpu().numpy().astype(np.float64)
        for q in range(parts):
            sl = got[:, :, q * S:min(cols, (q + 1) * S)]   # the stored bf16 values of Y
            w = np.einsum("bik,bjk->bij", sl, sl)
            np.testing.assert_allclose(g[:, q], w, rtol=1e-5, atol=1e-5 * max(1.0, np.abs(w).max()))


def _bf16_host(t):
    return t.float().cpu().numpy().astype(np.float64)


def _collapse_reference(a, steps, scale, eps):
    """fp64 M of qkvnr_ns_collapse's definition from the Gram matrices a [blocks, d, d]."""
    d = a.shape[-1]
    n = np.sqrt(np.trace(a, axis1=1, axis2=2)) + eps
    A = a / (n * n)[:, None, None]
    M = None
    for _ in range(steps):
        P = 3.4445 * np.eye(d)[None] - 4.7750 * A + 2.0315 * np.matmul(A, A)
        M = P if M is None else np.matmul(P, M)
        A = np.matmul(np.matmul(P, A), P)
    return M * (scale / n)[:, None, None]


# both sides, one and several slices of partials (the last one empty, as 520 columns in 8 slices of 80
# leave it), one step, five and seven, the block scale.  Wide blocks only: M is compared itself, and on
# the null space of a rank-deficient G G^T it is free (p(0) = 3.4445 per step) while M G is not
# affected; the end-to-end test covers such blocks through M G.
@pytest.mark.parametrize("blocks,d,cols,parts,steps,scale", [(3, 128, 1000, 3, 5, 1.0), (48, 128, 4096, 5, 5, 1.0),
                                                             (2, 64, 1064, 2, 1, 1.25), (1, 128, 520, 8, 7, 1.0),
                                                             (5, 64, 512, 1, 5, 1.5)])
def test_ns_collapse_matches_the_definition(blocks, d, cols, parts, steps, scale):
    # the Gram partials of seeded N(0,1) blocks (condition about (1 + (d/cols)^0.5) / (1 - (d/cols)^0.5)),
    # against the recurrence in fp64 from the same fp32 partials.  Each of the 4 products a step is within
    # about 2^-14 of |a| |b| and these blocks do not amplify it: M within 2^-12 in Frobenius norm and
    # 2^-11 max|M| element-wise (a model of the kernel's arithmetic in numpy gives 2e-5 to 6e-5)
    rng = np.random.default_rng(blocks * d + cols + parts + steps)
    x = torch.from_numpy(rng.standard_normal((blocks, d, cols)).astype(np.float32)).cuda().to(torch.bfloat16)
    gram = torch.full((blocks, parts, d, d), float("nan"), device="cuda")
    qk.qkvnr_gram_partials(blocks, d, cols, x, parts, gram)
    m = torch.full((blocks, 2, d, d), float("nan"), device="cuda").to(torch.bfloat16)
    qk.qkvnr_ns_collapse(blocks, d, gram, parts, steps, scale, 1e-7, m)
    torch.cuda.synchronize()
    g = gram.cpu().numpy().astype(np.float64)
    want = _collapse_reference(sum(g[:, q] for q in range(parts)), steps, scale, 1e-7)
    mh = _bf16_host(m)
    got = mh[:, 0] + mh[:, 1]
    fro = float(np.linalg.norm(got - want) / np.linalg.norm(want))
    elem = float(np.abs(got - want).max() / np.abs(want).max())
    print(f"[collapse] {blocks} x {d} x {cols}, {parts} slices, {steps} steps: Frobenius {fro:.2e}, "
          f"element {elem:.2e}", flush=True)
    assert fro <= 2.0 ** -12 and elem <= 2.0 ** -11
    assert np.all(np.abs(mh[:, 1]) <= 2.0 ** -8 * np.abs(mh[:, 0]))   # lo is the rest of hi's rounding


# ragged chunk tails (1000, 1064, 40, 24 columns), an empty slice, both sides
@pytest.mark.parametrize("blocks,d,cols,parts", [(3, 128, 1000, 3), (48, 128, 4096, 5), (2, 64, 1064, 2),
                                                  (1, 128, 40, 4), (5, 64, 24, 1)])
def test_ns_apply_matches_the_products(blocks, d, cols, parts):
    rng = np.random.default_rng(blocks * d + cols + parts + 3)
    x = torch.from_numpy(rng.standard_normal((blocks, d, cols)).astype(np.float32)).cuda().to(torch.bfloat16)
    mv = rng.standard_normal((blocks, d, d)) / np.sqrt(d)
    hi = torch.from_numpy(mv.astype(np.float32)).to(torch.bfloat16)
    lo = torch.from_numpy((mv - hi.double().numpy()).astype(np.float32)).to(torch.bfloat16)
    m = torch.stack([hi, lo], dim=1).contiguous().cuda()
    y = torch.full_like(x, float("nan"))
    qk.qkvnr_ns_apply(blocks, d, cols, m, x, y, parts)
    torch.cuda.synchronize()
    xs, mh, got = _bf16_host(x), _bf16_host(m), _bf16_host(y)
    ms = mh[:, 0] + mh[:, 1]
    want = np.matmul(ms, xs)
    # one rounding to bf16 (2^-8 relative) of fp32 sums of 2 d products (2 d 2^-24 of the sum of |m||x|)
    acc_err = 2 * d * 2.0 ** -24 * (np.matmul(np.abs(mh[:, 0]), np.abs(xs)) + np.matmul(np.abs(mh[:, 1]), np.abs(xs)))
    assert np.all(np.abs(got - want) <= 2.0 ** -8 * np.abs(want) + 2 * acc_err + 1e-30)


def test_ns_apply_adds_the_lo_terms():
    # M given as its lo term alone (hi = 0): Y = lo X, so a product that left lo out would give zeros
    rng = np.random.default_rng(11)
    blocks, d, cols = 4, 128, 512
    x = torch.from_numpy(rng.standard_normal((blocks, d, cols)).astype(np.float32)).cuda().to(torch.bfloat16)
    lo = torch.from_numpy((rng.standard_normal((blocks, d, d)) * 2.0 ** -9).astype(np.float32)).to(torch.bfloat16)
    m = torch.stack([torch.zeros_like(lo), lo], dim=1).contiguous().cuda()
    y = torch.empty_like(x)
    qk.qkvnr_ns_apply(blocks, d, cols, m, x, y, 2)
    torch.cuda.synchronize()
    want = np.matmul(_bf16_host(lo), _bf16_host(x))
    assert np.all(np.abs(_bf16_host(y) - want) <= 2.0 ** -8 * np.abs(want) + 1e-6 * np.abs(want).max())


def test_collapse_and_apply_refuse_bad_arguments():
    x = torch.zeros((2, 64, 128), dtype=torch.bfloat16, device="cuda")
    gram = torch.zeros((2, 1, 64, 64), device="cuda")
    m = torch.zeros((2, 2, 64, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(qk.QkvnrError):
        qk.qkvnr_ns_collapse(2, 96, gram, 1, 5, 1.0, 1e-7, m)          # no kernel for side 96
    with pytest.raises(qk.QkvnrError):
        qk.qkvnr_ns_collapse(2, 64, gram, 1, 0, 1.0, 1e-7, m)          # no steps
    with pytest.raises(qk.QkvnrError):
        qk.qkvnr_ns_apply(2, 64, 128, m, x, x, 1)                      # y is x
    with pytest.raises(qk.QkvnrError):
        qk.qkvnr_ns_apply(2, 64, 128, m, x, m, 1)                      # y overlaps m


def test_weight_at_an_unaligned_offset():
    # a weight that is a view 2 bytes into a flat buffer: updated like an aligned copy of itself
    rng = np.random.default_rng(5)
    rows, cols = (4 + 2 * 2) * 64, 512
    flat = torch.from_numpy(rng.standard_normal(rows * cols + 1).astype(np.float32)).cuda().to(torch.bfloat16)
    g = flat[1:].view(rows, cols)
    assert g.data_ptr() % 16 != 0
    got = per_head_newton_schulz(g, 4, 2, 64)
    want = per_head_newton_schulz(g.clone(), 4, 2, 64)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))


def test_declined_weights_raise():
    g = torch.zeros((80, 64), device="cuda")   # the Falcon shape: config total 192 rows, weight 80
    with pytest.raises(qk.QkvnrError):
        per_head_newton_schulz(g, 8, 8, 8)
