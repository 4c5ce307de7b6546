"""GPU: per-head Newton-Schulz on fused QKV weights against the fp64 oracle.

DeepSpeed page "[muon] Per-head Newton-Schulz for fused QKV projections":
the sectioned and interleaved orders of one fused weight give the same update
up to the block permutation (here bitwise: every block goes through the same
batched products), and a weight whose rows are not the exact fused total is
declined.  Values: fp32 compute within 1e-4 * max(|ref|, rms) of the fp64
oracle, element by element and in Frobenius norm (five steps of products over
rows up to 4096 long, in fp32).  bf16 compute, as Muon runs it, stores X, P and
the Gram matrix in bf16 at every step (each a 2**-9 relative rounding, five
times over): within 2**-5 of the oracle in Frobenius norm and 2**-3 * max(|ref|,
rms) element by element (observed: up to about 6e-2 element-wise, the quintic
amplifies the roundings of the small singular values).
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


@pytest.mark.parametrize("n_q,n_kv,D,cols", [(32, 8, 128, 4096), (8, 2, 16, 64), (4, 1, 64, 32), (3, 0, 8, 40)])
@pytest.mark.parametrize("dtype,tol,normwise_tol", [(torch.float32, 1e-4, 1e-4), (torch.bfloat16, 2.0 ** -3, 2.0 ** -5)])
def test_per_head_matches_oracle(n_q, n_kv, D, cols, dtype, tol, normwise_tol):
    rng = np.random.default_rng(n_q * 100 + D)
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
