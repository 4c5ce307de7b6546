"""Host-side logic of the Python layer, on the CPU (no kernel is launched).

- ``pool_slots``: which tokens the staged MLA pool write may scatter.  Its rule
  must be the direct pool write's (TensorRT-LLM page "MLA DSpark: run each
  drafter layer's kv path beside its q path", Description and Test Coverage:
  the direct write and staged + scatter are bitwise equal), so a table entry
  the direct kernel skips (page id < 0 or >= num_pages, page index past the
  table row, negative position) must be refused by the staged path too.
- ``_keep_workspace_clean``: a backward call that fails after kernels may have
  been enqueued drops the module's cached workspace of that device.
- ``per_head_newton_schulz`` refuses zero steps before touching the device.
"""
import numpy as np
import pytest
import torch

import oracle
import qkv_split_head_amd._binding as bnd
from qkv_split_head_amd.mla_drafter import pool_slots, staged_slots


def _table(rng, B, per_req, num_pages):
    return rng.permutation(num_pages)[:B * per_req].reshape(B, per_req).astype(np.int32)


def test_pool_slots_match_brute_force_on_a_valid_table():
    rng = np.random.Generator(np.random.PCG64(5))
    B, T_req, P, num_pages = 3, 7, 16, 64
    ctx = rng.integers(0, 100, size=B)
    pos = np.concatenate([c + np.arange(T_req) for c in ctx]).astype(np.int32)
    bt = _table(rng, B, 8, num_pages)
    slot, ok = pool_slots(torch.from_numpy(pos), torch.from_numpy(bt), T_req, P, num_pages)
    page, off = oracle.paged_slots(pos, bt, T_req, P)
    assert bool(ok.all())
    assert np.array_equal(slot.numpy(), page.astype(np.int64) * P + off)


def test_pool_slots_refuse_pages_the_direct_write_skips():
    B, T_req, P, num_pages = 1, 6, 4, 10
    pos = torch.tensor([0, 4, 8, 12, 16, 21], dtype=torch.int32)  # page indices 0..5
    bt = torch.tensor([[3, num_pages, -1, num_pages + 7, 9, 2]], dtype=torch.int32)
    # the last token's page index (5) is inside the row; drop the row to 5 entries to push it out
    slot, ok = pool_slots(pos, bt[:, :5].contiguous(), T_req, P, num_pages)
    assert ok.tolist() == [True, False, False, False, True, False]
    assert slot[0].item() == 3 * P and slot[4].item() == 9 * P
    slot, ok = pool_slots(pos, bt, T_req, P, num_pages)
    assert ok.tolist() == [True, False, False, False, True, True]
    neg = pos.clone()
    neg[0] = -1
    _, ok = pool_slots(neg, bt, T_req, P, num_pages)
    assert not bool(ok[0])


def test_staged_slots_stay_inside_the_pool():
    pos = torch.tensor([0, 4, 8], dtype=torch.int32)
    bt = torch.tensor([[0, 99, -5]], dtype=torch.int32)
    s = staged_slots(pos, bt, 3, 4, 10 * 4)
    assert int(s.min()) >= 0 and int(s.max()) < 40


class _Ws:
    """Stand-in for a cached device workspace (never touched)."""


def test_failed_launch_drops_the_cached_workspace():
    ws = _Ws()
    bnd._workspaces[7] = ws

    def fail_launch():
        raise bnd.QkvnrError(bnd.EHIP, "launch failed")

    with pytest.raises(bnd.QkvnrError):
        bnd._keep_workspace_clean(fail_launch, ws, 7)
    assert 7 not in bnd._workspaces


def test_validation_error_keeps_the_cached_workspace():
    ws = _Ws()
    bnd._workspaces[7] = ws

    def reject():
        raise bnd.QkvnrError(bnd.EINVAL, "bad argument")

    try:
        with pytest.raises(bnd.QkvnrError):
            bnd._keep_workspace_clean(reject, ws, 7)
        assert bnd._workspaces.get(7) is ws
        other = _Ws()  # a caller's own workspace failing leaves the cached one alone
        with pytest.raises(bnd.QkvnrError):
            bnd._keep_workspace_clean(lambda: (_ for _ in ()).throw(bnd.QkvnrError(bnd.EHIP, "x")), other, 7)
        assert bnd._workspaces.get(7) is ws
    finally:
        bnd._workspaces.pop(7, None)



def test_newton_schulz_refuses_zero_steps():
    # every path folds the Frobenius normalisation into the first step, so no step is refused before any device work
    from qkv_split_head_amd.muon import per_head_newton_schulz
    with pytest.raises(ValueError, match="steps"):
        per_head_newton_schulz(torch.zeros((3 * 64, 128)), 1, 1, 64, steps=0)
