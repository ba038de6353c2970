"""The allocation-free balance (ultraep_balance_static) against ultraep_balance.

Two calls in a row share the library's static workspace: the single-layer
workload at full size (4,194,304 pairs), then the tiny workload's eight
layers batched (a smaller input, on a workspace holding the first call's
words).  Each must give the plan records, replica map and fused dispatch
layout of ultraep_balance bit for bit.  A request beyond the static
workspace fails on the host with ULTRAEP_ESCRATCH.
"""
import numpy as np
import pytest

import moe_expert_load_ultraep_amd as U
import workload as W
from gpu_common import routing_cached, run_balance, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
DEV = "cuda"


def _static(ctx, idx, wt, T, k):
    L = idx.shape[0]
    buf = U.Buffers(ctx, L, T, k, DEV)
    buf.inv.fill_(-7)
    d_idx = torch.from_numpy(np.array(idx, copy=True)).to(DEV)
    d_w = torch.from_numpy(np.array(wt, copy=True)).to(DEV)
    U.ultraep_balance_static(ctx, d_idx, T, k, buf.plans, buf.phys_idx, buf.pos, topk_w=d_w,
                             inv=buf.inv, w_perm=buf.w_perm, L=L)
    torch.cuda.synchronize()
    return {"plans": buf.plans.cpu().numpy(), "phys": buf.phys_idx.cpu().numpy(),
            "pos": buf.pos.cpu().numpy(), "inv": buf.inv.cpu().numpy(),
            "w_perm": buf.w_perm.cpu().numpy()}


def _compare(w, idx, wt):
    ctx = U.ultraep_create(w.E, w.R, w.S, w.D)
    got = _static(ctx, idx, wt, w.T, w.k)
    ref = run_balance(ctx, idx, wt, w.T, w.k)
    for key in ("plans", "phys", "pos", "inv", "w_perm"):
        assert np.array_equal(got[key].view(np.uint32), ref[key].view(np.uint32)), key


def test_static_workspace_two_calls():
    w = W.SINGLE
    say("static workspace: single-layer workload, full size")
    idx, wt = routing_cached(2, 0, 0)
    _compare(w, idx[None], wt[None])
    w = W.TINY
    say("static workspace: tiny workload, 8 layers")
    layers = [routing_cached(1, l, 0) for l in range(8)]
    _compare(w, np.stack([a for a, _ in layers]), np.stack([b for _, b in layers]))


def test_static_workspace_limit():
    """64 layers of the single-layer shape need 64 x 512 KiB = 32 MiB (fits);
    65 layers need more and are refused before any launch."""
    w = W.SINGLE
    ctx = U.ultraep_create(w.E, w.R, w.S, w.D)
    assert ctx.workspace_bytes(64, w.T, w.k) <= U.STATIC_WORKSPACE_BYTES
    assert ctx.workspace_bytes(65, w.T, w.k) > U.STATIC_WORKSPACE_BYTES
    d = torch.zeros(16, dtype=torch.int32, device=DEV)
    with pytest.raises(U.UltraEPError) as ei:
        U.ultraep_balance_static(ctx, d, w.T, w.k, d, d, d, L=65)
    assert ei.value.status == -5
