"""The balance call captured in a HIP graph: every replay equals the eager
call.  The entry points allocate nothing and never synchronise, so a caller
can capture them; each replay here follows eager work that overwrites the
outputs, and is checked in full."""
import numpy as np
import pytest

import workload as W
from gpu_common import routing_cached

torch = pytest.importorskip("torch")
import moe_expert_load_ultraep_amd as U  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_balance_graph_replays_equal_eager(mode):
    w = W.CONFIGS[2].with_(T=1024)
    idx, wt = routing_cached(2, 0, 0, 1024)
    ctx = U.ultraep_create(w.E, w.R, w.S, w.D, reroute_mode=mode)
    buf = U.Buffers(ctx, 1, w.T, w.k, "cuda")
    d_idx = torch.from_numpy(np.array(idx, copy=True)).cuda()
    d_w = torch.from_numpy(np.array(wt, copy=True)).cuda()

    def bal():
        U.ultraep_balance(ctx, d_idx, w.T, w.k, buf.workspace, buf.plans, buf.phys_idx, buf.pos,
                          topk_w=d_w, inv=buf.inv, w_perm=buf.w_perm, L=1)

    outs = (buf.plans, buf.phys_idx, buf.pos, buf.inv, buf.w_perm)

    def clear():
        # rows past the layout's end are not written: every run starts from
        # the same fill
        for t in outs[:4]:
            t.fill_(-7)
        buf.w_perm.fill_(-1.0)

    clear()
    bal()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bal()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bal()
    torch.cuda.synchronize()
    for rep in range(4):
        clear()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, outs):
            assert torch.equal(a, b), f"replay {rep} differs from the eager call"
