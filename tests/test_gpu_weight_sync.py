"""GPU parity of weight_sync and its relay plan through the C ABI.

The relay table is integer data: bit-exact against the oracle's.  The copy
is a bit copy: every replica slot must hold exactly its expert's master
bits (NaN payloads included), empty slots and slots outside the range must
stay untouched, and the two-stage relay copy must give the same bits as the
direct one.
"""
import numpy as np
import pytest

import moe_expert_load_ultraep_amd as U
import oracle as O
import workload as W
from gpu_common import routing_cached, run_balance, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
DEV = "cuda"
SENTINEL = 0x7FC3


def _plan(cfg, T=None):
    w = W.CONFIGS[cfg] if T is None else W.CONFIGS[cfg].with_(T=T)
    idx, wt = routing_cached(cfg, 0, 0, T)
    ctx = U.ultraep_create(w.E, w.R, w.S, w.D)
    got = run_balance(ctx, idx[None], None, w.T, w.k)
    c, dropped = O.count(idx, w.E)
    return w, ctx, got["buf"].plans[0], O.plan(c, w.E, w.R, w.S, w.D, dropped=dropped)


@pytest.mark.parametrize("cfg,T", [(1, None), (2, 2048), (3, 2048), (5, 2048)])
@pytest.mark.parametrize("mode,min_rep,domain", [(0, 4, None), (1, 4, None), (1, 2, None), (2, 4, None), (2, 4, 8)])
def test_relay_plan_matches_oracle(cfg, T, mode, min_rep, domain):
    w, ctx, d_plan, pl = _plan(cfg, T)
    say(f"relay plan cfg={cfg} mode={mode} min_replicas={min_rep} domain_gpus={domain}")
    relay = torch.full((2, w.R * w.S), 77, dtype=torch.int32, device=DEV)
    U.ultraep_weight_sync_plan(ctx, d_plan, relay, mode=mode, min_replicas=min_rep, domain_gpus=domain)
    torch.cuda.synchronize()
    src, stage = O.relay_plan(pl, mode, min_replicas=min_rep, domain_gpus=domain)
    got = relay.cpu().numpy()
    assert np.array_equal(got[0].astype(np.int64), src)
    assert np.array_equal(got[1].astype(np.int64), stage)


def _sync_and_check(w, ctx, d_plan, pl, numel, s0, s1, relay=None, null_expert=None, offset=0):
    rng = np.random.default_rng([w.cfg_id, numel, s0, s1])
    masters = rng.integers(0, 1 << 16, size=(w.E, numel + offset), dtype=np.uint16)
    d_m = torch.from_numpy(masters.view(np.int16)).to(DEV)
    ptrs = [d_m[e, offset:].data_ptr() for e in range(w.E)]
    if null_expert is not None:
        ptrs[null_expert] = 0
    d_ptrs = torch.tensor(ptrs, dtype=torch.int64, device=DEV)
    reps = torch.full((s1 - s0, numel), SENTINEL, dtype=torch.int16, device=DEV)
    U.ultraep_weight_sync(ctx, d_plan, d_ptrs, reps, numel, s0, s1, relay=relay)
    torch.cuda.synchronize()
    got = reps.cpu().numpy().view(np.uint16)
    want = O.weight_sync({e: masters[e, offset:] for e in range(w.E)}, pl, s0, s1)
    for s in range(s0, s1):
        e = int(pl.slot_expert[s])
        if s in want and e != null_expert:
            assert got[s - s0].tobytes() == want[s].tobytes(), s
        else:
            assert (got[s - s0] == SENTINEL).all(), s
    return got


@pytest.mark.parametrize("numel,offset", [(4096, 0), (1000, 0), (4096, 1), (8, 0)])
def test_weight_sync_direct(numel, offset):
    """Vector path (numel % 8 == 0, aligned), scalar path (odd size or an
    unaligned master), all slots and a sub-range."""
    w, ctx, d_plan, pl = _plan(2, 2048)
    say(f"weight sync numel={numel} offset={offset}")
    _sync_and_check(w, ctx, d_plan, pl, numel, 0, w.R * w.S, offset=offset)
    _sync_and_check(w, ctx, d_plan, pl, numel, 37, 90, offset=offset)


def test_weight_sync_relay_equals_direct():
    w, ctx, d_plan, pl = _plan(3, 2048)
    relay = torch.empty((2, w.R * w.S), dtype=torch.int32, device=DEV)
    U.ultraep_weight_sync_plan(ctx, d_plan, relay, mode=U.RELAY_FORCE)
    torch.cuda.synchronize()
    assert (relay[1] == 2).any(), "the forced plan must use a second stage"
    a = _sync_and_check(w, ctx, d_plan, pl, 2048, 0, w.R * w.S, relay=relay)
    b = _sync_and_check(w, ctx, d_plan, pl, 2048, 0, w.R * w.S)
    assert a.tobytes() == b.tobytes()


def test_weight_sync_null_master_entry_leaves_slots():
    w, ctx, d_plan, pl = _plan(1)
    hot = int(pl.slot_expert[pl.slot_expert >= 0][0])
    _sync_and_check(w, ctx, d_plan, pl, 64, 0, w.R * w.S, null_expert=hot)


def test_weight_sync_full_size_fc1_whole_group():
    """Single-layer workload at full size: fc1 of a 4096 x 1536 expert
    (12,582,912 bf16) into all 128 slots, direct and adaptive relay; checked
    on the device slot by slot against the master buffers."""
    w = W.SINGLE
    idx, _ = routing_cached(2, 0, 0)
    ctx = U.ultraep_create(w.E, w.R, w.S, w.D)
    got = run_balance(ctx, idx[None], None, w.T, w.k)
    pl = ctx.decode_plan(got["plans"][0])
    numel = 2 * 4096 * 1536
    gen = torch.Generator(device=DEV).manual_seed(5)
    masters = torch.randint(-32768, 32767, (w.E, numel), generator=gen, dtype=torch.int16, device=DEV)
    ptrs = torch.tensor([masters[e].data_ptr() for e in range(w.E)], dtype=torch.int64, device=DEV)
    for mode in (None, U.RELAY_FORCE):
        say(f"full size weight sync relay mode {mode}")
        reps = torch.zeros((w.R * w.S, numel), dtype=torch.int16, device=DEV)
        relay = None
        if mode is not None:
            relay = torch.empty((2, w.R * w.S), dtype=torch.int32, device=DEV)
            U.ultraep_weight_sync_plan(ctx, got["buf"].plans[0], relay, mode=mode)
        U.ultraep_weight_sync(ctx, got["buf"].plans[0], ptrs, reps, numel, 0, w.R * w.S, relay=relay)
        torch.cuda.synchronize()
        for s, e in enumerate(pl["slot_expert"]):
            if e >= 0:
                assert torch.equal(reps[s], masters[int(e)]), s
            else:
                assert not reps[s].any(), s
