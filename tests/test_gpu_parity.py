"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bit-exact for the histogram, plan record, replica map, layout indices,
permuted weights and permuted bf16 rows; the fold within 1e-6 of the fp64
oracle relative to |master| + sum |replica|.
"""
import json
import os

import numpy as np
import pytest

import moe_expert_load_ultraep_amd as U
import oracle as O
import workload as W
from gpu_common import assert_layer_equal, assert_plan_equal, routing_cached, run_balance, say
from pins import check_layout, check_plan_invariants, load_golden

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
DEV = "cuda"


def _ctx(w, **kw):
    return U.ultraep_create(w.E, w.R, w.S, w.D, **kw)


# ---------------------------------------------------------- block order ---
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_reroute_block_order_tail_several_layers(mode):
    """The reroute kernels take their (layer, tile) from the workgroup index
    in XCD order, and the grid's last (workgroups mod 8) keep their index.
    Three layers of 12 tiles each (six ranks of two tiles, the second one
    ragged) make 36 workgroups, 4 past the last group of eight: every layer
    is compared in full, in each reroute mode, with the layout fused."""
    E, R, S, D, T, k, L = 24, 6, 2, 3, 2000, 8, 3
    rng = np.random.default_rng(7100 + mode)
    idx, wt = [], []
    for _ in range(L):
        p = rng.dirichlet(np.full(E, 0.4))
        keys = np.log(np.maximum(p, 1e-12))[None, :] + rng.gumbel(size=(R * T, E))
        idx.append(np.argsort(-keys, axis=1)[:, :k].astype(np.int32))
        wt.append(rng.random((R * T, k), dtype=np.float32))
    idx, wt = np.stack(idx), np.stack(wt)
    say(f"block order: E={E} R={R} S={S} D={D} T={T} k={k} L={L} mode={mode}")
    ctx = U.ultraep_create(E, R, S, D, reroute_mode=mode)
    got = run_balance(ctx, idx, wt, T, k)
    for l in range(L):
        assert_layer_equal(ctx, got, l, idx[l], wt[l], E, R, S, D)


# ------------------------------------------------------------------ tiny ---
def test_tiny_full_path_eight_layers():
    """Tiny workload: 8 independent layers balanced in one batched call,
    everything compared in full, then permute and fold of every rank."""
    w = W.TINY
    say("tiny: 8 layers")
    layers = [routing_cached(1, l, 0) for l in range(8)]
    idx = np.stack([a for a, _ in layers])
    wt = np.stack([b for _, b in layers])
    ctx = _ctx(w)
    got = run_balance(ctx, idx, wt, w.T, w.k)
    hid = W.hidden(w)
    d_hid = torch.from_numpy(hid.view(np.int16)).to(DEV)
    P1 = w.M + w.S
    for l in range(8):
        pl, phys, pos = assert_layer_equal(ctx, got, l, idx[l], wt[l], w.E, w.R, w.S, w.D)
        inv = got["buf"].inv[l]
        plan = got["buf"].plans[l]
        for r in range(w.R):
            rows = int(pl.phys_off[(r + 1) * P1] - pl.phys_off[r * P1])
            out = torch.full((rows + 3, w.H), 0x5A5A, dtype=torch.int16, device=DEV)
            U.ultraep_permute(ctx, plan, inv, w.k, d_hid, r * P1, (r + 1) * P1, out)
            o = out.cpu().numpy().view(np.uint16)
            want = O.permute(hid, got["inv"][l][:pl.total], w.k, pl, r * P1, (r + 1) * P1)
            assert np.array_equal(o[:rows], want)
            assert (o[rows:] == 0x5A5A).all(), "rows beyond the segment must stay untouched"
        # fold: every slot of the layer into its master
        numel = w.numel
        nslot = w.R * w.S
        masters = W.grads(w, w.E, stream=10 + l)
        reps = W.grads(w, nslot, stream=100 + l)
        d_m = torch.from_numpy(masters).to(DEV)
        d_r = torch.from_numpy(reps).to(DEV)
        ptrs = torch.tensor([d_m[e].data_ptr() for e in range(w.E)], dtype=torch.int64, device=DEV)
        U.ultraep_fold_grads(ctx, plan, ptrs, d_r, numel, 0, nslot)
        want = O.fold({e: masters[e] for e in range(w.E)}, reps, pl, 0, nslot)
        gotm = d_m.cpu().numpy()
        for e in range(w.E):
            if e in want:
                scale = np.abs(masters[e].astype(np.float64)) + sum(
                    np.abs(reps[s].astype(np.float64)) for s in range(nslot) if pl.slot_expert[s] == e)
                assert (np.abs(gotm[e].astype(np.float64) - want[e]) <= 1e-6 * scale).all()
            else:
                assert np.array_equal(gotm[e], masters[e])


def test_hand_worked_plans_on_gpu():
    """The hand-worked plans (tests/golden) reproduced by the device solver
    from routings with exactly those counts."""
    for case in load_golden("hand_plans.json")["cases"]:
        c = np.array(case["c"])
        E, R, S, D = case["E"], case["R"], case["S"], case["D"]
        ids = np.repeat(np.arange(E, dtype=np.int32), c)
        T = max(1, -(-ids.size // R))
        k = 1
        idx = np.full(R * T * k, -1, dtype=np.int32)
        idx[:ids.size] = np.random.default_rng(0).permutation(ids)
        ctx = U.ultraep_create(E, R, S, D, allow_zero_master=case.get("allow_zero_master", False),
                               threshold=tuple(case.get("threshold", (1, 1))),
                               min_tokens=case.get("min_tokens", 1), replica_lean=case.get("lean", False))
        got = run_balance(ctx, idx.reshape(1, R * T, k), None, T, k)
        g = ctx.decode_plan(got["plans"][0])
        assert g["Q_star"] == case["Q_star"] and g["grid_index"] == case["grid_index"], case["name"]
        for key in ("slot_expert", "slot_quota", "master_quota", "phys_load", "phys_off", "inst_ptr",
                    "inst_phys", "inst_end", "rank_after"):
            if key in case:
                n = len(case[key]) if key.startswith("inst_") else len(g[key])
                assert g[key][:n].tolist() == case[key], (case["name"], key)


# -------------------------------------------------------- edge cases ------
@pytest.mark.parametrize("E,R,S,D,T,k,invalid,allow_zero", [
    (8, 4, 1, 4, 0, 2, 0.0, False),        # empty layer
    (8, 4, 1, 4, 1, 1, 0.0, False),        # one token per rank
    (12, 4, 2, 2, 333, 3, 0.05, False),    # ragged tile, dropped ids, two domains
    (16, 4, 0, 4, 500, 2, 0.0, False),     # no slots
    (16, 4, 2, 1, 500, 2, 0.0, False),     # domain of one rank
    (32, 8, 3, 4, 2049, 4, 0.01, True),    # zero-quota masters allowed
    (64, 64, 1, 64, 700, 1, 0.0, False),   # k = 1, M = 1
    (1024, 64, 8, 64, 512, 16, 0.0, False),    # M = 16, S = 8 (largest register tiles)
    (512, 512, 2, 64, 32, 8, 0.0, False),      # R*S = 1024 (slot limit), 8 domains
    (1024, 512, 1, 64, 32, 8, 0.0, False),     # E = 1024 with 512 slots
    (1024, 1024, 1, 64, 16, 8, 0.0, False),    # E = 1024 and R*S = 1024 together
    (512, 512, 1, 8, 32, 8, 0.0, False),       # 64 domains: more items than waves
    (160, 40, 3, 8, 1000, 8, 0.0, False),
    (3, 3, 2, 3, 3000, 2, 0.02, False),    # odd expert count, two experts per token
])
@pytest.mark.parametrize("fused", [True, False])
def test_edge_shapes(E, R, S, D, T, k, invalid, allow_zero, fused):
    say(f"edge E={E} R={R} S={S} D={D} T={T} k={k} fused={fused}")
    rng = np.random.default_rng([E, R, S, D, T, k])
    p = rng.dirichlet(np.full(E, 0.2))
    N = R * T * k
    idx = rng.choice(E, size=N, p=p).astype(np.int32)
    if invalid:
        idx = np.where(rng.random(N) < invalid, rng.choice([-1, E, 1 << 30], size=N), idx).astype(np.int32)
    idx = idx.reshape(R * T, k)
    wt = rng.random((R * T, k)).astype(np.float32)
    ctx = U.ultraep_create(E, R, S, D, allow_zero_master=allow_zero)
    got = run_balance(ctx, idx[None], wt[None], T, k, fused=fused)
    pl, phys, pos = assert_layer_equal(ctx, got, 0, idx, wt, E, R, S, D, allow_zero_master=allow_zero)
    check_plan_invariants(pl, pl.c, allow_zero)


def _degenerate_routing(kind, E, R, T, k):
    """Routing patterns with extreme structure: every pair on one expert
    (one run covers whole tiles), two experts alternating (every chunk holds
    both), every pair on the experts of rank 0 (the other ranks all spare),
    and every id invalid (no load at all)."""
    g = np.arange(R * T, dtype=np.int64)[:, None]
    j = np.arange(k, dtype=np.int64)[None, :]
    if kind == "one_expert":
        idx = np.full((R * T, k), 3, dtype=np.int64)
    elif kind == "two_experts":
        idx = np.where((g + j) % 2 == 0, 0, 5) + 0 * g
    elif kind == "rank0_experts":
        M = E // R
        idx = (g * k + j) % M
    elif kind == "all_invalid":
        idx = np.where((g + j) % 3 == 0, -1, E) + 0 * g
    else:
        raise ValueError(kind)
    return idx.astype(np.int32)


@pytest.mark.parametrize("kind", ["one_expert", "two_experts", "rank0_experts", "all_invalid"])
@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("fused", [True, False])
def test_degenerate_routing(kind, mode, fused):
    E, R, S, D, T, k = 16, 4, 2, 4, 5000, 4  # 20,000 pairs per rank: three tiles, the last ragged
    say(f"degenerate {kind} mode={mode} fused={fused}")
    idx = _degenerate_routing(kind, E, R, T, k)
    wt = np.random.default_rng(11).random((R * T, k)).astype(np.float32)
    ctx = U.ultraep_create(E, R, S, D, reroute_mode=mode)
    got = run_balance(ctx, idx[None], wt[None], T, k, fused=fused)
    pl, phys, pos = assert_layer_equal(ctx, got, 0, idx, wt, E, R, S, D)
    check_plan_invariants(pl, pl.c, False)


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_degenerate_layers_in_one_call(mode):
    """Four layers of different structure in one batched call: each layer's
    plan, replica map and layout must come out as if it were balanced alone."""
    E, R, S, D, T, k = 16, 4, 2, 4, 3000, 4
    say(f"degenerate layers mode={mode}")
    kinds = ["all_invalid", "one_expert", "two_experts", "rank0_experts"]
    idx = np.stack([_degenerate_routing(kd, E, R, T, k) for kd in kinds])
    wt = np.random.default_rng(12).random(idx.shape).astype(np.float32)
    ctx = U.ultraep_create(E, R, S, D, reroute_mode=mode)
    got = run_balance(ctx, idx, wt, T, k)
    for l in range(len(kinds)):
        assert_layer_equal(ctx, got, l, idx[l], wt[l], E, R, S, D)


@pytest.mark.parametrize("thr", [(101, 100), (105, 100), (3, 2)])
def test_threshold_single_layer(thr):
    """The early-stop target above 1 on the single-layer workload (1024
    tokens per rank) and the pages' EP64 table shape."""
    w = W.SINGLE.with_(T=1024)
    idx, wt = routing_cached(2, 0, 0, 1024)
    ctx = _ctx(w, threshold=thr)
    got = run_balance(ctx, idx[None], wt[None], w.T, w.k)
    assert_layer_equal(ctx, got, 0, idx, wt, w.E, w.R, w.S, w.D, thr_num=thr[0], thr_den=thr[1])


@pytest.mark.parametrize("cfg,T,mt", [(2, 1024, 1024), (2, None, 1024), (6, None, 1024), (8, None, 4096)])
def test_minimum_tokens_per_replica(cfg, T, mt):
    """Replicas below the minimum are not created (the pages' default 1024)."""
    w = W.CONFIGS[cfg] if T is None else W.CONFIGS[cfg].with_(T=T)
    idx, wt = routing_cached(cfg, 0, 0, T)
    ctx = _ctx(w, min_tokens=mt)
    got = run_balance(ctx, idx[None], wt[None], w.T, w.k)
    pl, _, _ = assert_layer_equal(ctx, got, 0, idx, wt, w.E, w.R, w.S, w.D, min_tokens=mt)
    check_plan_invariants(pl, pl.c, False, mt)


@pytest.mark.parametrize("cfg,T,mt", [(2, None, 1), (2, None, 1024), (6, None, 1024), (7, None, 1024),
                                      (8, None, 1024), (5, 2048, 1)])
def test_replica_lean(cfg, T, mt):
    """The lean planner (no chain step) at full size: plan record, replica
    map and fused layout equal to the oracle's; at the pages' table shape
    within 1.15 times the table's replicas at max/mean 1.01."""
    w = W.CONFIGS[cfg] if T is None else W.CONFIGS[cfg].with_(T=T)
    say(f"lean cfg={cfg} T={w.T} min={mt}")
    idx, wt = routing_cached(cfg, 0, 0, T)
    ctx = _ctx(w, min_tokens=mt, replica_lean=True)
    got = run_balance(ctx, idx[None], wt[None], w.T, w.k)
    pl, _, _ = assert_layer_equal(ctx, got, 0, idx, wt, w.E, w.R, w.S, w.D, min_tokens=mt, lean=True)
    check_plan_invariants(pl, pl.c, False, mt)
    if cfg in (6, 7, 8):
        table = load_golden("pages_ep64_table.json")
        assert pl.imbalance_after() <= 1.01 + 1e-9
        assert pl.n_replicas <= 1.15 * table["replicas_total"][cfg - 6]


@pytest.mark.parametrize("mode", [1, 2])
def test_minimum_tokens_with_locality(mode):
    w = W.CONFIGS[2].with_(T=1024)
    idx, wt = routing_cached(2, 0, 0, 1024)
    ctx = _ctx(w, min_tokens=1024, reroute_mode=mode)
    got = run_balance(ctx, idx[None], wt[None], w.T, w.k)
    assert_layer_equal(ctx, got, 0, idx, wt, w.E, w.R, w.S, w.D, min_tokens=1024)


def test_large_counts_take_the_unpacked_probe():
    """One expert with more than 2^22 pairs at 16 masters per rank: the
    planner's packed selection keys cannot hold such pieces, so it takes its
    general selection path; the plan must be the same."""
    E, R, S, D, T, k = 64, 4, 1, 4, 1_200_000, 1
    say(f"large counts E={E} R={R} T={T}")
    rng = np.random.default_rng([64, 4, 1, 4, 1_200_000])
    p = np.full(E, 0.1 / (E - 1))
    p[5] = 0.9
    idx = rng.choice(E, size=(R * T, k), p=p).astype(np.int32)
    assert np.bincount(idx.ravel(), minlength=E).max() >= 1 << 22
    wt = rng.random((R * T, k)).astype(np.float32)
    ctx = U.ultraep_create(E, R, S, D)
    got = run_balance(ctx, idx[None], wt[None], T, k)
    pl, _, _ = assert_layer_equal(ctx, got, 0, idx, wt, E, R, S, D)
    check_plan_invariants(pl, pl.c, False)


def test_determinism_and_streams():
    """Two runs on different streams give bit-identical results."""
    w = W.SINGLE.with_(T=1024)
    idx, wt = routing_cached(2, 0, 0, 1024)
    ctx = _ctx(w)
    a = run_balance(ctx, idx[None], wt[None], w.T, w.k)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = run_balance(ctx, idx[None], wt[None], w.T, w.k)
    torch.cuda.synchronize()
    for key in ("plans", "phys", "pos", "inv", "w_perm"):
        assert np.array_equal(a[key].view(np.uint32), b[key].view(np.uint32)), key


# ---------------------------------------------------- full-size configs ---
def _full_config(cfg_id, layers, check_layers, mb=0):
    w = W.CONFIGS[cfg_id]
    say(f"config {cfg_id}: generating {len(layers)} layers")
    data = [routing_cached(cfg_id, l, mb) for l in layers]
    idx = np.stack([a for a, _ in data])
    wt = np.stack([b for _, b in data])
    ctx = _ctx(w)
    say(f"config {cfg_id}: balancing L={len(layers)} on the GPU")
    got = run_balance(ctx, idx, wt, w.T, w.k)
    for li, l in enumerate(layers):
        c, dropped = O.count(idx[li], w.E)
        pl = O.plan(c, w.E, w.R, w.S, w.D, dropped=dropped)
        assert_plan_equal(ctx, got["plans"][li], pl, w.N)
        if l in check_layers:
            say(f"config {cfg_id}: full layout parity, layer {l}")
            assert_layer_equal(ctx, got, li, idx[li], wt[li], w.E, w.R, w.S, w.D)
    return w, ctx, got, idx


def test_config2_single_layer_full():
    w, ctx, got, idx = _full_config(2, [0], {0})
    # the separate layout call gives the same rows
    wt = routing_cached(2, 0, 0)[1]
    sep = run_balance(ctx, idx, wt[None], w.T, w.k, fused=False)
    for key in ("inv", "w_perm"):
        assert np.array_equal(sep[key].view(np.uint32), got[key].view(np.uint32)), key
    g = ctx.decode_plan(got["plans"][0])
    assert g["rank_after"].max() * w.R / g["total"] <= 1.04


def test_config3_61_layers():
    _full_config(3, list(range(61)), {0, 30, 60})


def test_config4_stream_sample():
    """32 instances of the non-stationary stream (two layers, every
    microbatch of the walk) batched in one call."""
    w = W.STREAM
    insts = [(l, mb) for l in (0, 31) for mb in range(16)]
    data = [routing_cached(4, l, mb) for l, mb in insts]
    idx = np.stack([a for a, _ in data])
    wt = np.stack([b for _, b in data])
    ctx = _ctx(w)
    got = run_balance(ctx, idx, wt, w.T, w.k)
    for i, (l, mb) in enumerate(insts):
        c, dropped = O.count(idx[i], w.E)
        pl = O.plan(c, w.E, w.R, w.S, w.D, dropped=dropped)
        assert_plan_equal(ctx, got["plans"][i], pl, w.N)
        assert pl.imbalance_after() <= 1.04
    for i in (0, 21):
        assert_layer_equal(ctx, got, i, idx[i], wt[i], w.E, w.R, w.S, w.D)


def test_config5_topology_full():
    w, ctx, got, idx = _full_config(5, [0], {0})
    g = ctx.decode_plan(got["plans"][0])
    floor = g["floor"] * w.R / g["total"]
    assert floor > 1.0 and g["rank_after"].max() * w.R / g["total"] <= floor + 0.01


@pytest.mark.parametrize("cfg_id", [2, 3, 5])
def test_permute_full_size_segments(cfg_id):
    """Permute at full size: the most loaded rank's segment and rank 0's, in
    the launch configuration the benchmark times, compared row by row."""
    w = W.CONFIGS[cfg_id]
    idx, wt = routing_cached(cfg_id, 0, 0)
    ctx = _ctx(w)
    got = run_balance(ctx, idx[None], wt[None], w.T, w.k)
    c, dropped = O.count(idx, w.E)
    pl = O.plan(c, w.E, w.R, w.S, w.D, dropped=dropped)
    say(f"config {cfg_id}: hidden {w.tokens}x{w.H}")
    hid = W.hidden(w, workers=16)
    d_hid = torch.from_numpy(hid.view(np.int16)).to(DEV)
    P1 = w.M + w.S
    inv = got["inv"][0][:pl.total]
    for r in sorted({int(np.argmax(pl.rank_after)), 0}):
        rows = int(pl.phys_off[(r + 1) * P1] - pl.phys_off[r * P1])
        out = torch.empty((rows, w.H), dtype=torch.int16, device=DEV)
        U.ultraep_permute(ctx, got["buf"].plans[0], got["buf"].inv[0], w.k, d_hid, r * P1, (r + 1) * P1, out)
        o = out.cpu().numpy().view(np.uint16)
        assert np.array_equal(o, O.permute(hid, inv, w.k, pl, r * P1, (r + 1) * P1)), r
    del d_hid


def test_permute_random_bits_and_capacity():
    """Raw 16-bit patterns (NaN payloads, infinities, subnormals) survive,
    a short capacity stops at the bound, and a tiny H works."""
    w = W.TINY
    idx, wt = routing_cached(1, 3, 0)
    ctx = _ctx(w)
    got = run_balance(ctx, idx[None], wt[None], w.T, w.k)
    pl, _, _ = O.balance(idx, w.E, w.R, w.S, w.D)
    inv = got["inv"][0][:pl.total]
    for H in (8, 24, 520):
        hid = W.random_bits_hidden(w.tokens, H, seed=H)
        d_hid = torch.from_numpy(hid.view(np.int16)).to(DEV)
        want = O.permute(hid, inv, w.k, pl, 0, pl.P)
        cap = pl.total - 5
        out = torch.full((cap, H), 0x1234, dtype=torch.int16, device=DEV)
        U.ultraep_permute(ctx, got["buf"].plans[0], got["buf"].inv[0], w.k, d_hid, 0, pl.P, out)
        assert np.array_equal(out.cpu().numpy().view(np.uint16), want[:cap])


@pytest.mark.parametrize("cfg_id,numel", [(3, None), (2, 4097 * 3 + 1), (5, None), (2, None),
                                           (2, 4 * (1024 * 37 + 5))])
def test_fold_full_size(cfg_id, numel):
    """One rank's slots folded at full size (vector path: several rounds per
    workgroup at workloads 3 and 5, one round at workload 2), an odd numel
    (scalar path), and a one-round grid whose last workgroup covers only 5
    vectors (the ragged end of the one-round store form)."""
    w = W.CONFIGS[cfg_id]
    idx, _ = routing_cached(cfg_id, 0, 0)
    c, dropped = O.count(idx, w.E)
    pl = O.plan(c, w.E, w.R, w.S, w.D, dropped=dropped)
    ctx = _ctx(w)
    got = run_balance(ctx, idx[None], None, w.T, w.k)
    numel = w.numel if numel is None else numel
    r = int(np.argmax([(pl.slot_expert[q * w.S:(q + 1) * w.S] >= 0).sum() for q in range(w.R)]))
    s0, s1 = r * w.S, (r + 1) * w.S
    experts = sorted({int(e) for e in pl.slot_expert[s0:s1] if e >= 0})
    assert experts, "the chosen rank hosts replicas"
    say(f"config {cfg_id}: fold slots [{s0},{s1}) experts {experts} numel {numel}")
    masters = W.grads(w, len(experts), stream=1, numel=numel)
    reps = W.grads(w, s1 - s0, stream=2, numel=numel)
    d_m = torch.from_numpy(masters).to(DEV)
    d_r = torch.from_numpy(reps).to(DEV)
    table = [0] * w.E
    for i, e in enumerate(experts):
        table[e] = d_m[i].data_ptr()
    ptrs = torch.tensor(table, dtype=torch.int64, device=DEV)
    U.ultraep_fold_grads(ctx, got["buf"].plans[0], ptrs, d_r, numel, s0, s1)
    want = O.fold({e: masters[i] for i, e in enumerate(experts)}, reps, pl, s0, s1)
    gm = d_m.cpu().numpy()
    for i, e in enumerate(experts):
        scale = np.abs(masters[i].astype(np.float64)) + sum(
            np.abs(reps[s - s0].astype(np.float64)) for s in range(s0, s1) if pl.slot_expert[s] == e)
        assert (np.abs(gm[i].astype(np.float64) - want[e]) <= 1e-6 * scale).all(), e


# ------------------------------------------- locality-aware reroute -------
@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("cfg,T", [(1, None), (2, 512), (3, 256), (5, 256)])
@pytest.mark.parametrize("fused", [True, False])
def test_locality_reroute_workloads(mode, cfg, T, fused):
    """Locality-aware reroute (mode 1) and its interleave (mode 2) against
    the oracle's reroute_local, with the layout fused or separate."""
    w = W.CONFIGS[cfg] if T is None else W.CONFIGS[cfg].with_(T=T)
    say(f"locality mode={mode} cfg={cfg} T={w.T} fused={fused}")
    idx, wt = routing_cached(cfg, 0, 0, T)
    ctx = _ctx(w, reroute_mode=mode)
    got = run_balance(ctx, idx[None], wt[None], w.T, w.k, fused=fused)
    assert_layer_equal(ctx, got, 0, idx, wt, w.E, w.R, w.S, w.D)


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("E,R,S,D,T,k,invalid,allow_zero", [
    (12, 4, 2, 2, 333, 3, 0.05, False),   # ragged tiles, dropped ids, two domains
    (16, 4, 0, 4, 500, 2, 0.0, False),    # no slots: every instance is a master
    (32, 8, 3, 4, 2049, 4, 0.01, True),   # zero-quota masters allowed
    (1024, 64, 8, 64, 256, 16, 0.0, False),  # M = 16, S = 8 (layout by a separate scatter)
    (64, 64, 1, 64, 20000, 1, 0.0, False),   # several tiles per rank (T*k > 8192)
    (512, 64, 4, 64, 512, 8, 0.0, False),    # fused layout in 8-wave workgroups
    (1024, 64, 1, 64, 256, 8, 0.01, False),  # fused layout in 4-wave workgroups
    (4, 2, 2, 2, 3000, 2, 0.0, False),       # tables too small to hold the write-out's words
    (3, 3, 2, 3, 3000, 2, 0.02, False),      # the same with an odd expert count
])
def test_locality_reroute_edge_shapes(mode, E, R, S, D, T, k, invalid, allow_zero):
    say(f"locality edge mode={mode} E={E} R={R} S={S} D={D} T={T} k={k}")
    rng = np.random.default_rng([E, R, S, D, T, k, 7])
    p = rng.dirichlet(np.full(E, 0.2))
    N = R * T * k
    idx = rng.choice(E, size=N, p=p).astype(np.int32)
    if invalid:
        idx = np.where(rng.random(N) < invalid, rng.choice([-1, E, 1 << 30], size=N), idx).astype(np.int32)
    idx = idx.reshape(R * T, k)
    wt = rng.random((R * T, k)).astype(np.float32)
    ctx = U.ultraep_create(E, R, S, D, allow_zero_master=allow_zero, reroute_mode=mode)
    got = run_balance(ctx, idx[None], wt[None], T, k)
    assert_layer_equal(ctx, got, 0, idx, wt, E, R, S, D, allow_zero_master=allow_zero)


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("fused", [True, False])
def test_locality_several_layers_one_call(mode, fused):
    """Eight layers of the tiny workload and three of the topology workload
    (several tiles per rank) in one batched call each."""
    for cfg, n, T in ((1, 8, None), (5, 3, 2048)):
        w = W.CONFIGS[cfg] if T is None else W.CONFIGS[cfg].with_(T=T)
        say(f"locality layers mode={mode} fused={fused} cfg={cfg} L={n}")
        layers = [routing_cached(cfg, l, 0, T) for l in range(n)]
        idx = np.stack([x for x, _ in layers])
        wt = np.stack([y for _, y in layers])
        ctx = _ctx(w, reroute_mode=mode)
        got = run_balance(ctx, idx, wt, w.T, w.k, fused=fused)
        for l in range(n):
            assert_layer_equal(ctx, got, l, idx[l], wt[l], w.E, w.R, w.S, w.D)


@pytest.mark.parametrize("mode", [1, 2])
def test_locality_single_layer_full_size(mode):
    """Modes 1 and 2 on the full single-layer workload (4,194,304 pairs)."""
    w = W.SINGLE
    idx, wt = routing_cached(2, 0, 0)
    ctx = _ctx(w, reroute_mode=mode)
    got = run_balance(ctx, idx[None], wt[None], w.T, w.k)
    assert_layer_equal(ctx, got, 0, idx, wt, w.E, w.R, w.S, w.D)
