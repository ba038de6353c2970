"""Pins of the oracle's locality-aware reroute and its interleave (CPU).

Hand-worked cases (golden file), the structure every such layout must have
(own expert, promised loads, a bijection onto the layout, local pairs first
in pair order, pool pairs after them in pool order), the local count at its
bound and never below the plain reroute's, and the interleave's owner
sequence rebuilt in closed form (round t gives one pool pair to every
instance with more than t remaining, in instance order) instead of by the
oracle's simulation.
"""
import json
import os

import numpy as np
import pytest

import oracle as O
import workload as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_locality.json")
CASES = json.load(open(GOLDEN))["cases"]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_locality_hand_worked(case):
    idx = np.array(case["topk_idx"], dtype=np.int32).reshape(-1, 1)
    c, _ = O.count(idx, case["E"])
    pl = O.plan(c, case["E"], case["R"], case["S"], case["D"])
    assert pl.phys_load.tolist() == case["phys_load"]
    for mode, fn in (("plain", lambda: O.reroute(idx, pl)),
                     ("local", lambda: O.reroute_local(idx, pl, False)),
                     ("interleave", lambda: O.reroute_local(idx, pl, True))):
        phys, pos = fn()
        assert phys.tolist() == case[mode]["phys"], mode
        assert pos.tolist() == case[mode]["pos"], mode


def _rank_counts(idx, pl):
    ids = np.asarray(idx).reshape(-1)
    TK = ids.size // pl.R
    rc = np.zeros((pl.R, pl.E), dtype=np.int64)
    for n, e in enumerate(ids):
        if 0 <= e < pl.E:
            rc[n // TK, e] += 1
    return rc


def _local_count(idx, pl, phys):
    ids = np.asarray(idx).reshape(-1)
    TK = ids.size // pl.R
    ok = phys >= 0
    return int(((np.arange(ids.size) // TK)[ok] == phys[ok] // (pl.M + pl.S)).sum())


def _closed_form_owner(rem):
    """Pool owners of round-robin with removal, built round by round from
    the sorted remaining quotas (not by walking the pool)."""
    seq = []
    levels = sorted(set(v for v in rem if v > 0))
    prev = 0
    for lv in levels:
        active = [i for i, v in enumerate(rem) if v >= lv]
        for _ in range(prev, lv):
            seq += active
        prev = lv
    return seq


def check_local_layout(idx, pl, phys, pos, interleave):
    ids = np.asarray(idx).reshape(-1)
    N = ids.size
    valid = (ids >= 0) & (ids < pl.E)
    assert (phys[~valid] == -1).all() and (pos[~valid] == -1).all()
    P1 = pl.M + pl.S
    pv = phys[valid]
    r, j = pv // P1, pv % P1
    m = j < pl.M
    assert (r[m] * pl.M + j[m] == ids[valid][m]).all()
    assert (pl.slot_expert[r[~m] * pl.S + j[~m] - pl.M] == ids[valid][~m]).all()
    assert np.array_equal(np.bincount(pv, minlength=pl.P), pl.phys_load)
    assert np.array_equal(np.sort(pos[valid]), np.arange(valid.sum()))
    assert (pos[valid] >= pl.phys_off[pv]).all() and (pos[valid] < pl.phys_off[pv + 1]).all()
    rc = _rank_counts(idx, pl)
    a = O.local_takes(pl, rc)
    TK = N // pl.R
    src = np.arange(N) // TK
    for e in range(pl.E):
        insts = list(range(pl.inst_ptr[e], pl.inst_ptr[e + 1]))
        pool = []                     # pool pairs of e in pair order
        taken = {}
        for n in np.nonzero(ids == e)[0]:
            i = next((i for i in insts if pl.inst_phys[i] // P1 == src[n]), None)
            if i is not None and taken.get(i, 0) < a[i]:
                taken[i] = taken.get(i, 0) + 1
                assert phys[n] == pl.inst_phys[i]                 # local pairs stay local
                assert pos[n] - pl.phys_off[phys[n]] == taken[i] - 1
            else:
                pool.append(n)
        start, rem = 0, []
        for i in insts:
            q = int(pl.inst_end[i]) - start
            start = int(pl.inst_end[i])
            rem.append(q - int(a[i]))
        owner = _closed_form_owner(rem) if interleave else [k for k, v in enumerate(rem) for _ in range(v)]
        assert len(owner) == len(pool)
        seen = [0] * len(insts)
        for u, n in enumerate(pool):
            i = insts[owner[u]]
            assert phys[n] == pl.inst_phys[i]
            assert pos[n] - pl.phys_off[phys[n]] == a[i] + seen[owner[u]]
            seen[owner[u]] += 1
    return a


@pytest.mark.parametrize("cfg,T", [(1, None), (2, 256), (3, 256), (5, 128)])
@pytest.mark.parametrize("interleave", [False, True])
def test_locality_structure_on_workloads(cfg, T, interleave):
    w = W.CONFIGS[cfg] if T is None else W.CONFIGS[cfg].with_(T=T)
    idx, _, _ = W.routing(w, 0, 0)
    c, dropped = O.count(idx, w.E)
    pl = O.plan(c, w.E, w.R, w.S, w.D, dropped=dropped)
    phys, pos = O.reroute_local(idx, pl, interleave)
    a = check_local_layout(idx, pl, phys, pos, interleave)
    local = _local_count(idx, pl, phys)
    assert local == int(a.sum())
    plain_phys, _ = O.reroute(idx, pl)
    assert local >= _local_count(idx, pl, plain_phys)


@pytest.mark.parametrize("seed", range(6))
def test_locality_random_shapes_with_dropped(seed):
    rng = np.random.default_rng(900 + seed)
    R = int(rng.choice([2, 4, 8]))
    M, S = int(rng.integers(1, 4)), int(rng.integers(1, 3))
    D = int(rng.choice([d for d in (1, 2, 4, 8) if R % d == 0]))
    E, k, T = R * M, 2, int(rng.integers(1, 30))
    idx = W.random_ids(rng, E, R * T * k, invalid_frac=0.1).reshape(-1, k)
    idx[rng.random(idx.shape[0]) < 0.5, 0] = 0               # one hot expert
    pl = O.balance(idx, E, R, S, D)[0]
    for il in (False, True):
        phys, pos = O.reroute_local(idx, pl, il)
        check_local_layout(idx, pl, phys, pos, il)
