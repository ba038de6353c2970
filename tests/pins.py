"""Checks that pin the CPU oracle to facts outside itself.

Each check takes the oracle as a parameter (an object with the oracle's
functions), so the same checks can be run against deliberately broken copies
of the oracle to show that they catch plausible mistakes.

None of these re-type the oracle's formulas: they use hand-worked values,
brute force written a different way, closed-form special cases, invariants,
and the numbers the pages print.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# brute force, written as plain loops
# ---------------------------------------------------------------------------
def brute_counts(ids, E):
    c = [0] * E
    dropped = 0
    for x in np.asarray(ids).reshape(-1).tolist():
        if 0 <= x < E:
            c[x] += 1
        else:
            dropped += 1
    return c, dropped


def brute_ordinals(ids, E):
    flat = np.asarray(ids).reshape(-1).tolist()
    seen = {}
    out = []
    for x in flat:
        if 0 <= x < E:
            out.append(seen.get(x, 0))
            seen[x] = seen.get(x, 0) + 1
        else:
            out.append(-1)
    return out


def brute_segment_tokens(phys, k, p_begin, p_end):
    """Tokens of the pairs on physical experts [p_begin, p_end), grouped by
    physical expert and in pair order inside each (the dispatch order)."""
    phys = np.asarray(phys).reshape(-1).tolist()
    toks = []
    for p in range(p_begin, p_end):
        for n, q in enumerate(phys):
            if q == p:
                toks.append(n // k)
    return toks


def hall_min_quota(c, hosts_of, R):
    """Smallest integer Q such that the loads c can be split over the allowed
    hosts with every rank at most Q (Hall's condition on the expert->rank
    graph: every expert set X needs sum c(X) <= Q * |hosts(X)|)."""
    E = len(c)
    best = 0
    for mask in range(1, 1 << E):
        load = 0
        hosts = 0
        for e in range(E):
            if mask >> e & 1:
                load += c[e]
                hosts |= hosts_of[e]
        if load:
            n = bin(hosts).count("1")
            best = max(best, -(-load // n))
    return best


def brute_optimum(c, E, R, S, D):
    """Best possible max rank load over every placement of at most S foreign
    in-domain replicas per rank (splits ignore the keep-one rule, so this is a
    lower bound for any valid plan)."""
    M = E // R
    choices = []
    for r in range(R):
        d = r // D
        foreign = [e for e in range(d * D * M, (d + 1) * D * M) if e // M != r]
        opts = []
        for n in range(0, S + 1):
            opts.extend(itertools.combinations(foreign, n))
        choices.append(opts)
    best = None
    for placement in itertools.product(*choices):
        hosts_of = [1 << (e // M) for e in range(E)]
        for r, chosen in enumerate(placement):
            for e in chosen:
                hosts_of[e] |= 1 << r
        q = hall_min_quota(c, hosts_of, R)
        best = q if best is None else min(best, q)
    return best


# ---------------------------------------------------------------------------
# invariants of a plan
# ---------------------------------------------------------------------------
def check_plan_invariants(pl, c, allow_zero_master=False, min_tokens=1):
    E, R, S, D, M = pl.E, pl.R, pl.S, pl.D, pl.M
    c = np.asarray(c, dtype=np.int64)
    assert np.array_equal(pl.c, c)
    assert pl.total == int(c.sum())
    H = c.reshape(R, M).sum(axis=1)
    assert np.array_equal(pl.rank_before, H)
    assert pl.Q_max == int(H.max()) if E else True
    assert pl.Q_lb <= pl.Q_star <= pl.Q_max
    assert pl.Q_star >= math.ceil(pl.total / R)
    # every slot: an expert of its own domain, not homed on the slot's rank
    hosted = {}
    for s in range(R * S):
        e = int(pl.slot_expert[s])
        r = s // S
        if e < 0:
            assert pl.slot_quota[s] == 0
            continue
        assert 0 <= e < E
        assert pl.slot_quota[s] >= max(1, min_tokens)
        assert e // M != r, "replica on its own home rank"
        assert (e // M) // D == r // D, "replica outside its domain"
        assert e not in hosted.setdefault(r, set()), "two replicas of one expert on a rank"
        hosted[r].add(e)
    # conservation per expert
    per_expert = np.zeros(E, dtype=np.int64)
    for s in range(R * S):
        if pl.slot_expert[s] >= 0:
            per_expert[pl.slot_expert[s]] += pl.slot_quota[s]
    assert np.array_equal(pl.master_quota + per_expert, c)
    keep = np.where((c > 0) & (not allow_zero_master), 1, 0)
    assert (pl.master_quota >= keep).all()
    # physical loads, offsets, rank loads
    assert pl.phys_load.sum() == pl.total
    assert pl.phys_off[0] == 0 and np.array_equal(np.diff(pl.phys_off), pl.phys_load)
    assert np.array_equal(pl.rank_after, pl.phys_load.reshape(R, M + S).sum(axis=1))
    assert int(pl.rank_after.max(initial=0)) <= pl.Q_star
    # instances: each expert's master plus its replicas, ascending physical id
    for e in range(E):
        inst = pl.instances(e)
        phys = [p for p, _, _ in inst]
        assert phys == sorted(phys)
        master_p = (e // M) * (M + S) + e % M
        assert master_p in phys
        rep_p = sorted((s // S) * (M + S) + M + s % S for s in range(R * S) if pl.slot_expert[s] == e)
        assert sorted(phys) == sorted([master_p] + rep_p)
        prev = 0
        for p, start, end in inst:
            assert start == prev and end - start == pl.phys_load[p]
            prev = end
        assert prev == c[e]


def check_layout(topk_idx, topk_w, pl, phys, pos, inv, w_perm, E, k):
    """Layout properties that hold at any size."""
    ids = np.asarray(topk_idx).reshape(-1)
    n = ids.size
    valid = (ids >= 0) & (ids < E)
    phys = np.asarray(phys).reshape(-1)
    pos = np.asarray(pos).reshape(-1)
    assert (phys[~valid] == -1).all() and (pos[~valid] == -1).all()
    M, S = pl.M, pl.S
    # each pair on an instance of its own expert
    pv = phys[valid]
    r, j = pv // (M + S), pv % (M + S)
    is_master = j < M
    assert (r[is_master] * M + j[is_master] == ids[valid][is_master]).all()
    slot = r[~is_master] * S + (j[~is_master] - M)
    assert (pl.slot_expert[slot] == ids[valid][~is_master]).all()
    # physical loads are what the plan promised
    assert np.array_equal(np.bincount(pv, minlength=pl.P), pl.phys_load)
    # pos is a bijection onto the layout, inside each expert's segment,
    # in pair order: the layout is the (phys, pair) order of the valid pairs
    nv = np.nonzero(valid)[0]
    order = nv[np.lexsort((nv, phys[nv]))]
    expect_pos = np.empty(n, dtype=np.int64)
    expect_pos[order] = np.arange(order.size)
    assert np.array_equal(pos[valid], expect_pos[valid])
    assert np.array_equal(np.asarray(inv)[:order.size], order)
    w = np.asarray(topk_w, dtype=np.float32).reshape(-1)
    assert np.array_equal(np.asarray(w_perm)[:order.size].view(np.uint32), w[order].view(np.uint32))
