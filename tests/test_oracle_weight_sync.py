"""Pins of the oracle's weight_sync and relay plan (CPU).

The copy is pinned by bit patterns (NaN payloads included) and slot ranges.
The relay plan is pinned by hand-worked fan-out costs (golden file), by
simulating the produced two-stage schedule send by send and comparing its
critical fan-out with every other relay count, and by its structural rules
on the workloads' plans.
"""
import json
import os

import numpy as np
import pytest

import oracle as O
import workload as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "relay_costs.json")


class StubPlan:
    """Just enough of a plan for the relay rules: expert 0 has n replicas on
    ranks 1..n (one slot each), every other expert none."""

    def __init__(self, n, D=None):
        self.R, self.S, self.M = n + 1, 1, 1
        self.E = self.R
        self.D = D if D is not None else 64
        self.slot_expert = np.full(self.R, -1)
        self.slot_expert[1:] = 0

    def instances(self, e):
        P1 = self.M + self.S
        if e != 0:
            return [(e * P1, 0, 0)]
        return [(0, 0, 0)] + [(r * P1 + 1, 0, 0) for r in range(1, self.R)]


def simulate(src, stage, reps):
    """Critical fan-out of one expert's schedule, counted send by send."""
    sends_master = sum(1 for s in reps if src[s] == -1 and stage[s] == 1)
    per_relay = {}
    for s in reps:
        if stage[s] == 2:
            per_relay[src[s]] = per_relay.get(src[s], 0) + 1
    return sends_master + (max(per_relay.values()) if per_relay else 0)


def round_robin_cost(n, m):
    """Fan-out with m relays by dealing the other n - m replicas one by one."""
    load = [0] * m
    for i in range(n - m):
        load[i % m] += 1
    return m + max(load)


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: f"n{c['n']}")
def test_relay_costs_hand_worked(case):
    pl = StubPlan(case["n"])
    reps = O.replica_slots(pl, 0)
    assert len(reps) == case["n"]
    src, stage = O.relay_plan(pl, O.RELAY_FORCE)
    relays = [s for s in reps if stage[s] == 1]
    assert len(relays) == case["m"]
    assert simulate(src, stage, reps) == case["cost"]
    assert case["cost"] == min(round_robin_cost(case["n"], m) for m in range(1, min(8, case["n"] - 1) + 1))
    src_a, stage_a = O.relay_plan(pl, O.RELAY_ADAPTIVE)
    assert bool((stage_a[reps] == 2).any()) == case["adaptive_relays"]
    # a domain of at most 8 GPUs always copies directly
    src_d, stage_d = O.relay_plan(StubPlan(case["n"], D=8), O.RELAY_FORCE)
    assert (src_d[reps] == -1).all() and (stage_d[reps] == 1).all()


def test_relay_schedule_structure_on_workload_plans():
    for cfg, T in ((2, 1024), (3, 1024), (4, 1024)):
        w = W.CONFIGS[cfg].with_(T=T)
        idx, _, _ = W.routing(w, 0, 0)
        c, _ = O.count(idx, w.E)
        pl = O.plan(c, w.E, w.R, w.S, w.D)
        for mode in (O.RELAY_DIRECT, O.RELAY_ADAPTIVE, O.RELAY_FORCE):
            src, stage = O.relay_plan(pl, mode, min_replicas=3)
            empty = pl.slot_expert < 0
            assert (src[empty] == -2).all() and (stage[empty] == 0).all()
            for e in range(w.E):
                reps = O.replica_slots(pl, e)
                if mode == O.RELAY_DIRECT:
                    assert all(src[s] == -1 and stage[s] == 1 for s in reps)
                    continue
                relays = [s for s in reps if stage[s] == 1]
                assert relays == reps[:len(relays)], "relays are the lowest-id replicas"
                loads = {}
                for s in reps:
                    if stage[s] == 2:
                        assert src[s] in relays and pl.slot_expert[src[s]] == e
                        loads[src[s]] = loads.get(src[s], 0) + 1
                if loads:
                    assert max(loads.values()) - min(loads.values()) <= 1
                    best = min(round_robin_cost(len(reps), m) for m in range(1, min(8, len(reps) - 1) + 1))
                    assert simulate(src, stage, reps) == best
                    if mode == O.RELAY_ADAPTIVE:
                        assert len(reps) >= 3 and len(reps) >= 2 * best


def test_weight_sync_copies_bits():
    w = W.TINY
    idx, _, _ = W.routing(w, 0, 0)
    c, _ = O.count(idx, w.E)
    pl = O.plan(c, w.E, w.R, w.S, w.D)
    rng = np.random.default_rng(31)
    master = {e: rng.integers(0, 1 << 16, size=1000, dtype=np.uint16) for e in range(w.E)}
    out = O.weight_sync(master, pl, 0, w.R * w.S)
    filled = [s for s in range(w.R * w.S) if pl.slot_expert[s] >= 0]
    assert sorted(out) == filled
    for s in filled:
        assert out[s].tobytes() == master[int(pl.slot_expert[s])].tobytes()
        assert out[s] is not master[int(pl.slot_expert[s])]
    sub = O.weight_sync(master, pl, 1, 3)
    assert sorted(sub) == [s for s in (1, 2) if pl.slot_expert[s] >= 0]
