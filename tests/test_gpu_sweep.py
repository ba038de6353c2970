"""Seeded random-shape sweep of the whole balance path on the GPU.

The project README's "Tests" section describes solving runs on synthesized
skewed loads at many imbalance levels; this sweep draws 200 small shapes
(E <= 64, R <= 16, S <= 4, D dividing R, k <= 4, T <= 3000 tokens per rank,
so a rank's pairs span one or two tiles) with Dirichlet loads of random
concentration, some invalid ids, and random planning options, and compares
the plan record, the replica map and the fused dispatch layout with the
oracle in all three reroute modes.  The first mismatch stops the test and
names the shape.
"""
import numpy as np
import pytest

import moe_expert_load_ultraep_amd as U
import oracle as O
from gpu_common import assert_layer_equal, run_balance, say
from pins import check_plan_invariants

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

N_SHAPES = 200
CHUNKS = 4


def sweep_case(i):
    """Shape, options and routing of sweep case i (seeded by i alone)."""
    rng = np.random.default_rng([20261203, i])
    R = int(rng.choice([1, 2, 3, 4, 6, 8, 8, 12, 16, 16]))
    M = int(rng.choice([m for m in (1, 2, 3, 4, 5, 8) if R * m <= 64]))
    E = R * M
    # mostly domains of two ranks or more, where replicas can be placed
    wide = [d for d in range(2, R + 1) if R % d == 0]
    D = int(rng.choice(wide)) if wide and rng.random() > 0.15 else 1
    S = int(rng.choice([0, 1, 1, 2, 2, 2, 3, 4]))
    k = int(rng.integers(1, min(4, E) + 1))
    u = rng.random()   # empty layers, ranks of more than one tile, else log-uniform
    T = 0 if u < 0.05 else int(rng.integers(2049, 3001)) if u < 0.2 else \
        int(np.exp(rng.uniform(0.0, np.log(3001.0)))) - 1
    alpha = float(np.exp(rng.uniform(np.log(0.05), np.log(2.0))))
    p = np.maximum(rng.dirichlet(np.full(E, alpha)), 1e-12)
    p /= p.sum()
    N = R * T * k
    idx = rng.choice(E, size=N, p=p).astype(np.int32)
    if rng.random() < 0.3:
        bad = rng.random(N) < rng.uniform(0.0, 0.05)
        idx = np.where(bad, rng.choice([-1, E, 1 << 30], size=N), idx).astype(np.int32)
    wt = rng.random(N).astype(np.float32)
    opts = {"allow_zero_master": bool(rng.random() < 0.2)}
    if rng.random() < 0.2:
        opts["thr_num"], opts["thr_den"] = [(101, 100), (11, 10), (3, 2)][int(rng.integers(3))]
    if rng.random() < 0.2:
        opts["eps_num"], opts["eps_den"] = [(0, 1), (1, 20), (1, 1000)][int(rng.integers(3))]
    if rng.random() < 0.25:
        opts["min_tokens"] = int(rng.choice([2, 3, 8, 50, 400]))
    if rng.random() < 0.25:
        opts["lean"] = True
    return dict(E=E, R=R, S=S, D=D, k=k, T=T, idx=idx.reshape(R * T, k), wt=wt.reshape(R * T, k),
                opts=opts)


def _ctx(c, mode):
    o = c["opts"]
    return U.ultraep_create(c["E"], c["R"], c["S"], c["D"],
                            eps=(o.get("eps_num", 1), o.get("eps_den", 100)),
                            allow_zero_master=o["allow_zero_master"],
                            threshold=(o.get("thr_num", 1), o.get("thr_den", 1)), reroute_mode=mode,
                            min_tokens=o.get("min_tokens", 1), replica_lean=o.get("lean", False))


@pytest.mark.parametrize("chunk", range(CHUNKS))
def test_random_shape_sweep(chunk):
    per = N_SHAPES // CHUNKS
    for i in range(chunk * per, (chunk + 1) * per):
        c = sweep_case(i)
        E, R, S, D, k, T = c["E"], c["R"], c["S"], c["D"], c["k"], c["T"]
        tag = f"case {i}: E={E} R={R} S={S} D={D} k={k} T={T} opts={c['opts']}"
        pl, _, _ = O.balance(c["idx"], E, R, S, D, **c["opts"])
        check_plan_invariants(pl, pl.c, c["opts"]["allow_zero_master"], c["opts"].get("min_tokens", 1))
        for mode in (0, 1, 2):
            ctx = _ctx(c, mode)
            got = run_balance(ctx, c["idx"][None], c["wt"][None], T, k, fused=(i + mode) % 3 != 0)
            try:
                assert_layer_equal(ctx, got, 0, c["idx"], c["wt"], E, R, S, D, **c["opts"])
            except AssertionError:
                say(f"sweep mismatch, {tag}, reroute mode {mode}")
                raise
    say(f"sweep chunk {chunk}: {per} shapes x 3 modes equal")
