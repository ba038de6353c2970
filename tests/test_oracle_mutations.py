"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case edits one line of a copy of the oracle's source (a dropped term, a
flipped tie-break, an off-by-one, a wrong operand), loads the copy as a
module, swaps it in for ``oracle`` and runs a fast subset of the pins.  The
test passes only if at least one pin fails on the broken copy.
"""
import inspect
import json
import sys
import types

import numpy as np
import pytest

import oracle
import oracle.ultraep_oracle as base
import test_oracle_combine as C
import test_oracle_locality as LC
import test_oracle_weight_sync as WS
import test_oracle_pins as P

MUTATIONS = [
    ("count keeps id E", "valid = (ids >= 0) & (ids < E)\n    c = np.bincount",
     "valid = (ids >= 0) & (ids <= E)\n    c = np.bincount"),
    ("ordinal off by one", 'run_start = np.searchsorted(key[order], key[order], side="left")',
     'run_start = np.searchsorted(key[order], key[order], side="right")'),
    ("no domain floor", "Q_lb = min(max(Q_mean, floor), Q_max)", "Q_lb = min(Q_mean, Q_max)"),
    ("minimum ignored", "    m = max(1, int(min_tokens))", "    m = 1"),
    ("lean plan still chains", "don = [] if lean else [f for f in piece", "don = [] if False else [f for f in piece"),
    ("lean option ignored", "hosted = feasible(c, Q, E, R, S, D, allow_zero_master, min_tokens, lean)",
     "hosted = feasible(c, Q, E, R, S, D, allow_zero_master, min_tokens)"),
    ("minimum: small shed dropped, not raised", "t = m if avail >= m else 0", "t = 0"),
    ("minimum: fill takes the whole spare", "                x = min(spare[r], a - m)\n                if x < m:",
     "                x = spare[r]\n                if x < m:"),
    ("minimum: chain fill takes the whole spare", "x = min(spare[r2], a - m)", "x = spare[r2]"),
    ("minimum: donor may leave less than the minimum",
     "                if 0 < a - x < m:              # what stays queued is at least m\n                    x = a - m\n", ""),
    ("target ignored", "Q_mean = _ceil_div(total * thr_num, R * thr_den)", "Q_mean = _ceil_div(total, R)"),
    ("tolerance not per rank", "tol = max(1, (total * eps_num) // (R * eps_den))",
     "tol = max(1, (total * eps_num) // eps_den)"),
    ("shed coldest first", "key=lambda f: (-c[f], f)", "key=lambda f: (c[f], f)"),
    ("keep nothing", "return 1 if (c[e] > 0 and not allow_zero_master) else 0",
     "return 0 if (c[e] > 0 and not allow_zero_master) else 0"),
    ("piece tie by higher id", "e = max(piece, key=lambda f: (piece[f], -f))",
     "e = max(piece, key=lambda f: (piece[f], f))"),
    ("loosest fit", "r = min(fit, key=lambda q: (spare[q], q))", "r = min(fit, key=lambda q: (-spare[q], q))"),
    ("roomiest tie by higher rank", "r = max(rec, key=lambda q: (spare[q], -q))",
     "r = max(rec, key=lambda q: (spare[q], q))"),
    ("chain does not grow the donor piece", "piece[f] += x", "piece[f] += 0"),
    ("no chain branch", "if don:", "if False:"),
    ("replica may sit on its home", "return r != home and free[r] > 0", "return free[r] > 0"),
    ("instances in creation order", "for p in sorted(phys):", "for p in phys:"),
    ("offset not prefix", "phys_off[1:] = np.cumsum(phys_load)", "phys_off[1:] = phys_load"),
    ("instance lookup left", 'i = np.searchsorted(inst_gend, expert_base[e] + o[valid], side="right")',
     'i = np.searchsorted(inst_gend, expert_base[e] + o[valid], side="left")'),
    ("layout weight of row", "    w_perm[pos[n]] = w[n]\n    return inv, w_perm",
     "    w_perm[pos[n]] = w[pos[n]]\n    return inv, w_perm"),
    ("permute token from slot", "[np.asarray(inv)[lo:hi] // k]", "[np.asarray(inv)[lo:hi] % k]"),
    ("permute segment shifted", "lo, hi = int(pl.phys_off[p_begin]), int(pl.phys_off[p_end])",
     "lo, hi = int(pl.phys_off[p_begin]), int(pl.phys_off[p_end - 1])"),
    ("fold in fp32", "acc = np.asarray(master[e], dtype=np.float64).copy()",
     "acc = np.asarray(master[e], dtype=np.float32).copy()"),
    ("fold drops range end", "slots = [s for s in range(slot_begin, slot_end) if",
     "slots = [s for s in range(slot_begin, slot_end - 1) if"),
    ("combine ignores the weight", "out[g - token_begin] += (1.0 if w is None else w[n]) * rows[p[n]]",
     "out[g - token_begin] += rows[p[n]]"),
    ("combine keeps rows past the layout", "            if 0 <= p[n] < nrows:\n                out[",
     "            if 0 <= p[n] <= nrows - 0 and p[n] != -1:\n                out["),
    ("row gradient without the weight", "grad_rows[int(p[n])] = w[n] * dy[g - token_begin]",
     "grad_rows[int(p[n])] = dy[g - token_begin]"),
    ("weight gradient from the pair's own index", "float(np.dot(dy[g - token_begin], rows[p[n]]))",
     "float(np.dot(dy[g - token_begin], rows[n % nrows]))"),
    ("bf16 ties round up", "q = np.rint(x / spacing) * spacing", "q = np.floor(x / spacing + 0.5) * spacing"),
    ("bf16 one bit short", "spacing = np.exp2(np.maximum(e - 7, -133.0))", "spacing = np.exp2(np.maximum(e - 6, -133.0))"),
    ("relay count ties to the larger", "if best is None or cost < best[0]:", "if best is None or cost <= best[0]:"),
    ("relays are the highest-id replicas", "            if not relay or i < m:", "            if not relay or i >= n - m:"),
    ("relay gain not checked", "(n >= min_replicas and n >= min_gain * cost)", "(n >= min_replicas)"),
    ("relay ignores the domain size", "domain_gpus > 8 and n >= 2", "domain_gpus > 0 and n >= 2"),
    ("local take not capped by the quota", "a[i] = min(q, int(rank_counts[h, e]))", "a[i] = int(rank_counts[h, e])"),
    ("pool rows before local rows", "row = int(a[i]) + pool_seen[i]", "row = pool_seen[i]"),
    ("interleave in reverse instance order", "                for i in insts:\n                    if left[i] > 0:",
     "                for i in reversed(insts):\n                    if left[i] > 0:"),
    ("weight sync from the wrong master", "{s: np.array(master[int(pl.slot_expert[s])], copy=True)",
     "{s: np.array(master[int(pl.slot_expert[s]) ^ 1], copy=True)"),
]

PIN_SUBSET = [
    (P.test_count_hand_example, {}),
    (P.test_count_brute_force_with_invalid_ids, {"seed": 0}),
    (P.test_ordinals_brute_force, {"seed": 1}),
    (P.test_plan_hand_layout_example, {}),
    *[(P.test_plan_hand_worked, {"case": c}) for c in P.HAND],
    (P.test_plan_single_hot_expert_wraps, {"N": 77, "R": 5, "M": 3, "S": 1}),
    (P.test_plan_two_ranks_closed_form, {"seed": 1}),
    (P.test_plan_uniform_home_load, {}),
    (P.test_plan_threshold_stops_at_the_target, {"which": 1, "thr": (105, 100)}),
    (P.test_plan_minimum_tokens_per_replica, {"cfg": 2, "mt": 1024}),
    (P.test_plan_minimum_single_hot_expert_wraps, {"N": 50, "R": 8, "m": 6}),
    (P.test_plan_lean_invariants_random_shapes, {"seed": 0}),
    (P.test_plan_no_replication_possible, {"seed": 0, "S": 0, "D": 4}),
    (P.test_plan_invariants_random_shapes, {"seed": 3}),
    (P.test_layout_properties_workloads, {"cfg": 1, "layer": 0}),
    (P.test_layout_properties_random_with_dropped, {"seed": 2}),
    (P.test_layout_without_replication_is_stable_sort_by_expert, {}),
    (P.test_permute_brute_force, {"seed": 0}),
    (P.test_fold_exact_integers_and_untouched, {}),
    (P.test_fold_rounds_once_from_fp64, {}),
    (P.test_plan_against_brute_force_optimum_tiny, {"seed": 0}),
    (P.test_topology_floor_is_reached, {}),
    (C.test_bf16_rounding_fixed_cases, {}),
    (C.test_combine_matches_dense_matrix_product, {"seed": 0}),
    (C.test_dropped_pairs_add_nothing, {}),
    (C.test_combine_backward_is_the_adjoint, {"seed": 0}),
    (C.test_weight_gradient_is_a_finite_difference, {"seed": 0}),
    (C.test_unweighted_combine_is_the_adjoint_of_the_dispatch_gather, {}),
    *[(WS.test_relay_costs_hand_worked, {"case": c}) for c in json.load(open(WS.GOLDEN))["cases"]],
    (WS.test_relay_schedule_structure_on_workload_plans, {}),
    (WS.test_weight_sync_copies_bits, {}),
    *[(LC.test_locality_hand_worked, {"case": c}) for c in LC.CASES],
    (LC.test_locality_structure_on_workloads, {"cfg": 1, "T": None, "interleave": True}),
    (LC.test_locality_random_shapes_with_dropped, {"seed": 0}),
]


def _mutant(old, new):
    src = inspect.getsource(base)
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    sys.modules["oracle_mutant"] = mod       # dataclasses look their module up
    try:
        exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    finally:
        del sys.modules["oracle_mutant"]
    return mod


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(name, old, new, monkeypatch):
    mod = _mutant(old, new)
    for attr in oracle.__dict__:
        if not attr.startswith("_") and hasattr(mod, attr):
            monkeypatch.setattr(P.O, attr, getattr(mod, attr))
    failed = []
    for fn, kw in PIN_SUBSET:
        try:
            fn(**kw)
        except (AssertionError, IndexError, ValueError, KeyError, TypeError):
            failed.append(fn.__name__)
    assert failed, f"no pin caught the planted mistake: {name}"


def test_unmutated_oracle_passes_subset():
    for fn, kw in PIN_SUBSET:
        fn(**kw)
