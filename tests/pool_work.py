"""Host work the GPU tests hand to a process pool: drawing seeded routings
and running the CPU oracle on them.

The pool is started with the "spawn" method: every worker is a fresh
interpreter that imports only NumPy, the generators and the oracle (never
torch or the HIP library), so it holds no GPU state, and a test can use it
after earlier tests have touched the GPU.
"""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

import oracle as O
import workload as W


def pool(n_tasks: int, cap: int = 16):
    """A spawn pool sized to the task count and the host's usable cores
    (at most ``cap``)."""
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    return mp.get_context("spawn").Pool(max(1, min(cap, cores, n_tasks)))


def routing_and_plan(args):
    """(topk_idx, topk_w or None, oracle plan) of one (workload, layer,
    microbatch) instance; the weights only when asked for."""
    cfg_id, layer, mb, want_w = args
    w = W.CONFIGS[cfg_id]
    idx, wt, _ = W.routing(w, layer, mb)
    c, dropped = O.count(idx, w.E)
    pl = O.plan(c, w.E, w.R, w.S, w.D, dropped=dropped)
    return idx, (wt if want_w else None), pl
