"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and compare it with the CPU oracle on the same seeded inputs."""
from __future__ import annotations

import functools
import sys

import numpy as np

import moe_expert_load_ultraep_amd as U
import oracle as O
import workload as W


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=None)
def routing_cached(cfg_id: int, layer: int, mb: int, T: int | None = None):
    w = W.CONFIGS[cfg_id]
    if T is not None:
        w = w.with_(T=T)
    idx, wt, _ = W.routing(w, layer, mb)
    idx.setflags(write=False)
    wt.setflags(write=False)
    return idx, wt


def run_balance(ctx, idx_layers: np.ndarray, w_layers: np.ndarray | None, T: int, k: int, dev="cuda",
                fused: bool = True):
    """Balance (and, with weights, lay out) L layers; returns host copies.

    fused: the layout is written by ultraep_balance itself; otherwise by a
    separate ultraep_dispatch_layout call."""
    import torch
    L = idx_layers.shape[0]
    buf = U.Buffers(ctx, L, T, k, dev)
    d_idx = torch.from_numpy(np.array(idx_layers, copy=True)).to(dev)
    out = {"buf": buf}
    buf.inv.fill_(-7)
    if w_layers is not None:
        d_w = torch.from_numpy(np.array(w_layers, copy=True)).to(dev)
        if fused:
            U.ultraep_balance(ctx, d_idx, T, k, buf.workspace, buf.plans, buf.phys_idx, buf.pos,
                              topk_w=d_w, inv=buf.inv, w_perm=buf.w_perm, L=L)
        else:
            U.ultraep_balance(ctx, d_idx, T, k, buf.workspace, buf.plans, buf.phys_idx, buf.pos, L=L)
            U.ultraep_dispatch_layout(ctx, T, k, buf.pos, d_w, buf.inv, buf.w_perm, L=L)
    else:
        U.ultraep_balance(ctx, d_idx, T, k, buf.workspace, buf.plans, buf.phys_idx, buf.pos, L=L)
    torch.cuda.synchronize()
    out["plans"] = buf.plans.cpu().numpy()
    out["phys"] = buf.phys_idx.cpu().numpy()
    out["pos"] = buf.pos.cpu().numpy()
    if w_layers is not None:
        out["inv"] = buf.inv.cpu().numpy()
        out["w_perm"] = buf.w_perm.cpu().numpy()
    return out


def assert_plan_equal(ctx, words: np.ndarray, pl: O.Plan, N: int):
    g = ctx.decode_plan(words)
    assert g["magic"] == U.PLAN_MAGIC
    for key, want in (("E", pl.E), ("R", pl.R), ("S", pl.S), ("D", pl.D), ("M", pl.M), ("P", pl.P),
                      ("N", N), ("total", pl.total), ("dropped", pl.dropped), ("Q_star", pl.Q_star),
                      ("Q_lb", pl.Q_lb), ("Q_max", pl.Q_max), ("tol", pl.tol),
                      ("grid_index", pl.grid_index), ("floor", pl.floor),
                      ("replicas", pl.n_replicas)):
        assert g[key] == want, (key, g[key], want)
    for key in ("counts", "master_quota", "slot_expert", "slot_quota", "phys_load", "phys_off",
                "inst_ptr", "rank_before", "rank_after"):
        want = pl.c if key == "counts" else getattr(pl, key)
        assert np.array_equal(g[key].astype(np.int64), np.asarray(want, dtype=np.int64)), key
    n = int(pl.inst_ptr[-1])
    assert np.array_equal(g["inst_phys"][:n].astype(np.int64), pl.inst_phys)
    assert np.array_equal(g["inst_end"][:n].astype(np.int64), pl.inst_end)
    # layout row of ordinal o on instance i is inst_base[i] + o
    start = pl.inst_end - pl.phys_load[pl.inst_phys]
    assert np.array_equal(g["inst_base"][:n].astype(np.int64), pl.phys_off[pl.inst_phys] - start)
    # the unused tail has fixed values
    assert (g["inst_phys"][n:] == -1).all() and (g["inst_end"][n:] == 0).all() and (g["inst_base"][n:] == 0).all()
    return g


def rank_counts(idx: np.ndarray, R: int, E: int) -> np.ndarray:
    """Pairs of each expert from each rank's tokens (pairs are rank-major)."""
    ids = np.asarray(idx).reshape(-1).astype(np.int64)
    src = np.arange(ids.size) // max(1, ids.size // R)
    ok = (ids >= 0) & (ids < E)
    rc = np.zeros((R, E), dtype=np.int64)
    np.add.at(rc, (src[ok], ids[ok]), 1)
    return rc


def assert_layer_equal(ctx, got: dict, layer: int, idx: np.ndarray, wt: np.ndarray | None,
                       E: int, R: int, S: int, D: int, **opts):
    pl, phys, pos = O.balance(idx, E, R, S, D, **opts)
    mode = getattr(ctx, "reroute_mode", 0)
    if mode:
        phys, pos = O.reroute_local(idx, pl, interleave=(mode == 2))
    N = idx.size
    assert_plan_equal(ctx, got["plans"][layer], pl, N)
    g = ctx.decode_plan(got["plans"][layer])
    n = int(pl.inst_ptr[-1])
    assert np.array_equal(g["inst_local"][:n].astype(np.int64), O.local_takes(pl, rank_counts(idx, R, E)))
    assert (g["inst_local"][n:] == 0).all()
    assert np.array_equal(got["phys"][layer].astype(np.int64), phys)
    assert np.array_equal(got["pos"][layer].astype(np.int64), pos)
    if wt is not None:
        inv, wp = O.layout(pos, wt, pl.total)
        assert np.array_equal(got["inv"][layer][:pl.total].astype(np.int64), inv)
        assert (got["inv"][layer][pl.total:] == -7).all(), "rows beyond total must stay untouched"
        assert np.array_equal(got["w_perm"][layer][:pl.total].view(np.uint32), wp.view(np.uint32))
    return pl, phys, pos


def fold_tolerance_ok(got: np.ndarray, master: np.ndarray, reps: list) -> bool:
    want = master.astype(np.float64) + sum(r.astype(np.float64) for r in reps)
    scale = np.abs(master.astype(np.float64)) + sum(np.abs(r.astype(np.float64)) for r in reps)
    return bool((np.abs(got.astype(np.float64) - want) <= 1e-6 * scale + 1e-30).all())
