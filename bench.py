"""Benchmark of the exact-load rebalancing hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic routing:
  ultraep_balance          count + quota plan + reroute (phys_idx, pos) and the
                           dispatch layout (inverse index, permuted weights),
                           for every layer of the batch in one call
  ultraep_permute          bf16 rows of the most loaded rank's receive segment
                           (first layer of the batch)
  ultraep_fold_grads       that layer's redundant-slot gradients of the rank
                           with the most filled slots, into their masters
All inputs are resident in HBM before the timed region.  Each call is timed
with HIP events on the stream it runs on; the permute kernel is the dominant
one and its roofline is reported against the 8 TB/s HBM peak.

Beside the timed steps, the balance call is timed warm (back to back on the
same input) and cold (a 1 GiB scratch write before each repetition evicts the
256 MB Infinity Cache and the L2s); permute and fold are timed cold the same
way; every cold figure also comes as mean, median, p99 and max
(cold_distribution_us).  The balance is timed again at the pages' default
knobs (locality-aware decomposition with interleave, at least 1024 pairs per
replica: pages_defaults) and with the replica-lean planner option
(replica_lean: its plan quality and the weight_sync of its fewer slots).  The CPU oracle is timed stage by stage on the host
on the same workload (cpu_baseline).  Workloads of several layers or
microbatches also report each instance's max/mean before and after
(load_trace; --load-trace writes every rank and expert load).  Prints ONE
JSON line.

Workloads (--config):
  2  single layer, E=128 R=64 S=2 D=64 T=8192 top-8 (the default)
  3  61 layers, E=256 R=64 S=2 D=64 T=4096 top-8, balanced in one call;
     per-layer figures are the call's time / 61
  4  non-stationary stream, 32 layers x 16 microbatches of the single-layer
     shape, one balance call per instance; the cold balance time is also
     reported as median and p99 over the instances
  5  topology-constrained prefill, E=160 R=40 S=3 D=8 T=16384 top-8
  1  tiny (launch-bound; no roofline claim)
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "balance+reroute µs/layer; routed pairs/s; permute/fold HBM GB/s vs peak"
FLUSH_MIB = 1024


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, help="workload id (2 = single layer, the headline)")
    ap.add_argument("--cold-reps", type=int, default=100, help="repetitions of each cold / warm timing")
    ap.add_argument("--instances", type=int, default=0,
                    help="workload 4: instances used (0 = all 32 x 16)")
    ap.add_argument("--workers", type=int, default=16, help="host processes generating inputs")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget for the oracle timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--threshold", default="1/1",
                    help="early-stop target of the quota search as num/den (the pages' default 1.0)")
    ap.add_argument("--min-tokens", type=int, default=1,
                    help="smallest replica quota the plan keeps (the pages' default is 1024)")
    ap.add_argument("--reroute-mode", type=int, default=0, choices=(0, 1, 2),
                    help="0: ordinal ranges; 1: locality-aware; 2: locality-aware with interleave")
    ap.add_argument("--no-weight-sync", action="store_true",
                    help="skip the weight_sync timing (needs master and replica weight buffers)")
    ap.add_argument("--no-combine", action="store_true",
                    help="skip the combine / combine-backward timing (needs two layout-sized buffers)")
    ap.add_argument("--copy-mib", type=int, default=1024,
                    help="size of the runtime device-to-device copy timed for context")
    ap.add_argument("--no-pages-defaults", action="store_true",
                    help="skip the balance timing at the pages' default knobs (locality with "
                         "interleave, minimum 1024 pairs per replica)")
    ap.add_argument("--load-trace", default="",
                    help="write per-(layer, microbatch) rank and expert loads before and after "
                         "balancing to this file (JSON lines)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_single_layer_E128_R64_T8192.md")
KERNEL_SOURCE = os.path.join(ROOT, "moe_expert_load_ultraep_amd", "csrc", "ultraep_kernels.hip")


def permute_source_sha256():
    """Hash of the permute kernel's source (its constants, helpers and body,
    not its comment block), so recorded counters go stale only when the
    code changes; None when the kernel cannot be found."""
    import hashlib
    text = open(KERNEL_SOURCE).read()
    try:
        start = text.index("constexpr int kPermThreads")
        end = text.index("\n}\n", text.index("void permute_kernel(", start)) + 3
    except ValueError:
        return None
    return hashlib.sha256(text[start:end].encode()).hexdigest()


def recorded_traffic(config):
    """HBM bytes per permute launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary, or None when the kernel source changed since or the
    summary covers another workload."""
    import re
    if config != 2:
        return None
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    src = permute_source_sha256()
    m_src = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_val = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_src or not m_val or m_src.group(1) != src:
        return None
    return float(m_val.group(1))


def device_copy_rate(torch, dev, mib):
    """Rate of the runtime's own device-to-device copy (torch copy_, read +
    write bytes / time), the best of a few relative placements of source
    and destination.  Context only: it is not a ceiling (the permute kernel
    moves rows faster than this copy)."""
    n = mib << 20
    pad = 8 << 20
    buf = torch.empty(2 * n + pad, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    a = buf[:n]
    best = 0.0
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for off in (0, 64 << 10, (1 << 20) + (4 << 10), (4 << 20) + (12 << 10)):
        b = buf[n + off:2 * n + off]
        for _ in range(2):
            b.copy_(a)
        reps = 8
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(reps):
            b.copy_(a)
        ev[1].record()
        torch.cuda.synchronize()
        best = max(best, 2 * n / (ev[0].elapsed_time(ev[1]) / reps * 1e-3) / 1e9)
    del buf, a, b
    return best


def dist_us(ms, per=1):
    """Mean, median, p99 and max (in µs, divided by per) of a run of timings
    in ms, so a bimodal or heavy-tailed run shows beside its mean."""
    us = np.asarray(ms, dtype=np.float64) * 1e3 / per
    return {"mean": float(us.mean()), "median": float(np.median(us)),
            "p99": float(np.percentile(us, 99)), "max": float(us.max()), "n": int(us.size)}


def host_info():
    model = platform.processor() or ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cpus": usable}


def _route(a):
    import workload as W
    cfg, layer, mb = a
    idx, wt, _ = W.routing(W.CONFIGS[cfg], layer, mb)
    return idx, wt


def routing_instances(w, insts, workers):
    """Routing of every (layer, microbatch) in insts, generated by a process
    pool before the GPU is touched (the generator is seeded per instance, so
    the result does not depend on the pool)."""
    if workers <= 1 or len(insts) == 1:
        return [_route((w.cfg_id, l, m)) for l, m in insts]
    import multiprocessing as mp
    with mp.get_context("fork").Pool(min(workers, len(insts))) as pool:
        return pool.map(_route, [(w.cfg_id, l, m) for l, m in insts], chunksize=1)


def quality(ctx, plans, w):
    """Balance quality of decoded plan records: max/mean rank load before and
    after, the domain floor, replicas, probes."""
    rows = []
    for pl in plans:
        mean = pl["total"] / w.R
        reps = np.bincount(pl["slot_expert"][pl["slot_expert"] >= 0], minlength=w.E)
        rows.append({"before": pl["rank_before"].max() / mean, "after": pl["rank_after"].max() / mean,
                     "floor": pl["floor"] / mean, "replicas": pl["replicas"],
                     "max_per_expert": int(reps.max()), "grid_index": pl["grid_index"],
                     "rounds": pl["rounds"]})
    if len(rows) == 1:
        r = rows[0]
        return {"imbalance_before": r["before"], "imbalance_after": r["after"],
                "domain_floor": r["floor"], "replicas": r["replicas"],
                "replicas_max_per_expert": r["max_per_expert"], "grid_index": r["grid_index"],
                "probe_rounds": r["rounds"]}
    col = lambda k: np.array([r[k] for r in rows], dtype=np.float64)  # noqa: E731
    return {"plans": len(rows),
            "imbalance_before_min_median_max": [col("before").min(), float(np.median(col("before"))),
                                                col("before").max()],
            "imbalance_after_median_max": [float(np.median(col("after"))), col("after").max()],
            "domain_floor_max": col("floor").max(),
            "replicas_median_max": [float(np.median(col("replicas"))), int(col("replicas").max())],
            "replicas_max_per_expert": int(col("max_per_expert").max()),
            "grid_index_max": int(col("grid_index").max()), "probe_rounds_max": int(col("rounds").max())}


def dispatch_traffic(phys, w):
    """Where the first layer's pairs travel: the fraction served on their
    own token's rank, and the R x R matrix of pairs sent from each token's
    rank to each serving rank (off the diagonal) as max over mean."""
    ids = np.asarray(phys).reshape(-1)
    ok = ids >= 0
    src = (np.arange(ids.size) // (w.T * w.k))[ok]
    dst = ids[ok] // (w.M + w.S)
    m = np.bincount(src * w.R + dst, minlength=w.R * w.R).reshape(w.R, w.R).astype(np.float64)
    off = m[~np.eye(w.R, dtype=bool)]
    return {"local_fraction": float(np.trace(m) / m.sum()),
            "remote_pairs": int(off.sum()),
            "remote_matrix_max_over_mean": float(off.max() / off.mean()) if off.mean() > 0 else None,
            "max_remote_pairs_received_by_a_rank": int((m.sum(axis=0) - np.diag(m)).max())}


def stale_plan_imbalance(prev, cur, w):
    """Max/mean rank load when an instance is served by the previous
    instance's placement, every expert's pairs split evenly over the ranks
    that hold it (a history-based balancer's view), against the exact
    counts of the current instance."""
    P1 = w.M + w.S
    counts = cur["counts"].astype(np.float64)
    load = np.zeros(w.R)
    ptr, phys = prev["inst_ptr"], prev["inst_phys"]
    for e in range(w.E):
        ranks = phys[ptr[e]:ptr[e + 1]] // P1
        load[ranks] += counts[e] / len(ranks)
    return float(load.max() * w.R / counts.sum())


# The pages' EP64 test table ([README] "Tests"), for the workloads at its shape.
PAGES_TABLE = {6: {"initial": 1.51, "final": 1.01, "replicas_max_per_expert": 4, "replicas_total": 38,
                   "update_placement_ms": 0.067, "reroute_ms": 0.039},
               7: {"initial": 2.01, "final": 1.01, "replicas_max_per_expert": 5, "replicas_total": 46,
                   "update_placement_ms": 0.072, "reroute_ms": 0.037},
               8: {"initial": 3.03, "final": 1.01, "replicas_max_per_expert": 6, "replicas_total": 51,
                   "update_placement_ms": 0.078, "reroute_ms": 0.036}}


def cpu_baseline(w, L, routes, hidden, seg, masters, reps, slots, budget_s, thr=(1, 1), min_tokens=1):
    """Time the oracle (unchanged) on the host, stage by stage, on the same
    arrays: count, plan, reroute and layout per layer (the batch's layers or
    instances in order, as many as the budget allows), permute of the same
    rank segment and fold of the same slots of the first layer.  The step
    estimate is L layers of balance plus one permute and one fold, as on the
    GPU."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(1)
    except Exception:  # pragma: no cover
        limiter = None
    p_begin, p_end = seg
    s0, s1 = slots
    st = {"count": [], "plan": [], "reroute": [], "layout": [], "permute": [], "fold": []}
    t_start = time.perf_counter()
    i = 0
    while True:
        idx, wt = routes[i % len(routes)]
        t0 = time.perf_counter()
        c, dropped = O.count(idx, w.E)
        t1 = time.perf_counter()
        pl = O.plan(c, w.E, w.R, w.S, w.D, dropped=dropped, thr_num=thr[0], thr_den=thr[1],
                    min_tokens=min_tokens)
        t2 = time.perf_counter()
        phys, pos = O.reroute(idx, pl)
        t3 = time.perf_counter()
        inv, _ = O.layout(pos, wt, pl.total)
        t4 = time.perf_counter()
        st["count"].append(t1 - t0)
        st["plan"].append(t2 - t1)
        st["reroute"].append(t3 - t2)
        st["layout"].append(t4 - t3)
        if i == 0:
            t5 = time.perf_counter()
            O.permute(hidden, inv, w.k, pl, p_begin, p_end)
            t6 = time.perf_counter()
            O.fold(masters, reps, pl, s0, s1)
            t7 = time.perf_counter()
            st["permute"].append(t6 - t5)
            st["fold"].append(t7 - t6)
        i += 1
        if time.perf_counter() - t_start > budget_s or i >= 20:
            break
    if limiter is not None:
        limiter.unregister()
    med = {k: float(np.median(v)) for k, v in st.items()}
    layer_s = med["count"] + med["plan"] + med["reroute"] + med["layout"]
    step_s = L * layer_s + med["permute"] + med["fold"]
    return {"value": L * w.N / step_s, "unit": "pairs/s", "cores": 1, "kind": "oracle",
            "sample": f"{i} layer(s) of the same workload through count, plan, reroute and layout, "
                      f"one permute of the same rank segment and one fold of the same slots; "
                      f"medians combined as {L} layer(s) + permute + fold = {step_s * 1e3:.0f} ms "
                      f"per step; NumPy, one thread",
            "stage_ms": {k: v * 1e3 for k, v in med.items()}}


def gbps_fn(b, ms):
    return b / (ms * 1e-3) / 1e9


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the EP group is simulated as logical ranks on a "
              "single MI355X, so --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import moe_expert_load_ultraep_amd as U
    import workload as W

    w = W.CONFIGS[args.config]
    # ---- inputs: generated on the host before the GPU is touched (untimed)
    if args.config == 3:
        insts = [(l, 0) for l in range(w.layers)]
        L = w.layers
    elif args.config == 4:
        insts = [(l, m) for l in range(w.layers) for m in range(w.microbatches)]
        if args.instances > 0:
            insts = insts[:args.instances]
        L = 1
    else:
        insts = [(0, 0)]
        L = 1
    routes = routing_instances(w, insts, args.workers)
    hidden = W.hidden(w, workers=args.workers)

    import torch
    if not os.path.exists(U.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    dev = torch.device("cuda:0")
    thr = tuple(int(x) for x in args.threshold.split("/"))
    ctx = U.ultraep_create(w.E, w.R, w.S, w.D, threshold=thr, reroute_mode=args.reroute_mode,
                           min_tokens=args.min_tokens)
    buf = U.Buffers(ctx, L, w.T, w.k, dev)
    if args.config == 3:
        d_idx = [torch.from_numpy(np.stack([r[0] for r in routes])).to(dev)]
        d_w = [torch.from_numpy(np.stack([r[1] for r in routes])).to(dev)]
    else:
        d_idx = [torch.from_numpy(r[0]).to(dev) for r in routes]
        d_w = [torch.from_numpy(r[1]).to(dev) for r in routes]
    n_inst = len(d_idx)
    d_hid = torch.from_numpy(hidden.view(np.int16)).to(dev)

    def balance(i):
        U.ultraep_balance(ctx, d_idx[i], w.T, w.k, buf.workspace, buf.plans, buf.phys_idx, buf.pos,
                          topk_w=d_w[i], inv=buf.inv, w_perm=buf.w_perm, L=L)

    # ---- sizing pass (untimed): every instance's plans, for the permute
    # segment's capacity, the fold's masters and the quality figures
    plans = []
    for i in range(n_inst):
        balance(i)
        host = buf.plans.cpu().numpy()
        plans.append([ctx.decode_plan(host[l]) for l in range(L)])
    first = plans[0][0]
    P1 = w.M + w.S
    r_max = int(np.argmax(first["rank_after"]))
    seg = (r_max * P1, (r_max + 1) * P1)
    seg_rows = [int(p[0]["phys_off"][seg[1]] - p[0]["phys_off"][seg[0]]) for p in plans]
    out = torch.empty((max(seg_rows), w.H), dtype=torch.int16, device=dev)
    # fold unit: the redundant slots of the rank with the most filled slots
    # (lowest such rank) in the first plan.  Every expert those slots hold in
    # any instance gets a master buffer; the first plan's come from the seeded
    # generator (the oracle folds those), the others copy the first one.
    filled = (first["slot_expert"].reshape(w.R, w.S) >= 0).sum(axis=1)
    r_fold = int(np.argmax(filled))
    slots = (r_fold * w.S, (r_fold + 1) * w.S)
    held = [p[0]["slot_expert"][slots[0]:slots[1]] for p in plans]
    first_experts = sorted({int(e) for e in held[0] if e >= 0})
    all_experts = sorted({int(e) for h in held for e in h if e >= 0})
    masters_h = W.grads(w, max(1, len(first_experts)), stream=1)
    reps_h = W.grads(w, w.S, stream=2)
    d_m = {e: torch.from_numpy(masters_h[i]).to(dev) for i, e in enumerate(first_experts)}
    for e in all_experts:
        if e not in d_m:
            d_m[e] = d_m[first_experts[0]].clone()
    d_r = torch.from_numpy(reps_h).to(dev)
    table = [0] * w.E
    for e, t in d_m.items():
        table[e] = t.data_ptr()
    d_ptrs = torch.tensor(table, dtype=torch.int64, device=dev)
    n_fold_slots = [int((h >= 0).sum()) for h in held]
    n_fold_experts = [len({int(e) for e in h if e >= 0}) for h in held]
    scratch = torch.empty(FLUSH_MIB << 20, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def permute():
        U.ultraep_permute(ctx, buf.plans[0], buf.inv[0], w.k, d_hid, seg[0], seg[1], out)

    def fold():
        U.ultraep_fold_grads(ctx, buf.plans[0], d_ptrs, d_r, w.numel, slots[0], slots[1])

    def step(i, ev=None):
        if ev is not None:
            ev[0].record(stream)
        balance(i)
        if ev is not None:
            ev[1].record(stream)
        permute()
        if ev is not None:
            ev[2].record(stream)
        fold()
        if ev is not None:
            ev[3].record(stream)

    # ---- timed steps: K steps, synchronised on both sides
    for s in range(args.warmup):
        step(s % n_inst)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(s % n_inst, events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps

    def ev_ms(evs, a, b):
        return np.array([e[a].elapsed_time(e[b]) for e in evs])

    t_bal, t_perm, t_fold = ev_ms(events, 0, 1), ev_ms(events, 1, 2), ev_ms(events, 2, 3)
    step_insts = [s % n_inst for s in range(args.steps)]

    # ---- cold and warm repetitions, outside the timed steps
    def timed(fn, reps, flush):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for r in range(reps):
            if flush:
                scratch.fill_(r & 0xFF)
            evs[r][0].record(stream)
            fn(r)
            evs[r][1].record(stream)
        torch.cuda.synchronize()
        return ev_ms(evs, 0, 1)

    bal_cold = timed(lambda r: balance(r % n_inst), n_inst if args.config == 4 else args.cold_reps, True)
    bal_warm = timed(lambda r: balance(0), args.cold_reps, False)
    perm_cold = timed(lambda r: permute(), args.cold_reps, True)
    fold_cold = timed(lambda r: fold(), args.cold_reps, True)

    # ---- the pages' default knobs ([README] "Replication planning": the
    # locality-aware quota decomposition and the reroute interleave on, and a
    # minimum of 1024 pairs per replica): the same balance call on the same
    # inputs, timed cold and warm, with its plan quality and dispatch traffic
    pdef = None
    if not args.no_pages_defaults:
        ctx_p = U.ultraep_create(w.E, w.R, w.S, w.D, threshold=thr, reroute_mode=U.REROUTE_INTERLEAVE,
                                 min_tokens=1024)
        buf_p = U.Buffers(ctx_p, L, w.T, w.k, dev)

        def balance_p(i):
            U.ultraep_balance(ctx_p, d_idx[i], w.T, w.k, buf_p.workspace, buf_p.plans, buf_p.phys_idx,
                              buf_p.pos, topk_w=d_w[i], inv=buf_p.inv, w_perm=buf_p.w_perm, L=L)

        plans_p = []
        for i in range(n_inst):
            balance_p(i)
            host = buf_p.plans.cpu().numpy()
            plans_p.append([ctx_p.decode_plan(host[l]) for l in range(L)])
        p_cold = timed(lambda r: balance_p(r % n_inst), n_inst if args.config == 4 else args.cold_reps, True)
        p_warm = timed(lambda r: balance_p(0), args.cold_reps, False)
        balance_p(0)
        torch.cuda.synchronize()
        pdef = {"reroute_mode": U.REROUTE_INTERLEAVE, "min_tokens_per_replica": 1024,
                "threshold": f"{thr[0]}/{thr[1]}",
                "balance_reroute_us_per_layer": float(np.mean(p_cold)) * 1e3 / L,
                "balance_reroute_us_per_layer_warm": float(np.mean(p_warm)) * 1e3 / L,
                "cold_distribution_us": dist_us(p_cold, L)}
        pdef.update(quality(ctx_p, [p[l] for p in plans_p for l in range(L)], w))
        pdef["dispatch_traffic"] = dispatch_traffic(buf_p.phys_idx[0].cpu().numpy(), w)
        del buf_p

    # ---- replica-lean planning (an option: the greedy without its chain
    # step), at the pages' minimum of 1024 pairs per replica: the balance
    # timed cold, its plan quality, and below the weight_sync of its slots
    lean = None
    buf_l = None
    if not args.no_pages_defaults:
        ctx_l = U.ultraep_create(w.E, w.R, w.S, w.D, threshold=thr, min_tokens=1024, replica_lean=True)
        buf_l = U.Buffers(ctx_l, L, w.T, w.k, dev)

        def balance_l(i):
            U.ultraep_balance(ctx_l, d_idx[i], w.T, w.k, buf_l.workspace, buf_l.plans, buf_l.phys_idx,
                              buf_l.pos, topk_w=d_w[i], inv=buf_l.inv, w_perm=buf_l.w_perm, L=L)

        plans_l = []
        for i in range(n_inst):
            balance_l(i)
            host = buf_l.plans.cpu().numpy()
            plans_l.append([ctx_l.decode_plan(host[l]) for l in range(L)])
        l_cold = timed(lambda r: balance_l(r % n_inst), n_inst if args.config == 4 else args.cold_reps, True)
        balance_l(0)
        torch.cuda.synchronize()
        lean = {"replica_lean": True, "min_tokens_per_replica": 1024, "reroute_mode": 0,
                "balance_reroute_us_per_layer": float(np.mean(l_cold)) * 1e3 / L,
                "cold_distribution_us": dist_us(l_cold, L)}
        lean.update(quality(ctx_l, [p[l] for p in plans_l for l in range(L)], w))

    # ---- combine and its backward (after the experts; not part of the step):
    # the tokens of the permuted rank against the whole layout of the first
    # layer, expert outputs and output gradients drawn on the GPU
    comb = None
    if not args.no_combine:
        total0 = int(first["total"])
        gen = torch.Generator(device=dev).manual_seed(7)
        x_rows = torch.randn((total0, w.H), generator=gen, device=dev, dtype=torch.bfloat16).view(torch.int16)
        g_rows = torch.empty_like(x_rows)
        g0c, g1c = r_max * w.T, (r_max + 1) * w.T
        dy = torch.randn((w.T, w.H), generator=gen, device=dev, dtype=torch.bfloat16).view(torch.int16)
        y = torch.empty((w.T, w.H), dtype=torch.int16, device=dev)
        gw = torch.empty((w.T, w.k), dtype=torch.float32, device=dev)
        pos0, w0 = buf.pos[0], d_w[0].reshape(-1)
        balance(0)

        def comb_fwd(r):
            U.ultraep_combine(ctx, pos0, w0, w.k, x_rows, g0c, g1c, y)

        def comb_bwd(r):
            U.ultraep_combine_backward(ctx, pos0, w0, w.k, x_rows, dy, g0c, g1c, g_rows, gw)

        for _ in range(2):
            comb_fwd(0)
            comb_bwd(0)
        t_cf = timed(comb_fwd, args.cold_reps, True)
        t_cb = timed(comb_bwd, args.cold_reps, True)
        ctok = g1c - g0c
        cf_bytes = ctok * (w.k * 2 * w.H + 2 * w.H + w.k * 8)           # rows, out, pos + w
        cb_bytes = ctok * (2 * w.H + 2 * w.k * 2 * w.H + w.k * 12)      # dy, rows r + w, pos + w + dw
        comb = {"tokens": f"rank {r_max} ({ctok} tokens x {w.k} rows of the first layer)",
                "combine_us": float(np.mean(t_cf)) * 1e3,
                "combine_GBps": gbps_fn(cf_bytes, float(np.mean(t_cf))),
                "combine_backward_us": float(np.mean(t_cb)) * 1e3,
                "combine_backward_GBps": gbps_fn(cb_bytes, float(np.mean(t_cb))),
                "combine_bytes": cf_bytes, "combine_backward_bytes": cb_bytes,
                "cold_distribution_us": {"combine": dist_us(t_cf), "combine_backward": dist_us(t_cb)}}
        comb["combine_frac_of_peak"] = comb["combine_GBps"] / HBM_PEAK_GBPS
        comb["combine_backward_frac_of_peak"] = comb["combine_backward_GBps"] / HBM_PEAK_GBPS
        del x_rows, g_rows, dy, y, gw

    # ---- weight_sync: master fc1 / fc2 bf16 weights into the replica slots
    # of the first layer's plan: the fold rank's slots (one GPU's share) and
    # every slot of the group, direct and with the adaptive relay plan
    wsync = None
    if not args.no_weight_sync and w.ffn > 0:
        balance(0)
        numels = (2 * w.H * w.ffn, w.H * w.ffn)
        gen = torch.Generator(device=dev).manual_seed(11)
        mast = [torch.randint(-32768, 32767, (w.E, n), generator=gen, dtype=torch.int16, device=dev)
                for n in numels]
        ptrs = [torch.tensor([m[e].data_ptr() for e in range(w.E)], dtype=torch.int64, device=dev)
                for m in mast]
        nslot = w.R * w.S
        reps_w = [torch.empty((nslot, n), dtype=torch.int16, device=dev) for n in numels]
        relay = torch.empty((2, nslot), dtype=torch.int32, device=dev)
        U.ultraep_weight_sync_plan(ctx, buf.plans[0], relay)
        slot_e = first["slot_expert"]

        def ws(s0, s1, rl):
            for q in range(2):
                U.ultraep_weight_sync(ctx, buf.plans[0], ptrs[q], reps_w[q][s0:s1] if rl is None else reps_w[q],
                                      numels[q], s0, s1, relay=rl)

        def ws_bytes(s0, s1):
            held = [int(e) for e in slot_e[s0:s1] if e >= 0]
            return sum(n * 2 * (len(held) + len(set(held))) for n in numels)

        for _ in range(2):
            ws(slots[0], slots[1], None)
            ws(0, nslot, None)
            ws(0, nslot, relay)
        t_rank = timed(lambda r: ws(slots[0], slots[1], None), args.cold_reps, True)
        t_all = timed(lambda r: ws(0, nslot, None), args.cold_reps, True)
        t_rel = timed(lambda r: ws(0, nslot, relay), args.cold_reps, True)
        if lean is not None:
            # every filled slot of the lean plan (fewer replicas: fewer copies)
            def ws_lean(r):
                for q in range(2):
                    U.ultraep_weight_sync(ctx_l, buf_l.plans[0], ptrs[q], reps_w[q], numels[q], 0, nslot)
            ws_lean(0)
            t_lean = timed(ws_lean, args.cold_reps, True)
            lean_e = [int(e) for e in plans_l[0][0]["slot_expert"] if e >= 0]
            lean_b = sum(n * 2 * (len(lean_e) + len(set(lean_e))) for n in numels)
            lean["weight_sync_all_slots_us"] = float(np.mean(t_lean)) * 1e3
            lean["weight_sync_all_slots_bytes"] = lean_b
            lean["weight_sync_all_slots_GBps"] = gbps_fn(lean_b, float(np.mean(t_lean)))
        rel = relay.cpu().numpy()
        b_rank, b_all = ws_bytes(slots[0], slots[1]), ws_bytes(0, nslot)
        wsync = {"expert_weights": f"fc1 2x{w.H}x{w.ffn} + fc2 {w.H}x{w.ffn} bf16 per expert",
                 "rank_slots_us": float(np.mean(t_rank)) * 1e3,
                 "rank_slots_GBps": gbps_fn(b_rank, float(np.mean(t_rank))),
                 "all_slots_us": float(np.mean(t_all)) * 1e3,
                 "all_slots_GBps": gbps_fn(b_all, float(np.mean(t_all))),
                 "all_slots_relay_us": float(np.mean(t_rel)) * 1e3,
                 "relayed_slots": int((rel[1] == 2).sum()), "filled_slots": int((rel[1] > 0).sum()),
                 "rank_slots_bytes": b_rank, "all_slots_bytes": b_all,
                 "cold_distribution_us": {"rank_slots": dist_us(t_rank), "all_slots": dist_us(t_all),
                                          "all_slots_relay": dist_us(t_rel)}}
        wsync["all_slots_frac_of_peak"] = wsync["all_slots_GBps"] / HBM_PEAK_GBPS
        wsync["rank_slots_frac_of_peak"] = wsync["rank_slots_GBps"] / HBM_PEAK_GBPS
        del mast, ptrs, reps_w, relay
    del scratch, buf_l

    # ---- algorithmic bytes
    row_bytes = 2 * 2 * w.H + 4                            # read row, write row, read inv
    fold_bytes = [(n_fold_experts[i] * 2 + n_fold_slots[i]) * w.numel * 4 for i in range(n_inst)]
    bal_bytes = L * w.N * (4 + 4 + 4 + 16)   # idx read twice, w read; phys, pos, inv, w_perm written
    gbps = lambda b, ms: b / (ms * 1e-3) / 1e9             # noqa: E731

    perm_b = np.array([seg_rows[i] * row_bytes for i in step_insts], dtype=np.float64)
    fold_b = np.array([fold_bytes[i] for i in step_insts], dtype=np.float64)
    perm_gbps = float(perm_b.sum() / (t_perm.sum() * 1e-3) / 1e9)
    fold_gbps = float(fold_b.sum() / (t_fold.sum() * 1e-3) / 1e9)
    copy_rate = device_copy_rate(torch, dev, args.copy_mib) if args.copy_mib > 0 else None
    bal_cold_us = float(np.mean(bal_cold)) * 1e3 / L
    result = {
        "metric": METRIC,
        "value": L * w.N / (ms_step * 1e-3),
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32+bf16+f32",
        "data": "synthetic",
        "config": {"workload": w.name, "E": w.E, "R": w.R, "S": w.S, "D": w.D, "top_k": w.k,
                   "tokens_per_rank": w.T, "hidden": w.H, "layers_per_step": L, "instances": n_inst,
                   "permute_segment": f"rank {r_max} of the first layer ({seg_rows[0]} rows)",
                   "fold": f"rank {r_fold} slots {slots[0]}..{slots[1] - 1} ({n_fold_slots[0]} filled), "
                           f"{w.fold_rows}x{w.fold_cols} fp32 per slot",
                   "parallelism": "1 GPU; EP group simulated as logical ranks"},
        "balance_reroute_us_per_layer": bal_cold_us,
        "balance_reroute_us_per_layer_warm": float(np.mean(bal_warm)) * 1e3 / L,
        "balance_reroute_us_per_layer_in_step": float(np.mean(t_bal)) * 1e3 / L,
        "routed_pairs_per_s_balance_layout": w.N / (bal_cold_us * 1e-6),
        "balance_layout_GBps": gbps(bal_bytes, float(np.mean(bal_cold))),
        "permute_us": float(np.mean(t_perm)) * 1e3,
        "permute_us_cold": float(np.mean(perm_cold)) * 1e3,
        "permute_GBps": perm_gbps,
        "permute_frac_of_peak": perm_gbps / HBM_PEAK_GBPS,
        "fold_us": float(np.mean(t_fold)) * 1e3,
        "fold_us_cold": float(np.mean(fold_cold)) * 1e3,
        "fold_GBps": fold_gbps,
        "fold_GBps_cold": gbps(fold_bytes[0], float(np.mean(fold_cold))),
        "fold_frac_of_peak": fold_gbps / HBM_PEAK_GBPS,
        "device_copy_GBps": copy_rate,
        "cold_distribution_us": {"balance_per_layer": dist_us(bal_cold, L), "permute": dist_us(perm_cold),
                                 "fold": dist_us(fold_cold)},
        "roofline": {"bound": "hbm", "kernel": "permute_kernel", "achieved": perm_gbps,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": perm_gbps / HBM_PEAK_GBPS,
                     "traffic": recorded_traffic(args.config),
                     "algorithmic_bytes_per_launch": float(perm_b.mean())},
        "host": host_info(),
    }
    if args.config == 4:
        per = bal_cold * 1e3
        result["balance_reroute_us_per_layer_cold_median_p99"] = [float(np.median(per)),
                                                                  float(np.percentile(per, 99))]
    if comb is not None:
        result["combine"] = comb
    if wsync is not None:
        result["weight_sync"] = wsync
    result.update(quality(ctx, [p[l] for p in plans for l in range(L)], w))
    result["threshold"] = f"{thr[0]}/{thr[1]}"
    result["reroute_mode"] = args.reroute_mode
    result["min_tokens_per_replica"] = args.min_tokens
    balance(0)
    torch.cuda.synchronize()
    result["dispatch_traffic"] = dispatch_traffic(buf.phys_idx[0].cpu().numpy(), w)
    if args.config == 4 and n_inst > 1:
        stale = [stale_plan_imbalance(plans[i - 1][0], plans[i][0], w) for i in range(1, n_inst)]
        result["stale_plan_imbalance_median_max"] = [float(np.median(stale)), float(np.max(stale))]
    if pdef is not None:
        result["pages_defaults"] = pdef
    if lean is not None:
        result["replica_lean"] = lean
    # per-(layer, microbatch) loads before and after balancing (the pages'
    # load profiler records the same per microbatch: [README] "Load profiler
    # and viewer"): max/mean per instance in the line, every rank and expert
    # load in --load-trace
    flat = [(insts[i * L + l], plans[i][l]) for i in range(n_inst) for l in range(L)]
    if len(flat) > 1:
        result["load_trace"] = [
            {"layer": lm[0], "mb": lm[1], "before": float(p["rank_before"].max() * w.R / max(1, p["total"])),
             "after": float(p["rank_after"].max() * w.R / max(1, p["total"])), "replicas": p["replicas"]}
            for lm, p in flat]
    if args.load_trace:
        with open(args.load_trace, "w") as f:
            for lm, p in flat:
                f.write(json.dumps({"layer": lm[0], "mb": lm[1], "expert_load": p["counts"].tolist(),
                                    "rank_before": p["rank_before"].tolist(),
                                    "rank_after": p["rank_after"].tolist(),
                                    "phys_load": p["phys_load"].tolist()}) + "\n")
    if args.config in PAGES_TABLE:
        result["pages_table_context"] = PAGES_TABLE[args.config]
    if not args.no_cpu_baseline:
        masters = {e: masters_h[i] for i, e in enumerate(first_experts)}
        result["cpu_baseline"] = cpu_baseline(w, L, routes, hidden, seg, masters, reps_h, slots,
                                              args.cpu_seconds, thr, args.min_tokens)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
