"""Benchmark of the exact-load rebalancing hot path on one MI355X.

One step = one pass of the whole path over one layer of synthetic routing:
  ultraep_balance          count + quota plan + reroute (phys_idx, pos) and the
                           dispatch layout (inverse index, permuted weights)
  ultraep_permute          bf16 rows of the most loaded rank's receive segment
  ultraep_fold_grads       that rank's redundant-slot gradients into masters
All inputs are resident in HBM before the timed region.  Each call is timed
with HIP events on the stream it runs on; the permute kernel is the dominant
one and its roofline is reported against the 8 TB/s HBM peak.

The CPU oracle is timed on the host on the same workload (cpu_baseline).
Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "balance+reroute µs/layer; routed pairs/s; permute/fold HBM GB/s vs peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, help="workload id (2 = single layer, the headline)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget for the oracle timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-mib", type=int, default=1024,
                    help="size of the device-to-device copy that measures the HBM copy ceiling")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "permute_kernel_traffic_single_layer.md")
KERNEL_SOURCE = os.path.join(ROOT, "moe_expert_load_ultraep_amd", "csrc", "ultraep_kernels.hip")


def permute_source_sha256():
    """Hash of the permute kernel's source (its comment block, constants,
    helpers and body), so recorded counters go stale only when it changes."""
    import hashlib
    text = open(KERNEL_SOURCE).read()
    start = text.index("// One wave per output row")
    end = text.index("\n}\n", text.index("void permute_kernel(", start)) + 3
    return hashlib.sha256(text[start:end].encode()).hexdigest()


def recorded_traffic():
    """HBM bytes per permute launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary, or None when the kernel source changed since."""
    import hashlib
    import re
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


def copy_ceiling(torch, dev, mib):
    """Device-to-device copy rate (read + write bytes / time): the practical
    HBM ceiling a streaming kernel is compared with."""
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    reps = 10
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(reps):
        b.copy_(a)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    del a, b
    return 2 * n / (ms * 1e-3) / 1e9


def cpu_baseline(w, idx, wt, hidden, seg, masters, reps, slots, budget_s):
    """Time the oracle (unchanged) on the host: the same step on the same arrays."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(1)
    except Exception:  # pragma: no cover
        limiter = None
    p_begin, p_end = seg
    s0, s1 = slots
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        pl, phys, pos = O.balance(idx, w.E, w.R, w.S, w.D)
        inv, wp = O.layout(pos, wt, pl.total)
        O.permute(hidden, inv, w.k, pl, p_begin, p_end)
        O.fold(masters, reps, pl, s0, s1)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= 20:
            break
    if limiter is not None:
        limiter.unregister()
    t = float(np.median(times))
    return {"value": w.N / t, "unit": "pairs/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(times)} full steps of the same workload (count, plan, reroute, layout, "
                      f"permute of one rank segment, fold of one rank's slots), median "
                      f"{t * 1e3:.0f} ms/step, NumPy single thread"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the EP group is simulated as logical ranks on a "
              "single MI355X, so --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import moe_expert_load_ultraep_amd as U
    import workload as W

    if not os.path.exists(U.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    dev = torch.device("cuda:0")
    w = W.CONFIGS[args.config]
    L = 1

    # ---- inputs (host generation is not timed) -------------------------
    idx, wt, _ = W.routing(w)
    hidden = W.hidden(w, workers=16)
    ctx = U.ultraep_create(w.E, w.R, w.S, w.D)
    buf = U.Buffers(ctx, L, w.T, w.k, dev)
    d_idx = torch.from_numpy(idx).to(dev)
    d_w = torch.from_numpy(wt).to(dev)
    d_hid = torch.from_numpy(hidden.view(np.int16)).to(dev)

    # one balance to size the permute / fold targets (outside the timing)
    U.ultraep_balance(ctx, d_idx, w.T, w.k, buf.workspace, buf.plans, buf.phys_idx, buf.pos, L=L)
    torch.cuda.synchronize()
    plan = ctx.decode_plan(buf.plans[0].cpu().numpy())
    P1 = w.M + w.S
    r_max = int(np.argmax(plan["rank_after"]))
    seg = (r_max * P1, (r_max + 1) * P1)
    seg_rows = int(plan["phys_off"][seg[1]] - plan["phys_off"][seg[0]])
    out = torch.empty((seg_rows, w.H), dtype=torch.int16, device=dev)
    # fold unit: the redundant slots of the rank with the most filled slots
    # (lowest such rank); each filled slot is one replica to fold
    filled = (plan["slot_expert"].reshape(w.R, w.S) >= 0).sum(axis=1)
    r_fold = int(np.argmax(filled))
    slots = (r_fold * w.S, (r_fold + 1) * w.S)
    fold_experts = sorted({int(e) for e in plan["slot_expert"][slots[0]:slots[1]] if e >= 0})
    n_fold_slots = int(filled[r_fold])
    masters_h = W.grads(w, max(1, len(fold_experts)), stream=1)
    reps_h = W.grads(w, w.S, stream=2)
    d_m = torch.from_numpy(masters_h).to(dev)
    d_r = torch.from_numpy(reps_h).to(dev)
    table = [0] * w.E
    for i, e in enumerate(fold_experts):
        table[e] = d_m[i].data_ptr()
    d_ptrs = torch.tensor(table, dtype=torch.int64, device=dev)

    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        U.ultraep_balance(ctx, d_idx, w.T, w.k, buf.workspace, buf.plans, buf.phys_idx, buf.pos,
                          topk_w=d_w, inv=buf.inv, w_perm=buf.w_perm, L=L)
        if ev is not None:
            ev[1].record(stream)
            ev[2].record(stream)
        U.ultraep_permute(ctx, buf.plans[0], buf.inv[0], w.k, d_hid, seg[0], seg[1], out)
        if ev is not None:
            ev[3].record(stream)
        U.ultraep_fold_grads(ctx, buf.plans[0], d_ptrs, d_r, w.numel, slots[0], slots[1])
        if ev is not None:
            ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps

    def avg_ms(a, b):
        return float(np.mean([e[a].elapsed_time(e[b]) for e in events]))

    t_bal, t_lay, t_perm, t_fold = avg_ms(0, 1), avg_ms(1, 2), avg_ms(2, 3), avg_ms(3, 4)

    # algorithmic bytes
    perm_bytes = seg_rows * (2 * 2 * w.H + 4)                       # read row, write row, read inv
    fold_bytes = (len(fold_experts) * 2 + n_fold_slots) * w.numel * 4  # masters r+w, replicas r
    bal_bytes = w.N * (4 + 4 + 4 + 16)   # idx read twice, w read; phys, pos, inv, w_perm written
    gbps = lambda b, ms: b / (ms * 1e-3) / 1e9                       # noqa: E731

    total = plan["total"]
    ceiling = copy_ceiling(torch, dev, args.copy_mib) if args.copy_mib > 0 else None
    traffic = recorded_traffic()
    result = {
        "metric": METRIC,
        "value": w.N / (ms_step * 1e-3),
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
                   "tokens_per_rank": w.T, "hidden": w.H, "layers_per_step": L,
                   "permute_segment": f"rank {r_max} ({seg_rows} rows)",
                   "fold": f"rank {r_fold} slots {slots[0]}..{slots[1] - 1} ({n_fold_slots} filled), "
                           f"{w.fold_rows}x{w.fold_cols} fp32 per slot",
                   "parallelism": "1 GPU; EP group simulated as logical ranks"},
        "balance_reroute_us_per_layer": (t_bal + t_lay) * 1e3 / L,
        "routed_pairs_per_s_balance_layout": w.N / ((t_bal + t_lay) * 1e-3),
        "balance_layout_GBps": gbps(bal_bytes, t_bal + t_lay),
        "permute_us": t_perm * 1e3,
        "permute_GBps": gbps(perm_bytes, t_perm),
        "permute_frac_of_peak": gbps(perm_bytes, t_perm) / HBM_PEAK_GBPS,
        "fold_us": t_fold * 1e3,
        "fold_GBps": gbps(fold_bytes, t_fold),
        "fold_frac_of_peak": gbps(fold_bytes, t_fold) / HBM_PEAK_GBPS,
        "imbalance_before": plan["rank_before"].max() * w.R / total,
        "imbalance_after": plan["rank_after"].max() * w.R / total,
        "replicas": plan["replicas"],
        "hbm_copy_ceiling_GBps": ceiling,
        "permute_frac_of_copy_ceiling": gbps(perm_bytes, t_perm) / ceiling if ceiling else None,
        "roofline": {"bound": "hbm", "kernel": "permute_kernel", "achieved": gbps(perm_bytes, t_perm),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps(perm_bytes, t_perm) / HBM_PEAK_GBPS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": perm_bytes},
    }
    if not args.no_cpu_baseline:
        masters = {e: masters_h[i] for i, e in enumerate(fold_experts)}
        result["cpu_baseline"] = cpu_baseline(w, idx, wt, hidden, seg, masters, reps_h, slots,
                                              args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
