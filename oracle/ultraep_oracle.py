"""Plain CPU oracle for UltraEP's per-layer exact-load rebalancing path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test suite, the package smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code, table or helper with
the HIP library; the two meet only through the seeded inputs of ``workload``.

Every function is the slow, obvious definition of one step, written with
NumPy primitives (bincount, stable argsort, fancy indexing, fp64 sums) and
pure-Python loops over the small per-expert / per-rank state.

Sources (web pages on UltraEP; cited by title and section):
  [README]  "UltraEP" project README (mirror kd.iw.mk/studio-dots-ai/UltraEP)
  [NEWS]    "Xiaohongshu's UltraEP Balances MoE Experts in 300 µs, Reaching
            94.3% of Ideal" (news.hamidun.com, English)
  [WEEKLY]  "UltraEP: Real-Time Load Balancing for Large-Scale MoE Training
            and Inference" (aikit weekly article)

Shapes and notation (readings where the pages are silent are marked R#; the
full list is kept with the design notes):
  R logical EP ranks, T tokens per rank (R1), token g = r*T + t, top-k
  routing ``idx[R*T, k]``; pair n = g*k + j; N = R*T*k.
  E experts, M = E/R masters per rank, expert e homed on rank e // M (R2).
  S redundant slots per rank ([README] Interface / Initialization: the same
  number of redundant-expert slots on every rank).  Domain size D: rank r is
  in domain r // D (R3); replicas stay inside the domain ([README] principles,
  "Topology-aware replication").
  Load = number of (token, k) pairs (R4).
  Physical experts P = R*(M+S), rank-major: p = r*(M+S) + j; j < M is the
  master of expert r*M + j, j >= M is redundant slot j-M of rank r (R12).
  Redundant slot id s = r*S + j-M.

Parity: count, reroute, layout, permute and fold are pinned by closed forms
and brute force in the tests.  The plan is pinned by invariants, special
cases with closed-form answers, hand-worked examples, the pages' 1.01-1.04
post-balance band and a brute-force optimum on tiny shapes; its tie-break
rules are this build's own reading (the pages give no algorithm), so the
exact choice among equally valid plans is parity unpinned by the pages.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np


# ---------------------------------------------------------------------------
# count
# ---------------------------------------------------------------------------
def count(topk_idx: np.ndarray, E: int) -> Tuple[np.ndarray, int]:
    """Exact number of (token, k) pairs routed to each expert.

    [WEEKLY] "Technical Details": each expert's load is computed from the
    exact routing before the forward pass; [README] intro and Interface /
    "Forward and backward": ``update_placement`` plans from the exact
    post-gating routing map.  Ids outside [0, E) are dropped pairs (R13).
    """
    ids = np.asarray(topk_idx).reshape(-1).astype(np.int64)
    valid = (ids >= 0) & (ids < E)
    c = np.bincount(ids[valid], minlength=E).astype(np.int64)
    return c, int(ids.size - valid.sum())


# ---------------------------------------------------------------------------
# plan
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class Plan:
    E: int
    R: int
    S: int
    D: int
    M: int
    P: int
    c: np.ndarray                 # [E] pairs per expert
    total: int                    # valid pairs
    dropped: int
    rank_before: np.ndarray       # [R] home load H[r]
    Q_lb: int
    Q_max: int
    tol: int
    floor: int                    # max over domains of ceil(domain load / D)
    grid_index: int
    Q_star: int
    slot_expert: np.ndarray       # [R*S] expert hosted in redundant slot, -1 empty
    slot_quota: np.ndarray        # [R*S] pairs served by that slot
    master_quota: np.ndarray      # [E]
    phys_load: np.ndarray         # [P]
    phys_off: np.ndarray          # [P+1] exclusive prefix of phys_load
    inst_ptr: np.ndarray          # [E+1] CSR of each expert's instances
    inst_phys: np.ndarray         # [E + R*S] physical id of each instance (ascending per expert)
    inst_end: np.ndarray          # [E + R*S] cumulative ordinal end of each instance
    rank_after: np.ndarray        # [R]

    @property
    def n_replicas(self) -> int:
        return int((self.slot_expert >= 0).sum())

    def instances(self, e: int) -> List[Tuple[int, int, int]]:
        """(phys, start, end) ordinal ranges of expert e, in instance order."""
        out, start = [], 0
        for i in range(self.inst_ptr[e], self.inst_ptr[e + 1]):
            out.append((int(self.inst_phys[i]), start, int(self.inst_end[i])))
            start = int(self.inst_end[i])
        return out

    def imbalance_before(self) -> float:
        return 1.0 if self.total == 0 else float(self.rank_before.max() * self.R / self.total)

    def imbalance_after(self) -> float:
        return 1.0 if self.total == 0 else float(self.rank_after.max() * self.R / self.total)


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def quota_grid(total: int, H: List[int], R: int, D: int, eps_num: int, eps_den: int,
               thr_num: int = 1, thr_den: int = 1):
    """The quota values a plan may settle on, in the order they are tried.

    [README] "Performance Tuning / Replication planning": the balancing ratio
    is searched with an early-stop target of 1.0 and a numerical tolerance
    eps (default 0.01).  Read as an integer grid (R6): start at the lowest
    quota any placement could reach -- the mean rank load, or the mean rank
    load of the most loaded domain, since replicas cannot leave their domain
    ([README] principles, "Topology-aware replication"; R7) -- and step by
    eps * mean until the no-replication load max H is reached; that last
    quota is always feasible.  (The domain term is never below the global
    mean, so it alone sets the start; the mean is kept for readability.)

    The early-stop target (default 1.0) is read as the lowest max/mean the
    search aims at: with a target thr = thr_num / thr_den the grid starts at
    ceil(thr * total / R) instead of the mean, so a plan stops replicating
    once every rank is within thr of the mean (R26).
    """
    Q_mean = _ceil_div(total * thr_num, R * thr_den)
    floor = max(_ceil_div(sum(H[d * D:(d + 1) * D]), D) for d in range(R // D))
    Q_max = max(H)
    Q_lb = min(max(Q_mean, floor), Q_max)   # the clamp only acts for a target above 1
    tol = max(1, (total * eps_num) // (R * eps_den))
    grid = []
    q = Q_lb
    while q < Q_max:
        grid.append(q)
        q += tol
    grid.append(Q_max)
    return grid, Q_lb, Q_max, tol, floor


def feasible(c: List[int], Q: int, E: int, R: int, S: int, D: int,
             allow_zero_master: bool = False, min_tokens: int = 1,
             lean: bool = False) -> Optional[Dict[int, List[Tuple[int, int]]]]:
    """Try to bring every rank's load to at most Q with <= S replicas per rank.

    Returns, per rank, the replicas it hosts as (expert, quota) in arrival
    order (arrival index = redundant slot index), or None if this greedy
    cannot reach Q.  The pages name a quota-driven scheduler ([NEWS] "How
    balancing in 300 microseconds works") that replicates hot experts onto
    idle devices and merges cold ones ([WEEKLY] "Technical Details") but give
    no procedure; this greedy is this build's reading (R8-R10):

    1. Shedding.  A rank above Q gives up its excess from its hottest experts
       first (pairs desc, id asc).  A master keeps at least one pair unless
       zero-quota masters are allowed ([README] "Replication planning").
       Each shed amount is a queued piece; ``room[e]`` is how much more of e
       its master could still give up.
    2. Placement, per domain.  Receivers have ``spare = Q - load`` and S free
       slots.  Repeatedly take the largest piece (ties: lower expert id):
       a. if a receiver can take it whole, the tightest one does (smallest
          spare, then lowest rank);
       b. else, if some other shedding rank could host it, pick the largest
          queued piece q whose home could (ties: lower id): first fill the
          roomiest receiver, then swap the rest onto q's home rank, which
          sheds that much more of q's expert (its load is unchanged);
       c. else fill the roomiest receiver and queue the remainder;
       d. else fail.
       Every step fills one slot, so a domain takes at most D*S steps.

    Minimum tokens per replica m ([README] "Replication planning": a replica
    is allocated at least a minimal load; R34).  Every amount the greedy
    moves is at least m: a shed piece below m is raised to m when its expert
    has room for m (the rank then ends below Q) and dropped when it has not;
    a receiver takes part of a piece only with a spare of at least m, and a
    queued piece serves as chain donor only with room for m more; a partial
    placement leaves at least m queued (the roomiest receiver takes
    min(spare, a - m), skipped in a chain when that is below m; the donor's
    part is cut so the rest is 0 or at least m); a placement below m fails
    the probe.  With m = 1 every rule is the plain greedy's.

    Replica-lean planning (``lean``, R35): step b is left out, so only ranks
    with spare take replicas; a piece that fits no receiver goes in part to
    the roomiest one (step c).  Each chain splits a piece over two ranks and
    grows the donor's piece; without them the large domains need about a
    third fewer replicas at the same quota, while small ones may need a
    higher quota.
    """
    m = max(1, int(min_tokens))
    M = E // R
    H = [sum(c[r * M:(r + 1) * M]) for r in range(R)]

    def keep(e: int) -> int:
        return 1 if (c[e] > 0 and not allow_zero_master) else 0

    hosted: Dict[int, List[Tuple[int, int]]] = {r: [] for r in range(R)}
    for d in range(R // D):
        ranks = list(range(d * D, (d + 1) * D))
        piece: Dict[int, int] = {}
        room: Dict[int, int] = {}
        for r in ranks:
            X = H[r] - Q
            if X <= 0:
                continue
            for e in sorted(range(r * M, (r + 1) * M), key=lambda f: (-c[f], f)):
                if X <= 0:
                    break
                avail = c[e] - keep(e)
                t = min(X, avail)
                if t < m:                      # a piece is never below the minimum
                    t = m if avail >= m else 0
                if t > 0:
                    piece[e] = t
                    room[e] = avail - t
                    X -= t
            if X > 0:
                return None
        spare = {r: max(0, Q - H[r]) for r in ranks}
        free = {r: S for r in ranks}

        def place(e: int, r: int, x: int) -> None:
            assert x >= m and free[r] > 0
            hosted[r].append((e, x))
            free[r] -= 1

        while piece:
            e = max(piece, key=lambda f: (piece[f], -f))
            a = piece.pop(e)
            home = e // M

            def elig(r: int) -> bool:
                return r != home and free[r] > 0 and all(x != e for x, _ in hosted[r])

            rec = [r for r in ranks if elig(r) and spare[r] >= m]
            fit = [r for r in rec if spare[r] >= a]
            if fit:
                r = min(fit, key=lambda q: (spare[q], q))
                place(e, r, a)
                spare[r] -= a
                continue
            don = [] if lean else [f for f in piece if elig(f // M) and room[f] >= m]
            if don:
                f = max(don, key=lambda g: (piece[g], -g))
                if rec:
                    r2 = max(rec, key=lambda q: (spare[q], -q))
                    assert r2 != f // M
                    x = min(spare[r2], a - m)
                    if x >= m:
                        place(e, r2, x)
                        spare[r2] -= x
                        a -= x
                x = min(a, room[f])
                if 0 < a - x < m:              # what stays queued is at least m
                    x = a - m
                if x < m:
                    return None
                place(e, f // M, x)
                piece[f] += x
                room[f] -= x
                a -= x
                if a > 0:
                    piece[e] = a
            elif rec:
                r = max(rec, key=lambda q: (spare[q], -q))
                x = min(spare[r], a - m)
                if x < m:
                    return None
                place(e, r, x)
                spare[r] -= x
                piece[e] = a - x
            else:
                return None
    return hosted


def plan(c: np.ndarray, E: int, R: int, S: int, D: int, *, dropped: int = 0,
         eps_num: int = 1, eps_den: int = 100, allow_zero_master: bool = False,
         thr_num: int = 1, thr_den: int = 1, min_tokens: int = 1, lean: bool = False) -> Plan:
    """Replication plan from the exact per-expert load ([README] Interface /
    "Forward and backward": ``update_placement``).

    Q* is the first grid quota (see ``quota_grid``) that ``feasible`` reaches.
    Each expert's instances are its master and its replicas, ordered by
    ascending physical id (R10); instance i serves the ordinals
    [start_i, start_i + quota_i) of that expert's pairs, cumulatively.

    [README] "Replication planning": a minimal load is allocated to a
    replica (default 1024 there).  ``feasible`` enforces it inside the greedy
    (R34), so Q* is the first grid quota reachable with every replica at
    ``min_tokens`` pairs or more, and every rank still ends at Q* or below.
    The default 1 changes nothing.

    ``lean`` plans without the greedy's chain step (R35; see ``feasible``).
    """
    if E % R or R % D or S < 0:
        raise ValueError("bad shape")
    M = E // R
    P = R * (M + S)
    c = [int(x) for x in c]
    total = sum(c)
    H = [sum(c[r * M:(r + 1) * M]) for r in range(R)]
    grid, Q_lb, Q_max, tol, floor = quota_grid(total, H, R, D, eps_num, eps_den, thr_num, thr_den)
    for gi, Q in enumerate(grid):
        hosted = feasible(c, Q, E, R, S, D, allow_zero_master, min_tokens, lean)
        if hosted is not None:
            break
    assert hosted is not None, "no replication at Q_max must always be feasible"

    slot_expert = np.full(R * S, -1, dtype=np.int64)
    slot_quota = np.zeros(R * S, dtype=np.int64)
    for r in range(R):
        for s, (e, x) in enumerate(hosted[r]):
            slot_expert[r * S + s] = e
            slot_quota[r * S + s] = x
    master_quota = np.array(c, dtype=np.int64)
    for s in range(R * S):
        if slot_expert[s] >= 0:
            master_quota[slot_expert[s]] -= slot_quota[s]

    phys_load = np.zeros(P, dtype=np.int64)
    for r in range(R):
        for j in range(M):
            phys_load[r * (M + S) + j] = master_quota[r * M + j]
        for j in range(S):
            phys_load[r * (M + S) + M + j] = slot_quota[r * S + j]
    phys_off = np.zeros(P + 1, dtype=np.int64)
    phys_off[1:] = np.cumsum(phys_load)

    inst_ptr = [0]
    inst_phys: List[int] = []
    inst_end: List[int] = []
    for e in range(E):
        home = e // M
        phys = [home * (M + S) + (e % M)]
        for s in range(R * S):
            if slot_expert[s] == e:
                r, j = divmod(s, S)
                phys.append(r * (M + S) + M + j)
        end = 0
        for p in sorted(phys):
            end += int(phys_load[p])
            inst_phys.append(p)
            inst_end.append(end)
        assert end == c[e]
        inst_ptr.append(len(inst_phys))

    rank_after = phys_load.reshape(R, M + S).sum(axis=1)
    return Plan(E=E, R=R, S=S, D=D, M=M, P=P, c=np.array(c, dtype=np.int64), total=total,
                dropped=int(dropped), rank_before=np.array(H, dtype=np.int64), Q_lb=Q_lb,
                Q_max=Q_max, tol=tol, floor=floor, grid_index=gi, Q_star=grid[gi],
                slot_expert=slot_expert, slot_quota=slot_quota, master_quota=master_quota,
                phys_load=phys_load, phys_off=phys_off,
                inst_ptr=np.array(inst_ptr, dtype=np.int64),
                inst_phys=np.array(inst_phys, dtype=np.int64),
                inst_end=np.array(inst_end, dtype=np.int64), rank_after=rank_after)


# ---------------------------------------------------------------------------
# reroute + dispatch layout
# ---------------------------------------------------------------------------
def ordinals(topk_idx: np.ndarray, E: int) -> np.ndarray:
    """o[n] = number of pairs n' < n routed to the same expert (-1 if dropped).

    Read off a stable sort by expert id: within one expert's run the pairs
    keep their order, so a pair's place in the run is its ordinal.
    """
    ids = np.asarray(topk_idx).reshape(-1).astype(np.int64)
    valid = (ids >= 0) & (ids < E)
    key = np.where(valid, ids, E)
    order = np.argsort(key, kind="stable")
    run_start = np.searchsorted(key[order], key[order], side="left")
    o = np.empty(ids.size, dtype=np.int64)
    o[order] = np.arange(ids.size) - run_start
    o[~valid] = -1
    return o


def reroute(topk_idx: np.ndarray, pl: Plan) -> Tuple[np.ndarray, np.ndarray]:
    """Physical expert and dispatch row of every pair.

    [README] Interface / "Forward and backward": ``reroute`` expands the
    logical routing to physical replicas.  Pair n of expert e with ordinal o
    goes to the instance whose range holds o (R11); its row in the
    replica-contiguous layout is ``phys_off[p] + o - start``.  Dropped pairs
    get -1 in both.
    """
    ids = np.asarray(topk_idx).reshape(-1).astype(np.int64)
    o = ordinals(ids, pl.E)
    valid = o >= 0
    # Lay every expert's ordinal range end to end (experts ascending, each
    # expert's instances in instance order); the instance holding a pair is
    # then the first whose cumulative end lies beyond the pair's place.
    expert_base = np.concatenate([[0], np.cumsum(pl.c)])
    inst_expert = np.repeat(np.arange(pl.E), np.diff(pl.inst_ptr))
    inst_gend = expert_base[inst_expert] + pl.inst_end
    inst_start = pl.inst_end - pl.phys_load[pl.inst_phys]
    e = ids[valid]
    i = np.searchsorted(inst_gend, expert_base[e] + o[valid], side="right")
    phys = np.full(ids.size, -1, dtype=np.int64)
    pos = np.full(ids.size, -1, dtype=np.int64)
    phys[valid] = pl.inst_phys[i]
    pos[valid] = pl.phys_off[pl.inst_phys[i]] + o[valid] - inst_start[i]
    return phys, pos


def local_takes(pl: Plan, rank_counts: np.ndarray) -> np.ndarray:
    """Pairs each instance takes from its own rank's pairs of its expert.

    [README] "Replication planning": the locality-aware per-rank quota
    decomposition cuts remote traffic.  Read as (R31): instance i of expert e,
    hosted on rank h_i with quota q_i, first serves min(q_i, pairs of e whose
    token lives on h_i).  rank_counts[r, e] = pairs of e from rank r.
    Returns one value per instance entry (inst_phys order).
    """
    a = np.zeros(len(pl.inst_phys), dtype=np.int64)
    for e in range(pl.E):
        start = 0
        for i in range(pl.inst_ptr[e], pl.inst_ptr[e + 1]):
            q = int(pl.inst_end[i]) - start
            start = int(pl.inst_end[i])
            h = int(pl.inst_phys[i]) // (pl.M + pl.S)
            a[i] = min(q, int(rank_counts[h, e]))
    return a


def reroute_local(topk_idx: np.ndarray, pl: Plan, interleave: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """Physical expert and dispatch row of every pair, locality first.

    [README] "Replication planning": locality-aware per-rank quota
    decomposition to cut remote traffic, and reroute interleave to spread
    the token order over the replicas against congestion in the dispatch
    that follows.  Reading (R31, R32):
      - the pairs of expert e split by the rank of their token into R
        blocks, each in pair order;
      - instance i (host rank h_i, quota q_i) first takes the first a_i =
        min(q_i, |block h_i|) pairs of block h_i (``local_takes``);
      - the remaining pairs of all blocks, in pair order, form e's pool;
        the instances' remaining quotas q_i - a_i take the pool
        contiguously in instance order, or, with interleave, round by
        round: in round t every instance with more than t remaining pairs
        takes the next pool pair, in instance order;
      - instance i's rows hold its local pairs first (in pair order), then
        its pool pairs in pool order.
    The token's rank is n // (N / R): pairs are rank-major.
    """
    ids = np.asarray(topk_idx).reshape(-1).astype(np.int64)
    N = ids.size
    E, R = pl.E, pl.R
    TK = N // R if R else 0
    valid = (ids >= 0) & (ids < E)
    src = np.arange(N) // max(TK, 1)
    rank_counts = np.zeros((R, E), dtype=np.int64)
    np.add.at(rank_counts, (src[valid], ids[valid]), 1)
    a = local_takes(pl, rank_counts)
    phys = np.full(N, -1, dtype=np.int64)
    pos = np.full(N, -1, dtype=np.int64)
    for e in range(E):
        insts = list(range(pl.inst_ptr[e], pl.inst_ptr[e + 1]))
        host = {int(pl.inst_phys[i]) // (pl.M + pl.S): i for i in insts}
        start = 0
        rem = {}
        for i in insts:
            rem[i] = int(pl.inst_end[i]) - start - int(a[i])
            start = int(pl.inst_end[i])
        # the pool's owner sequence
        owner: List[int] = []
        if interleave:
            left = dict(rem)
            while any(left[i] > 0 for i in insts):
                for i in insts:
                    if left[i] > 0:
                        owner.append(i)
                        left[i] -= 1
        else:
            for i in insts:
                owner += [i] * rem[i]
        taken = {i: 0 for i in insts}     # local pairs handed out so far
        pool_seen = {i: 0 for i in insts}  # pool pairs handed out so far
        u = 0
        for n in np.nonzero(ids == e)[0]:
            r = int(src[n])
            i = host.get(r)
            if i is not None and taken[i] < a[i]:
                row = taken[i]
                taken[i] += 1
            else:
                i = owner[u]
                u += 1
                row = int(a[i]) + pool_seen[i]
                pool_seen[i] += 1
            phys[n] = pl.inst_phys[i]
            pos[n] = pl.phys_off[pl.inst_phys[i]] + row
    return phys, pos


def layout(pos: np.ndarray, topk_w: np.ndarray, total: int) -> Tuple[np.ndarray, np.ndarray]:
    """Inverse index and permuted weights of the dispatch layout.

    inv[pos[n]] = n and w_perm[pos[n]] = w[n] for every valid pair; the
    layout holds ``total`` rows.
    """
    pos = np.asarray(pos).reshape(-1)
    w = np.asarray(topk_w, dtype=np.float32).reshape(-1)
    inv = np.full(total, -1, dtype=np.int64)
    w_perm = np.zeros(total, dtype=np.float32)
    n = np.nonzero(pos >= 0)[0]
    inv[pos[n]] = n
    w_perm[pos[n]] = w[n]
    return inv, w_perm


# ---------------------------------------------------------------------------
# permute
# ---------------------------------------------------------------------------
def permute(hidden_bits: np.ndarray, inv: np.ndarray, k: int, pl: Plan,
            p_begin: int, p_end: int) -> np.ndarray:
    """bf16 rows of the physical experts [p_begin, p_end), in layout order.

    Row i of the segment is the hidden row of the token that owns pair
    inv[phys_off[p_begin] + i].  Rows are moved as raw 16-bit patterns.
    """
    lo, hi = int(pl.phys_off[p_begin]), int(pl.phys_off[p_end])
    return np.asarray(hidden_bits)[np.asarray(inv)[lo:hi] // k]


# ---------------------------------------------------------------------------
# fold
# ---------------------------------------------------------------------------
def fold(master: Dict[int, np.ndarray], replica_grads: np.ndarray, pl: Plan,
         slot_begin: int, slot_end: int) -> Dict[int, np.ndarray]:
    """Fold replica gradients back into their masters.

    [README] Interface / "Forward and backward": ``grad_reduce`` reduces
    replica weight gradients into the master experts' gradients;
    "Performance Tuning / Expert communication": deterministic, non-atomic
    reduction by default.  For each expert with a replica among the slots
    [slot_begin, slot_end): master + the sum of those replicas, in fp64,
    rounded once to fp32.  ``replica_grads[s - slot_begin]`` is slot s.
    Returns the new master buffers of the touched experts.
    """
    out: Dict[int, np.ndarray] = {}
    for e in range(pl.E):
        slots = [s for s in range(slot_begin, slot_end) if pl.slot_expert[s] == e]
        if not slots:
            continue
        acc = np.asarray(master[e], dtype=np.float64).copy()
        for s in slots:
            acc += np.asarray(replica_grads[s - slot_begin], dtype=np.float64)
        out[e] = acc.astype(np.float32)
    return out


# ---------------------------------------------------------------------------
# weight_sync: master weights into the replica slots
# ---------------------------------------------------------------------------
RELAY_DIRECT, RELAY_ADAPTIVE, RELAY_FORCE = 0, 1, 2


def weight_sync(master: Dict[int, np.ndarray], pl: Plan, slot_begin: int,
                slot_end: int) -> Dict[int, np.ndarray]:
    """Replica weights of the slots [slot_begin, slot_end).

    [README] Interface, "Forward and backward": weight_sync materialises the
    plan by distributing master weights to the replica slots.  Slot s holding
    expert e receives a bit copy of e's master weights; empty slots get
    nothing.  Returns {slot: weights}.
    """
    return {s: np.array(master[int(pl.slot_expert[s])], copy=True)
            for s in range(slot_begin, slot_end) if pl.slot_expert[s] >= 0}


def replica_slots(pl: Plan, e: int) -> List[int]:
    """Redundant slots holding expert e, in ascending physical id."""
    out = []
    for p, _, _ in pl.instances(e):
        r, j = divmod(p, pl.M + pl.S)
        if j >= pl.M:
            out.append(r * pl.S + (j - pl.M))
    return out


def relay_plan(pl: Plan, mode: int = RELAY_ADAPTIVE, min_replicas: int = 4, max_relays: int = 8,
               min_gain: int = 2, domain_gpus: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Where each replica slot's weights come from, and in which stage.

    [README] "Performance Tuning", "Expert communication": the weight
    distribution plan is direct, adaptive or forced relay; adaptive relay
    needs a minimum replica count per expert, uses at most a maximum number
    of relays and is taken only for a minimum fan-out gain; plans are direct
    when the scale-up domain has at most 8 GPUs.  [NEWS] "What problem does
    UltraEP solve": the relay keeps the master's fan-out from overloading.

    Reading (the pages give the switches, not the schedule): an expert with
    n replicas either copies all of them from its master in one stage
    (fan-out n) or picks m relays -- its m lowest-physical-id replicas --
    that copy from the master in stage 1 while the other n - m copy from the
    relays in stage 2, relay (i - m) mod m serving the i-th replica.  The
    critical fan-out is then m + ceil((n - m) / m); m is the smallest value in
    [1, min(max_relays, n - 1)] that minimises it, and the gain is n over it.
    Relay is used under RELAY_FORCE (n >= 2), or under RELAY_ADAPTIVE when
    n >= min_replicas and n >= min_gain * critical fan-out; never when the
    domain has at most 8 GPUs (domain_gpus defaults to D, one GPU per rank).

    Returns (src, stage), each [R*S]: src -1 = the master, >= 0 = the relay
    slot, -2 = empty slot; stage 1 or 2, 0 for an empty slot.
    """
    if domain_gpus is None:
        domain_gpus = pl.D
    nslots = pl.R * pl.S
    src = np.full(nslots, -2, dtype=np.int64)
    stage = np.zeros(nslots, dtype=np.int64)
    for e in range(pl.E):
        reps = replica_slots(pl, e)
        n = len(reps)
        relay = False
        m = 0
        if mode != RELAY_DIRECT and domain_gpus > 8 and n >= 2 and max_relays >= 1:
            best = None
            for cand in range(1, min(max_relays, n - 1) + 1):
                cost = cand + _ceil_div(n - cand, cand)
                if best is None or cost < best[0]:
                    best = (cost, cand)
            cost, m = best
            relay = mode == RELAY_FORCE or (n >= min_replicas and n >= min_gain * cost)
        for i, s in enumerate(reps):
            if not relay or i < m:
                src[s], stage[s] = -1, 1
            else:
                src[s], stage[s] = reps[(i - m) % m], 2
    return src, stage


# ---------------------------------------------------------------------------
# the whole path for one layer
# ---------------------------------------------------------------------------
def balance(topk_idx: np.ndarray, E: int, R: int, S: int, D: int, **opts):
    """count -> plan -> reroute for one layer; returns (plan, phys, pos)."""
    c, dropped = count(topk_idx, E)
    pl = plan(c, E, R, S, D, dropped=dropped, **opts)
    phys, pos = reroute(topk_idx, pl)
    return pl, phys, pos


# ---------------------------------------------------------------------------
# combine, and the gradient gathers of the backward pass
# ---------------------------------------------------------------------------
# [README] Interface, "Forward and backward": after the experts run on the
# dispatched rows, combine brings each token's k expert outputs back to the
# token, weighted by its routing probabilities; in the backward pass reroute
# gathers the gradients of the physical replicas back to the logical experts.
# With routing held as (token, k) pairs the weights stay attached to their
# pair, so the gradient of each pair's weight comes back in pair order; the
# token gradient of the dispatch is the sum of its k rows' gradients.

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Values of bf16 bit patterns (a bf16 is the top half of an fp32)."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 (nearest, ties to even) in one step.

    bf16 keeps 8 significand bits and fp32's exponent range: the spacing of
    bf16 values around |x| in [2^e, 2^(e+1)) is 2^(e-7), and 2^-133 below the
    smallest normal 2^-126.  Rounding happens on the exact fp64 value, never
    through an intermediate fp32.  Finite inputs only; results beyond the
    largest bf16 become infinities.
    """
    x = np.asarray(x, dtype=np.float64)
    mag = np.abs(x)
    e = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
    spacing = np.exp2(np.maximum(e - 7, -133.0))
    q = np.rint(x / spacing) * spacing           # rint: halves go to even
    q32 = q.astype(np.float32)                   # exact: q has <= 8 significant bits
    return (q32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def combine(rows_bits: np.ndarray, pos: np.ndarray, topk_w: Optional[np.ndarray], k: int,
            token_begin: int, token_end: int) -> np.ndarray:
    """y[g] = sum_j w[g, j] * rows[pos[g*k + j]] for g in [token_begin, token_end), in fp64.

    rows_bits: the expert outputs in layout order, bf16 bit patterns
    [layout_rows, H].  Pairs whose pos is outside [0, layout_rows) (dropped
    pairs) add nothing.  With topk_w None every weight is 1: the sum of a
    token's k row gradients, which is the backward of the dispatch gather.
    """
    rows = bf16_bits_to_f64(rows_bits)
    nrows, H = rows.shape
    p = np.asarray(pos).reshape(-1).astype(np.int64)
    w = None if topk_w is None else np.asarray(topk_w, dtype=np.float64).reshape(-1)
    out = np.zeros((token_end - token_begin, H), dtype=np.float64)
    for g in range(token_begin, token_end):
        for j in range(k):
            n = g * k + j
            if 0 <= p[n] < nrows:
                out[g - token_begin] += (1.0 if w is None else w[n]) * rows[p[n]]
    return out


def combine_backward(rows_bits: np.ndarray, pos: np.ndarray, topk_w: np.ndarray, k: int,
                     grad_out_bits: np.ndarray, token_begin: int, token_end: int):
    """Gradients of combine for the tokens [token_begin, token_end), in fp64.

    grad_out_bits: dL/dy as bf16 bit patterns [token_end - token_begin, H].
    Returns (grad_rows, grad_w): grad_rows maps each layout row that a pair
    of the range points to onto w[n] * dy[g] (the gradient of that expert
    output row); grad_w[g - token_begin, j] = <dy[g], rows[pos[g*k + j]]>
    (the gradient of the pair's routing weight, in logical pair order), 0
    for a dropped pair.
    """
    rows = bf16_bits_to_f64(rows_bits)
    nrows = rows.shape[0]
    dy = bf16_bits_to_f64(grad_out_bits)
    p = np.asarray(pos).reshape(-1).astype(np.int64)
    w = np.asarray(topk_w, dtype=np.float64).reshape(-1)
    grad_rows: Dict[int, np.ndarray] = {}
    grad_w = np.zeros((token_end - token_begin, k), dtype=np.float64)
    for g in range(token_begin, token_end):
        for j in range(k):
            n = g * k + j
            if 0 <= p[n] < nrows:
                grad_rows[int(p[n])] = w[n] * dy[g - token_begin]
                grad_w[g - token_begin, j] = float(np.dot(dy[g - token_begin], rows[p[n]]))
    return grad_rows, grad_w
