"""Seeded synthetic inputs for the exact-load rebalancing path.

This module only draws random inputs. It holds none of the method's
arithmetic (no counting, planning, rerouting, permuting or folding), so the
CPU oracle and the HIP path can both be fed from it without sharing any of
the computation they are compared on.

The pages give no dataset for this path.  The project README's "Tests"
section runs its solver on one GPU over made-up, Zipf-skewed expert loads
tuned to chosen max/mean rank imbalances; these generators stand in for
those inputs.  The five workloads below follow the routing shapes named there
(256 experts, top-8, EP64, 8k tokens per rank) and the model scales the news
pages list (106B to 671B parameter MoE models, EP40/EP64 prefill).

Conventions shared by every workload
------------------------------------
* ``R`` logical EP ranks each own ``T`` tokens; token ``g = r*T + t`` is
  rank-major.  ``topk_idx`` is int32 ``[R*T, k]``; pair ``n = g*k + j``.
* Top-k experts are drawn per token *without replacement*, each next expert
  with probability proportional to its popularity among the experts not yet
  taken (the Plackett-Luce law that Gumbel-top-k also samples).  Duplicates
  are redrawn; a row that keeps hitting taken experts switches to an explicit
  draw from the renormalised remainder, which is the same law because
  rejection is memoryless.
* Routing weights: softmax over ``k`` i.i.d. N(0,1) logits, fp64, stored fp32.
* Hidden rows: N(0,1) fp32 rounded to bf16 (nearest-even), returned as the
  uint16 bit pattern.  Generated in blocks of ``HIDDEN_BLOCK`` rows, each
  block from its own seed, so any subset of rows can be regenerated alone.
* Gradients: N(0,1) fp32.
* Seeds: ``np.random.default_rng([cfg_id, layer, microbatch])`` for routing,
  drawn in the order popularity, experts, weights.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

HIDDEN_BLOCK = 4096
_HIDDEN_STREAM = 7_000_003
_GRAD_STREAM = 9_000_011
_WALK_STREAM = 5_000_017
_HOTDOM_STREAM = 3_000_007


@dataclasses.dataclass(frozen=True)
class Workload:
    cfg_id: int
    name: str
    E: int            # experts
    R: int            # logical EP ranks
    S: int            # redundant slots per rank
    D: int            # scale-up domain size (ranks)
    k: int            # top-k
    T: int            # tokens per rank
    H: int            # hidden size (bf16 elements per row)
    layers: int
    microbatches: int
    fold_rows: int    # one slot's gradient is fold_rows x fold_cols fp32
    fold_cols: int
    ffn: int = 0      # expert FFN width: fc1 holds 2*H*ffn weights, fc2 H*ffn

    @property
    def M(self) -> int:
        return self.E // self.R

    @property
    def N(self) -> int:
        return self.R * self.T * self.k

    @property
    def tokens(self) -> int:
        return self.R * self.T

    @property
    def numel(self) -> int:
        return self.fold_rows * self.fold_cols

    @property
    def instances(self) -> int:
        return self.layers * self.microbatches

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads.  T is per rank for all of them.
TINY = Workload(1, "tiny: T=256/rank E=8 top-2 R=4 S=1 D=4 H=64",
                E=8, R=4, S=1, D=4, k=2, T=256, H=64, layers=1, microbatches=1,
                fold_rows=64, fold_cols=64, ffn=64)
SINGLE = Workload(2, "single layer 235B-class: E=128 top-8 R=64 S=2 D=64 T=8192 H=4096 Dirichlet(0.3)",
                  E=128, R=64, S=2, D=64, k=8, T=8192, H=4096, layers=1, microbatches=1,
                  fold_rows=2048, fold_cols=4096, ffn=1536)
DEEP = Workload(3, "671B-class 61 layers: E=256 top-8 R=64 S=2 D=64 T=4096 H=7168 Zipf s~U[0.6,1.4]",
                E=256, R=64, S=2, D=64, k=8, T=4096, H=7168, layers=61, microbatches=1,
                fold_rows=2048, fold_cols=7168, ffn=2048)
STREAM = Workload(4, "non-stationary stream 32 layers x 16 mb: E=128 top-8 R=64 S=2 D=64 T=8192 H=4096",
                  E=128, R=64, S=2, D=64, k=8, T=8192, H=4096, layers=32, microbatches=16,
                  fold_rows=2048, fold_cols=4096, ffn=1536)
TOPO = Workload(5, "topology-constrained prefill: E=160 top-8 R=40 S=3 D=8 T=16384 H=5120 hot in 2 domains",
                E=160, R=40, S=3, D=8, k=8, T=16384, H=5120, layers=1, microbatches=1,
                fold_rows=2048, fold_cols=5120, ffn=1536)

# The project README's EP64 test table ("Tests"): 256 experts, 4 masters and
# 2 redundant slots per rank, top-8, 8k tokens per rank, loads synthesized
# at initial max/mean 1.51, 2.01 and 3.03 (hidden and FFN widths of the
# 256-expert model class, which the table does not give).
TABLE_IMBALANCE = {6: 1.51, 7: 2.01, 8: 3.03}
TABLE = [Workload(cid, f"pages' EP64 table shape: E=256 top-8 R=64 S=2 D=64 T=8192, initial max/mean {r}",
                  E=256, R=64, S=2, D=64, k=8, T=8192, H=7168, layers=1, microbatches=1,
                  fold_rows=2048, fold_cols=7168, ffn=2048)
         for cid, r in TABLE_IMBALANCE.items()]

CONFIGS = {w.cfg_id: w for w in (TINY, SINGLE, DEEP, STREAM, TOPO, *TABLE)}


def _zipf(E: int, s: float) -> np.ndarray:
    return np.arange(1, E + 1, dtype=np.float64) ** (-s)


def _walk_alphas(n: int) -> np.ndarray:
    """Dirichlet concentration per microbatch for the non-stationary stream.

    One walk over the microbatches, shared by every layer: log(alpha) starts
    uniform in [log 0.1, log 2] and moves by N(0, 0.5^2) steps, reflected back
    into that interval.
    """
    rng = np.random.default_rng([4, _WALK_STREAM])
    lo, hi = math.log(0.1), math.log(2.0)
    x = rng.uniform(lo, hi)
    out = []
    for _ in range(n):
        out.append(math.exp(x))
        x = x + rng.normal(0.0, 0.5)
        while x < lo or x > hi:          # reflect into [lo, hi]
            x = 2 * lo - x if x < lo else 2 * hi - x
    return np.array(out)


def hot_domains(w: Workload) -> np.ndarray:
    """The two domains that hold the hottest experts in the topology workload."""
    rng = np.random.default_rng([w.cfg_id, _HOTDOM_STREAM])
    return np.sort(rng.choice(w.R // w.D, size=2, replace=False))


def zipf_at_imbalance(target: float, E: int, R: int, rng: np.random.Generator) -> np.ndarray:
    """Zipf popularity over a seeded permutation of the experts, its exponent
    bisected so that the expected max/mean home-rank load is ``target``."""
    perm = rng.permutation(E)

    def law(s):
        z = _zipf(E, s)
        q = np.empty(E)
        q[perm] = z / z.sum()
        return q.reshape(R, -1).sum(axis=1).max() * R, q

    lo, hi = 0.0, 4.0
    for _ in range(60):
        mid = (lo + hi) / 2
        if law(mid)[0] < target:
            lo = mid
        else:
            hi = mid
    return law(lo)[1]


def dealt_topk(rng: np.random.Generator, counts: np.ndarray, ntok: int, k: int) -> np.ndarray:
    """A top-k routing with exactly ``counts`` pairs per expert.

    The pairs, sorted by expert, are dealt column by column: pair i goes to
    token i mod ntok, slot i div ntok.  No expert has more pairs than there
    are tokens, so two pairs of one expert never meet in a token.  Tokens and
    the slots inside each token are then shuffled."""
    assert counts.sum() == ntok * k and counts.max() <= ntok
    ids = np.repeat(np.arange(counts.size), counts)
    out = ids.reshape(k, ntok).T.copy()
    out = out[rng.permutation(ntok)]
    return np.take_along_axis(out, rng.random((ntok, k)).argsort(axis=1), axis=1)


def popularity(w: Workload, layer: int, mb: int, rng: np.random.Generator) -> np.ndarray:
    """Expert popularity p (sums to 1, every entry >= 1e-30) for one instance."""
    E = w.E
    if w.cfg_id in TABLE_IMBALANCE:         # Zipf tuned to the table's initial max/mean
        return zipf_at_imbalance(TABLE_IMBALANCE[w.cfg_id], E, w.R, rng)
    if w.cfg_id == 1:                       # Zipf(1.2), seeded permutation
        z = _zipf(E, 1.2)
        p = np.empty(E)
        p[rng.permutation(E)] = z
    elif w.cfg_id == 2:                     # Dirichlet(0.3)
        p = rng.dirichlet(np.full(E, 0.3))
    elif w.cfg_id == 3:                     # per-layer Zipf, s ~ U[0.6, 1.4]
        s = rng.uniform(0.6, 1.4)
        z = _zipf(E, s)
        p = np.empty(E)
        p[rng.permutation(E)] = z
    elif w.cfg_id == 4:                     # Dirichlet(alpha_t), alpha_t a random walk
        alpha = _walk_alphas(w.microbatches)[mb]
        p = rng.dirichlet(np.full(E, alpha))
    elif w.cfg_id == 5:                     # Zipf(1.2), hottest experts in 2 domains
        z = _zipf(E, 1.2)                   # descending
        doms = hot_domains(w)
        per_dom = w.D * w.M
        hot_experts = np.concatenate([np.arange(d * per_dom, (d + 1) * per_dom) for d in doms])
        cold_experts = np.setdiff1d(np.arange(E), hot_experts)
        p = np.empty(E)
        p[rng.permutation(hot_experts)] = z[: len(hot_experts)]
        p[rng.permutation(cold_experts)] = z[len(hot_experts):]
    else:
        raise ValueError(f"unknown workload {w.cfg_id}")
    p = np.maximum(p, 1e-30)
    return p / p.sum()


def sample_topk(rng: np.random.Generator, p: np.ndarray, ntok: int, k: int,
                max_rounds: int = 16) -> np.ndarray:
    """k distinct experts per token, drawn sequentially proportional to p."""
    E = p.shape[0]
    if k > E:
        raise ValueError("k > E")
    cdf = np.cumsum(p)
    cdf /= cdf[-1]
    out = np.empty((ntok, k), dtype=np.int64)
    for j in range(k):
        col = np.minimum(np.searchsorted(cdf, rng.random(ntok), side="right"), E - 1)
        dup = (out[:, :j] == col[:, None]).any(axis=1) if j else np.zeros(ntok, bool)
        rounds = 0
        while dup.any() and rounds < max_rounds:
            rows = np.nonzero(dup)[0]
            redraw = np.minimum(np.searchsorted(cdf, rng.random(rows.size), side="right"), E - 1)
            col[rows] = redraw
            dup[rows] = (out[rows, :j] == redraw[:, None]).any(axis=1)
            rounds += 1
        if dup.any():
            rows = np.nonzero(dup)[0]
            q = np.broadcast_to(p, (rows.size, E)).copy()
            np.put_along_axis(q, out[rows, :j], 0.0, axis=1)
            cq = np.cumsum(q, axis=1)
            u = rng.random(rows.size) * cq[:, -1]
            col[rows] = np.minimum((cq <= u[:, None]).sum(axis=1), E - 1)
        out[:, j] = col
    return out


def routing(w: Workload, layer: int = 0, mb: int = 0):
    """(topk_idx int32 [R*T, k], topk_w fp32 [R*T, k], p float64 [E]) for one instance."""
    rng = np.random.default_rng([w.cfg_id, layer, mb])
    p = popularity(w, layer, mb, rng)
    if w.cfg_id in TABLE_IMBALANCE:         # exact multinomial counts, dealt to tokens
        counts = rng.multinomial(w.N, p)
        idx = dealt_topk(rng, counts, w.tokens, w.k).astype(np.int32)
    else:
        idx = sample_topk(rng, p, w.tokens, w.k).astype(np.int32)
    logits = rng.standard_normal((w.tokens, w.k))
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    wts = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    return idx, wts, p


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


def hidden_block(w: Workload, block: int) -> np.ndarray:
    """Rows [block*HIDDEN_BLOCK, ...) of the workload's hidden matrix (uint16 bf16 bits)."""
    rows = min(HIDDEN_BLOCK, w.tokens - block * HIDDEN_BLOCK)
    rng = np.random.default_rng([w.cfg_id, _HIDDEN_STREAM, block])
    return f32_to_bf16_bits(rng.standard_normal((rows, w.H), dtype=np.float32))


def hidden(w: Workload, out: np.ndarray | None = None, workers: int = 8) -> np.ndarray:
    """The whole hidden matrix [R*T, H] as uint16 bf16 bit patterns.

    Blocks are independent streams, so they are filled by a thread pool; the
    result does not depend on ``workers``.
    """
    if out is None:
        out = np.empty((w.tokens, w.H), dtype=np.uint16)
    nblocks = (w.tokens + HIDDEN_BLOCK - 1) // HIDDEN_BLOCK

    def fill(b: int) -> None:
        out[b * HIDDEN_BLOCK:(b + 1) * HIDDEN_BLOCK] = hidden_block(w, b)

    if workers <= 1 or nblocks == 1:
        for b in range(nblocks):
            fill(b)
    else:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(nblocks)))
    return out


def hidden_rows(w: Workload, rows: np.ndarray) -> np.ndarray:
    """Only the requested rows of ``hidden(w)``, regenerating just their blocks."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, w.H), dtype=np.uint16)
    blocks = rows // HIDDEN_BLOCK
    for b in np.unique(blocks):
        sel = np.nonzero(blocks == b)[0]
        out[sel] = hidden_block(w, int(b))[rows[sel] - b * HIDDEN_BLOCK]
    return out


def random_bits_hidden(rows: int, H: int, seed: int) -> np.ndarray:
    """Uniformly random 16-bit patterns (NaN payloads, infinities, subnormals included)."""
    return np.random.default_rng([seed, _HIDDEN_STREAM]).integers(0, 1 << 16, size=(rows, H), dtype=np.uint16)


def grads(w: Workload, count: int, stream: int, numel: int | None = None) -> np.ndarray:
    """``count`` gradient buffers of ``numel`` fp32 each, N(0,1)."""
    n = w.numel if numel is None else numel
    rng = np.random.default_rng([w.cfg_id, _GRAD_STREAM, stream])
    return rng.standard_normal((count, n), dtype=np.float32)


def random_ids(rng: np.random.Generator, E: int, n: int, invalid_frac: float = 0.0) -> np.ndarray:
    """Uniform expert ids with a fraction replaced by out-of-range ids (edge-case inputs)."""
    ids = rng.integers(0, E, size=n).astype(np.int32)
    if invalid_frac > 0:
        bad = rng.random(n) < invalid_frac
        junk = rng.choice(np.array([-1, -7, E, E + 3, 2**31 - 1, -(2**31)], dtype=np.int64), size=n)
        ids[bad] = junk[bad].astype(np.int32)
    return ids
