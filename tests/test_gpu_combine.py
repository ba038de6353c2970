"""GPU parity of combine and its backward through the C ABI.

Both return bf16 (and fp32 weight gradients) computed in fp32, so they are
compared element by element with the fp64 oracle under the bound of that
arithmetic: k fp32 additions (each off by at most 2^-24 of the running sum
of magnitudes) plus one rounding to bf16 (half a bf16 unit in the last
place); the weight gradient's dot product over H columns is off by at most
(H/64 + 6) * 2^-24 of the sum of magnitudes (each lane adds its H/64
columns, then six tree steps combine the lanes).  The layout positions come
from the oracle, so the only HIP code under test is the combine's.
"""
import numpy as np
import pytest

import moe_expert_load_ultraep_amd as U
import oracle as O
import workload as W
from gpu_common import routing_cached, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
DEV = "cuda"
U24 = 2.0 ** -24
SENTINEL = 0x7FC1  # a NaN pattern no result can take


def ulp_bf16(x):
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.exp2(np.maximum(e - 7, -133.0))


def bf16_normal(rng, shape):
    return W.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def to_dev(a):
    a = np.array(a, copy=True, order="C")  # writable: torch shares the buffer
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def check_combine(got_bits, rows_bits, pos, w, k, g0, g1):
    exact = O.combine(rows_bits, pos, w, k, g0, g1)
    mag = O.combine(rows_bits & np.uint16(0x7FFF), pos, None if w is None else np.abs(w), k, g0, g1)
    delta = k * U24 * mag
    bound = ulp_bf16(np.abs(exact) + delta) + 2 * delta
    got = O.bf16_bits_to_f64(got_bits)
    bad = np.abs(got - exact) > bound
    assert not bad.any(), (np.argwhere(bad)[:5], got[bad][:5], exact[bad][:5])


def check_backward(grad_rows_bits, gw, rows_bits, pos, w, k, dy_bits, g0, g1, H):
    want_rows, want_w = O.combine_backward(rows_bits, pos, w, k, dy_bits, g0, g1)
    for r, v in want_rows.items():
        got = O.bf16_bits_to_f64(grad_rows_bits[r])
        bound = ulp_bf16(v) + 2.0 ** -23 * np.abs(v)
        assert (np.abs(got - v) <= bound).all(), r
    _, mag = O.combine_backward(rows_bits & np.uint16(0x7FFF), pos, np.abs(w), k,
                                dy_bits & np.uint16(0x7FFF), g0, g1)
    bound = 2 * (H / 64 + 6) * U24 * mag + 1e-30
    assert (np.abs(gw.astype(np.float64) - want_w) <= bound).all()
    return set(want_rows)


def run_case(rng, T, k, H, nrows, g0, g1, drop=0.0, weighted=True):
    pos = rng.permutation(nrows)[:T * k].astype(np.int32) if nrows >= T * k else \
        rng.integers(0, nrows, T * k).astype(np.int32)
    if drop:
        sel = rng.random(T * k) < drop
        pos[sel] = rng.choice(np.array([-1, nrows, 1 << 30], dtype=np.int32), size=int(sel.sum()))
    w = rng.random((T, k)).astype(np.float32)
    rows = bf16_normal(rng, (nrows, H))
    dy = bf16_normal(rng, (g1 - g0, H))
    ctx = U.ultraep_create(64, 4, 1, 4)
    d_pos, d_w, d_rows, d_dy = to_dev(pos), to_dev(w), to_dev(rows), to_dev(dy)
    out = torch.full((g1 - g0, H), SENTINEL, dtype=torch.int16, device=DEV)
    U.ultraep_combine(ctx, d_pos, d_w if weighted else None, k, d_rows, g0, g1, out)
    grad_rows = torch.full((nrows, H), SENTINEL, dtype=torch.int16, device=DEV)
    gw = torch.full((g1 - g0, k), float("nan"), dtype=torch.float32, device=DEV)
    U.ultraep_combine_backward(ctx, d_pos, d_w, k, d_rows, d_dy, g0, g1, grad_rows, gw)
    torch.cuda.synchronize()
    check_combine(out.cpu().numpy().view(np.uint16), rows, pos, w if weighted else None, k, g0, g1)
    gr = grad_rows.cpu().numpy().view(np.uint16)
    touched = check_backward(gr, gw.cpu().numpy(), rows, pos, w, k, dy, g0, g1, H)
    untouched = np.setdiff1d(np.arange(nrows), np.fromiter(touched, dtype=np.int64))
    assert (gr[untouched] == SENTINEL).all(), "rows of other tokens must stay untouched"


@pytest.mark.parametrize("T,k,H,nrows,g0,g1,drop,weighted", [
    (300, 8, 4096, 2600, 0, 300, 0.0, True),      # eight 1 KiB column chunks a token, full range
    (300, 8, 4096, 2600, 0, 300, 0.0, False),     # unweighted: backward of the dispatch
    (257, 6, 136, 1600, 13, 250, 0.05, True),     # ragged H (one partial chunk), sub-range, dropped pairs
    (64, 1, 8, 64, 0, 64, 0.0, True),             # k = 1, one 16-byte vector per row
    (40, 64, 64, 2600, 0, 40, 0.02, True),        # k = 64 (eight groups of eight rows)
    (50, 3, 7168, 200, 7, 7, 0.0, True),          # empty range
    (700, 2, 1000, 1400, 100, 700, 0.0, True),    # H / 8 % 64 != 0: a partial second chunk
])
def test_combine_cases(T, k, H, nrows, g0, g1, drop, weighted):
    say(f"combine T={T} k={k} H={H} rows={nrows} range=[{g0},{g1}) drop={drop} weighted={weighted}")
    run_case(np.random.default_rng([T, k, H, nrows, g0]), T, k, H, nrows, g0, g1, drop, weighted)


def test_combine_tiny_workload_layout():
    """The tiny workload end to end: its oracle layout, all tokens."""
    w = W.TINY
    idx, wt = routing_cached(1, 0, 0)
    pl, _, pos = O.balance(idx, w.E, w.R, w.S, w.D)
    rng = np.random.default_rng(21)
    rows = bf16_normal(rng, (pl.total, w.H))
    dy = bf16_normal(rng, (w.tokens, w.H))
    ctx = U.ultraep_create(w.E, w.R, w.S, w.D)
    d_pos, d_w, d_rows = to_dev(pos.astype(np.int32)), to_dev(wt), to_dev(rows)
    out = torch.empty((w.tokens, w.H), dtype=torch.int16, device=DEV)
    U.ultraep_combine(ctx, d_pos, d_w, w.k, d_rows, 0, w.tokens, out)
    grad_rows = torch.empty((pl.total, w.H), dtype=torch.int16, device=DEV)
    gw = torch.empty((w.tokens, w.k), dtype=torch.float32, device=DEV)
    U.ultraep_combine_backward(ctx, d_pos, d_w, w.k, d_rows, to_dev(dy), 0, w.tokens, grad_rows, gw)
    torch.cuda.synchronize()
    check_combine(out.cpu().numpy().view(np.uint16), rows, pos, wt, w.k, 0, w.tokens)
    touched = check_backward(grad_rows.cpu().numpy().view(np.uint16), gw.cpu().numpy(), rows, pos, wt,
                             w.k, dy, 0, w.tokens, w.H)
    assert touched == set(range(pl.total))      # the layout is a bijection onto its rows


def test_combine_full_size_single_layer_sampled():
    """Single-layer workload at full size: rank 1's 8192 tokens against the
    whole 4,194,304-row layout (34 GB of bf16 expert outputs, drawn on the
    GPU by a seeded generator); the oracle checks a seeded sample of tokens
    from host copies of just the rows they read."""
    w = W.SINGLE
    idx, wt = routing_cached(2, 0, 0)
    pl, _, pos = O.balance(idx, w.E, w.R, w.S, w.D)
    g0, g1 = w.T, 2 * w.T
    gen = torch.Generator(device=DEV).manual_seed(2024)
    say("full size: drawing the layout rows")
    rows = torch.randn((pl.total, w.H), generator=gen, device=DEV, dtype=torch.bfloat16)
    dy = torch.randn((g1 - g0, w.H), generator=gen, device=DEV, dtype=torch.bfloat16)
    ctx = U.ultraep_create(w.E, w.R, w.S, w.D)
    d_pos, d_w = to_dev(pos.astype(np.int32)), to_dev(wt)
    out = torch.empty((g1 - g0, w.H), dtype=torch.int16, device=DEV)
    U.ultraep_combine(ctx, d_pos, d_w, w.k, rows.view(torch.int16), g0, g1, out)
    grad_rows = torch.full((pl.total, w.H), SENTINEL, dtype=torch.int16, device=DEV)
    gw = torch.empty((g1 - g0, w.k), dtype=torch.float32, device=DEV)
    U.ultraep_combine_backward(ctx, d_pos, d_w, w.k, rows.view(torch.int16), dy.view(torch.int16), g0, g1,
                               grad_rows, gw)
    torch.cuda.synchronize()
    say("full size: checking sampled tokens")
    sample = np.sort(np.random.default_rng(22).choice(g1 - g0, size=48, replace=False))
    for t in sample:
        g = g0 + int(t)
        p = pos[g * w.k:(g + 1) * w.k]
        sub = rows[torch.from_numpy(p.astype(np.int64)).to(DEV)].view(torch.int16).cpu().numpy().view(np.uint16)
        local_pos = np.arange(w.k, dtype=np.int32)
        wt_t = wt[g:g + 1]
        check_combine(out[t:t + 1].cpu().numpy().view(np.uint16), sub, local_pos, wt_t, w.k, 0, 1)
        gr = grad_rows[torch.from_numpy(p.astype(np.int64)).to(DEV)].cpu().numpy().view(np.uint16)
        dyt = dy[t:t + 1].view(torch.int16).cpu().numpy().view(np.uint16)
        check_backward(gr, gw[t:t + 1].cpu().numpy(), sub, local_pos, wt_t, w.k, dyt, 0, 1, w.H)
    # rows that belong to other ranks' tokens are untouched (a sample of them)
    others = np.concatenate([pos[:g0 * w.k], pos[g1 * w.k:]])
    probe = np.random.default_rng(23).choice(others, size=256, replace=False)
    assert (grad_rows[torch.from_numpy(probe.astype(np.int64)).to(DEV)].cpu().numpy() == SENTINEL).all()
