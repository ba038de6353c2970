"""Pins of the oracle's combine, its backward and the bf16 rounding (CPU).

Each pin checks the oracle against something other than its own formula:
fixed rounding cases, a dense-matrix formulation of the same sum, adjoint
identities that tie the backward to the forward (and the unweighted combine
to the already pinned dispatch gather), and a finite difference for the
weight gradient.  Integer-valued rows and dyadic weights keep every fp64 sum
exact, so the identities hold bit for bit.
"""
import numpy as np
import pytest

import oracle as O
import workload as W


def _int_rows(rng, n, H, lo=-8, hi=9):
    """bf16 bit patterns of small integers (exact in bf16 and in fp64 sums)."""
    vals = rng.integers(lo, hi, size=(n, H)).astype(np.float32)
    return (vals.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _dyadic(rng, shape):
    return (rng.integers(-16, 17, size=shape) / 16.0).astype(np.float32)


def test_bf16_rounding_fixed_cases():
    cases = [
        (1.0, 0x3F80),
        (1.0 + 2.0 ** -8, 0x3F80),          # tie -> even (down)
        (1.0 + 3 * 2.0 ** -8, 0x3F82),      # tie -> even (up)
        (1.0 + 3 * 2.0 ** -9, 0x3F81),      # above the tie
        (1.0 + 2.0 ** -8 - 2.0 ** -40, 0x3F80),  # just below a tie: no double rounding
        (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),  # just above
        (-2.5, 0xC020),
        (2.0 ** -130, 0x0008),              # subnormal: spacing 2^-133
        (0.0, 0x0000),
        (3.0e38, 0x7F62),
    ]
    got = O.f64_to_bf16_bits(np.array([c[0] for c in cases]))
    assert [int(x) for x in got] == [c[1] for c in cases]
    assert (O.bf16_bits_to_f64(np.array([0x3F80, 0xC020, 0x0008], dtype=np.uint16)) ==
            np.array([1.0, -2.5, 2.0 ** -130])).all()


def test_bf16_rounding_agrees_with_fp32_rounding_on_fp32_inputs():
    """On values that are already fp32 there is one rounding either way, so
    the direct fp64 rounding must match the integer fp32 rounding trick the
    input generator uses."""
    x = np.random.default_rng(5).standard_normal(200_000).astype(np.float32) * 1e3
    assert np.array_equal(O.f64_to_bf16_bits(x.astype(np.float64)), W.f32_to_bf16_bits(x))


@pytest.mark.parametrize("seed", [0, 1])
def test_combine_matches_dense_matrix_product(seed):
    rng = np.random.default_rng([seed, 11])
    T, k, H, nrows = 37, 3, 24, 140
    rows = _int_rows(rng, nrows, H)
    pos = rng.integers(-1, nrows, size=T * k)
    w = _dyadic(rng, (T, k))
    A = np.zeros((T, nrows))
    for n in range(T * k):
        if pos[n] >= 0:
            A[n // k, pos[n]] += w.reshape(-1)[n]
    want = A @ O.bf16_bits_to_f64(rows)
    assert np.array_equal(O.combine(rows, pos, w, k, 0, T), want)
    # a token sub-range is the same rows of the full result
    assert np.array_equal(O.combine(rows, pos, w, k, 5, 20), want[5:20])
    # unweighted: the incidence (count) matrix
    A1 = np.zeros((T, nrows))
    for n in range(T * k):
        if pos[n] >= 0:
            A1[n // k, pos[n]] += 1
    assert np.array_equal(O.combine(rows, pos, None, k, 0, T), A1 @ O.bf16_bits_to_f64(rows))


def test_combine_k1_unit_weights_is_the_row_gather():
    rng = np.random.default_rng(3)
    rows = _int_rows(rng, 50, 16)
    pos = rng.permutation(50)[:20]
    got = O.combine(rows, pos, np.ones(20, np.float32), 1, 0, 20)
    assert np.array_equal(got, O.bf16_bits_to_f64(rows[pos]))


def test_dropped_pairs_add_nothing():
    rng = np.random.default_rng(4)
    rows = _int_rows(rng, 30, 8)
    pos = rng.permutation(30)[:24]
    w = _dyadic(rng, (8, 3))
    pos_drop = pos.copy()
    pos_drop[[1, 7, 14]] = [-1, 30, 1 << 20]
    w_zero = w.reshape(-1).copy()
    w_zero[[1, 7, 14]] = 0
    assert np.array_equal(O.combine(rows, pos_drop, w, 3, 0, 8), O.combine(rows, pos, w_zero, 3, 0, 8))
    gr, gw = O.combine_backward(rows, pos_drop, w, 3, _int_rows(rng, 8, 8), 0, 8)
    assert set(gr) == set(int(p) for p in pos_drop if 0 <= p < 30)
    assert gw.reshape(-1)[[1, 7, 14]].tolist() == [0, 0, 0]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_combine_backward_is_the_adjoint(seed):
    """<combine(X), dy> = sum over rows <X[row], grad_rows[row]> (exact)."""
    rng = np.random.default_rng([seed, 12])
    T, k, H = 40, 4, 32
    nrows = T * k + 10
    rows = _int_rows(rng, nrows, H)
    pos = rng.permutation(nrows)[:T * k]
    pos[rng.random(T * k) < 0.1] = -1
    w = _dyadic(rng, (T, k))
    dy = _int_rows(rng, T, H)
    y = O.combine(rows, pos, w, k, 0, T)
    lhs = float((y * O.bf16_bits_to_f64(dy)).sum())
    gr, _ = O.combine_backward(rows, pos, w, k, dy, 0, T)
    X = O.bf16_bits_to_f64(rows)
    rhs = sum(float((X[r] * v).sum()) for r, v in gr.items())
    assert lhs == rhs


@pytest.mark.parametrize("seed", [0, 1])
def test_weight_gradient_is_a_finite_difference(seed):
    """<combine(X; w + d e_n), dy> - <combine(X; w), dy> = d * grad_w[n] (exact)."""
    rng = np.random.default_rng([seed, 13])
    T, k, H = 12, 3, 16
    nrows = T * k
    rows = _int_rows(rng, nrows, H)
    pos = rng.permutation(nrows)
    w = _dyadic(rng, (T, k))
    dy = _int_rows(rng, T, H)
    _, gw = O.combine_backward(rows, pos, w, k, dy, 0, T)
    base = float((O.combine(rows, pos, w, k, 0, T) * O.bf16_bits_to_f64(dy)).sum())
    d = 0.25
    for n in rng.choice(T * k, size=10, replace=False):
        w2 = w.reshape(-1).copy()
        w2[n] += d
        bumped = float((O.combine(rows, pos, w2, k, 0, T) * O.bf16_bits_to_f64(dy)).sum())
        assert bumped - base == d * gw.reshape(-1)[n]


def test_unweighted_combine_is_the_adjoint_of_the_dispatch_gather():
    """Over the whole layout, <permute(h), G> = <h, combine(G, unweighted)>:
    the token gradient of the dispatch is the unweighted sum of its rows'
    gradients.  Ties the new function to the pinned permute oracle."""
    w = W.TINY
    idx, _, _ = W.routing(w, 0, 0)
    pl, _, pos = O.balance(idx, w.E, w.R, w.S, w.D)
    inv, _ = O.layout(pos, np.ones(idx.shape, np.float32), pl.total)
    rng = np.random.default_rng(14)
    h = _int_rows(rng, w.tokens, 8)
    G = _int_rows(rng, pl.total, 8)
    P = O.permute(h, inv, w.k, pl, 0, pl.P)
    lhs = float((O.bf16_bits_to_f64(P) * O.bf16_bits_to_f64(G)).sum())
    back = O.combine(G, pos, None, w.k, 0, w.tokens)
    rhs = float((O.bf16_bits_to_f64(h) * back).sum())
    assert lhs == rhs
