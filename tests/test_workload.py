"""The seeded input generators (no GPU)."""
import numpy as np
import pytest

import workload as W


@pytest.mark.parametrize("cfg", [1, 2, 5])
def test_routing_is_seeded_and_well_formed(cfg):
    w = W.CONFIGS[cfg]
    if cfg != 1:
        w = w.with_(T=256)
    a = W.routing(w)
    b = W.routing(w)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    idx, wt, p = a
    assert idx.shape == (w.tokens, w.k) and idx.dtype == np.int32
    assert wt.shape == idx.shape and wt.dtype == np.float32
    assert ((idx >= 0) & (idx < w.E)).all()
    s = np.sort(idx, axis=1)
    assert (s[:, 1:] != s[:, :-1]).all(), "top-k experts of a token must be distinct"
    assert np.allclose(wt.sum(axis=1), 1.0, atol=1e-6)
    assert abs(p.sum() - 1) < 1e-12 and (p > 0).all()
    assert not np.array_equal(W.routing(w, layer=1)[0], idx)


def test_sampler_follows_sequential_law():
    """First pick ~ p; second pick ~ sum_i p_i p_j / (1 - p_i) (sampling
    without replacement)."""
    rng = np.random.default_rng(0)
    p = np.array([0.5, 0.25, 0.15, 0.1])
    n = 200_000
    idx = W.sample_topk(rng, p, n, 2)
    first = np.bincount(idx[:, 0], minlength=4) / n
    second = np.bincount(idx[:, 1], minlength=4) / n
    want2 = np.array([sum(p[i] * p[j] / (1 - p[i]) for i in range(4) if i != j) for j in range(4)])
    assert np.abs(first - p).max() < 0.005
    assert np.abs(second - want2).max() < 0.005


def test_sampler_concentrated_mass_still_distinct():
    rng = np.random.default_rng(1)
    p = np.full(16, 1e-30)
    p[3] = 1.0
    p /= p.sum()
    idx = W.sample_topk(rng, p, 1000, 4)
    assert (idx[:, 0] == 3).all()
    s = np.sort(idx, axis=1)
    assert (s[:, 1:] != s[:, :-1]).all()


def test_bf16_rounding_nearest_even():
    x = np.array([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -2.5, 1 + 2.0 ** -8 + 2.0 ** -20], dtype=np.float32)
    assert W.f32_to_bf16_bits(x).tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F81]


def test_hidden_rows_match_whole():
    w = W.TINY.with_(T=W.HIDDEN_BLOCK // 2 + 7)   # two blocks, ragged
    full = W.hidden(w, workers=2)
    rows = np.array([0, 5, W.HIDDEN_BLOCK - 1, W.HIDDEN_BLOCK, w.tokens - 1])
    assert np.array_equal(W.hidden_rows(w, rows), full[rows])
    assert np.array_equal(W.hidden(w, workers=1), full)


def test_walk_alphas_in_range():
    a = W._walk_alphas(16)
    assert ((a >= 0.1 - 1e-12) & (a <= 2.0 + 1e-12)).all() and len(set(a.round(12))) == 16


def test_topology_hot_domains_hold_hottest_experts():
    w = W.TOPO
    rng = np.random.default_rng([w.cfg_id, 0, 0])
    p = W.popularity(w, 0, 0, rng)
    doms = W.hot_domains(w)
    per = w.D * w.M
    hot = np.concatenate([np.arange(d * per, (d + 1) * per) for d in doms])
    assert p[hot].min() > np.delete(p, hot).max()
