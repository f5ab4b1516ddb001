"""Pins of the oracle's softmax statistics against closed forms, brute force and library routines.

Each case is chosen so that a plausible slip in the oracle (a dropped term, a wrong sign, an off-by-one
in k, a wrong tie rule, a transposed operand) fails at least one of them.
"""
import itertools
import math

import numpy as np
import pytest
import scipy.special

from oracle import kvprof_oracle as O

VIDEO_BOUNDS = [0, 1560, 3900, 6240]


def _row(s):
    s = np.asarray(s, dtype=np.float64)
    return s, O.softmax_row(s)


@pytest.mark.parametrize("n", [50, 100, 128, 6240])
def test_uniform_row(n):
    s, p = _row(np.zeros(n))
    assert O.entropy_support(p, n) == pytest.approx(1.0, abs=1e-12)
    for pct in O.TOP_PCTS:
        assert O.top_mass(p, n, pct) == pytest.approx(pct / 100.0, abs=1e-12)
    assert O.strict_zero_count(s, n) == 0
    # ties resolve to the lowest indices
    assert list(O.top32(s, n)[: min(32, n)]) == list(range(min(32, n)))


def test_uniform_region_and_frame_masses():
    s, p = _row(np.zeros(6240))
    reg = O.segment_masses(p, VIDEO_BOUNDS)
    assert np.allclose(reg, [0.25, 0.375, 0.375], atol=1e-12)
    fr = O.segment_masses(p, O.frame_bounds(390, 16))
    assert np.allclose(fr, 1 / 16, atol=1e-12)
    # frames 0-3 / 4-9 / 10-15 make up the three regions
    assert np.allclose([fr[:4].sum(), fr[4:10].sum(), fr[10:].sum()], reg, atol=1e-12)


@pytest.mark.parametrize("n", [128, 6240])
def test_one_hot_row(n):
    s = np.zeros(n)
    s[7] = 200.0
    s, p = _row(s)
    assert O.entropy_support(p, n) == pytest.approx(1.0 / n, rel=1e-9)
    for pct in O.TOP_PCTS:
        assert O.top_mass(p, n, pct) == pytest.approx(1.0, abs=1e-12)
    assert O.strict_zero_count(s, n) == n - 1
    t = O.top32(s, n)
    assert t[0] == 7 and list(t[1:]) == [j for j in range(n) if j != 7][:31]


@pytest.mark.parametrize("a,n", [(1, 16), (5, 128), (422, 6240), (6240, 6240)])
def test_flat_support_closed_form(a, n):
    """a keys share all the mass equally (others 1000 nats lower): H = ln a, support = a/n."""
    s = np.full(n, -1000.0)
    s[:a] = 0.0
    s, p = _row(s)
    assert O.entropy_support(p, n) == pytest.approx(a / n, rel=1e-12)


def test_strict_zero_boundary():
    """Two keys, s = [0, -x]: p_2 = e^-x / (1 + e^-x) is an fp32 zero iff p_2 <= 2^-150."""
    for x, zero in [(103.9, 0), (104.1, 1), (150.0, 1), (50.0, 0)]:
        s = np.array([0.0, -x])
        exact = -x - math.log1p(math.exp(-x))
        assert (exact <= -150 * math.log(2)) == bool(zero)
        assert O.strict_zero_count(s, 2) == zero


def test_softmax_and_lse_match_scipy():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((7, 16))
    k = rng.standard_normal((40, 16))
    res = O.row_stats(q, k, scale=0.25)
    s = 0.25 * q @ k.T
    assert np.allclose(res["p"], scipy.special.softmax(s, axis=1), atol=1e-15)
    assert np.allclose(res["row_lse"], scipy.special.logsumexp(s, axis=1), atol=1e-12)
    assert np.allclose(res["row_max"], s.max(axis=1))


def _brute_top_mass(p, pct):
    n = len(p)
    kf, rem = divmod(n * pct, 100)
    best = 0.0
    for sub in itertools.combinations(range(n), kf):
        best = max(best, sum(p[list(sub)]))
    # the next-largest element: the largest outside the best subset of size kf+1 minus best
    if kf < n:
        best1 = max(sum(p[list(sub)]) for sub in itertools.combinations(range(n), kf + 1))
        return best + (rem / 100.0) * (best1 - best)
    return best


@pytest.mark.parametrize("seed", range(4))
def test_top_mass_brute_force(seed):
    rng = np.random.default_rng(seed)
    for n in (10, 12, 16):
        s = rng.standard_normal(n) * 2
        _, p = _row(s)
        for pct in (10, 25, 50):  # pct values that give floor(k) >= 1 at these n
            assert O.top_mass(p, n, pct) == pytest.approx(_brute_top_mass(p, pct), abs=1e-12)


def _brute_top32(s):
    n = len(s)
    inside = [j for j in range(n)
              if sum(1 for i in range(n) if s[i] > s[j] or (s[i] == s[j] and i < j)) < 32]
    return set(inside)


@pytest.mark.parametrize("seed", range(3))
def test_top32_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    n = 40
    s = np.round(rng.standard_normal(n), 1)  # rounding creates ties
    t = O.top32(s, n)
    assert set(int(x) for x in t) == _brute_top32(s)
    # output order: score descending, ties by lower index
    for a, b in zip(t[:-1], t[1:]):
        assert s[a] > s[b] or (s[a] == s[b] and a < b)


def test_top32_short_row_pads():
    s = np.arange(10, dtype=np.float64)
    t = O.top32(s, 10)
    assert list(t[:10]) == list(range(9, -1, -1)) and all(t[10:] == -1)


def test_duplicate_keys_pick_lowest_indices():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 8))
    k = rng.standard_normal((40, 8))
    k[20:] = k[0]  # 21 copies of key 0
    k[1:20] = -k[0]  # 19 copies of its negation, below
    if float(q[0] @ k[0]) < 0:
        q = -q
    res = O.row_stats(q, k, scale=1.0)
    order = list(res["top32"][0])
    assert order[:21] == [0, *range(20, 40)]
    assert order[21:] == list(range(1, 12))


def test_bias_closed_form_region_masses():
    """Q = 0 with +0.5 on the current chunk: sink = 1560/D, recent = 2340/D, current = 2340 e^0.5/D,
    D = 3900 + 2340 e^0.5."""
    q = np.zeros((2, 8))
    k = np.random.default_rng(1).standard_normal((6240, 8))
    bias = np.zeros(6240)
    bias[3900:] = 0.5
    res = O.row_stats(q, k, scale=1.0, key_bias=bias, region_bounds=VIDEO_BOUNDS, frame_len=390,
                      n_frames=16)
    D = 3900 + 2340 * math.exp(0.5)
    assert np.allclose(res["region_mass"][0], [1560 / D, 2340 / D, 2340 * math.exp(0.5) / D],
                       atol=1e-12)
    assert np.allclose(res["frame_mass"].sum(axis=1), 1.0, atol=1e-12)
    assert np.allclose(res["region_mass"].sum(axis=1), 1.0, atol=1e-12)


def test_output_closed_forms():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((64, 8))
    k = rng.standard_normal((64, 8))
    q_uniform = np.zeros((1, 8))
    res = O.row_stats(q_uniform, k, scale=1.0, v=v)
    assert np.allclose(res["o"][0], v.mean(axis=0), atol=1e-14)
    # one-hot: key 5 made dominant through the bias
    bias = np.zeros(64)
    bias[5] = 500.0
    res = O.row_stats(q_uniform, k, scale=1.0, key_bias=bias, v=v)
    assert np.allclose(res["o"][0], v[5], atol=1e-14)


def test_causal_visibility():
    n = O.visible_counts(4, 10, True, 3)
    assert list(n) == [4, 5, 6, 7]
    rng = np.random.default_rng(4)
    q = rng.standard_normal((4, 8))
    k = rng.standard_normal((10, 8))
    res = O.row_stats(q, k, scale=1.0, causal=True, q_pos0=3)
    for i in range(4):
        assert np.all(res["p"][i, n[i]:] == 0)
        assert res["p"][i, : n[i]].sum() == pytest.approx(1.0)
        # stats computed on the visible prefix equal those of the truncated problem
        sub = O.row_stats(q[i:i + 1], k[: n[i]], scale=1.0)
        assert res["support"][i] == pytest.approx(sub["support"][0], rel=1e-12)


def test_heatmap_and_histograms():
    rng = np.random.default_rng(5)
    fm = rng.dirichlet(np.ones(16), size=96)
    groups = np.repeat(np.arange(6), 16)
    hm = O.heatmap(fm, groups, 6)
    assert hm.shape == (6, 16)
    assert np.allclose(hm.sum(axis=1), 1.0)
    assert np.allclose(hm[2], fm[32:48].mean(axis=0))
    x = np.array([0.0, 0.0999, 0.1, 0.25, 0.999, 1.0])
    h = O.histogram100(x)
    assert h.sum() == 6 and h[0] == 1 and h[9] == 1 and h[10] == 1 and h[25] == 1 and h[99] == 2
