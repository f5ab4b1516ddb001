"""Pins of the oracle's local output ablation (drop a key range, renormalise P, compare O) against
closed forms, brute force and vector identities.

The video regions are sink [0, 1560), recent [1560, 3900) and current [3900, 6240); the three ablations
drop the sink, the recent region, or all history ([0, 3900)).
"""
import math

import numpy as np
import pytest

from oracle import kvprof_oracle as O

SK = 6240
DROPS = {"drop_sink": (0, 1560), "drop_recent": (1560, 3900), "drop_history": (0, 3900)}


def _video_bias():
    b = np.zeros(SK)
    b[3900:] = 0.5
    return b


def test_empty_drop_is_the_full_output():
    rng = np.random.default_rng(0)
    q, k, v = rng.standard_normal((5, 16)), rng.standard_normal((40, 16)), rng.standard_normal((40, 16))
    full = O.row_stats(q, k, scale=0.25, v=v)["o"]
    abl = O.ablated_output(q, k, v, scale=0.25, drop=(7, 7))
    assert np.allclose(abl, full, rtol=0, atol=1e-13)
    m = O.ablation_metrics(abl, full)
    assert np.allclose(m["rel_l2_row"], 0.0, atol=1e-12)
    assert np.allclose(m["cos_row"], 1.0, atol=1e-12)


def test_one_kept_key_gives_its_value():
    rng = np.random.default_rng(1)
    q, k, v = rng.standard_normal((4, 8)), rng.standard_normal((30, 8)), rng.standard_normal((30, 8))
    for lo, hi, j in ((0, 29, 29), (1, 30, 0)):
        abl = O.ablated_output(q, k, v, scale=1.0, drop=(lo, hi))
        assert np.array_equal(abl, np.broadcast_to(v[j], abl.shape))


def test_nothing_kept_is_rejected():
    z = np.zeros((3, 4))
    with pytest.raises(ValueError):
        O.ablated_output(z, z, z, scale=1.0, drop=(0, 3))


@pytest.mark.parametrize("name", list(DROPS))
def test_zero_query_closed_form(name):
    """Q = 0 leaves only the key bias in the scores, so O is a bias-weighted mean of the kept values:
    weight 1 on sink and recent keys, e^0.5 on current keys."""
    rng = np.random.default_rng(2)
    v = rng.standard_normal((SK, 4))
    k = rng.standard_normal((SK, 4))
    lo, hi = DROPS[name]
    abl = O.ablated_output(np.zeros((2, 4)), k, v, scale=0.1, key_bias=_video_bias(), drop=(lo, hi))
    num, den = np.zeros(4), 0.0
    for j in range(SK):
        if lo <= j < hi:
            continue
        w = math.exp(0.5) if j >= 3900 else 1.0
        num += w * v[j]
        den += w
    assert np.allclose(abl, num / den, rtol=1e-12, atol=1e-14)


def test_brute_force_tiny():
    rng = np.random.default_rng(3)
    q, k, v = rng.standard_normal((3, 5)), rng.standard_normal((12, 5)), rng.standard_normal((12, 5))
    bias = rng.standard_normal(12)
    abl = O.ablated_output(q, k, v, scale=0.7, key_bias=bias, drop=(2, 6))
    for i in range(3):
        w = [math.exp(0.7 * sum(q[i, c] * k[j, c] for c in range(5)) + bias[j]) if not 2 <= j < 6 else 0.0
             for j in range(12)]
        z = sum(w)
        ref = [sum(w[j] * v[j, c] for j in range(12)) / z for c in range(5)]
        assert np.allclose(abl[i], ref, rtol=1e-12, atol=1e-14)


def test_large_negative_bias_encodes_the_drop_exactly():
    """A bias of -1e4 on the dropped keys makes their exponentials underflow to exactly 0 (in float64
    and in float32), so softmax over all keys with that bias is the renormalised softmax over the kept
    keys: the encoding the library uses for the ablation."""
    rng = np.random.default_rng(4)
    q, k, v = rng.standard_normal((6, 16)), rng.standard_normal((64, 16)), rng.standard_normal((64, 16))
    bias = rng.standard_normal(64)
    for lo, hi in ((0, 16), (16, 40), (0, 40)):
        b2 = bias.copy()
        b2[lo:hi] += -1.0e4
        via_bias = O.row_stats(q, k, scale=0.25, key_bias=b2, v=v)["o"]
        abl = O.ablated_output(q, k, v, scale=0.25, key_bias=bias, drop=(lo, hi))
        assert np.allclose(via_bias, abl, rtol=1e-13, atol=1e-14)
        assert np.float32(np.exp(np.float32(-1.0e4 + 40.0))) == 0.0


def test_cosine_and_rel_l2_identities():
    rng = np.random.default_rng(5)
    a = rng.standard_normal((7, 9))
    b = rng.standard_normal((7, 9))
    assert np.allclose(O.cosine_rows(a, 3.0 * a), 1.0, atol=1e-14)
    assert np.allclose(O.cosine_rows(a, -0.5 * a), -1.0, atol=1e-14)
    e = np.eye(9)
    assert np.allclose(O.cosine_rows(e[:3], e[3:6]), 0.0, atol=0)
    assert O.cosine_rows(np.zeros((1, 9)), a[:1])[0] == 0.0
    # |a - b|^2 = |a|^2 + |b|^2 - 2 |a| |b| cos
    na, nb = np.linalg.norm(a, axis=1), np.linalg.norm(b, axis=1)
    lhs = (O.rel_l2_rows(a, b) * nb) ** 2
    rhs = na ** 2 + nb ** 2 - 2 * na * nb * O.cosine_rows(a, b)
    assert np.allclose(lhs, rhs, rtol=1e-12)
    m = O.ablation_metrics(a, b)
    assert m["rel_l2"] == pytest.approx(math.sqrt(((a - b) ** 2).sum() / (b ** 2).sum()), rel=1e-13)
    assert m["cos"] == pytest.approx((a * b).sum() / math.sqrt((a * a).sum() * (b * b).sum()), rel=1e-13)
