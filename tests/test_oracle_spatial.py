"""Pins of the oracle's spatial-heatmap functions (P1 "Temporal & spatial heatmaps", Figures 9-10; P3
run manifest: heatmap pool shape and quantile sample cap) against closed forms, hand-worked values and
library routines."""
import numpy as np
import pytest
import torch

from oracle import kvprof_oracle as O


def test_percentile_hand_worked():
    # 200 values 0..199: position 199 * 0.995 = 198.005 -> 198 + 0.005 * (199 - 198)
    assert O.percentile_linear(np.arange(200.0), 99.5) == pytest.approx(198.005, abs=1e-12)
    assert O.percentile_linear(np.array([4.0, 1.0, 3.0, 2.0]), 50) == 2.5
    assert O.percentile_linear(np.array([7.0]), 99.5) == 7.0
    # order does not matter, and the 100th percentile is the maximum
    x = np.array([0.3, 0.1, 0.9, 0.5])
    assert O.percentile_linear(x, 100) == 0.9 and O.percentile_linear(x, 0) == 0.1


@pytest.mark.parametrize("n", [1, 2, 17, 390, 6240])
def test_percentile_matches_numpy_linear(n):
    rng = np.random.default_rng(n)
    x = rng.exponential(size=n)
    for pct in (0.0, 12.5, 50.0, 99.5, 100.0):
        assert O.percentile_linear(x, pct) == pytest.approx(float(np.percentile(x, pct)), rel=1e-14, abs=1e-300)


def test_quantile_sample_cap():
    x = np.arange(10)
    assert np.array_equal(O.quantile_sample(x, cap=10), x)
    assert np.array_equal(O.quantile_sample(x, cap=4), np.array([0, 3, 6, 9]))  # stride ceil(10/4) = 3
    assert np.array_equal(O.quantile_sample(x, cap=5), np.array([0, 2, 4, 6, 8]))
    big = np.arange(2 * O.QUANTILE_SAMPLE_CAP + 1)
    s = O.quantile_sample(big)
    assert s.size == -(-big.size // 3) and s.size <= O.QUANTILE_SAMPLE_CAP and s[1] == 3


def test_region_maps_constant_scores_are_uniform():
    # equal scores: every visible key gets 1/n, so a region made of whole frames has a flat map
    fl, nf = 6, 5
    q = np.zeros((4, 8))
    k = np.zeros((fl * nf, 8))
    p = O.probabilities(q, k, scale=1.0)
    maps = O.region_spatial_maps(p, [0, fl, 3 * fl, fl * nf], fl)
    assert maps.shape == (3, fl)
    assert np.allclose(maps, 1.0 / fl, atol=0, rtol=1e-14)


def test_region_maps_hand_worked():
    # frame_len 3, two frames, regions [0, 3) and [3, 6); rows pooled before normalising
    p = np.array([[0.1, 0.2, 0.1, 0.3, 0.2, 0.1],
                  [0.0, 0.5, 0.1, 0.1, 0.1, 0.2]])
    maps = O.region_spatial_maps(p, [0, 3, 6], 3)
    assert np.allclose(maps[0], np.array([0.1, 0.7, 0.2]) / 1.0)
    assert np.allclose(maps[1], np.array([0.4, 0.3, 0.3]) / 1.0)
    # a region that does not start at a frame boundary folds by the key's cell j mod frame_len
    m2 = O.region_spatial_maps(p, [2, 5], 3)
    assert np.allclose(m2[0], np.array([0.4, 0.3, 0.2]) / 0.9)


def test_region_maps_sum_to_one_and_zero_region():
    rng = np.random.default_rng(5)
    p = rng.dirichlet(np.ones(60), size=7)
    p[:, 40:50] = 0.0
    maps = O.region_spatial_maps(p, [0, 20, 40, 50, 60], 10)
    assert np.allclose(maps[[0, 1, 3]].sum(axis=1), 1.0, atol=1e-14)
    assert np.all(maps[2] == 0.0)  # a region without mass gives a zero map


def test_key_mass_and_spatial_relation():
    rng = np.random.default_rng(6)
    p = rng.dirichlet(np.ones(48), size=5)
    km = O.key_mass(p)
    assert np.allclose(km.sum(), 5.0)
    m = O.region_spatial_maps(p, [0, 48], 12)
    assert np.allclose(m[0], km.reshape(4, 12).sum(axis=0) / 5.0)


@pytest.mark.parametrize("shape,out", [((128, 192), (64, 96)), ((96, 6240), (64, 96)), ((2340, 6240), (64, 96)),
                                       ((5, 7), (3, 4)), ((64, 96), (64, 96))])
def test_pooled_map_matches_adaptive_avg_pool(shape, out):
    rng = np.random.default_rng(shape[0] + shape[1])
    a = rng.random(shape)
    ref = torch.nn.functional.adaptive_avg_pool2d(torch.from_numpy(a)[None, None], out)[0, 0].numpy()
    assert np.allclose(O.pooled_map(a, out), ref, rtol=1e-12, atol=0)


def test_pooled_map_divisible_is_block_mean():
    a = np.arange(12 * 20, dtype=np.float64).reshape(12, 20)
    blocks = a.reshape(4, 3, 5, 4).mean(axis=(1, 3))
    assert np.array_equal(O.pooled_map(a, (4, 5)), blocks)


def test_key_frame_heatmaps_clip():
    rng = np.random.default_rng(9)
    p = rng.dirichlet(np.full(16 * 390, 0.2))
    maps, clip = O.key_frame_heatmaps(p, 390, 16)
    assert maps.shape == (16, 390)
    assert clip == pytest.approx(float(np.percentile(p, 99.5)), rel=1e-14)
    assert np.all(maps <= clip)
    flat = p.reshape(16, 390)
    below = flat <= clip
    assert np.array_equal(maps[below], flat[below])
    # about 0.5 % of the cells lie above the clip
    assert abs((~below).sum() - 0.005 * p.size) <= 1.0
