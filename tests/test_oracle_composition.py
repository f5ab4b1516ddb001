"""Pins of the oracle's composed functions: row_stats' top-f masses and mx_row_stats as a whole.

The pieces (top_mass, pack_mxfp8, p_path, tv_distance, argmax_low) have their own pins; these tests
check that the composed functions wire them as the pages define ("Catnip Week 10 KV Cache Attention
Study", the Effective MXFP8 definition and the section on Q/K and probability quantization): every
statistic of the MX mode is taken on the MX row, TV and the reference argmax against the unrotated
bf16 row, and the P-path on the MX probabilities. A brute-force recomputation on a tiny head rebuilds
every output from the definitions with independent arithmetic (torch's E4M3 cast, plain Python loops).
"""
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import kvprof_oracle as O
from quantized_kv_amd import inputs


def _bf16(a):
    return inputs.bf16_values(inputs.to_bf16(np.asarray(a, dtype=np.float32)))


def _brute_top_mass(p, pct):
    """Largest sum over floor(k)-subsets plus frac(k) times the next-largest value, by enumeration."""
    n = len(p)
    kf, rem = divmod(n * pct, 100)
    best = max((sum(p[list(c)]) for c in itertools.combinations(range(n), kf)), default=0.0)
    if kf >= n:
        return best
    best1 = max(sum(p[list(c)]) for c in itertools.combinations(range(n), kf + 1))
    return best + (rem / 100.0) * (best1 - best)


@pytest.mark.parametrize("causal", [False, True])
def test_row_stats_top_mass_is_top_mass(causal):
    rng = np.random.default_rng(11)
    q = _bf16(rng.standard_normal((7, 32)) * 2)
    k = _bf16(rng.standard_normal((150, 32)))
    bias = rng.standard_normal(150) * 0.5
    res = O.row_stats(q, k, scale=0.2, key_bias=bias, causal=causal, q_pos0=3)
    for i in range(q.shape[0]):
        n = int(res["n_visible"][i])
        want = [O.top_mass(res["p"][i], n, pct) for pct in O.TOP_PCTS]
        assert list(res["top_mass"][i]) == want


def test_row_stats_top_mass_brute_force_tiny_rows():
    rng = np.random.default_rng(12)
    q = _bf16(rng.standard_normal((3, 8)) * 3)
    k = _bf16(rng.standard_normal((14, 8)))
    res = O.row_stats(q, k, scale=0.5, causal=True, q_pos0=9)  # rows see 10, 11, 12 keys
    for i in range(3):
        n = int(res["n_visible"][i])
        p = res["p"][i][:n]
        for t, pct in enumerate(O.TOP_PCTS):
            assert res["top_mass"][i][t] == pytest.approx(_brute_top_mass(p, pct), abs=1e-12)
    # uniform rows give exactly the fraction, at fractional k too (1.28 / 6.4 / 12.8 keys at n=128)
    res = O.row_stats(np.zeros((1, 8)), k[:1].repeat(128, 0), scale=1.0)
    assert res["top_mass"][0] == pytest.approx([0.01, 0.05, 0.10], abs=1e-15)


def _torch_e4m3_value(v):
    return float(torch.tensor([v], dtype=torch.float32).to(torch.float8_e4m3fn).to(torch.float64)[0])


def _brute_mx_values(x, signs):
    """Rotation by the dense matrix, then per-32 blocks: the smallest e with amax <= 448 2^e, each
    element rounded by torch's E4M3 cast of y 2^-e (all |y 2^-e| <= 448), times 2^e."""
    d = x.shape[1]
    H = np.ones((1, 1))
    while H.shape[0] < d:
        H = np.block([[H, H], [H, -H]])
    y = x if signs is None else ((x * signs) @ H * float.fromhex("0x1.6a09e667f3bccp-4")).astype(np.float32)
    y = np.asarray(y, dtype=np.float64)
    out = np.zeros_like(y)
    for r in range(y.shape[0]):
        for b in range(0, d, 32):
            blk = y[r, b:b + 32]
            amax = float(np.max(np.abs(blk)))
            e = -127
            while e < 127 and amax > 448.0 * 2.0 ** e:
                e += 1
            for c in range(blk.shape[0]):
                out[r, b + c] = _torch_e4m3_value(blk[c] * 2.0 ** -e) * 2.0 ** e
    return out


def _brute_p_path(p32):
    """P-path by hand: p rounded to float32, per-32 block exponent by the same rule, torch E4M3 cast."""
    ph = np.zeros_like(p32)
    for b in range(0, len(p32), 32):
        blk = p32[b:b + 32]
        amax = float(np.max(blk))
        e = -127
        while e < 127 and amax > 448.0 * 2.0 ** e:
            e += 1
        for c in range(blk.shape[0]):
            ph[b + c] = _torch_e4m3_value(blk[c] * 2.0 ** -e) * 2.0 ** e
    return ph


def test_mx_row_stats_brute_force_tiny():
    rng = np.random.default_rng(13)
    d, mq, sk = 128, 3, 45  # a partial last 32-key block on the P-path
    q = _bf16(rng.standard_normal((mq, d)) * 2)
    k = _bf16(rng.standard_normal((sk, d)))
    signs = inputs.hadamard_signs(4)
    scale = 1 / math.sqrt(d)
    bias = np.where(np.arange(sk) >= 30, 0.5, 0.0)
    res = O.mx_row_stats(q, k, signs, scale=scale, key_bias=bias, region_bounds=[0, 20, 45],
                         frame_len=15, n_frames=3)
    qd, kd = _brute_mx_values(q, signs), _brute_mx_values(k, signs)
    for i in range(mq):
        s_mx = [scale * sum(qd[i, c] * kd[j, c] for c in range(d)) + bias[j] for j in range(sk)]
        s_rf = [scale * sum(q[i, c] * k[j, c] for c in range(d)) + bias[j] for j in range(sk)]
        for s_row, key in ((s_mx, "scores"), (s_rf, "ref_scores")):
            assert np.allclose(res[key][i], s_row, rtol=1e-12, atol=1e-12)
        m_mx, m_rf = max(s_mx), max(s_rf)
        z_mx = sum(math.exp(s - m_mx) for s in s_mx)
        z_rf = sum(math.exp(s - m_rf) for s in s_rf)
        p_mx = [math.exp(s - m_mx) / z_mx for s in s_mx]
        p_rf = [math.exp(s - m_rf) / z_rf for s in s_rf]
        # statistics of the MX row
        H = -sum(p * math.log(p) for p in p_mx if p > 0)
        assert res["support"][i] == pytest.approx(math.exp(H) / sk, rel=1e-12)
        assert res["region_mass"][i] == pytest.approx([sum(p_mx[:20]), sum(p_mx[20:])], abs=1e-12)
        assert res["frame_mass"][i] == pytest.approx([sum(p_mx[f * 15:(f + 1) * 15]) for f in range(3)], abs=1e-12)
        order = sorted(range(sk), key=lambda j: (-s_mx[j], j))
        assert [int(x) for x in res["top32"][i]] == order[:32]
        # TV and argmax against the unrotated bf16 row
        assert res["tv_qk"][i] == pytest.approx(0.5 * sum(abs(a - b) for a, b in zip(p_mx, p_rf)), abs=1e-12)
        assert res["argmax"][i] == order[0]
        assert res["argmax_ref"][i] == min(range(sk), key=lambda j: (-s_rf[j], j))
        # P-path on the MX probabilities
        p32 = np.array(p_mx, dtype=np.float32).astype(np.float64)
        ph = _brute_p_path(p32)
        assert res["p_zero_frac"][i] == pytest.approx(sum(1 for a, b in zip(p32, ph) if a > 0 and b == 0) / sk, abs=0)
        assert res["tv_p"][i] == pytest.approx(0.5 * sum(abs(a - b) for a, b in zip(ph, p_mx)), abs=1e-12)
        assert res["p_rowsum"][i] == pytest.approx(float(np.sum(ph)), abs=1e-12)


def test_mx_row_stats_representable_without_rotation():
    """Q/K already exact in E4M3 blocks with a 448 2^-8 element per block, no rotation: the MX row is
    the bf16 row, so TV = 0 and both argmaxes agree; the P-path equals p_path of the MX row."""
    rng = np.random.default_rng(14)
    grid = np.array([O.e4m3_decode(c) for c in range(0, 0x7E) if O.e4m3_decode(c) * 2.0 ** -8 == _bf16([O.e4m3_decode(c) * 2.0 ** -8])[0]])
    q = rng.choice(grid, (5, 128)) * 2.0 ** -8 * rng.choice([-1, 1], (5, 128))
    k = rng.choice(grid, (70, 128)) * 2.0 ** -8 * rng.choice([-1, 1], (70, 128))
    q[:, ::32] = 448 * 2.0 ** -8
    k[:, ::32] = 448 * 2.0 ** -8
    assert np.array_equal(_bf16(q), q) and np.array_equal(_bf16(k), k)
    res = O.mx_row_stats(q, k, None, scale=0.05)
    assert np.array_equal(res["scores"], res["ref_scores"])
    assert np.all(res["tv_qk"] == 0.0)
    assert np.array_equal(res["argmax"], res["argmax_ref"])
    for i in range(5):
        assert (res["p_zero_frac"][i], res["tv_p"][i], res["p_rowsum"][i]) == O.p_path(res["p"][i], 70)


def test_mx_row_stats_wiring_is_not_swapped():
    """With rotation on random data the MX and reference rows differ. Each output must come from its
    own row: swapping the reference for the rotated copy, running the P-path on p_ref, or taking the
    argmax on the other score matrix would each fail one of these assertions."""
    rng = np.random.default_rng(15)
    q = _bf16(rng.standard_normal((40, 128)) * 2.5)
    k = _bf16(rng.standard_normal((96, 128)))
    signs = inputs.hadamard_signs(4)
    res = O.mx_row_stats(q, k, signs, scale=1 / math.sqrt(128))
    # the reference row is the unrotated bf16 product, bit for bit
    assert np.array_equal(res["ref_scores"], O.scores(q, k, 1 / math.sqrt(128)))
    rot = O.signed_hadamard_rotate(q, signs) @ O.signed_hadamard_rotate(k, signs).T / math.sqrt(128)
    assert not np.array_equal(res["ref_scores"], rot)
    assert np.all(res["tv_qk"] > 0)
    diff_argmax = 0
    diff_path = 0
    for i in range(40):
        assert res["argmax"][i] == O.argmax_low(res["scores"][i], 96)
        assert res["argmax_ref"][i] == O.argmax_low(res["ref_scores"][i], 96)
        diff_argmax += O.argmax_low(res["scores"][i], 96) != O.argmax_low(res["ref_scores"][i], 96)
        mine = O.p_path(res["p"][i], 96)
        assert (res["p_zero_frac"][i], res["tv_p"][i], res["p_rowsum"][i]) == mine
        diff_path += mine != O.p_path(res["ref_p"][i], 96)
        assert res["tv_qk"][i] == O.tv_distance(res["p"][i], res["ref_p"][i])
    assert diff_argmax > 0 and diff_path > 0  # the data tell the rows apart
