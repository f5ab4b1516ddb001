"""Pins of the oracle's signed-Hadamard rotation and MXFP8 E4M3/E8M0 codec."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import kvprof_oracle as O
from quantized_kv_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_sylvester_matches_popcount_definition():
    H = O.sylvester_hadamard(128)
    i = np.arange(128)
    pc = np.vectorize(lambda x: bin(x).count("1"))(i[:, None] & i[None, :])
    assert np.array_equal(H, (-1.0) ** pc)
    assert np.array_equal(H @ H.T, 128 * np.eye(128))


def test_rotation_constant_is_nearest_double():
    c = O.ROT_C
    exact = 1 / math.sqrt(128)
    assert abs(c - exact) <= math.ulp(exact) / 2 * 1.0000001
    assert abs(c * c * 128 - 1) < 4e-16


def _fwht(x):
    """Iterative fast Walsh-Hadamard butterfly (natural order)."""
    x = x.copy()
    h = 1
    while h < x.shape[-1]:
        for i in range(0, x.shape[-1], 2 * h):
            a = x[..., i:i + h].copy()
            b = x[..., i + h:i + 2 * h].copy()
            x[..., i:i + h] = a + b
            x[..., i + h:i + 2 * h] = a - b
        h *= 2
    return x


def test_rotation_equals_butterfly_and_preserves_dots():
    signs = inputs.hadamard_signs(4)
    rng = np.random.default_rng(0)
    x = inputs.bf16_values(inputs.to_bf16(rng.standard_normal((8, 128)).astype(np.float32)))
    y = O.signed_hadamard_rotate(x, signs)
    t = _fwht(x * signs)  # exact in float64 for bf16 inputs
    assert np.array_equal(y, (t * O.ROT_C).astype(np.float32).astype(np.float64))
    R = np.diag(signs.astype(np.float64)) @ O.sylvester_hadamard(128) / math.sqrt(128)
    assert np.allclose(R @ R.T, np.eye(128), atol=1e-14)
    q, k = x[:4], x[4:]
    assert np.allclose((q @ R) @ (k @ R).T, q @ k.T, rtol=1e-12, atol=1e-12)


def _torch_e4m3(vals):
    t = torch.tensor(vals, dtype=torch.float32).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_cast():
    # every bf16 value with |v| <= 448 (covers subnormal, normal and tie cases of E4M3 rounding)
    bits = np.arange(0, 1 << 16, dtype=np.uint32) << 16
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= 448)]
    mine = np.array([O.e4m3_encode(float(v)) for v in vals], dtype=np.uint8)
    assert np.array_equal(mine, _torch_e4m3(vals))
    # random float32 values too
    r = np.random.default_rng(1).standard_normal(20000).astype(np.float32) * 30
    mine = np.array([O.e4m3_encode(float(v)) for v in r], dtype=np.uint8)
    assert np.array_equal(mine, _torch_e4m3(r))


def test_e4m3_decode_matches_torch_and_round_trips():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    mine = np.array([O.e4m3_decode(c) for c in codes])
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert np.array_equal(mine, ref.astype(np.float64))
    assert all(O.e4m3_encode(v) == c for v, c in zip(mine, codes))


def test_worked_codes():
    cases = json.load(open(os.path.join(GOLDEN, "mx_worked_codes.json")))["cases"]
    for c in cases:
        e = O.e8m0_exponent(c["amax"])
        assert e + 127 == c["scale_byte"], c
        if c["amax"] > 0:
            assert O.e4m3_encode(math.ldexp(c["value"], -e)) == c["code"], c


def test_e8m0_rule_is_smallest_non_saturating_exponent():
    rng = np.random.default_rng(2)
    for amax in np.abs(rng.standard_normal(2000)) * 10.0 ** rng.integers(-20, 20, 2000):
        e = O.e8m0_exponent(float(amax))
        assert amax <= 448 * 2.0 ** e and amax > 448 * 2.0 ** (e - 1)


def test_representable_blocks_round_trip():
    rng = np.random.default_rng(3)
    finite = [O.e4m3_decode(c) for c in range(256) if (c & 0x7F) != 0x7F]
    for e in (-20, -8, 0, 5):
        blk = np.array(rng.choice(finite, 32)) * 2.0 ** e
        blk[5] = 448 * 2.0 ** e  # fixes the block exponent at e
        codes, scales = O.mx_quantize(blk[None, :])
        assert scales[0, 0] == e + 127
        assert np.array_equal(O.mx_dequantize(codes, scales)[0], blk)


def test_mx_scores_equal_reference_on_representable_inputs():
    """Q/K built from E4M3 values with a 448-scale element per block and no rotation: the MX row
    equals the bf16 row, so TV = 0 and the argmax agrees."""
    rng = np.random.default_rng(4)
    grid = np.array([O.e4m3_decode(c) for c in range(0, 0x7E)])
    q = rng.choice(grid, (6, 128)) * 2.0 ** -8 * rng.choice([-1, 1], (6, 128))
    k = rng.choice(grid, (40, 128)) * 2.0 ** -8 * rng.choice([-1, 1], (40, 128))
    q[:, ::32] = 448 * 2.0 ** -8
    k[:, ::32] = 448 * 2.0 ** -8
    ones = np.ones(128, dtype=np.int8)
    # identity rotation: signs of +1 with H would rotate, so quantize without rotation directly
    qc, qs = O.mx_quantize(q)
    kc, ks = O.mx_quantize(k)
    assert np.array_equal(O.mx_dequantize(qc, qs), q)
    assert np.array_equal(O.mx_dequantize(kc, ks), k)
    res = O.row_stats(O.mx_dequantize(qc, qs), O.mx_dequantize(kc, ks), scale=0.1)
    ref = O.row_stats(q, k, scale=0.1)
    assert max(O.tv_distance(a, b) for a, b in zip(res["p"], ref["p"])) == 0.0
    del ones


def test_p_path_closed_forms():
    # a block that is exactly representable: TV_p = 0, row sum = 1 (values sum to one)
    p = np.zeros(64)
    p[:4] = [0.5, 0.25, 0.125, 0.125]
    z, tvp, rs = O.p_path(p, 64)
    assert tvp == 0.0 and rs == 1.0 and z == 0.0
    # block {1 - eps, 31 tiny values 2^-20}: amax -> e = -8, tiny/2^-8 = 2^-12 < 2^-10 -> zero
    p = np.full(32, 2.0 ** -20)
    p[0] = 1.0 - 31 * 2.0 ** -20
    z, tvp, rs = O.p_path(p, 32)
    assert z == pytest.approx(31 / 32)
    assert tvp == pytest.approx(0.5 * (31 * 2.0 ** -20 + abs(1.0 - p[0])), rel=1e-9)


def test_tv_distance_extremes():
    a = np.array([1.0, 0.0])
    b = np.array([0.0, 1.0])
    assert O.tv_distance(a, a) == 0.0 and O.tv_distance(a, b) == 1.0
