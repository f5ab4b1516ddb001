"""Pins of the rolling residual window (P2 "適用邊界": KIVI-style movement of the oldest float32 tokens
into the grouped 4-bit part) and of the short-head attention protocol's oracle pieces."""
import numpy as np
import pytest

from oracle import kvprof_oracle as O
from quantized_kv_amd import inputs


def _kv(seed, n, d):
    rng = np.random.default_rng(seed)
    k = inputs.bf16_values(inputs.to_bf16(rng.standard_normal((n, d), dtype=np.float32)))
    v = inputs.bf16_values(inputs.to_bf16(rng.standard_normal((n, d), dtype=np.float32)))
    return k, v


def test_rolled_window_rule():
    assert O.rolled_window(16, 0, 16) == 16
    assert O.rolled_window(16, 31, 16) == 47       # below R + 32: nothing moves
    assert O.rolled_window(16, 32, 16) == 16       # one whole group moves
    assert O.rolled_window(16, 100, 16) == 20      # 116 -> three groups move
    assert O.rolled_window(0, 5, 0) == 5
    assert O.rolled_window(0, 64, 0) == 0
    for r_in in range(0, 80, 7):
        for t in range(0, 100, 9):
            r = O.rolled_window(r_in, t, 16)
            assert (r_in + t - r) % 32 == 0 and r <= r_in + t
            assert r_in + t < 48 or 16 <= r < 48


@pytest.mark.parametrize("d", [32, 64])
@pytest.mark.parametrize("n0,r0,t,R", [(64, 0, 1, 16), (64, 16, 40, 16), (32, 47, 1, 16), (96, 20, 77, 16),
                                       (0, 0, 128, 0), (64, 64, 0, 16), (128, 3, 200, 64)])
def test_append_equals_one_shot_pack(d, n0, r0, t, R):
    """Appending to a packed head gives exactly the blob that packing every token at once with the
    resulting window gives: the moved tokens are quantized from their float32 copies, which hold the
    bf16 values exactly."""
    N0 = n0 + r0
    k, v = _kv(7 + n0 + t, N0 + t, d)
    blob = O.pack_int4kv(k[:N0], v[:N0], r0)
    out = O.int4kv_append(blob, k[N0:], v[N0:], R)
    r_out = O.rolled_window(r0, t, R)
    assert np.array_equal(out, O.pack_int4kv(k, v, r_out))


def test_token_by_token_matches_pack():
    d, R = 32, 16
    k, v = _kv(11, 150, d)
    blob = O.pack_int4kv(k[:0], v[:0], 0)
    for i in range(150):
        blob = O.int4kv_append(blob, k[i:i + 1], v[i:i + 1], R)
        r = int(blob[8:12].view("<i4")[0])
        assert np.array_equal(blob, O.pack_int4kv(k[:i + 1], v[:i + 1], r)), i
        if i + 1 >= R + 32:
            assert R <= r < R + 32


def test_append_rejects_partial_groups():
    k, v = _kv(3, 128, 32)
    with pytest.raises(ValueError):
        O.int4kv_append(O.pack_int4kv(k, v, 16), k[:1], v[:1], 16)  # 112 = 3.5 groups
