"""The MXFP8 probability path rounds each probability to the E4M3 grid with a branch-free form (round
the float32 mantissa to 3 bits on the bit pattern, or onto the 2^-9 grid below 2^-6). This CPU test
restates that form in numpy and checks it against the oracle's E4M3 encode and decode ("Catnip Week
10 KV Cache Attention Study", experiment design, MXFP8 E4M3 elements) on sampled float32 values and
on every rounding tie and carry boundary of the format."""
import numpy as np

from oracle import kvprof_oracle as O


def grid_rounding(v: np.ndarray) -> np.ndarray:
    a = np.abs(v).astype(np.float32)
    ab = a.view(np.uint32).astype(np.uint64)
    nrm = (((ab + 0x7FFFF + ((ab >> 20) & 1)) & 0xFFF00000).astype(np.uint32)).view(np.float32)
    sub = (np.rint(a * np.float32(512.0)) * np.float32(2.0 ** -9)).astype(np.float32)
    return np.copysign(np.where(a < np.float32(2.0 ** -6), sub, nrm), v).astype(np.float32)


def reference(v: np.ndarray) -> np.ndarray:
    return np.array([O.e4m3_decode(O.e4m3_encode(float(x))) for x in v], dtype=np.float32)


def test_sampled_values():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 0x43E00001, size=60000, dtype=np.uint32)  # |v| <= 448
    v = bits.view(np.float32)
    v = np.concatenate([v, -v[:5000]])
    assert np.array_equal(grid_rounding(v).view(np.uint32), reference(v).view(np.uint32))


def test_ties_and_carries():
    vals = []
    for e in range(-6, 9):  # normal binades of E4M3 (2^-6 .. 2^8)
        for keep in range(8):
            base = (e + 127) << 23 | keep << 20
            for rem in (0, 1, 0x7FFFF, 0x80000, 0x80001, 0xFFFFF):
                vals.append(base | rem)
    v = np.array(vals, dtype=np.uint32).view(np.float32)
    v = v[np.abs(v) <= 448]
    sub = (np.arange(0, 8 * 4 + 1, dtype=np.float32) / np.float32(4.0)) * np.float32(2.0 ** -9)  # quarter steps below 2^-6
    v = np.concatenate([v, sub, -v, np.float32([0.0, -0.0, 448.0])])
    got, want = grid_rounding(v), reference(v)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
