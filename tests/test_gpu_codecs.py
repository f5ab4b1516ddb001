"""GPU parity of the codecs through the C ABI: MXFP8 codes/scales and int4 KV blobs must be bit-exact
with the oracle."""
import numpy as np
import pytest
import torch

from oracle import kvprof_oracle as O
from quantized_kv_amd import binding as B
from quantized_kv_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _np(t):
    return t.detach().cpu().numpy()


@pytest.mark.parametrize("rotate", [True, False])
def test_pack_mxfp8_tiny_variants(kvprof_lib, rotate):
    Q, K, _ = inputs.tiny_inputs(1)
    x = torch.cat([Q.reshape(-1, 128), K.reshape(-1, 128)])  # 768 rows (all three variants)
    signs = inputs.hadamard_signs(4)
    codes, scales = B.kvprof_pack_mxfp8(x.to(DEV), torch.from_numpy(signs).to(DEV) if rotate else None)
    torch.cuda.synchronize()
    oc, os_ = O.pack_mxfp8(inputs.bf16_values(x), signs if rotate else None)
    assert np.array_equal(_np(scales), os_)
    assert np.array_equal(_np(codes), oc)
    deq = _np(B.kvprof_unpack_mxfp8(codes, scales))
    assert np.array_equal(deq.astype(np.float64), O.mx_dequantize(oc, os_))


@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_pack_mxfp8_widths_and_extremes(kvprof_lib, d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((37, d)).astype(np.float32) * 10.0 ** rng.integers(-30, 30, (37, 1))
    x[0] = 0.0  # all-zero block -> scale byte 0
    x[1, :32] = -0.0
    x[2, :] = 448.0
    signs = (2 * rng.integers(0, 2, d) - 1).astype(np.int8)
    for sg in (signs, None):
        # the sign of an exactly-zero rotated sum depends on summation order: zero rows are checked
        # without the rotation only
        xb = inputs.to_bf16(x[3:] if sg is not None else x)
        codes, scales = B.kvprof_pack_mxfp8(xb.to(DEV), None if sg is None else torch.from_numpy(sg).to(DEV))
        torch.cuda.synchronize()
        oc, os_ = O.pack_mxfp8(inputs.bf16_values(xb), sg)
        assert np.array_equal(_np(scales), os_)
        assert np.array_equal(_np(codes), oc)


def test_pack_mxfp8_many_rows(kvprof_lib):
    """More rows than one pass of the d = 128 kernel's grid covers (262,144 rows per pass): sampled
    rows from the first pass, the second pass and the ragged end."""
    rng = np.random.default_rng(7)
    n = 262144 + 37
    xb = inputs.to_bf16(rng.standard_normal((n, 128), dtype=np.float32))
    signs = inputs.hadamard_signs(4)
    codes, scales = B.kvprof_pack_mxfp8(xb.to(DEV), torch.from_numpy(signs).to(DEV))
    torch.cuda.synchronize()
    rows = np.r_[0:40, 131072:131080, 262136:n]
    oc, os_ = O.pack_mxfp8(inputs.bf16_values(xb[rows]), signs)
    assert np.array_equal(_np(scales)[rows], os_)
    assert np.array_equal(_np(codes)[rows], oc)


def test_pack_mxfp8_empty(kvprof_lib):
    codes, scales = B.kvprof_pack_mxfp8(torch.empty((0, 128), dtype=torch.bfloat16, device=DEV))
    assert codes.shape == (0, 128)


@pytest.mark.parametrize("N,d,R", [(128, 32, 0), (128, 32, 16), (128, 32, 64), (100, 64, 16),
                                   (4096, 128, 0), (4096, 128, 16), (4096, 128, 64), (64, 128, 64)])
def test_pack_int4kv_bit_exact(kvprof_lib, N, d, R):
    rng = np.random.default_rng(N * 7 + d + R)
    heads = 2
    k = inputs.to_bf16(rng.standard_normal((heads, N, d)).astype(np.float32))
    v = inputs.to_bf16(rng.standard_normal((heads, N, d)).astype(np.float32))
    blob = B.kvprof_pack_int4kv(k.to(DEV), v.to(DEV), R)
    torch.cuda.synchronize()
    assert blob.shape[1] == O.int4kv_bytes(N, d, R)
    got = _np(blob)
    for h in range(heads):
        want = O.pack_int4kv(inputs.bf16_values(k[h]), inputs.bf16_values(v[h]), R)
        assert np.array_equal(got[h], want), f"head {h}: first diff at byte {np.argmax(got[h] != want)}"
    kh, vh = B.kvprof_unpack_int4kv(blob, N, d, R)
    torch.cuda.synchronize()
    for h in range(heads):
        ok, ov = O.unpack_int4kv(got[h])
        assert np.allclose(_np(kh[h]), ok, rtol=0, atol=1e-6 * np.abs(ok).max())
        assert np.allclose(_np(vh[h]), ov, rtol=0, atol=1e-6 * np.abs(ov).max())


def test_int4_payload_pins_on_device(kvprof_lib):
    rng = np.random.default_rng(9)
    k = inputs.to_bf16(rng.standard_normal((1, 128, 32)).astype(np.float32)).to(DEV)
    for R, nbytes in ((0, 5136), (16, 8912), (64, 18960)):
        assert B.kvprof_pack_int4kv(k, k, R).shape == (1, nbytes)
