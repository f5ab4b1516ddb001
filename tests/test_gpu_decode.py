"""GPU parity of decode-shaped attention (at most 16 query rows per KV head, attention outputs only),
through the C ABI, against the oracle — on the row kernel up to 6,272 keys and on the split-key path
beyond (6,273 to 8,192 keys): O, top-32, region masses, row max and
log-sum-exp, over bf16 and packed 4-bit K/V, including the exact fallback for rows whose top-32
candidates overflow a chunk ("KV residual window": attention over the dequantized cache and the
recent-window mass; the MiniCPM5-2B predictor study, section 0: GQA decode and recall@32)."""
import numpy as np
import pytest
import torch

from oracle import kvprof_oracle as O
from quantized_kv_amd import binding as B
from quantized_kv_amd import inputs
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
WANT = ("o", "top32", "region_mass", "row_max", "row_lse")


def _np(d):
    return {k: v.detach().cpu().numpy() for k, v in d.items() if isinstance(v, torch.Tensor)}


def _check(g, qv, kv, vv, Hkv, scale, **kw):
    Bn, Hq, Mq, _ = qv.shape
    grp = Hq // Hkv
    for b in range(Bn):
        for h in range(Hq):
            ref = O.row_stats(qv[b, h], kv[b, h // grp], scale=scale, v=vv[b, h // grp], **kw)
            sl = slice((b * Hq + h) * Mq, (b * Hq + h + 1) * Mq)
            P.check_rows({k: v[sl] for k, v in g.items()}, ref)


@pytest.mark.parametrize("n_k", [2048, 3000, 7000, 8192])
def test_decode_bf16_gqa_causal_bias(kvprof_lib, n_k):
    """Two positions x 8 query heads per KV head (16 rows), causal, key bias, a ragged last chunk."""
    Bn, Hq, Hkv, Mq = 2, 16, 2, 2
    print(f"decode bf16 n_k={n_k}", flush=True)
    Q, K, V = inputs.generic_inputs(100 + n_k, (Bn, Hq, Mq, 128), (Bn, Hkv, n_k, 128), q_scale=1.5)
    bias = (np.random.default_rng(101).standard_normal(n_k) * 0.5).astype(np.float32)
    rb = [0, 700, n_k - 64, n_k]
    kw = dict(causal=True, q_pos0=n_k - Mq - 1, region_bounds=rb)
    g = _np(B.run(Q.to(DEV), K.to(DEV), V.to(DEV), want=WANT, attend=True, scale=0.09,
                  key_bias=torch.from_numpy(bias).to(DEV), **kw))
    torch.cuda.synchronize()
    _check(g, inputs.bf16_values(Q), inputs.bf16_values(K), inputs.bf16_values(V), Hkv, 0.09, key_bias=bias, **kw)


@pytest.mark.parametrize("R", [0, 16, 64])
def test_decode_int4_batch_every_window(kvprof_lib, R):
    """The batched decode step (one position per sequence, 16 query heads over 2 packed KV heads of
    4,096 keys) at every residual window, on three sequences."""
    import bench

    L, n_seq = inputs.DECODE_L, 3
    print(f"decode int4 batch R={R}", flush=True)
    Q, packed = bench.decode_batch_inputs(n_seq, R, DEV)
    rb = [0, L - R, L] if R else [0, L]
    g = _np(B.run(Q, None, want=WANT, attend=True, mode=B.MODE_INT4KV, kv_packed=packed, r_window=R, n_k=L,
                  n_heads_kv=2, causal=True, q_pos0=L - 1, region_bounds=rb))
    torch.cuda.synchronize()
    for s in range(n_seq):
        q, k, v = inputs.decode_inputs(bench.DECODE_BATCH_SEED0 + s, mq=1)
        qv = inputs.bf16_values(q)
        for hk in range(2):
            khat, vhat = O.unpack_int4kv(O.pack_int4kv(inputs.bf16_values(k[hk]), inputs.bf16_values(v[hk]), R))
            for h in range(8 * hk, 8 * hk + 8):
                ref = O.row_stats(qv[h], khat, scale=128 ** -0.5, causal=True, q_pos0=L - 1, region_bounds=rb, v=vhat)
                sl = slice(s * 16 + h, s * 16 + h + 1)
                P.check_rows({k_: v_[sl] for k_, v_ in g.items()}, ref)


def test_decode_fallback_ties_and_peaked(kvprof_lib):
    """Rows that overflow a chunk's candidate list go through the exact fallback: q = 0 makes every
    score equal (top-32 = the 32 lowest indices); a very large query scale leaves fewer than 32 keys
    within 32 log2 units of a chunk's max."""
    Bn, Hq, Hkv, Mq, n_k = 1, 8, 1, 2, 8192
    Q, K, V = inputs.generic_inputs(110, (Bn, Hq, Mq, 128), (Bn, Hkv, n_k, 128))
    q = Q.float()
    q[0, :4] = 0.0           # ties
    q[0, 4:] *= 60.0         # peaked
    Q = q.to(torch.bfloat16)
    print("decode fallback rows", flush=True)
    g = _np(B.run(Q.to(DEV), K.to(DEV), V.to(DEV), want=WANT, attend=True, scale=128 ** -0.5))
    torch.cuda.synchronize()
    assert np.array_equal(g["top32"][:8], np.tile(np.arange(32), (8, 1)))
    _check(g, inputs.bf16_values(Q), inputs.bf16_values(K), inputs.bf16_values(V), Hkv, 128 ** -0.5)


@pytest.mark.parametrize("R", [0, 16, 64])
def test_decode_int4_split_keys(kvprof_lib, R):
    """Packed 4-bit K/V of 7,000 keys (split-key path, a ragged last chunk and window) for one GQA group
    at two positions."""
    Bn, Hq, Hkv, Mq, n_k = 1, 8, 1, 2, 7000
    print(f"decode int4 split R={R}", flush=True)
    Q, K, V = inputs.generic_inputs(120 + R, (Bn, Hq, Mq, 128), (Bn, Hkv, n_k, 128))
    packed = B.kvprof_pack_int4kv(K[0].to(DEV), V[0].to(DEV), R)
    rb = [0, n_k - R, n_k] if R else [0, n_k]
    kw = dict(causal=True, q_pos0=n_k - Mq, region_bounds=rb)
    g = _np(B.run(Q.to(DEV), None, want=WANT, attend=True, mode=B.MODE_INT4KV, kv_packed=packed, r_window=R, n_k=n_k,
                  n_heads_kv=Hkv, scale=128 ** -0.5, **kw))
    torch.cuda.synchronize()
    khat, vhat = O.unpack_int4kv(O.pack_int4kv(inputs.bf16_values(K[0, 0]), inputs.bf16_values(V[0, 0]), R))
    _check(g, inputs.bf16_values(Q), khat[None, None], vhat[None, None], Hkv, 128 ** -0.5, **kw)
