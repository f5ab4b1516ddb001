"""GPU parity of kvprof_row_stats on every row of wider cases, through the C ABI.

Beyond the row samples of test_gpu_rowstats: every row of several 16-row blocks with a ragged last one,
GQA, a key count that is not a multiple of 16 or 32, per-key random bias, causal rows, regions and key
frames whose boundaries fall inside key tiles, rows from near-uniform to very peaked in one block, and
all 32 heads of a full sampled video record (3,072 rows x 6,240 keys) with the heatmap compared to the
oracle's definition on the oracle's frame masses and the histograms compared bin by bin."""
import numpy as np
import pytest
import torch

from oracle import kvprof_oracle as O
from quantized_kv_amd import binding as B
from quantized_kv_amd import inputs
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ALL = ("support", "top_mass", "top32", "strict_zero", "row_max", "row_lse", "region_mass", "frame_mass")


def _np(d):
    return {k: v.detach().cpu().numpy() for k, v in d.items() if isinstance(v, torch.Tensor)}


def _check(g, Q, K, *, Hkv, scale, **kw):
    Bn, Hq, Mq, _ = Q.shape
    grp = Hq // Hkv
    qv, kv = inputs.bf16_values(Q), inputs.bf16_values(K)
    for b in range(Bn):
        for h in range(Hq):
            ref = O.row_stats(qv[b, h], kv[b, h // grp], scale=scale, **kw)
            gh = {k: v.reshape((Bn, Hq, Mq) + v.shape[1:])[b, h] for k, v in g.items()
                  if k not in ("heatmap", "heatmap_mean", "hist")}
            P.check_rows(gh, ref)


@pytest.mark.parametrize("causal", [False, True])
def test_wide_ragged_gqa_bias_causal(kvprof_lib, causal):
    Bn, Hq, Hkv, Mq, Sk = 2, 4, 2, 61, 1500
    print(f"wide case causal={causal} B={Bn} Hq={Hq} Hkv={Hkv} Mq={Mq} Sk={Sk}", flush=True)
    Q, K, _ = inputs.generic_inputs(51, (Bn, Hq, Mq, 128), (Bn, Hkv, Sk, 128), q_scale=2.0)
    bias = (np.random.default_rng(52).standard_normal(Sk) * 0.7).astype(np.float32)
    rb = [0, 400, 901, Sk]
    groups = (np.arange(Mq) % 3).astype(np.int32)
    kw = dict(key_bias=bias, causal=causal, q_pos0=Sk - Mq - 5, region_bounds=rb, frame_len=150, n_frames=10)
    g = B.run(Q.to(DEV), K.to(DEV), want=ALL, scale=0.09, heatmap=True, hist=True,
              row_group=torch.from_numpy(groups).to(DEV), n_groups=3,
              **{**kw, "key_bias": torch.from_numpy(bias).to(DEV)})
    torch.cuda.synchronize()
    gn = _np(g)
    _check(gn, Q, K, Hkv=Hkv, scale=0.09, **kw)
    fm = gn["frame_mass"].reshape(Bn, Hq, Mq, 10)
    for b in range(Bn):
        for h in range(Hq):
            P.check_close("heatmap", gn["heatmap"][b, h], O.heatmap(fm[b, h], groups, 3), atol=1e-6)


def test_wide_uniform_bias_exact_fit(kvprof_lib):
    """96 rows per (batch, KV head) and 1,024 keys: one full workgroup each, no bias, no regions."""
    Q, K, _ = inputs.generic_inputs(53, (1, 2, 96, 128), (1, 2, 1024, 128), q_scale=1.0)
    print("wide case uniform 96x1024", flush=True)
    g = _np(B.run(Q.to(DEV), K.to(DEV), want=ALL[:6], scale=128 ** -0.5))
    torch.cuda.synchronize()
    _check(g, Q, K, Hkv=2, scale=128 ** -0.5)


def test_wide_wide_and_flat_rows(kvprof_lib):
    """Rows from near-uniform (tiny temperature) to very peaked (large temperature) in one workgroup,
    with the video key bias: the histogram window and reference moves of the streaming path."""
    rng = np.random.default_rng(54)
    Sk = 2048
    k = rng.standard_normal((1, 1, Sk, 128)).astype(np.float32)
    tau = np.geomspace(0.02, 12.0, 96).astype(np.float32)
    q = rng.standard_normal((1, 1, 96, 128)).astype(np.float32) * tau[None, None, :, None]
    Q, K = inputs.to_bf16(q), inputs.to_bf16(k)
    bias = np.where(np.arange(Sk) >= 1400, 0.5, 0.0).astype(np.float32)
    print("wide case wide/flat rows", flush=True)
    g = _np(B.run(Q.to(DEV), K.to(DEV), want=ALL[:6] + ("region_mass",), scale=128 ** -0.5,
                  key_bias=torch.from_numpy(bias).to(DEV), region_bounds=[0, 700, 1400, Sk]))
    torch.cuda.synchronize()
    _check(g, Q, K, Hkv=1, scale=128 ** -0.5, key_bias=bias, region_bounds=[0, 700, 1400, Sk])


def test_wide_video_record_all_heads(kvprof_lib):
    """Sampled-query record 0 at full size, every one of the 32 heads against the oracle, with the
    heatmap compared to the oracle's definition on the oracle's frame masses and the histograms
    compared bin by bin (rows within the mass tolerance of a bin edge may move one bin)."""
    rec = inputs.video_record(0, with_v=False, sampled=True)
    bias = inputs.video_key_bias()
    groups = inputs.video_sample_groups()
    kw = dict(region_bounds=inputs.VIDEO_REGION_BOUNDS, frame_len=inputs.LF_TOKENS, n_frames=inputs.N_KEY_FRAMES)
    print("wide case video record 0, 32 heads", flush=True)
    g = _np(B.run(rec.q[None].to(DEV), rec.k[None].to(DEV), want=ALL, scale=128 ** -0.5,
                  key_bias=torch.from_numpy(bias).to(DEV), row_group=torch.from_numpy(groups).to(DEV),
                  n_groups=6, heatmap=True, hist=True, **kw))
    torch.cuda.synchronize()
    qv, kv = inputs.bf16_values(rec.q), inputs.bf16_values(rec.k)
    sup, reg = [], []
    for h in range(32):
        ref = O.row_stats(qv[h], kv[h], scale=128 ** -0.5, key_bias=bias, **kw)
        gh = {k: v.reshape((32, 96) + v.shape[1:])[h] for k, v in g.items()
              if k not in ("heatmap", "heatmap_mean", "hist")}
        P.check_rows(gh, ref)
        P.check_close("heatmap", g["heatmap"][0, h], O.heatmap(ref["frame_mass"], groups, 6), atol=2e-3)
        sup.append(ref["support"])
        reg.append(ref["region_mass"])
    sup, reg = np.concatenate(sup), np.concatenate(reg)
    for col, vals, tol in [(0, sup, 1e-3 * sup)] + [(1 + q, reg[:, q], 2e-3) for q in range(3)]:
        want = O.histogram100(vals)
        lo = O.histogram100(np.clip(vals - tol, 0, 1))
        hi = O.histogram100(np.clip(vals + tol, 0, 1))
        got = g["hist"][0, col]
        assert got.sum() == 3072 and want.sum() == 3072
        # rows below each bin edge: at least as many as with every value raised by the tolerance, at
        # most as many as with every value lowered by it
        assert np.all(np.cumsum(hi) <= np.cumsum(got)) and np.all(np.cumsum(got) <= np.cumsum(lo)), col


def test_wide_full_rows_one_head(kvprof_lib):
    """One head of full-row record 0 (2,340 queries x 6,240 keys), every row against the oracle, and the
    record's support / region-mass histograms of that head compared bin by bin (rows within the
    tolerance of a bin edge may move one bin)."""
    rec = inputs.video_record(0, heads=1, with_v=False)
    bias = inputs.video_key_bias()
    kw = dict(region_bounds=inputs.VIDEO_REGION_BOUNDS, frame_len=inputs.LF_TOKENS, n_frames=inputs.N_KEY_FRAMES)
    print("wide case full rows, one head", flush=True)
    g = _np(B.run(rec.q[None].to(DEV), rec.k[None].to(DEV), want=ALL, scale=128 ** -0.5,
                  key_bias=torch.from_numpy(bias).to(DEV), hist=True, **kw))
    torch.cuda.synchronize()
    qv, kv = inputs.bf16_values(rec.q), inputs.bf16_values(rec.k)
    ref = O.row_stats(qv[0], kv[0], scale=128 ** -0.5, key_bias=bias, **kw)
    gh = {k: v for k, v in g.items() if k != "hist"}
    P.check_rows(gh, ref)
    for col, vals, tol in [(0, ref["support"], 1e-3 * ref["support"])] + \
            [(1 + q, ref["region_mass"][:, q], 2e-3) for q in range(3)]:
        lo = O.histogram100(np.clip(vals - tol, 0, 1))
        hi = O.histogram100(np.clip(vals + tol, 0, 1))
        got = g["hist"][0, col]
        assert got.sum() == 2340
        assert np.all(np.cumsum(hi) <= np.cumsum(got)) and np.all(np.cumsum(got) <= np.cumsum(lo)), col
