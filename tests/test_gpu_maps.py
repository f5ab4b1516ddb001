"""GPU parity of the probability maps (key mass, region-normalised key spatial maps, pooled probability
matrices, one row's probabilities) and of the percentile clip, through the C ABI, against the oracle
("Catnip Week 10 KV Cache Attention Study", "Temporal & spatial heatmaps", Figures 9-10; the run
manifest's heatmap pool shape and quantile sample cap)."""
import numpy as np
import pytest
import torch

from oracle import kvprof_oracle as O
from quantized_kv_amd import binding as B
from quantized_kv_amd import inputs
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MAPS = ("key_mass", "spatial", "spatial_mean")


def _np(d):
    return {k: v.detach().cpu().numpy() for k, v in d.items() if isinstance(v, torch.Tensor)}


def _oracle_p(Q, K, Hkv, scale, **kw):
    Bn, Hq, Mq, _ = Q.shape
    grp = Hq // Hkv
    qv, kv = inputs.bf16_values(Q), inputs.bf16_values(K)
    return [[O.probabilities(qv[b, h], kv[b, h // grp], scale=scale, **kw) for h in range(Hq)] for b in range(Bn)]


def _check_maps(g, p, rb, fl, pool, p_row):
    Bn, Hq = len(p), len(p[0])
    Mq = p[0][0].shape[0]
    for b in range(Bn):
        for h in range(Hq):
            P.check_close(f"key_mass[{b},{h}]", g["key_mass"][b, h], O.key_mass(p[b][h]), rtol=1e-4, atol=1e-9)
            P.check_close(f"spatial[{b},{h}]", g["spatial"][b, h], O.region_spatial_maps(p[b][h], rb, fl),
                          rtol=1e-4, atol=1e-7)
            if pool is not None:
                P.check_close(f"pooled[{b},{h}]", g["pooled"][b, h], O.pooled_map(p[b][h], pool), rtol=1e-3,
                              atol=1e-9)
        P.check_close(f"spatial_mean[{b}]", g["spatial_mean"][b],
                      O.region_spatial_maps(np.concatenate(p[b]), rb, fl), rtol=1e-4, atol=1e-7)
    if p_row is not None:
        b, rem = divmod(p_row, Hq * Mq)
        h, i = divmod(rem, Mq)
        P.check_close("p_row", g["p_row_out"], p[b][h][i], rtol=1e-4, atol=1e-12)


@pytest.mark.parametrize("q_pos0", [950, 100])
def test_maps_ragged_gqa_causal_bias(kvprof_lib, q_pos0):
    """45 rows (a ragged 32-row block), 1,000 keys (a ragged 32-key tile), GQA 4/2, random key bias,
    a region boundary inside a frame; with q_pos0 = 100 the last region sees no key at all."""
    Bn, Hq, Hkv, Mq, Sk = 2, 4, 2, 45, 1000
    print(f"maps ragged case q_pos0={q_pos0}", flush=True)
    Q, K, _ = inputs.generic_inputs(61, (Bn, Hq, Mq, 128), (Bn, Hkv, Sk, 128), q_scale=2.0)
    bias = (np.random.default_rng(62).standard_normal(Sk) * 0.7).astype(np.float32)
    rb, fl, pool, p_row = [0, 200, 610, Sk], 50, (16, 24), 3 * Mq + 17
    g = _np(B.run(Q.to(DEV), K.to(DEV), want=("row_lse",), scale=0.09, key_bias=torch.from_numpy(bias).to(DEV),
                  causal=True, q_pos0=q_pos0, region_bounds=rb, frame_len=fl, maps_want=MAPS, pool=pool,
                  p_row=p_row))
    torch.cuda.synchronize()
    p = _oracle_p(Q, K, Hkv, 0.09, key_bias=bias, causal=True, q_pos0=q_pos0)
    _check_maps(g, p, rb, fl, pool, p_row)
    if q_pos0 == 100:
        assert np.all(g["spatial"][:, :, 2] == 0) and np.all(g["key_mass"][:, :, 145:] == 0)


def test_maps_without_row_outputs_and_deterministic(kvprof_lib):
    """Maps alone (row_lse from the workspace), one 32-row block per head, and bitwise-identical repeats."""
    Q, K, _ = inputs.generic_inputs(63, (1, 2, 32, 128), (1, 2, 640, 128), q_scale=1.5)
    print("maps alone, repeated", flush=True)
    outs = []
    for _ in range(2):
        g = B.run(Q.to(DEV), K.to(DEV), want=(), scale=128 ** -0.5, region_bounds=[0, 320, 640], frame_len=64,
                  maps_want=MAPS, pool=(8, 10))
        torch.cuda.synchronize()
        outs.append(_np(g))
    for k in ("key_mass", "spatial", "spatial_mean", "pooled"):
        assert np.array_equal(outs[0][k], outs[1][k]), k
    p = _oracle_p(Q, K, 2, 128 ** -0.5)
    _check_maps(outs[0], p, [0, 320, 640], 64, (8, 10), None)


def test_maps_video_record_all_heads(kvprof_lib):
    """Sampled-query record 0 (32 heads x 96 queries x 6,240 keys, the current-chunk bias): key masses,
    the sink / recent / current spatial maps of every head and of the record, the 64 x 96 pooled map of
    every head, and one query's 16 key-frame maps with the 99.5th-percentile clip."""
    rec = inputs.video_record(0, with_v=False, sampled=True)
    bias = inputs.video_key_bias()
    rb, fl, nf = inputs.VIDEO_REGION_BOUNDS, inputs.LF_TOKENS, inputs.N_KEY_FRAMES
    p_row = 23 * 96 + 50
    print("maps video record 0, 32 heads", flush=True)
    g = B.run(rec.q[None].to(DEV), rec.k[None].to(DEV), want=("row_lse",), scale=128 ** -0.5,
              key_bias=torch.from_numpy(bias).to(DEV), region_bounds=rb, frame_len=fl, n_frames=nf,
              maps_want=MAPS, pool=(64, 96), p_row=p_row)
    clip, y = B.kvprof_percentile_clip(g["p_row_out"][: nf * fl].contiguous(), 99.5)
    torch.cuda.synchronize()
    gn = _np(g)
    qv, kv = inputs.bf16_values(rec.q), inputs.bf16_values(rec.k)
    p = [[O.probabilities(qv[h], kv[h], scale=128 ** -0.5, key_bias=bias) for h in range(32)]]
    _check_maps(gn, p, rb, fl, (64, 96), p_row)
    maps, want_clip = O.key_frame_heatmaps(p[0][23][50], fl, nf)
    assert abs(float(clip.item()) - want_clip) <= 1e-4 * want_clip
    P.check_close("clipped maps", y.cpu().numpy().reshape(nf, fl), maps, rtol=1e-4, atol=1e-12)


def test_maps_full_rows_one_head(kvprof_lib):
    """One head of full-row record 0 (2,340 queries): 64 x 96 pooling with overlapping row windows."""
    rec = inputs.video_record(0, heads=1, with_v=False)
    bias = inputs.video_key_bias()
    rb, fl = inputs.VIDEO_REGION_BOUNDS, inputs.LF_TOKENS
    print("maps full-row head", flush=True)
    g = _np(B.run(rec.q[None].to(DEV), rec.k[None].to(DEV), want=(), scale=128 ** -0.5,
                  key_bias=torch.from_numpy(bias).to(DEV), region_bounds=rb, frame_len=fl, maps_want=MAPS,
                  pool=(64, 96)))
    torch.cuda.synchronize()
    p = [[O.probabilities(inputs.bf16_values(rec.q)[0], inputs.bf16_values(rec.k)[0], scale=128 ** -0.5,
                          key_bias=bias)]]
    _check_maps(g, p, rb, fl, (64, 96), None)


def test_maps_no_queries(kvprof_lib):
    """n_q = 0: no key receives mass and every spatial map is zero."""
    Q = torch.zeros((1, 2, 0, 128), dtype=torch.bfloat16, device=DEV)
    K = torch.zeros((1, 2, 64, 128), dtype=torch.bfloat16, device=DEV)
    g = B.run(Q, K, want=(), region_bounds=[0, 32, 64], frame_len=16, maps_want=MAPS)
    torch.cuda.synchronize()
    for k in MAPS:
        assert torch.all(g[k] == 0), k


@pytest.mark.parametrize("n", [1, 2, 17, 6240, 65536, 65537, 200001])
def test_percentile_clip_exact(kvprof_lib, n):
    """Order statistics are exact and the interpolation runs in float64 on both sides, so the clip value
    equals the oracle's rounded to float32, bit for bit; the clipped array is min(x, clip)."""
    rng = np.random.default_rng(n)
    x = rng.standard_normal(n).astype(np.float32)
    if n > 20:
        x[::7] = x[3]  # ties
        x[5] = -0.0
    xd = torch.from_numpy(x).to(DEV)
    print(f"percentile n={n}", flush=True)
    for cap in (O.QUANTILE_SAMPLE_CAP, 1000):
        for pct in (0.0, 50.0, 99.5, 100.0):
            clip, y = B.kvprof_percentile_clip(xd, pct, cap=cap)
            torch.cuda.synchronize()
            want = np.float32(O.percentile_linear(O.quantile_sample(x.astype(np.float64), cap), pct))
            got = clip.cpu().numpy()[0]
            assert got == want, (n, cap, pct, got, want)
            assert np.array_equal(y.cpu().numpy(), np.minimum(x, got)), (n, cap, pct)
