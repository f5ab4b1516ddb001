"""GPU parity of kvprof_row_stats / kvprof_attend (bf16 mode) against the oracle, through the C ABI.

Sizes span several 16-key tiles and several 16-row workgroups with ragged tails; the video-workload
cases run at full size (6,240 keys) and compare a sample of rows the oracle can compute one by one."""
import numpy as np
import pytest
import torch

from oracle import kvprof_oracle as O
from quantized_kv_amd import binding as B
from quantized_kv_amd import inputs
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ALL = ("support", "top_mass", "top32", "strict_zero", "row_max", "row_lse")


def _np(d):
    return {k: v.detach().cpu().numpy() for k, v in d.items() if isinstance(v, torch.Tensor)}


def _head(g, b, h, Hq, Mq):
    out = {}
    for k, v in g.items():
        if k in ("heatmap", "heatmap_mean", "hist"):
            continue
        out[k] = v.reshape((-1, Hq, Mq) + v.shape[1:])[b, h]
    return out


def _compare_all(g, Q, K, V, *, scale, Hkv, heads=None, rows=None, **kw):
    Bn, Hq, Mq, _ = Q.shape
    grp = Hq // Hkv
    qv, kv = inputs.bf16_values(Q), inputs.bf16_values(K)
    vv = inputs.bf16_values(V) if V is not None else None
    for b in range(Bn):
        for h in (range(Hq) if heads is None else heads):
            qq = qv[b, h] if rows is None else qv[b, h][rows]
            ref = O.row_stats(qq, kv[b, h // grp], scale=scale, v=None if vv is None else vv[b, h // grp], **kw)
            gh = _head(g, b, h, Hq, Mq)
            if rows is not None:
                gh = {k: v[rows] for k, v in gh.items()}
            P.check_rows(gh, ref)


def test_tiny_variants_all_stats_and_o(kvprof_lib):
    Q, K, V = inputs.tiny_inputs(1)
    rb = [0, inputs.TINY_EARLY, inputs.TINY_N]
    g = B.run(Q.to(DEV), K.to(DEV), V.to(DEV), want=ALL + ("region_mass", "o"), region_bounds=rb)
    torch.cuda.synchronize()
    _compare_all(_np(g), Q, K, V, scale=128 ** -0.5, Hkv=1, region_bounds=rb)


@pytest.mark.parametrize("causal", [False, True])
def test_ragged_gqa_bias_frames_heatmap_hist(kvprof_lib, causal):
    rng = np.random.default_rng(11)
    Bn, Hq, Hkv, Mq, Sk = 2, 4, 2, 37, 1000
    Q, K, V = inputs.generic_inputs(21, (Bn, Hq, Mq, 128), (Bn, Hkv, Sk, 128), q_scale=1.5)
    bias = rng.standard_normal(Sk).astype(np.float32)
    rb = [0, 250, 600, 1000]
    groups = (np.arange(Mq) % 5).astype(np.int32)
    kw = dict(scale=0.09, key_bias=torch.from_numpy(bias).to(DEV), causal=causal, q_pos0=Sk - Mq,
              region_bounds=rb, frame_len=100, n_frames=10, row_group=torch.from_numpy(groups).to(DEV),
              n_groups=5)
    g = B.run(Q.to(DEV), K.to(DEV), V.to(DEV), want=ALL + ("region_mass", "frame_mass", "o"), heatmap=True,
              hist=True, attend=True, **kw)
    torch.cuda.synchronize()
    gn = _np(g)
    _compare_all(gn, Q, K, V, scale=0.09, Hkv=Hkv, key_bias=bias, causal=causal, q_pos0=Sk - Mq,
                 region_bounds=rb, frame_len=100, n_frames=10)
    # heatmap from the GPU's own frame masses vs the oracle's definition
    fm = gn["frame_mass"].reshape(Bn, Hq, Mq, 10)
    for b in range(Bn):
        for h in range(Hq):
            P.check_close("heatmap", gn["heatmap"][b, h], O.heatmap(fm[b, h], groups, 5), atol=1e-6)
        P.check_close("heatmap_mean", gn["heatmap_mean"][b], gn["heatmap"][b].mean(axis=0), atol=1e-6)
    # histograms: counts per record sum to its rows; bins equal the oracle's binning of the GPU values
    hs = gn["hist"]
    sup = gn["support"].reshape(Bn, -1)
    reg = gn["region_mass"].reshape(Bn, -1, 3)
    for b in range(Bn):
        assert hs[b].sum(axis=1).tolist() == [Hq * Mq] * 4
        assert np.array_equal(hs[b, 0], O.histogram100(sup[b].astype(np.float64)))
        for q in range(3):
            assert np.array_equal(hs[b, 1 + q], O.histogram100(reg[b, :, q].astype(np.float64)))


def test_special_rows(kvprof_lib):
    """Uniform rows (Q = 0), one-hot rows (strict zeros), duplicated keys (ties to low indices)."""
    Sk = 300
    rng = np.random.default_rng(5)
    q = np.zeros((1, 1, 48, 128), np.float32)
    q[0, 0, 16:] = rng.standard_normal((32, 128)) * 3
    k = rng.standard_normal((1, 1, Sk, 128)).astype(np.float32)
    k[0, 0, 100:140] = k[0, 0, 7]  # duplicates of key 7
    q[0, 0, 16:32] = k[0, 0, 7] * 4  # rows that prefer key 7 and its copies
    Q, K = inputs.to_bf16(q), inputs.to_bf16(k)
    bias = np.zeros(Sk, np.float32)
    bias[299] = 200.0  # one-hot rows for the zero-query rows ... and near-one-hot elsewhere
    for b_ in (None, bias):
        kw = {} if b_ is None else dict(key_bias=torch.from_numpy(b_).to(DEV))
        g = _np(B.run(Q.to(DEV), K.to(DEV), want=ALL, scale=0.1, **kw))
        torch.cuda.synchronize()
        ref = O.row_stats(inputs.bf16_values(Q)[0, 0], inputs.bf16_values(K)[0, 0], scale=0.1, key_bias=b_)
        P.check_rows(g, ref)
        if b_ is None:
            assert np.allclose(g["support"][:16], 1.0, atol=1e-5)
            assert np.allclose(g["top_mass"][:16], [0.01, 0.05, 0.10], atol=1e-6)
            assert (g["top32"][:16] == np.arange(32)).all()
        else:
            assert (g["strict_zero"][:16] == Sk - 1).all()


def test_deterministic(kvprof_lib):
    Q, K, V = inputs.generic_inputs(3, (1, 2, 40, 128), (1, 2, 700, 128))
    a = _np(B.run(Q.to(DEV), K.to(DEV), V.to(DEV), want=ALL + ("o",), attend=True))
    b = _np(B.run(Q.to(DEV), K.to(DEV), V.to(DEV), want=ALL + ("o",), attend=True))
    for k in a:
        assert np.array_equal(a[k], b[k]), k


VIDEO_KW = dict(region_bounds=inputs.VIDEO_REGION_BOUNDS, frame_len=inputs.LF_TOKENS,
                n_frames=inputs.N_KEY_FRAMES)


def test_video_sampled_record(kvprof_lib):
    """Sampled-query record 0 at full size (32 heads x 96 queries x 6,240 keys): every row of every head
    against the oracle, the 6 x 16 heatmap of every head and their head mean cell by cell, and the
    record's four 100-bin histograms bin by bin (each count between those of the oracle's values moved
    down and up by the statistic's tolerance)."""
    rec = inputs.video_record(0, with_v=False, sampled=True)
    bias = inputs.video_key_bias()
    groups = inputs.video_sample_groups()
    print("video record 0, all heads", flush=True)
    g = B.run(rec.q[None].to(DEV), rec.k[None].to(DEV), want=ALL + ("region_mass", "frame_mass"),
              scale=128 ** -0.5, key_bias=torch.from_numpy(bias).to(DEV),
              row_group=torch.from_numpy(groups).to(DEV), n_groups=6, heatmap=True, hist=True, **VIDEO_KW)
    torch.cuda.synchronize()
    gn = _np(g)
    qv, kv = inputs.bf16_values(rec.q), inputs.bf16_values(rec.k)
    hm = gn["heatmap"][0]
    assert hm.shape == (32, 6, 16)
    sup, reg, hms = [], [], []
    for h in range(32):
        ref = O.row_stats(qv[h], kv[h], scale=128 ** -0.5, key_bias=bias, **VIDEO_KW)
        P.check_rows(_head(gn, 0, h, 32, 96), ref)
        want_hm = O.heatmap(ref["frame_mass"], groups, 6)
        P.check_close(f"heatmap[{h}]", hm[h], want_hm, atol=P.MASS_ATOL)
        hms.append(want_hm)
        sup.append(ref["support"])
        reg.append(ref["region_mass"])
    P.check_close("heatmap_mean", gn["heatmap_mean"][0], np.mean(hms, axis=0), atol=P.MASS_ATOL)
    sup, reg = np.concatenate(sup), np.concatenate(reg)
    hist = gn["hist"][0]
    assert hist.sum(axis=1).tolist() == [3072] * 4
    for col, vals, tol in [(0, sup, P.SUPPORT_RTOL * sup)] + [(1 + q, reg[:, q], P.MASS_ATOL) for q in range(3)]:
        lo = O.histogram100(np.clip(vals - tol, 0, 1))
        hi = O.histogram100(np.clip(vals + tol, 0, 1))
        got = hist[col]
        assert np.all(np.cumsum(hi) <= np.cumsum(got)) and np.all(np.cumsum(got) <= np.cumsum(lo)), col


def test_video_full_rows_sample(kvprof_lib):
    """Full-row record 0 (2,340 queries x 6,240 keys) on 2 heads; oracle on 178 rows of each; the sampled
    workload's rows equal the full workload's rows at the grid positions (row independence)."""
    rec = inputs.video_record(0, heads=2, with_v=False)
    bias = inputs.video_key_bias()
    g = _np(B.run(rec.q[None].to(DEV), rec.k[None].to(DEV), want=ALL + ("region_mass", "frame_mass"),
                  scale=128 ** -0.5, key_bias=torch.from_numpy(bias).to(DEV), **VIDEO_KW))
    torch.cuda.synchronize()
    rows = np.r_[0:48, 1000:1040, 1490:1530, 2290:2340]  # whole and ragged 16-row blocks, start and end
    _compare_all(g, rec.q[None], rec.k[None], None, scale=128 ** -0.5, Hkv=2, rows=rows, key_bias=bias,
                 **VIDEO_KW)
    srec = inputs.video_record(0, heads=2, with_v=False, sampled=True)
    gs = _np(B.run(srec.q[None].to(DEV), srec.k[None].to(DEV), want=ALL + ("region_mass", "frame_mass"),
                   scale=128 ** -0.5, key_bias=torch.from_numpy(bias).to(DEV), **VIDEO_KW))
    torch.cuda.synchronize()
    sel = inputs.video_sample_rows()
    for k in gs:
        full = g[k].reshape((2, 2340) + g[k].shape[1:])[:, sel].reshape(gs[k].shape)
        assert np.array_equal(full, gs[k]), k


def test_video_shape_ties_and_redo(kvprof_lib):
    """Full key count (6,240) with the selection's hard cases in one workgroup: uniform rows (every
    key tied: the slow path refines down to key indices), rows dominated by one key (the threshold
    keeps too few keys: the histogram is redone over all keys), rows whose boundary bins hold a block
    of 301 identical keys, and ordinary rows."""
    rng = np.random.default_rng(17)
    Sk = 6240
    k = rng.standard_normal((1, 1, Sk, 128)).astype(np.float32)
    k[0, 0, 100:401] = k[0, 0, 7]  # 301 copies of key 7
    q = rng.standard_normal((1, 1, 16, 128)).astype(np.float32)
    q[0, 0, 0:4] = 0.0
    q[0, 0, 4:8] = k[0, 0, 5000] * 3.0
    q[0, 0, 8:12] = k[0, 0, 7] * 0.4
    Q, K = inputs.to_bf16(q), inputs.to_bf16(k)
    bias = inputs.video_key_bias()
    g = _np(B.run(Q.to(DEV), K.to(DEV), want=ALL + ("region_mass", "frame_mass"), scale=128 ** -0.5,
                  key_bias=torch.from_numpy(bias).to(DEV), **VIDEO_KW))
    torch.cuda.synchronize()
    ref = O.row_stats(inputs.bf16_values(Q)[0, 0], inputs.bf16_values(K)[0, 0], scale=128 ** -0.5,
                      key_bias=bias, **VIDEO_KW)
    P.check_rows(g, ref)


def test_video_top_mass_interpolation_bound(kvprof_lib):
    """The kernel's in-bin estimate of the top-1/5/10 % masses is used only when its error bound is
    within 4e-4; on every row of a full sampled record (32 heads x 96 queries) the masses stay within
    that bound (plus float32 summation) of the oracle's exact rank definition."""
    rec = inputs.video_record(0, with_v=False, sampled=True)
    bias = inputs.video_key_bias()
    print("top-f mass bound, video record 0", flush=True)
    g = B.run(rec.q[None].to(DEV), rec.k[None].to(DEV), want=("top_mass",), scale=128 ** -0.5,
              key_bias=torch.from_numpy(bias).to(DEV), **VIDEO_KW)
    torch.cuda.synchronize()
    got = g["top_mass"].cpu().numpy().reshape(32, 96, 3)
    qv, kv = inputs.bf16_values(rec.q), inputs.bf16_values(rec.k)
    n = kv.shape[1]
    worst = 0.0
    for h in range(32):
        p = O.probabilities(qv[h], kv[h], scale=128 ** -0.5, key_bias=bias)
        want = np.array([[O.top_mass(p[i], n, pct) for pct in O.TOP_PCTS] for i in range(p.shape[0])])
        worst = max(worst, float(np.max(np.abs(got[h] - want))))
    print(f"max |top_mass - oracle| = {worst:.2e}", flush=True)
    assert worst <= 4e-4 + 5e-6


def test_o_with_large_magnitude_v(kvprof_lib):
    """V enters the P.V product as f16 (the header states the range limit |V| < 65520): values near the
    top of that range, and mixed with tiny ones, still give O within tolerance of the oracle, in bf16
    and in 4-bit mode (whose window keeps V as float32 and whose 4-bit part decodes into f16)."""
    rng = np.random.default_rng(31)
    Mq, Sk, R = 40, 700, 64
    q = rng.standard_normal((1, 1, Mq, 128)).astype(np.float32)
    k = rng.standard_normal((1, 1, Sk, 128)).astype(np.float32)
    v = np.clip(rng.standard_normal((1, 1, Sk, 128)).astype(np.float32) * 2e4, -6e4, 6e4)
    v[..., ::3] = np.clip(v[..., ::3] * 3.0, -6e4, 6e4)
    v[..., 5::7] *= 1e-6
    Q, K, V = inputs.to_bf16(q), inputs.to_bf16(k), inputs.to_bf16(v)
    print("large-magnitude V", flush=True)
    qv, kv, vv = inputs.bf16_values(Q)[0, 0], inputs.bf16_values(K)[0, 0], inputs.bf16_values(V)[0, 0]
    g = _np(B.run(Q.to(DEV), K.to(DEV), V.to(DEV), want=("o",), attend=True, scale=128 ** -0.5, causal=True,
                  q_pos0=Sk - Mq))
    ref = O.row_stats(qv, kv, scale=128 ** -0.5, causal=True, q_pos0=Sk - Mq, v=vv)
    P.check_o(g["o"], ref["o"])
    packed = B.kvprof_pack_int4kv(K.reshape(1, Sk, 128).to(DEV), V.reshape(1, Sk, 128).to(DEV), R)
    g4 = _np(B.run(Q.to(DEV), None, want=("o",), attend=True, mode=B.MODE_INT4KV, kv_packed=packed, r_window=R,
                   n_k=Sk, n_heads_kv=1, scale=128 ** -0.5, causal=True, q_pos0=Sk - Mq))
    torch.cuda.synchronize()
    kh, vh = O.unpack_int4kv(O.pack_int4kv(kv, vv, R))
    ref4 = O.row_stats(qv, kh, scale=128 ** -0.5, causal=True, q_pos0=Sk - Mq, v=vh)
    P.check_o(g4["o"], ref4["o"])
