"""GPU parity of the quantized modes: MXFP8 row statistics (tiny workload) and attention over the
packed 4-bit KV cache with the float32 recent window (decode-shaped GQA workload)."""
import numpy as np
import pytest
import torch

from oracle import kvprof_oracle as O
from quantized_kv_amd import binding as B
from quantized_kv_amd import inputs
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _np(d):
    return {k: v.detach().cpu().numpy() for k, v in d.items() if isinstance(v, torch.Tensor)}


def _check_zero_frac(got, p_ref, n):
    """Zero fraction of the P path: exact count except keys whose fp32 probability sits within the
    tie margin of the E4M3 underflow boundary (or in a block whose shared exponent is itself at a
    boundary)."""
    for r in range(len(got)):
        p32 = p_ref[r].astype(np.float32).astype(np.float64)
        lo = hi = 0
        for b0 in range(0, n, 32):
            blk = p32[b0:b0 + 32]
            amax = blk.max()
            e = O.e8m0_exponent(float(amax))
            edge = any(abs(amax - 448 * 2.0 ** ee) <= 1e-5 * amax for ee in (e - 1, e))
            x = blk * 2.0 ** -e
            zero = (blk > 0) & (x <= 2.0 ** -10)
            near = np.abs(x - 2.0 ** -10) <= 1e-5 * 2.0 ** -10
            if edge:
                hi += int(np.sum(blk > 0))
            else:
                lo += int(np.sum(zero & ~near))
                hi += int(np.sum(zero | near))
        cnt = int(round(got[r] * n))
        assert lo <= cnt <= hi, (r, cnt, lo, hi)


def _check_argmax(got, scores, name):
    for r in range(len(got)):
        srt = np.sort(scores[r])[::-1]
        if abs(srt[0] - srt[1]) < P.tie_margin(srt[0], srt[1]):
            continue
        assert got[r] == scores[r].argmax(), (name, r)


def test_mxfp8_tiny(kvprof_lib):
    Q, K, _ = inputs.tiny_inputs(1)
    signs = inputs.hadamard_signs(4)
    sg = torch.from_numpy(signs).to(DEV)
    qd, kd = Q.to(DEV), K.to(DEV)
    qc, qs = B.kvprof_pack_mxfp8(qd.reshape(-1, 128), sg)
    kc, ks = B.kvprof_pack_mxfp8(kd.reshape(-1, 128), sg)
    rb = [0, inputs.TINY_EARLY, inputs.TINY_N]
    want = ("support", "top_mass", "top32", "strict_zero", "region_mass", "tv_qk", "argmax", "argmax_ref",
            "p_zero_frac", "tv_p", "p_rowsum")
    g = _np(B.run(qd, kd, want=want, mode=B.MODE_MXFP8, q_codes=qc, q_scales=qs, k_codes=kc, k_scales=ks,
                  region_bounds=rb))
    torch.cuda.synchronize()
    for var in range(3):
        sl = slice(var * 128, (var + 1) * 128)
        ref = O.mx_row_stats(inputs.bf16_values(Q[var, 0]), inputs.bf16_values(K[var, 0]), signs,
                             scale=128 ** -0.5, region_bounds=rb)
        gv = {k: v[sl] for k, v in g.items()}
        P.check_rows(gv, ref)
        P.check_close("tv_qk", gv["tv_qk"], ref["tv_qk"], atol=P.MASS_ATOL)
        P.check_close("tv_p", gv["tv_p"], ref["tv_p"], atol=P.MASS_ATOL)
        P.check_close("p_rowsum", gv["p_rowsum"], ref["p_rowsum"], atol=P.MASS_ATOL)
        _check_zero_frac(gv["p_zero_frac"], ref["p"], 128)
        for name, sc in (("argmax", ref["scores"]), ("argmax_ref", ref["ref_scores"])):
            _check_argmax(gv[name], sc, name)
            assert np.array_equal(ref[name], sc.argmax(axis=1))  # the oracle's own argmax: lowest index


@pytest.mark.parametrize("R", [0, 16, 64])
def test_attend_int4_decode(kvprof_lib, R):
    Q, K, V = inputs.decode_inputs(5)
    L, Mq = inputs.DECODE_L, inputs.DECODE_MQ
    packed = B.kvprof_pack_int4kv(K.to(DEV), V.to(DEV), R)
    rb = [0, L - R, L] if R > 0 else None
    kw = dict(causal=True, q_pos0=L - Mq, region_bounds=rb)
    want = ("top32", "o") + (("region_mass",) if R else ())
    gq = _np(B.run(Q[None].to(DEV), None, want=want, attend=True, mode=B.MODE_INT4KV, kv_packed=packed,
                   r_window=R, n_k=L, n_heads_kv=2, **kw))
    gr = _np(B.run(Q[None].to(DEV), K[None].to(DEV), V[None].to(DEV), want=want, attend=True, **kw))
    torch.cuda.synchronize()
    qv = inputs.bf16_values(Q)
    # the oracle unpacks the blobs it packs itself (the codec parity test pins them to the device's)
    blobs = [O.pack_int4kv(inputs.bf16_values(K[h]), inputs.bf16_values(V[h]), R) for h in range(2)]
    assert all(np.array_equal(bl, dev) for bl, dev in zip(blobs, packed.cpu().numpy()))
    khat, vhat = zip(*[O.unpack_int4kv(bl) for bl in blobs])
    kref, vref = inputs.bf16_values(K), inputs.bf16_values(V)
    rows = np.r_[0:8, 120:128, 248:256]
    for h in (0, 7, 8, 15):
        sl = slice(h * Mq, (h + 1) * Mq)
        refq = O.row_stats(qv[h], khat[h // 8], scale=128 ** -0.5, causal=True, q_pos0=L - Mq,
                           region_bounds=rb, v=vhat[h // 8])
        refr = O.row_stats(qv[h], kref[h // 8], scale=128 ** -0.5, causal=True, q_pos0=L - Mq,
                           region_bounds=rb, v=vref[h // 8])
        for which, g, ref in (("int4", gq, refq), ("bf16", gr, refr)):
            print(f"decode R={R} head {h} {which}", flush=True)
            gh = {k: v[sl][rows] for k, v in g.items()}
            rh = {k: (v[rows] if getattr(v, "ndim", 0) >= 1 and len(v) == Mq else v) for k, v in ref.items()}
            P.check_top32(gh["top32"], rh["scores"], rh["n_visible"])
            P.check_o(gh["o"], rh["o"])
            if R:
                P.check_close("recent mass", gh["region_mass"][:, 1], rh["region_mass"][:, 1], atol=P.MASS_ATOL)
    # comparison kernel: relative L2 and recall@32 of the GPU outputs
    rel, rec, sums = B.kvprof_compare(torch.from_numpy(gq["o"]).to(DEV), torch.from_numpy(gr["o"]).to(DEV),
                                      torch.from_numpy(gq["top32"]).to(DEV), torch.from_numpy(gr["top32"]).to(DEV))
    torch.cuda.synchronize()
    rel, rec, sums = rel.cpu().numpy(), rec.cpu().numpy(), sums.cpu().numpy()
    ref_rel = np.linalg.norm(gq["o"].astype(np.float64) - gr["o"], axis=1) / np.linalg.norm(gr["o"].astype(np.float64), axis=1)
    assert np.allclose(rel, ref_rel, rtol=1e-5)
    ref_rec = np.array([O.recall32(a, b) for a, b in zip(gq["top32"], gr["top32"])])
    assert np.array_equal(rec, ref_rec.astype(np.float32))
    tensor_rel = np.sqrt(sums[0] / sums[1])
    assert tensor_rel == pytest.approx(O.rel_l2(gq["o"].astype(np.float64), gr["o"].astype(np.float64)), rel=1e-6)
    if R == 0:
        assert 0.02 < tensor_rel < 0.3  # 4-bit K/V: error of the order of ten percent


def test_mxfp8_video_sampled(kvprof_lib):
    """MXFP8 mode at the video shape (6,240 keys, bias, regions, frames): two heads of sampled record
    0 on the GPU, the oracle on 16 rows of each."""
    rec = inputs.video_record(0, with_v=False, sampled=True)
    heads = [0, 13]
    Q, K = rec.q[heads][None], rec.k[heads][None]  # [1, 2, 96, 128], [1, 2, 6240, 128]
    signs = inputs.hadamard_signs(4)
    sg = torch.from_numpy(signs).to(DEV)
    qd, kd = Q.to(DEV), K.to(DEV)
    qc, qs = B.kvprof_pack_mxfp8(qd.reshape(-1, 128), sg)
    kc, ks = B.kvprof_pack_mxfp8(kd.reshape(-1, 128), sg)
    bias = inputs.video_key_bias()
    kw = dict(region_bounds=inputs.VIDEO_REGION_BOUNDS, frame_len=inputs.LF_TOKENS, n_frames=inputs.N_KEY_FRAMES)
    want = ("support", "top_mass", "top32", "strict_zero", "region_mass", "frame_mass", "tv_qk", "argmax",
            "argmax_ref", "p_zero_frac", "tv_p", "p_rowsum")
    g = _np(B.run(qd, kd, want=want, mode=B.MODE_MXFP8, q_codes=qc, q_scales=qs, k_codes=kc, k_scales=ks,
                  scale=128 ** -0.5, key_bias=torch.from_numpy(bias).to(DEV), **kw))
    torch.cuda.synchronize()
    rows = np.r_[0:8, 88:96]
    qv, kv = inputs.bf16_values(Q[0]), inputs.bf16_values(K[0])
    for hi in range(2):
        ref = O.mx_row_stats(qv[hi][rows], kv[hi], signs, scale=128 ** -0.5, key_bias=bias, **kw)
        gv = {k: v[hi * 96:(hi + 1) * 96][rows] for k, v in g.items()}
        P.check_rows(gv, ref)
        P.check_close("tv_qk", gv["tv_qk"], ref["tv_qk"], atol=P.MASS_ATOL)
        P.check_close("tv_p", gv["tv_p"], ref["tv_p"], atol=P.MASS_ATOL)
        P.check_close("p_rowsum", gv["p_rowsum"], ref["p_rowsum"], atol=P.MASS_ATOL)
        _check_zero_frac(gv["p_zero_frac"], ref["p"], kv.shape[1])
        _check_argmax(gv["argmax"], ref["scores"], "argmax")
        _check_argmax(gv["argmax_ref"], ref["ref_scores"], "argmax_ref")


def test_mxfp8_ties_and_redo(kvprof_lib):
    """MXFP8 mode with the selection's hard cases (uniform rows, one dominant key, a block of 301
    identical keys at the top-32 boundary): those row blocks go through the redo kernel, which
    recomputes the ranks; the MX comparison outputs come from the main kernel."""
    rng = np.random.default_rng(23)
    Sk = 6240
    k = rng.standard_normal((1, 1, Sk, 128)).astype(np.float32)
    k[0, 0, 100:401] = k[0, 0, 7]
    q = rng.standard_normal((1, 1, 16, 128)).astype(np.float32)
    q[0, 0, 0:4] = 0.0
    q[0, 0, 4:8] = k[0, 0, 5000] * 3.0
    q[0, 0, 8:12] = k[0, 0, 7] * 0.4
    Q, K = inputs.to_bf16(q), inputs.to_bf16(k)
    signs = inputs.hadamard_signs(4)
    sg = torch.from_numpy(signs).to(DEV)
    qd, kd = Q.to(DEV), K.to(DEV)
    qc, qs = B.kvprof_pack_mxfp8(qd.reshape(-1, 128), sg)
    kc, ks = B.kvprof_pack_mxfp8(kd.reshape(-1, 128), sg)
    bias = inputs.video_key_bias()
    kw = dict(region_bounds=inputs.VIDEO_REGION_BOUNDS, frame_len=inputs.LF_TOKENS, n_frames=inputs.N_KEY_FRAMES)
    want = ("support", "top_mass", "top32", "strict_zero", "region_mass", "frame_mass", "tv_qk", "argmax",
            "argmax_ref", "p_zero_frac", "tv_p", "p_rowsum")
    res = B.run(qd, kd, want=want, mode=B.MODE_MXFP8, q_codes=qc, q_scales=qs, k_codes=kc, k_scales=ks,
                scale=128 ** -0.5, key_bias=torch.from_numpy(bias).to(DEV), **kw)
    torch.cuda.synchronize()
    # the workspace holds the decoded MX Q (16 x 128 bf16) and K (6240 x 128 bf16), then the redo list
    ws = res["_keepalive"][1].cpu().numpy()
    assert ws[4096 + Sk * 256:][:4].view(np.uint32)[0] == 1, "the row block was not redone"
    g = _np(res)
    ref = O.mx_row_stats(inputs.bf16_values(Q)[0, 0], inputs.bf16_values(K)[0, 0], signs, scale=128 ** -0.5,
                         key_bias=bias, **kw)
    P.check_rows(g, ref)
    P.check_close("tv_qk", g["tv_qk"], ref["tv_qk"], atol=P.MASS_ATOL)
    P.check_close("tv_p", g["tv_p"], ref["tv_p"], atol=P.MASS_ATOL)
    P.check_close("p_rowsum", g["p_rowsum"], ref["p_rowsum"], atol=P.MASS_ATOL)
    _check_zero_frac(g["p_zero_frac"], ref["p"], Sk)
    _check_argmax(g["argmax"], ref["scores"], "argmax")
    _check_argmax(g["argmax_ref"], ref["ref_scores"], "argmax_ref")


def test_attend_int4_decode_batch(kvprof_lib):
    """Several sequences in one launch, one query position each (the decode step): batch b reads
    only its own packed KV heads."""
    import bench

    R, L = 16, inputs.DECODE_L
    n_seq = 3
    Q, packed = bench.decode_batch_inputs(n_seq, R, DEV)
    rb = [0, L - R, L]
    g = _np(B.run(Q, None, want=("top32", "o", "region_mass"), attend=True, mode=B.MODE_INT4KV,
                  kv_packed=packed, r_window=R, n_k=L, n_heads_kv=2, causal=True, q_pos0=L - 1, region_bounds=rb))
    torch.cuda.synchronize()
    for s in range(n_seq):
        q, k, v = inputs.decode_inputs(bench.DECODE_BATCH_SEED0 + s, mq=1)
        qv = inputs.bf16_values(q)
        for hk in range(2):
            blob = O.pack_int4kv(inputs.bf16_values(k[hk]), inputs.bf16_values(v[hk]), R)
            assert np.array_equal(blob, packed[2 * s + hk].cpu().numpy())
            khat, vhat = O.unpack_int4kv(blob)
            for h in range(8 * hk, 8 * hk + 8):
                print(f"decode batch seq {s} head {h}", flush=True)
                ref = O.row_stats(qv[h], khat, scale=128 ** -0.5, causal=True, q_pos0=L - 1, region_bounds=rb,
                                  v=vhat)
                sl = slice(s * 16 + h, s * 16 + h + 1)
                P.check_top32(g["top32"][sl], ref["scores"], ref["n_visible"])
                P.check_o(g["o"][sl], ref["o"])
                P.check_close("recent mass", g["region_mass"][sl, 1], ref["region_mass"][:, 1], atol=P.MASS_ATOL)


def test_mxfp8_blocks_below_bf16_range(kvprof_lib):
    """MXFP8 blocks whose E8M0 exponent sits at the bottom of its range (query rows and keys scaled by
    1e-36, so the E4M3 subnormals times the block scale lie below bf16's smallest subnormal) next to
    ordinary rows and keys: the kernel takes MX products on bf16-decoded operands, which cannot hold
    those values, and every statistic must still agree with the oracle's exact decode to tolerance."""
    rng = np.random.default_rng(29)
    Sk, Mq = 2048, 32
    k = rng.standard_normal((1, 1, Sk, 128)).astype(np.float32)
    q = rng.standard_normal((1, 1, Mq, 128)).astype(np.float32) * 1.5
    q[0, 0, 0:8] *= 1e-36
    k[0, 0, 500:564] *= 1e-36
    k[0, 0, 1000:1032] *= 1e-30
    Q, K = inputs.to_bf16(q), inputs.to_bf16(k)
    signs = inputs.hadamard_signs(4)
    sg = torch.from_numpy(signs).to(DEV)
    qd, kd = Q.to(DEV), K.to(DEV)
    print("MXFP8 tiny blocks", flush=True)
    qc, qs = B.kvprof_pack_mxfp8(qd.reshape(-1, 128), sg)
    kc, ks = B.kvprof_pack_mxfp8(kd.reshape(-1, 128), sg)
    assert int(qs.cpu().numpy()[:8].min()) <= 1  # E8M0 bytes: exponent + 127
    kw = dict(region_bounds=[0, 512, 1024, Sk], frame_len=128, n_frames=16)
    want = ("support", "top_mass", "top32", "strict_zero", "region_mass", "frame_mass", "tv_qk", "argmax",
            "argmax_ref", "p_zero_frac", "tv_p", "p_rowsum")
    g = _np(B.run(qd, kd, want=want, mode=B.MODE_MXFP8, q_codes=qc, q_scales=qs, k_codes=kc, k_scales=ks,
                  scale=128 ** -0.5, **kw))
    torch.cuda.synchronize()
    ref = O.mx_row_stats(inputs.bf16_values(Q)[0, 0], inputs.bf16_values(K)[0, 0], signs, scale=128 ** -0.5, **kw)
    P.check_rows(g, ref)
    P.check_close("tv_qk", g["tv_qk"], ref["tv_qk"], atol=P.MASS_ATOL)
    P.check_close("tv_p", g["tv_p"], ref["tv_p"], atol=P.MASS_ATOL)
    P.check_close("p_rowsum", g["p_rowsum"], ref["p_rowsum"], atol=P.MASS_ATOL)
    _check_zero_frac(g["p_zero_frac"], ref["p"], Sk)
    _check_argmax(g["argmax"], ref["scores"], "argmax")
    _check_argmax(g["argmax_ref"], ref["ref_scores"], "argmax_ref")


def test_mxfp8_ragged_gqa_bias(kvprof_lib):
    """MXFP8 mode with ragged shapes: 45 rows per head (the last 16-row block a third full), 1,000 keys
    (the last 16-key tile half full, so the reference sweeps stop inside a wave's range), GQA 4/2, a
    random key bias, three regions and eight frames; every row of every head against the oracle."""
    Bn, Hq, Hkv, Mq, Sk = 1, 4, 2, 45, 1000
    Q, K, _ = inputs.generic_inputs(37, (Bn, Hq, Mq, 128), (Bn, Hkv, Sk, 128), q_scale=1.3)
    bias = (np.random.default_rng(38).standard_normal(Sk) * 0.6).astype(np.float32)
    signs = inputs.hadamard_signs(4)
    sg = torch.from_numpy(signs).to(DEV)
    qd, kd = Q.to(DEV), K.to(DEV)
    print("MXFP8 ragged GQA", flush=True)
    qc, qs = B.kvprof_pack_mxfp8(qd.reshape(-1, 128), sg)
    kc, ks = B.kvprof_pack_mxfp8(kd.reshape(-1, 128), sg)
    kw = dict(region_bounds=[0, 130, 610, Sk], frame_len=125, n_frames=8)
    want = ("support", "top_mass", "top32", "strict_zero", "region_mass", "frame_mass", "tv_qk", "argmax",
            "argmax_ref", "p_zero_frac", "tv_p", "p_rowsum")
    g = _np(B.run(qd, kd, want=want, mode=B.MODE_MXFP8, q_codes=qc, q_scales=qs, k_codes=kc, k_scales=ks,
                  scale=0.1, key_bias=torch.from_numpy(bias).to(DEV), **kw))
    torch.cuda.synchronize()
    qv, kv = inputs.bf16_values(Q)[0], inputs.bf16_values(K)[0]
    for h in range(Hq):
        ref = O.mx_row_stats(qv[h], kv[h // 2], signs, scale=0.1, key_bias=bias, **kw)
        gv = {k: v[h * Mq:(h + 1) * Mq] for k, v in g.items()}
        P.check_rows(gv, ref)
        P.check_close("tv_qk", gv["tv_qk"], ref["tv_qk"], atol=P.MASS_ATOL)
        P.check_close("tv_p", gv["tv_p"], ref["tv_p"], atol=P.MASS_ATOL)
        P.check_close("p_rowsum", gv["p_rowsum"], ref["p_rowsum"], atol=P.MASS_ATOL)
        _check_zero_frac(gv["p_zero_frac"], ref["p"], Sk)
        _check_argmax(gv["argmax"], ref["scores"], "argmax")
        _check_argmax(gv["argmax_ref"], ref["ref_scores"], "argmax_ref")
