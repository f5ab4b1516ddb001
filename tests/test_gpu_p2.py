"""GPU parity of the short-head attention path, the residual-window protocol and the rolling window,
through the C ABI ("KV residual window": the fixed-budget protocol at head dimension 32 — 3 seeds x 2
lengths x 3 distributions x R in {0, 16, 64}, relative L2 of the output and the reference's recent-window
mass — and the KIVI-style movement of the oldest window tokens that the study leaves out)."""
import numpy as np
import pytest
import torch

from oracle import kvprof_oracle as O
from quantized_kv_amd import binding as B
from quantized_kv_amd import inputs, p2
from tests import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SHORT = ("o", "row_max", "row_lse", "support", "region_mass")


def _np(d):
    return {k: v.detach().cpu().numpy() for k, v in d.items() if isinstance(v, torch.Tensor)}


def _attn(q, k, v, scale):
    p = O.probabilities(q, k, scale=scale)
    return p, p @ v


def test_p2_protocol_grid(kvprof_lib):
    """All 54 comparisons: every blob equals the oracle's byte for byte, every output O (reference and
    4-bit) matches the oracle's row by row, and every relative L2 and recent-window mass matches the
    oracle's value for the same input."""
    print("P2 grid", flush=True)
    summary = {}
    for variant in inputs.TINY_VARIANTS:
        for n in inputs.P2_LENGTHS:
            for seed in inputs.P2_SEEDS:
                q, k, v = inputs.p2_inputs(seed, n, variant)
                res = p2.run_case(q.to(DEV), k.to(DEV), v.to(DEV))
                qv, kv, vv = (inputs.bf16_values(t) for t in (q, k, v))
                scale = 32 ** -0.5
                p_ref, o_ref = _attn(qv, kv, vv, scale)
                P.check_o(res["o_ref"].cpu().numpy(), o_ref)
                for r in inputs.P2_WINDOWS:
                    blob = O.pack_int4kv(kv, vv, r)
                    assert np.array_equal(res["packed"][r].cpu().numpy()[0], blob), (variant, n, seed, r)
                    kh, vh = O.unpack_int4kv(blob)
                    _, o_q = _attn(qv, kh, vh, scale)
                    P.check_o(res["o"][r].cpu().numpy(), o_q)
                    want = O.rel_l2(o_q, o_ref)
                    assert abs(res["rel_l2"][r] - want) <= 5e-4 + 0.02 * want, (variant, n, seed, r, res["rel_l2"][r], want)
                    mass = float(np.mean(p_ref[:, n - r:].sum(axis=1))) if r else 0.0
                    assert abs(res["recent_mass"][r] - mass) <= 1e-5, (variant, n, seed, r)
                    summary.setdefault(variant, {}).setdefault(r, []).append((res["rel_l2"][r], res["recent_mass"][r]))
    for variant, per in summary.items():
        line = "  ".join(f"R={r}: relL2 {100 * np.mean([a for a, _ in x]):.3f}% mass {100 * np.mean([b for _, b in x]):.2f}%"
                         for r, x in per.items())
        print(f"P2 {variant:13s} {line}", flush=True)
    # the protocol's own sanity: the window helps recent_focus much more than early_focus
    rf = {r: np.mean([a for a, _ in summary["recent_focus"][r]]) for r in inputs.P2_WINDOWS}
    ef = {r: np.mean([a for a, _ in summary["early_focus"][r]]) for r in inputs.P2_WINDOWS}
    assert rf[16] < 0.5 * rf[0] and ef[16] > 0.8 * ef[0]


@pytest.mark.parametrize("d", [32, 64])
@pytest.mark.parametrize("mode", ["bf16", "int4"])
def test_short_head_parity(kvprof_lib, d, mode):
    """Short heads with GQA 4/2, 45 causal rows (ragged 16-row blocks), 1,000 keys (a ragged tile), key
    bias, three regions and the per-batch histograms, against the oracle's row statistics."""
    Bn, Hq, Hkv, Mq, Sk, R = 2, 4, 2, 45, 1000, 40
    print(f"short head d={d} mode={mode}", flush=True)
    Q, K, V = inputs.generic_inputs(70 + d, (Bn, Hq, Mq, d), (Bn, Hkv, Sk, d), q_scale=1.5)
    bias = (np.random.default_rng(71).standard_normal(Sk) * 0.5).astype(np.float32)
    rb = [0, 300, 640, Sk]
    kw = dict(causal=True, q_pos0=Sk - Mq - 5, region_bounds=rb)
    if mode == "int4":
        packed = B.kvprof_pack_int4kv(K.reshape(Bn * Hkv, Sk, d).to(DEV), V.reshape(Bn * Hkv, Sk, d).to(DEV), R)
        g = _np(B.run(Q.to(DEV), None, want=SHORT, attend=True, mode=B.MODE_INT4KV, kv_packed=packed, r_window=R,
                      n_k=Sk, n_heads_kv=Hkv, key_bias=torch.from_numpy(bias).to(DEV), scale=0.11, hist=True, **kw))
    else:
        g = _np(B.run(Q.to(DEV), K.to(DEV), V.to(DEV), want=SHORT, attend=True,
                      key_bias=torch.from_numpy(bias).to(DEV), scale=0.11, hist=True, **kw))
    torch.cuda.synchronize()
    qv, kv, vv = inputs.bf16_values(Q), inputs.bf16_values(K), inputs.bf16_values(V)
    sup, reg = [], []
    for b in range(Bn):
        for h in range(Hq):
            kk, vvv = kv[b, h // 2], vv[b, h // 2]
            if mode == "int4":
                kk, vvv = O.unpack_int4kv(O.pack_int4kv(kk, vvv, R))
            ref = O.row_stats(qv[b, h], kk, scale=0.11, key_bias=bias, v=vvv, **kw)
            sl = slice((b * Hq + h) * Mq, (b * Hq + h + 1) * Mq)
            P.check_rows({k_: v_[sl] for k_, v_ in g.items() if k_ != "hist"}, ref)
            sup.append(ref["support"])
            reg.append(ref["region_mass"])
    hist = g["hist"].reshape(Bn, 4, 100)
    sup = np.concatenate(sup).reshape(Bn, -1)
    reg = np.concatenate(reg).reshape(Bn, -1, 3)
    for b in range(Bn):
        assert hist[b].sum(axis=1).tolist() == [Hq * Mq] * 4
        for col, vals, tol in [(0, sup[b], 1e-3 * sup[b])] + [(1 + q, reg[b][:, q], 2e-3) for q in range(3)]:
            lo = O.histogram100(np.clip(vals - tol, 0, 1))
            hi = O.histogram100(np.clip(vals + tol, 0, 1))
            got = hist[b, col]
            assert np.all(np.cumsum(hi) <= np.cumsum(got)) and np.all(np.cumsum(got) <= np.cumsum(lo)), (b, col)


@pytest.mark.parametrize("d,n0,r0,t,R", [(32, 64, 16, 40, 16), (32, 96, 20, 77, 16), (64, 0, 0, 200, 64),
                                         (32, 128, 0, 0, 16), (64, 32, 47, 1, 16)])
def test_rolling_append(kvprof_lib, d, n0, r0, t, R):
    """Appending to packed heads on the GPU gives the blobs of the oracle's rolling append and of the
    library's own one-shot pack with the new window, byte for byte."""
    heads, N0 = 3, n0 + r0
    print(f"append d={d} n0={n0} r0={r0} t={t} R={R}", flush=True)
    _, K, V = inputs.generic_inputs(80 + t, (1, 1, 1, d), (heads, N0 + t, d))
    Kd, Vd = K.to(DEV), V.to(DEV)
    packed = B.kvprof_pack_int4kv(Kd[:, :N0].contiguous(), Vd[:, :N0].contiguous(), r0)
    out, r_out = B.kvprof_int4kv_append(packed, N0, d, r0, Kd[:, N0:].contiguous(), Vd[:, N0:].contiguous(), R)
    one = B.kvprof_pack_int4kv(Kd, Vd, r_out)
    torch.cuda.synchronize()
    assert r_out == O.rolled_window(r0, t, R)
    got = out.cpu().numpy()
    assert np.array_equal(got, one.cpu().numpy())
    kv, vv = inputs.bf16_values(K), inputs.bf16_values(V)
    for h in range(heads):
        want = O.int4kv_append(O.pack_int4kv(kv[h, :N0], vv[h, :N0], r0), kv[h, N0:], vv[h, N0:], R)
        assert np.array_equal(got[h], want), h


def test_rolling_token_by_token_decode(kvprof_lib):
    """Decode-style growth at head dimension 32: 100 single-token appends from 32 tokens; after each one
    the blob equals the one-shot pack and attention over it equals attention over the one-shot blob."""
    d, R, heads = 32, 16, 2
    _, K, V = inputs.generic_inputs(90, (1, 1, 1, d), (heads, 132, d))
    Q = inputs.generic_inputs(91, (1, heads, 1, d), (1, 1, 1, d))[0]
    Kd, Vd, Qd = K.to(DEV), V.to(DEV), Q.to(DEV)
    print("append token by token", flush=True)
    blob, r = B.kvprof_pack_int4kv(Kd[:, :32].contiguous(), Vd[:, :32].contiguous(), 0), 0
    for n in range(32, 132):
        blob, r = B.kvprof_int4kv_append(blob, n, d, r, Kd[:, n:n + 1].contiguous(), Vd[:, n:n + 1].contiguous(), R)
        if n % 9 == 0 or n == 131:
            one = B.kvprof_pack_int4kv(Kd[:, :n + 1].contiguous(), Vd[:, :n + 1].contiguous(), r)
            a = B.run(Qd, None, want=("o",), attend=True, mode=B.MODE_INT4KV, kv_packed=blob, r_window=r, n_k=n + 1,
                      n_heads_kv=heads, scale=d ** -0.5)
            b = B.run(Qd, None, want=("o",), attend=True, mode=B.MODE_INT4KV, kv_packed=one, r_window=r, n_k=n + 1,
                      n_heads_kv=heads, scale=d ** -0.5)
            torch.cuda.synchronize()
            assert torch.equal(blob, one), n
            assert torch.equal(a["o"], b["o"]), n
            assert n + 1 < R + 32 or R <= r < R + 32


def test_p2_batched_equals_per_input(kvprof_lib):
    """The batched runner (the inputs of one length in the batch dimension of each call) gives exactly the
    per-input runner's relative L2 and recent-window mass for every input and window."""
    print("P2 batched vs per input", flush=True)
    for n in inputs.P2_LENGTHS:
        keys = [(variant, seed) for variant in inputs.TINY_VARIANTS for seed in inputs.P2_SEEDS]
        qkv = [inputs.p2_inputs(seed, n, variant) for variant, seed in keys]
        q, k, v = (torch.stack([t[j] for t in qkv]).to(DEV) for j in range(3))
        batched = p2.run_batch(q, k, v)
        for i, (variant, seed) in enumerate(keys):
            one = p2.run_case(q[i], k[i], v[i])
            for r in inputs.P2_WINDOWS:
                assert batched[i]["rel_l2"][r] == one["rel_l2"][r], (n, variant, seed, r)
                assert abs(batched[i]["recent_mass"][r] - one["recent_mass"][r]) <= 1e-12, (n, variant, seed, r)
