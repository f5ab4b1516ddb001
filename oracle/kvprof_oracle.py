"""Plain CPU oracle of the KV-cache attention row profiler (NumPy, float64).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call this module. The library and its Python binding never do, and this
module imports nothing from them. Inputs come from ``quantized_kv_amd.inputs`` (seeded generators
that hold none of the method's arithmetic) as bf16 values promoted to float64.

Each function restates a definition from the pages, cited by page title and section:

* P1 = "Catnip Week 10 KV Cache Attention Study" (cappuccino.cafe/kv-attn.html)
* P2 = "KV residual window" (huhohoo.com/zh-TW/docs/llm/kv-residual-window)
* P3 = the run manifest of the fine-grained per-head KV-cache analysis (cappuccino.cafe/kv-fine.html)
* P4 = the MiniCPM5-2B attention-predictor study (bjdmk.com.cn/news/5855973)

Where a page is silent the reading taken is stated at the function; every reading is also listed
in the repository's design notes. The code favours obviousness over speed: per-row Python loops,
full sorts, dense matrices.

Parity status: every public function is pinned by ``tests/test_oracle_*.py`` against closed forms,
brute force, library routines or the pages' printed values. No function is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

LN2 = math.log(2.0)
TOP_PCTS = (1, 5, 10)  # top-1/5/10 % mass
TOPK = 32
E4M3_MAX = 448.0
MX_BLOCK = 32
INT4_GROUP = 32


# ----------------------------------------------------------------------------------------------
# Scores, softmax and the effective-sparsity statistics (P1, "实验设计 / From production boundary
# to statistics": Structural / Effective definitions; P1 "总体结论": support as exp(H)/Sk)
# ----------------------------------------------------------------------------------------------

def visible_counts(mq: int, sk: int, causal: bool, q_pos0: int) -> np.ndarray:
    """Number of keys row i may attend to. Causal: key j is visible iff j <= q_pos0 + i."""
    if not causal:
        return np.full(mq, sk, dtype=np.int64)
    return np.clip(q_pos0 + np.arange(mq, dtype=np.int64) + 1, 0, sk)


def scores(q: np.ndarray, k: np.ndarray, scale: float, key_bias=None, causal=False, q_pos0=0):
    """s_ij = scale * q_i . k_j + b_j over all cached keys; invisible keys get -inf.

    P1 reads post-RoPE Q/K after the KV concat and forms scaled dot products; P2 uses q.k/sqrt(d).
    Reading: an optional per-key additive bias is added after scaling.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    s = scale * (q @ k.T)
    if key_bias is not None:
        s = s + np.asarray(key_bias, dtype=np.float64)[None, :]
    n = visible_counts(q.shape[0], k.shape[0], causal, q_pos0)
    mask = np.arange(k.shape[0])[None, :] >= n[:, None]
    s[mask] = -np.inf
    return s


def softmax_row(s_row: np.ndarray) -> np.ndarray:
    """Stable softmax p_j = exp(s_j - m) / sum_k exp(s_k - m); -inf entries get p = 0."""
    m = np.max(s_row)
    e = np.exp(s_row - m)
    return e / np.sum(e)


def entropy_support(p_row: np.ndarray, n: int) -> float:
    """exp(H)/n with H = -sum p ln p (natural log, 0 ln 0 = 0) over the n visible keys."""
    pz = p_row[p_row > 0]
    H = -float(np.sum(pz * np.log(pz)))
    return math.exp(H) / n


def sorted_desc(values: np.ndarray) -> np.ndarray:
    """Indices ordered by value descending, ties by lowest index first."""
    idx = np.arange(values.shape[0])
    return np.lexsort((idx, -values))


def top_mass(p_row: np.ndarray, n: int, pct: int) -> float:
    """Mass carried by the top pct % of the n visible keys.

    k = n*pct/100 is in general fractional (1.28 keys at n=128, 62.4 at n=6,240). Reading: linear
    interpolation of the sorted-mass curve, M = sum of the floor(k) largest p + frac(k) times the next
    one. It is the plain sum when k is whole, and gives exactly pct/100 on a uniform row.
    k is formed exactly in integers: floor(k) = (n*pct) // 100, frac(k) = ((n*pct) % 100) / 100.
    """
    order = sorted_desc(p_row[:n])
    ps = p_row[:n][order]
    kf = (n * pct) // 100
    frac = ((n * pct) % 100) / 100.0
    m = float(np.sum(ps[:kf]))
    if kf < n:
        m += frac * float(ps[kf])
    return m


def top32(s_row: np.ndarray, n: int) -> np.ndarray:
    """Exact top-32 key indices: order by (score descending, index ascending), first 32; -1 pads
    rows with fewer than 32 visible keys. (Top-k indices: P1 "稀疏性很大吗"; recall@32: P4 section 0.)"""
    order = sorted_desc(s_row[:n])[:TOPK]
    out = np.full(TOPK, -1, dtype=np.int64)
    out[: order.shape[0]] = order
    return out


def strict_zero_count(s_row: np.ndarray, n: int) -> int:
    """Entries of the FP32 softmax that are exactly zero (P1: "Structural" sparsity).

    Reading: an fp32 probability is exactly 0 when the exact value is at most 2^-150 (half the smallest
    fp32 subnormal, which rounds to zero). Evaluated in float64 on log-probabilities:
    (s_j - m) - ln Z <= -150 ln 2.
    """
    s = s_row[:n]
    m = np.max(s)
    lnZ = math.log(float(np.sum(np.exp(s - m))))
    return int(np.sum((s - m) - lnZ <= -150.0 * LN2))


def segment_masses(p_row: np.ndarray, bounds) -> np.ndarray:
    """Sum of p over each [bounds[i], bounds[i+1]) key range (region or frame masses; P1 sink/recent/
    current banner and "Temporal attention heatmap": the 16 key-LF masses of a row sum to 100 %)."""
    b = list(bounds)
    return np.array([float(np.sum(p_row[b[i]:b[i + 1]])) for i in range(len(b) - 1)])


def frame_bounds(frame_len: int, n_frames: int):
    return [f * frame_len for f in range(n_frames + 1)]


def row_stats(q, k, *, scale, key_bias=None, causal=False, q_pos0=0, region_bounds=None,
              frame_len=0, n_frames=0, v=None):
    """All per-row statistics of one (batch, head): q [Mq, d], k [Sk, d] (bf16 values as float64).

    Returns a dict of per-row arrays: support, top_mass [Mq,3], top32 [Mq,32], strict_zero,
    region_mass [Mq, n_regions], frame_mass [Mq, n_frames], row_max, row_lse, and o [Mq, d] when v is
    given (O = P.V; P1 recommended local output ablation, P2 output error).
    """
    s = scores(q, k, scale, key_bias, causal, q_pos0)
    mq, sk = s.shape
    n = visible_counts(mq, sk, causal, q_pos0)
    out = {k_: [] for k_ in ("support", "top_mass", "top32", "strict_zero", "region_mass",
                             "frame_mass", "row_max", "row_lse", "p")}
    for i in range(mq):
        ni = int(n[i])
        p = softmax_row(s[i])
        out["p"].append(p)
        out["support"].append(entropy_support(p[:ni], ni))
        out["top_mass"].append([top_mass(p, ni, pct) for pct in TOP_PCTS])
        out["top32"].append(top32(s[i], ni))
        out["strict_zero"].append(strict_zero_count(s[i], ni))
        if region_bounds is not None:
            out["region_mass"].append(segment_masses(p, region_bounds))
        if n_frames:
            out["frame_mass"].append(segment_masses(p, frame_bounds(frame_len, n_frames)))
        m = float(np.max(s[i, :ni]))
        out["row_max"].append(m)
        out["row_lse"].append(m + math.log(float(np.sum(np.exp(s[i, :ni] - m)))))
    res = {key: np.asarray(val) for key, val in out.items() if len(val)}
    res["n_visible"] = n
    res["scores"] = s
    if v is not None:
        res["o"] = res["p"] @ np.asarray(v, dtype=np.float64)
    return res


def heatmap(frame_mass: np.ndarray, groups: np.ndarray, n_groups: int) -> np.ndarray:
    """Temporal heatmap of one head: mean frame mass over the rows of each query group (query LF).
    (P1 Figure 2: each query-LF row of the 6x16 map sums to 100 %.)"""
    return np.stack([frame_mass[groups == g].mean(axis=0) for g in range(n_groups)])


def histogram100(x: np.ndarray) -> np.ndarray:
    """Counts over 100 equal bins of [0, 1]; bin = min(floor(100 x), 99). Reading: 100 bins so that the
    cut points P1 quotes (10/25/75/80 %) are bin edges (P1 Figure 5 distributions)."""
    b = np.minimum(np.floor(np.asarray(x, dtype=np.float64) * 100.0), 99).astype(np.int64)
    b = np.maximum(b, 0)
    return np.bincount(b, minlength=100).astype(np.int64)


# ----------------------------------------------------------------------------------------------
# Signed Hadamard-128 rotation and MXFP8 E4M3/E8M0 K32 (P1 "实验设计" step 4 and
# "Q/K 与 probability quantization 的影响": production signed-H128 + E4M3/E8M0 K32 Q/K, and the
# per-K32 E4M3/E8M0 probability path)
# ----------------------------------------------------------------------------------------------

def sylvester_hadamard(n: int) -> np.ndarray:
    """H_1 = [1], H_2m = [[H, H], [H, -H]] (entries +-1, not normalised)."""
    H = np.ones((1, 1))
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


ROT_C = float.fromhex("0x1.6a09e667f3bccp-4")  # float64 nearest to 1/sqrt(128)


def signed_hadamard_rotate(x: np.ndarray, signs: np.ndarray) -> np.ndarray:
    """y = (s . x) H / sqrt(d) per row, returned as float32 values (in a float64 array).

    Reading: the sign flip is applied to the input channels before H; the sums are exact in float64
    (bf16 inputs); the product with the float64 constant 1/sqrt(d) is rounded to float64 and then to
    float32 (round to nearest even). d must be a power of two.
    """
    d = x.shape[-1]
    H = sylvester_hadamard(d)
    t = (np.asarray(x, dtype=np.float64) * np.asarray(signs, dtype=np.float64)) @ H
    c = ROT_C if d == 128 else 1.0 / math.sqrt(d)
    return (t * c).astype(np.float32).astype(np.float64)


def e8m0_exponent(amax: float) -> int:
    """Shared block exponent: the smallest integer e with amax <= 448 * 2^e, clamped to [-127, 127];
    amax = 0 gives -127. Reading ("ceil" rule): no element of the block saturates. P1's P row-sum median
    just under 1 (0.999392) fits it."""
    if amax == 0.0:
        return -127
    e = math.frexp(amax)[1] - 1 - 10  # floor(log2 amax) - 10: certainly too small
    while amax > E4M3_MAX * math.ldexp(1.0, e):
        e += 1
    return max(-127, min(127, e))


def e4m3_encode(v: float) -> int:
    """float -> E4M3FN byte, round to nearest even. Bias 7, 3 mantissa bits, subnormal step 2^-9,
    max 448, no infinities; the sign of zero is kept (-0 -> 0x80). |v| must not exceed 448."""
    sign = 0x80 if math.copysign(1.0, v) < 0 else 0
    a = abs(v)
    if a > E4M3_MAX:
        raise ValueError("E4M3 overflow")
    if a < 2.0 ** -6:
        n = int(np.rint(a * 2.0 ** 9))  # subnormal grid, 0..8
        if n == 8:
            return sign | (1 << 3)
        return sign | n
    E = math.frexp(a)[1] - 1  # a in [2^E, 2^(E+1))
    n = int(np.rint(a / 2.0 ** (E - 3)))  # 8..16, RNE
    if n == 16:
        E, n = E + 1, 8
    ef = E + 7
    if ef > 15 or (ef == 15 and n - 8 == 7):
        raise ValueError("E4M3 overflow after rounding")
    return sign | (ef << 3) | (n - 8)


def e4m3_decode(code: int) -> float:
    c = int(code) & 0xFF
    sgn = -1.0 if c & 0x80 else 1.0
    e = (c >> 3) & 0xF
    m = c & 7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return sgn * m * 2.0 ** -9
    return sgn * (8 + m) * 2.0 ** (e - 10)


def mx_quantize(y: np.ndarray):
    """Quantize the last axis in blocks of 32 (a final partial block uses its own amax):
    scale byte = e + 127, code = E4M3(RNE(y / 2^e)). Returns (codes uint8, scales uint8)."""
    y = np.asarray(y, dtype=np.float64)
    lead = y.shape[:-1]
    n = y.shape[-1]
    nb = (n + MX_BLOCK - 1) // MX_BLOCK
    flat = y.reshape(-1, n)
    codes = np.zeros(flat.shape, dtype=np.uint8)
    scales = np.zeros((flat.shape[0], nb), dtype=np.uint8)
    for r in range(flat.shape[0]):
        for b in range(nb):
            blk = flat[r, b * MX_BLOCK:(b + 1) * MX_BLOCK]
            e = e8m0_exponent(float(np.max(np.abs(blk))))
            scales[r, b] = e + 127
            for c, val in enumerate(blk):
                codes[r, b * MX_BLOCK + c] = e4m3_encode(math.ldexp(float(val), -e))
    return codes.reshape(lead + (n,)), scales.reshape(lead + (nb,))


def mx_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Element value = E4M3 value * 2^(scale byte - 127), exact in float64."""
    codes = np.asarray(codes)
    n = codes.shape[-1]
    flat_c = codes.reshape(-1, n)
    flat_s = np.asarray(scales).reshape(flat_c.shape[0], -1)
    out = np.zeros(flat_c.shape, dtype=np.float64)
    for r in range(flat_c.shape[0]):
        for j in range(n):
            out[r, j] = math.ldexp(e4m3_decode(flat_c[r, j]), int(flat_s[r, j // MX_BLOCK]) - 127)
    return out.reshape(codes.shape)


def pack_mxfp8(x: np.ndarray, signs=None):
    """Rotate (when signs are given) and MX-quantize rows of x: returns (codes, scales)."""
    y = signed_hadamard_rotate(x, signs) if signs is not None else np.asarray(x, dtype=np.float64)
    return mx_quantize(y)


def tv_distance(p: np.ndarray, q: np.ndarray) -> float:
    """Total variation 1/2 * sum |p - q|. Reading: the standard 1/2 factor (P1 does not print it)."""
    return 0.5 * float(np.sum(np.abs(np.asarray(p) - np.asarray(q))))


def argmax_low(s_row: np.ndarray, n: int) -> int:
    """Argmax with ties to the lowest index."""
    return int(sorted_desc(s_row[:n])[0])


def p_path(p_row: np.ndarray, n: int):
    """The per-K32 E4M3/E8M0 probability path (P1 "Numerical MXFP8" and Figure 7).

    The fp32 softmax row (the page's reconstructed FP32 softmax; the quantisation decisions are taken
    on float32 values) is MX-quantized in 32-key blocks along the keys. Returns (zero_frac, tv_p,
    rowsum): the fraction of keys with p > 0 whose dequantized value is 0, 1/2 sum |P_hat - p| against
    the unquantized row, and sum P_hat (not renormalised; P1 reports its median 0.999392).
    """
    p32 = p_row[:n].astype(np.float32).astype(np.float64)
    codes, scales = mx_quantize(p32[None, :])
    ph = mx_dequantize(codes, scales)[0]
    zero_frac = float(np.sum((p32 > 0) & (ph == 0))) / n
    return zero_frac, tv_distance(ph, p_row[:n]), float(np.sum(ph))


def mx_row_stats(q, k, signs, *, scale, key_bias=None, region_bounds=None, frame_len=0, n_frames=0):
    """MX mode for one head: Q and K rotated and MX-quantized, scores from the dequantized blocks
    (products exact in float64), every statistic of ``row_stats`` on the MX row, plus TV and argmax
    agreement against the unrotated bf16 reference row, and the P-path statistics."""
    qc, qs = pack_mxfp8(q, signs)
    kc, ks = pack_mxfp8(k, signs)
    qd = mx_dequantize(qc, qs)
    kd = mx_dequantize(kc, ks)
    res = row_stats(qd, kd, scale=scale, key_bias=key_bias, region_bounds=region_bounds,
                    frame_len=frame_len, n_frames=n_frames)
    ref = row_stats(q, k, scale=scale, key_bias=key_bias)
    mq, sk = res["scores"].shape
    tv, am, amr, zf, tvp, rs = [], [], [], [], [], []
    for i in range(mq):
        tv.append(tv_distance(res["p"][i], ref["p"][i]))
        am.append(argmax_low(res["scores"][i], sk))
        amr.append(argmax_low(ref["scores"][i], sk))
        z, t, r_ = p_path(res["p"][i], sk)
        zf.append(z)
        tvp.append(t)
        rs.append(r_)
    res.update(q_codes=qc, q_scales=qs, k_codes=kc, k_scales=ks, tv_qk=np.array(tv),
               argmax=np.array(am), argmax_ref=np.array(amr), p_zero_frac=np.array(zf),
               tv_p=np.array(tvp), p_rowsum=np.array(rs), ref_scores=ref["scores"], ref_p=ref["p"])
    return res


# ----------------------------------------------------------------------------------------------
# Grouped 4-bit KV with an fp32 recent-R residual window (P2: cache = [early N-R tokens, grouped
# 4-bit | last R tokens, float32]; group 32, K per channel over token groups, V per token over
# feature groups; payload table at N=128; cut = N - R so that R = 0 stores no tail)
# ----------------------------------------------------------------------------------------------

def int4kv_bytes(n_tokens: int, d: int, r_window: int) -> int:
    """Payload of one KV head's packed blob, counting group padding, scales and the shape header:
    16 (header) + G*32*d/2 (K codes, token groups padded) + G*d*4 (K scale+min per group and channel)
    + n*d/2 (V codes) + n*ceil(d/32)*4 (V scale+min per token and feature group) + 8*R*d (fp32 K and V
    residual), with n = N - R and G = ceil(n/32)."""
    n = n_tokens - r_window
    G = -(-n // INT4_GROUP)
    return (16 + G * INT4_GROUP * d // 2 + G * d * 4 + n * d // 2 + n * (-(-d // INT4_GROUP)) * 4
            + 8 * r_window * d)


def _int4_codes(x32: np.ndarray, lo32: np.ndarray, hi32: np.ndarray):
    """Asymmetric 4-bit codes with IEEE float32 arithmetic. Reading (KIVI-style min/scale, which P2
    names): scale = fp16(fp32(hi - lo) / 15), min = fp16(lo), code = clamp(rint((x - min) / scale),
    0, 15) with round-half-even, each operation in float32; a zero scale gives code 0."""
    scale32 = (hi32 - lo32) / np.float32(15.0)
    s_h = scale32.astype(np.float16)
    m_h = lo32.astype(np.float16)
    s32 = s_h.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = (x32 - m_h.astype(np.float32)) / s32
    q = np.where(s32 == 0, np.float32(0), q)
    codes = np.clip(np.rint(q), 0, 15).astype(np.uint8)
    return codes, s_h, m_h


def _pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Two codes per byte along the last axis: low nibble = even channel, high nibble = odd."""
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def pack_int4kv(k: np.ndarray, v: np.ndarray, r_window: int) -> np.ndarray:
    """Pack one KV head (k, v: [N, d] bf16 values) into the blob layout:
    int32[4] {N, d, R, 32}; K codes [G*32][d/2]; K meta [G][d] x (fp16 scale, fp16 min);
    V codes [n][d/2]; V meta [n][d/32] x (fp16 scale, fp16 min); K residual f32 [R][d];
    V residual f32 [R][d]. K groups run over tokens per channel (pad tokens excluded from min/max,
    their codes are 0); V groups run over 32 features per token."""
    k32 = np.asarray(k, dtype=np.float32)
    v32 = np.asarray(v, dtype=np.float32)
    N, d = k32.shape
    n = N - r_window
    G = -(-n // INT4_GROUP)
    kcodes = np.zeros((G * INT4_GROUP, d), dtype=np.uint8)
    kmeta = np.zeros((G, d, 2), dtype=np.float16)
    for g in range(G):
        blk = k32[g * INT4_GROUP:min((g + 1) * INT4_GROUP, n)]  # [t, d]
        lo, hi = blk.min(axis=0), blk.max(axis=0)
        c, s_h, m_h = _int4_codes(blk, lo[None, :], hi[None, :])
        kcodes[g * INT4_GROUP:g * INT4_GROUP + blk.shape[0]] = c
        kmeta[g, :, 0] = s_h[0]
        kmeta[g, :, 1] = m_h[0]
    nfg = -(-d // INT4_GROUP)
    vcodes = np.zeros((n, d), dtype=np.uint8)
    vmeta = np.zeros((n, nfg, 2), dtype=np.float16)
    for f in range(nfg):
        blk = v32[:n, f * INT4_GROUP:(f + 1) * INT4_GROUP]  # [n, 32]
        lo, hi = blk.min(axis=1), blk.max(axis=1)
        c, s_h, m_h = _int4_codes(blk, lo[:, None], hi[:, None])
        vcodes[:, f * INT4_GROUP:(f + 1) * INT4_GROUP] = c
        vmeta[:, f, 0] = s_h[:, 0]
        vmeta[:, f, 1] = m_h[:, 0]
    parts = [np.array([N, d, r_window, INT4_GROUP], dtype="<i4").view(np.uint8),
             _pack_nibbles(kcodes).reshape(-1), kmeta.astype("<f2").view(np.uint8).reshape(-1),
             _pack_nibbles(vcodes).reshape(-1), vmeta.astype("<f2").view(np.uint8).reshape(-1),
             k32[n:].astype("<f4").view(np.uint8).reshape(-1),
             v32[n:].astype("<f4").view(np.uint8).reshape(-1)]
    blob = np.concatenate(parts)
    assert blob.size == int4kv_bytes(N, d, r_window)
    return blob


def unpack_int4kv(blob: np.ndarray):
    """Inverse of pack_int4kv: x_hat = code * scale + min (exact in float64) for the first N - R tokens,
    the fp32 residual after. Returns (k_hat, v_hat) as float64 [N, d]."""
    blob = np.asarray(blob, dtype=np.uint8)
    N, d, R, grp = (int(x) for x in blob[:16].view("<i4"))
    n = N - R
    G = -(-n // grp)
    nfg = -(-d // grp)
    off = 16

    def take(nbytes):
        nonlocal off
        out = blob[off:off + nbytes]
        off += nbytes
        return out

    kc = take(G * grp * d // 2).reshape(G * grp, d // 2)
    km = take(G * d * 4).view("<f2").reshape(G, d, 2).astype(np.float64)
    vc = take(n * d // 2).reshape(n, d // 2)
    vm = take(n * nfg * 4).view("<f2").reshape(n, nfg, 2).astype(np.float64)
    kr = take(R * d * 4).view("<f4").reshape(R, d).astype(np.float64)
    vr = take(R * d * 4).view("<f4").reshape(R, d).astype(np.float64)

    def unnib(c):
        out = np.zeros((c.shape[0], c.shape[1] * 2), dtype=np.float64)
        out[:, 0::2] = c & 0xF
        out[:, 1::2] = c >> 4
        return out

    kcodes = unnib(kc)[:n]
    tok_g = np.arange(n) // grp
    k_hat = kcodes * km[tok_g, :, 0] + km[tok_g, :, 1]
    vcodes = unnib(vc)
    feat_g = np.arange(d) // grp
    v_hat = vcodes * vm[:, feat_g, 0] + vm[:, feat_g, 1]
    return np.concatenate([k_hat, kr]), np.concatenate([v_hat, vr])


def rolled_window(r_in: int, n_new: int, r_window: int) -> int:
    """Residual length after appending n_new tokens to a window of r_in float32 tokens when the oldest
    residual tokens move to the 4-bit part in whole 32-token groups. Reading (P2 "適用邊界" names KIVI's
    residual mechanism as what the static study leaves out): the window keeps at least the last
    r_window tokens in float32, and once it holds r_window + 32 or more, its oldest tokens move in whole
    groups, so afterwards it holds between r_window and r_window + 31 tokens. Below r_window + 32 nothing
    moves."""
    r = r_in + n_new
    if r < r_window + INT4_GROUP:
        return r
    return r - INT4_GROUP * ((r - r_window) // INT4_GROUP)


def int4kv_append(blob: np.ndarray, k_new: np.ndarray, v_new: np.ndarray, r_window: int) -> np.ndarray:
    """Append tokens (k_new, v_new: [t, d] bf16 values) to one packed head with rolling re-quantisation:
    the new tokens join the float32 window; then, while the window holds more than needed (see
    rolled_window), its oldest 32 tokens become one more K group (per channel over the 32 tokens) and 32
    more V rows (per token over each 32-feature group), with the same 4-bit arithmetic as the one-shot
    pack. The 4-bit part of the input must hold whole groups ((N - R) % 32 == 0)."""
    blob = np.asarray(blob, dtype=np.uint8)
    N, d, R, grp = (int(x) for x in blob[:16].view("<i4"))
    n = N - R
    if n % grp:
        raise ValueError("the 4-bit part must hold whole 32-token groups to take more")
    G = n // grp
    nfg = -(-d // grp)
    off = 16
    sizes = [G * grp * d // 2, G * d * 4, n * d // 2, n * nfg * 4, R * d * 4, R * d * 4]
    parts = []
    for sz in sizes:
        parts.append(blob[off:off + sz])
        off += sz
    kc, km, vc, vm, kr, vr = parts
    res_k = np.concatenate([kr.view("<f4").reshape(R, d), np.asarray(k_new, dtype=np.float32).reshape(-1, d)])
    res_v = np.concatenate([vr.view("<f4").reshape(R, d), np.asarray(v_new, dtype=np.float32).reshape(-1, d)])
    t = res_k.shape[0] - R
    r_out = rolled_window(R, t, r_window)
    moved = res_k.shape[0] - r_out  # a multiple of 32
    new_kc, new_km, new_vc, new_vm = [kc], [km], [vc], [vm]
    for g0 in range(0, moved, grp):
        blk = res_k[g0:g0 + grp]
        c, s_h, m_h = _int4_codes(blk, blk.min(axis=0)[None, :], blk.max(axis=0)[None, :])
        new_kc.append(_pack_nibbles(c).reshape(-1))
        meta = np.stack([s_h[0], m_h[0]], axis=1).astype("<f2")  # [d, 2]
        new_km.append(meta.view(np.uint8).reshape(-1))
    for tok in range(moved):
        codes = np.zeros(d, dtype=np.uint8)
        meta = np.zeros((nfg, 2), dtype=np.float16)
        for f in range(nfg):
            x = res_v[tok, f * grp:(f + 1) * grp]
            c, s_h, m_h = _int4_codes(x, x.min(), x.max())
            codes[f * grp:(f + 1) * grp] = c
            meta[f] = (s_h, m_h)
        new_vc.append(_pack_nibbles(codes))
        new_vm.append(meta.astype("<f2").view(np.uint8).reshape(-1))
    head = np.array([N + t, d, r_out, grp], dtype="<i4").view(np.uint8)
    out = np.concatenate([head] + new_kc + new_km + new_vc + new_vm
                         + [res_k[moved:].astype("<f4").view(np.uint8).reshape(-1),
                            res_v[moved:].astype("<f4").view(np.uint8).reshape(-1)])
    assert out.size == int4kv_bytes(N + t, d, r_out)
    return out


def attend(q, k, v, *, scale, causal=True, q_pos0=0, region_bounds=None):
    """O = softmax(scale q k^T, causal) V for one query head, with top-32 and region masses
    (P2: attention over the whole context with the dequantized cache; the recent-window mass of the
    unquantized reference)."""
    return row_stats(q, k, scale=scale, causal=causal, q_pos0=q_pos0, region_bounds=region_bounds,
                     v=v)


def rel_l2(o_q: np.ndarray, o_ref: np.ndarray) -> float:
    """||O_q - O_ref||_F / ||O_ref||_F (P2: relative L2 of the attention output)."""
    return float(np.linalg.norm(o_q - o_ref) / np.linalg.norm(o_ref))


def recall32(t_q: np.ndarray, t_ref: np.ndarray) -> float:
    """|T_q intersect T_ref| / 32 over valid entries (P4 section 0: recall@32)."""
    a = set(int(x) for x in t_q if x >= 0)
    b = set(int(x) for x in t_ref if x >= 0)
    return len(a & b) / float(TOPK)


# ----------------------------------------------------------------------------------------------
# Local output ablation (P1, "当前判断与下一步优化空间 / Recommended sequence", first item: drop the
# sink, the recent region or all history for the same sampled Q/K/V, renormalise P, and measure the
# relative L2 and the cosine of the attention output before the output projection)
# ----------------------------------------------------------------------------------------------

def ablated_output(q, k, v, *, scale, key_bias=None, drop=(0, 0)):
    """O_i = sum_j p'_ij v_j with p' the softmax over the keys outside the index range [lo, hi) only
    (P renormalised over what is kept). Non-causal rows; at least one key must be kept."""
    lo, hi = drop
    sk = k.shape[0]
    keep = np.ones(sk, dtype=bool)
    keep[lo:hi] = False
    if not keep.any():
        raise ValueError("the ablation must keep at least one key")
    kb = None if key_bias is None else np.asarray(key_bias, dtype=np.float64)[keep]
    s = scores(q, np.asarray(k, dtype=np.float64)[keep], scale, key_bias=kb)
    out = np.empty((s.shape[0], v.shape[1]), dtype=np.float64)
    vk = np.asarray(v, dtype=np.float64)[keep]
    for i in range(s.shape[0]):
        out[i] = softmax_row(s[i]) @ vk
    return out


def cosine_rows(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Per-row cosine a_i.b_i / (|a_i| |b_i|); 0 where either row is the zero vector (reading: the page
    gives no rule for a zero output)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    out = np.zeros(a.shape[0])
    for i in range(a.shape[0]):
        na, nb = np.linalg.norm(a[i]), np.linalg.norm(b[i])
        if na > 0 and nb > 0:
            out[i] = float(a[i] @ b[i]) / (na * nb)
    return out


def rel_l2_rows(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Per-row |a_i - b_i| / |b_i| (0 where b_i is the zero vector)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    num = np.linalg.norm(a - b, axis=1)
    den = np.linalg.norm(b, axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), 0.0)


def ablation_metrics(o_abl: np.ndarray, o_full: np.ndarray) -> dict:
    """Relative L2 and cosine of the ablated output against the full one: per row and over the whole
    tensor (flattened), as P2 reports its output error per input tensor."""
    fa = np.asarray(o_abl, dtype=np.float64).ravel()
    ff = np.asarray(o_full, dtype=np.float64).ravel()
    return {"rel_l2_row": rel_l2_rows(o_abl, o_full), "cos_row": cosine_rows(o_abl, o_full),
            "rel_l2": rel_l2(fa, ff), "cos": float(fa @ ff) / (np.linalg.norm(fa) * np.linalg.norm(ff))}


# ----------------------------------------------------------------------------------------------
# Spatial heatmaps (P1 "Temporal & spatial heatmaps": Figure 9, region spatial maps normalised inside
# each region; Figure 10, a representative query's per-key-frame 15x26 maps with the colour range
# clipped at the record's 99.5th percentile. P3, the run manifest's config block: a 64x96 heatmap pool
# shape and a cap of 65,536 values on the sample a quantile statistic is taken over.)
# ----------------------------------------------------------------------------------------------

QUANTILE_SAMPLE_CAP = 65536
POOL_SHAPE = (64, 96)


def region_spatial_maps(p_rows: np.ndarray, region_bounds, frame_len: int) -> np.ndarray:
    """Key spatial preference inside each region, pooled over the given rows.

    Key j sits at latent-grid cell j mod frame_len of its frame. For region [a, b):
    map[c] = (sum over rows and over keys j in [a, b) with j mod frame_len = c of p_j) / (sum over rows
    of the region's mass). Reading: the rows' probabilities are pooled before the normalisation (the
    map of the rows' mean attention restricted to the region), so each map sums to 1; a region with no
    mass gives an all-zero map. Returns [n_regions, frame_len].
    """
    p = np.asarray(p_rows, dtype=np.float64)
    b = list(region_bounds)
    out = np.zeros((len(b) - 1, frame_len))
    for q in range(len(b) - 1):
        for j in range(b[q], b[q + 1]):
            out[q, j % frame_len] += float(np.sum(p[:, j]))
        tot = float(np.sum(out[q]))
        if tot > 0:
            out[q] /= tot
    return out


def percentile_linear(values: np.ndarray, pct: float) -> float:
    """The pct-th percentile with linear interpolation between order statistics: sort ascending,
    position pos = (n - 1) pct / 100, value = v[floor(pos)] + frac(pos) (v[floor(pos) + 1] - v[floor(pos)])."""
    v = np.sort(np.asarray(values, dtype=np.float64).ravel())
    pos = (v.size - 1) * pct / 100.0
    lo = int(math.floor(pos))
    hi = min(lo + 1, v.size - 1)
    return float(v[lo] + (pos - lo) * (v[hi] - v[lo]))


def quantile_sample(values: np.ndarray, cap: int = QUANTILE_SAMPLE_CAP) -> np.ndarray:
    """At most `cap` values for a quantile statistic. Reading: all values when there are no more than
    cap of them, otherwise every ceil(n / cap)-th value in index order (a fixed stride, so the sample is
    reproducible)."""
    v = np.asarray(values).ravel()
    if v.size <= cap:
        return v
    return v[:: -(-v.size // cap)]


def key_frame_heatmaps(p_row: np.ndarray, frame_len: int, n_frames: int, pct: float = 99.5):
    """A query's probabilities as n_frames maps of frame_len cells, clipped at the pct-th percentile of
    the record's values (Figure 10). Reading: the record is the representative query's own
    n_frames x frame_len values. Returns (maps [n_frames, frame_len] = min(p, clip), clip)."""
    p = np.asarray(p_row, dtype=np.float64)[: n_frames * frame_len].reshape(n_frames, frame_len)
    clip = percentile_linear(quantile_sample(p), pct)
    return np.minimum(p, clip), clip


def pooled_map(a: np.ndarray, shape=POOL_SHAPE) -> np.ndarray:
    """Adaptive average pooling of a [M, N] attention map to shape (H, W): cell (i, j) is the mean of
    a[floor(i M / H) : ceil((i + 1) M / H), floor(j N / W) : ceil((j + 1) N / W)]."""
    a = np.asarray(a, dtype=np.float64)
    M, N = a.shape
    H, W = shape
    out = np.zeros((H, W))
    for i in range(H):
        r0, r1 = (i * M) // H, -(-((i + 1) * M) // H)
        for j in range(W):
            c0, c1 = (j * N) // W, -(-((j + 1) * N) // W)
            out[i, j] = float(np.mean(a[r0:r1, c0:c1]))
    return out


def key_mass(p_rows: np.ndarray) -> np.ndarray:
    """Attention mass each key receives from a set of rows: sum over the rows of p_j."""
    return np.sum(np.asarray(p_rows, dtype=np.float64), axis=0)


def probabilities(q, k, *, scale, key_bias=None, causal=False, q_pos0=0) -> np.ndarray:
    """The softmax probability matrix [Mq, Sk] of one head (invisible keys 0)."""
    s = scores(q, k, scale, key_bias, causal, q_pos0)
    return np.stack([softmax_row(s[i]) for i in range(s.shape[0])])
