"""Comparison helpers for the GPU parity tests: the tolerances and near-tie exemptions of the
profiler's contract, applied element by element against the oracle."""
import math

import numpy as np

MASS_ATOL = 2e-3  # every probability mass, TV, zero fraction, row sum
SUPPORT_RTOL = 1e-3
O_RTOL = 1e-3  # per row, ||dO|| / ||O||
TIE_REL = 1e-5  # near-tie margin on scores


def tie_margin(*vals):
    return TIE_REL * max(1.0, *(abs(v) for v in vals if np.isfinite(v)))


def check_top32(gpu_t32, scores, nvis, rows=None):
    """Exact top-32 sets, except where the oracle's 32nd and 33rd scores are within the tie margin:
    then the GPU set must hold every key scored above the 32nd by more than the margin."""
    gpu_t32 = np.asarray(gpu_t32)
    bad = []
    for r in range(gpu_t32.shape[0]) if rows is None else rows:
        n = int(nvis[r])
        s = scores[r, :n]
        order = np.lexsort((np.arange(n), -s))
        k = min(32, n)
        g = [int(x) for x in gpu_t32[r] if x >= 0]
        if len(g) != k or len(set(g)) != k or any(x >= n for x in g) or any(x != -1 for x in gpu_t32[r][k:]):
            bad.append((r, "malformed", g))
            continue
        want = set(int(x) for x in order[:k])
        if set(g) == want:
            continue
        if n > 32:
            s32, s33 = s[order[31]], s[order[32]]
            m = tie_margin(s32, s33)
            if abs(s32 - s33) < m:
                must = set(int(j) for j in np.nonzero(s > s32 + m)[0])
                if must <= set(g) and all(s[x] >= s33 - m for x in g):
                    continue
        bad.append((r, sorted(want - set(g))[:5], sorted(set(g) - want)[:5]))
    assert not bad, f"top-32 mismatches in {len(bad)} rows, first: {bad[:3]}"


def check_order(gpu_t32, scores, nvis):
    """GPU top-32 lists are sorted by score descending (within the tie margin)."""
    for r in range(gpu_t32.shape[0]):
        g = [int(x) for x in gpu_t32[r] if x >= 0]
        sc = scores[r, g]
        for a, b in zip(sc[:-1], sc[1:]):
            assert a >= b - tie_margin(a, b), (r, a, b)


def check_strict_zero(gpu, scores, nvis):
    for r in range(len(gpu)):
        n = int(nvis[r])
        s = scores[r, :n]
        m = s.max()
        lnZ = math.log(float(np.sum(np.exp(s - m))))
        x = (s - m) - lnZ + 150 * math.log(2)
        near = np.abs(x) < TIE_REL * np.maximum(1.0, np.abs(s))
        lo = int(np.sum((x <= 0) & ~near))
        assert lo <= int(gpu[r]) <= lo + int(np.sum(near)), (r, int(gpu[r]), lo, int(np.sum(near)))


def check_close(name, gpu, ref, atol=0.0, rtol=0.0):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(gpu - ref) - (atol + rtol * np.abs(ref))
    worst = np.unravel_index(np.argmax(err), err.shape) if err.size else None
    assert err.size == 0 or err.max() <= 0, (
        f"{name}: worst at {worst}: gpu {gpu[worst]} vs oracle {ref[worst]} (atol {atol}, rtol {rtol})")


def check_o(gpu_o, ref_o):
    gpu_o = np.asarray(gpu_o, dtype=np.float64)
    num = np.linalg.norm(gpu_o - ref_o, axis=1)
    den = np.maximum(np.linalg.norm(ref_o, axis=1), 1e-30)
    rel = num / den
    assert rel.max() <= O_RTOL, f"O relative error {rel.max():.3e} at row {int(rel.argmax())}"


def check_rows(gpu, ref, rows=None, masses=True):
    """Compare the scalar row outputs of one (batch, head) against oracle.row_stats."""
    sl = slice(None) if rows is None else rows
    n = ref["n_visible"][sl]
    if "support" in gpu:
        check_close("support", gpu["support"][sl], ref["support"][sl], rtol=SUPPORT_RTOL)
    if "top_mass" in gpu:
        check_close("top_mass", gpu["top_mass"][sl], ref["top_mass"][sl], atol=MASS_ATOL)
    if "region_mass" in gpu and "region_mass" in ref:
        check_close("region_mass", gpu["region_mass"][sl], ref["region_mass"][sl], atol=MASS_ATOL)
    if "frame_mass" in gpu and "frame_mass" in ref:
        check_close("frame_mass", gpu["frame_mass"][sl], ref["frame_mass"][sl], atol=MASS_ATOL)
    if "row_max" in gpu:
        check_close("row_max", gpu["row_max"][sl], ref["row_max"][sl], atol=2e-5, rtol=2e-5)
    if "row_lse" in gpu:
        check_close("row_lse", gpu["row_lse"][sl], ref["row_lse"][sl], atol=2e-5, rtol=2e-5)
    if "top32" in gpu:
        idx = np.arange(len(n)) if rows is None else None
        check_top32(gpu["top32"][sl], ref["scores"][sl], n)
        check_order(np.asarray(gpu["top32"][sl]), ref["scores"][sl], n)
    if "strict_zero" in gpu:
        check_strict_zero(gpu["strict_zero"][sl], ref["scores"][sl], n)
    if "o" in gpu and "o" in ref:
        check_o(gpu["o"][sl], ref["o"][sl])
