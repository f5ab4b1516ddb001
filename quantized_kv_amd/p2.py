"""The fixed-budget residual-window protocol ("KV residual window", section on the fixed budget and who
it protects): every input is attended by an unquantized bf16 reference and by the grouped 4-bit cache
with a float32 window of the last R tokens, R in {0, 16, 64}; each comparison reports the relative L2 of
the attention output over the whole input, and the reference's attention mass on the recent window.
3 seeds x 2 lengths x 3 distributions = 18 inputs, 54 comparisons, at head dimension 32.

Host orchestration only: every number comes from the library's kernels (kvprof_attend in BF16 and
INT4KV modes, kvprof_pack_int4kv, kvprof_compare) through the binding. run_case takes one input;
run_batch puts the inputs of one length into the batch dimension of each call.
"""
from __future__ import annotations

import math

from . import binding as B
from . import inputs


def run_case(q, k, v, windows=inputs.P2_WINDOWS, stream=None) -> dict:
    """q, k, v: bf16 [N, d] on the GPU. Non-causal attention over all N tokens with scale 1/sqrt(d).
    Returns {"recent_mass": {R: mean over queries of the reference mass on the last R tokens},
    "rel_l2": {R: ||O_R - O_ref|| / ||O_ref||}, "o_ref": tensor, "o": {R: tensor}, "packed": {R: tensor}}
    (tensors left on the GPU; the scalars are read after a synchronisation)."""
    import torch

    n, d = q.shape
    Q, K, V = q[None, None], k[None, None], v[None, None]
    bounds = sorted({0, n} | {n - r for r in windows if 0 < r < n})
    scale = 1.0 / math.sqrt(d)
    ref = B.run(Q, K, V, want=("o", "region_mass"), attend=True, scale=scale, region_bounds=bounds,
                stream=stream)
    out = {"o_ref": ref["o"], "o": {}, "packed": {}, "rel_l2": {}, "recent_mass": {}}
    sums = {}
    for r in windows:
        packed = B.kvprof_pack_int4kv(k[None], v[None], r, stream=stream)
        g = B.run(Q, None, want=("o",), attend=True, mode=B.MODE_INT4KV, kv_packed=packed, r_window=r, n_k=n,
                  n_heads_kv=1, scale=scale, stream=stream)
        _, _, s = B.kvprof_compare(g["o"], ref["o"], stream=stream)
        out["o"][r], out["packed"][r], sums[r] = g["o"], packed, s
    if stream is not None:
        stream.synchronize()
    else:
        torch.cuda.synchronize()
    rm = ref["region_mass"].double().mean(dim=0).cpu().tolist()  # mean over queries, per region
    for r in windows:
        s = sums[r].cpu().tolist()
        out["rel_l2"][r] = math.sqrt(s[0] / s[1]) if s[1] > 0 else 0.0
        first = bounds.index(n - r) if 0 < r <= n else len(bounds) - 1
        out["recent_mass"][r] = float(sum(rm[first:]))
    return out


def run_batch(q, k, v, windows=inputs.P2_WINDOWS, stream=None) -> list:
    """The same comparisons for several inputs of one length at once: q, k, v bf16 [nb, N, d] on the GPU,
    input i in batch entry i of each call (one reference attend, one pack and one 4-bit attend per R
    for all inputs, then one compare per input and R), one synchronisation. Returns run_case's scalars
    per input: [{"recent_mass": {R: x}, "rel_l2": {R: x}}, ...]."""
    import torch

    nb, n, d = q.shape
    Q, K, V = q[:, None], k[:, None], v[:, None]
    bounds = sorted({0, n} | {n - r for r in windows if 0 < r < n})
    scale = 1.0 / math.sqrt(d)
    ref = B.run(Q, K, V, want=("o", "region_mass"), attend=True, scale=scale, region_bounds=bounds,
                stream=stream)
    sums = {}
    for r in windows:
        packed = B.kvprof_pack_int4kv(k, v, r, stream=stream)
        g = B.run(Q, None, want=("o",), attend=True, mode=B.MODE_INT4KV, kv_packed=packed, r_window=r, n_k=n,
                  n_heads_kv=1, scale=scale, stream=stream)
        sums[r] = [B.kvprof_compare(g["o"][i * n:(i + 1) * n], ref["o"][i * n:(i + 1) * n], stream=stream)[2]
                   for i in range(nb)]
    if stream is not None:
        stream.synchronize()
    else:
        torch.cuda.synchronize()
    rm = ref["region_mass"].double().reshape(nb, n, -1).mean(dim=1).cpu().tolist()  # per input, per region
    out = []
    for i in range(nb):
        rec = {"rel_l2": {}, "recent_mass": {}}
        for r in windows:
            s = sums[r][i].cpu().tolist()
            rec["rel_l2"][r] = math.sqrt(s[0] / s[1]) if s[1] > 0 else 0.0
            first = bounds.index(n - r) if 0 < r <= n else len(bounds) - 1
            rec["recent_mass"][r] = float(sum(rm[i][first:]))
        out.append(rec)
    return out


def run_grid(seeds=inputs.P2_SEEDS, lengths=inputs.P2_LENGTHS, variants=inputs.TINY_VARIANTS,
             windows=inputs.P2_WINDOWS, device="cuda:0"):
    """All inputs of the protocol. Returns a list of records {seed, n, variant, rel_l2: {R: x},
    recent_mass: {R: x}} and the summary {variant: {"rel_l2": {R: mean}, "recent_mass": {R: mean}}} with
    means over the inputs of each distribution (equal weights)."""
    import torch

    records = []
    for n in lengths:  # the inputs of one length share each launch
        keys = [(variant, seed) for variant in variants for seed in seeds]
        qkv = [inputs.p2_inputs(seed, n, variant) for variant, seed in keys]
        q, k, v = (torch.stack([t[j] for t in qkv]).to(device) for j in range(3))
        for (variant, seed), res in zip(keys, run_batch(q, k, v, windows)):
            records.append({"seed": seed, "n": n, "variant": variant, "rel_l2": res["rel_l2"],
                            "recent_mass": res["recent_mass"]})
    summary = {}
    for variant in variants:
        recs = [r for r in records if r["variant"] == variant]
        summary[variant] = {key: {w: sum(r[key][w] for r in recs) / len(recs) for w in windows}
                            for key in ("rel_l2", "recent_mass")}
    return records, summary
