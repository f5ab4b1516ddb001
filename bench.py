"""Benchmark of the KV-cache attention row profiler on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload sampled|full_rows|decode|decode_batch|mx_sampled|ablation|tiny] [--no-cpu-baseline]
    python bench.py --copy-calibration     # 1 GiB device copy, for scaling the HBM byte counters

A step is one kvprof_row_stats call over the whole workload with every statistic the workload
reports, inputs already resident in HBM:

* sampled   (default): 42 records x 32 heads x 96 sampled queries against 6,240 cached keys (16 key
             frames x 390 tokens, [sink 4 | recent 6 | current 6] frames), +0.5 current-chunk bias;
             support, top-1/5/10 % mass, top-32 indices, strict zeros, region and frame masses,
             row max / lse, the 6x16 per-head temporal heatmaps and per-record histograms.
* full_rows: the same for all 2,340 queries per head, 42 records per step (3,144,960 rows); the
             default run also measures it and reports it under "full_rows" (--no-full-rows skips it).
* decode   : 16 query heads sharing 2 KV heads, 4,096 cached keys, last 256 positions, attention
             output over the packed 4-bit K/V (R = 16) with top-32 and recent-window mass.
* decode_batch: one decode step for 512 sequences (seeds 5000 + b): each sequence's last position,
             16 query heads over its own 2 packed 4-bit KV heads of 4,096 keys (R = 16); the same
             outputs. Every packed byte is read once per step.
* mx_sampled: the sampled workload in MXFP8 mode: each step packs Q and K (signed-H128 + E4M3/E8M0
             K32) and computes every statistic on the MX rows plus TV / argmax against the bf16
             rows and the P path.
* ablation : local output ablation over the sampled workload with V: O over all keys, then O with
             the sink, the recent region and all history dropped (P renormalised over the kept keys),
             each compared with the full O by per-row relative L2 and cosine.

* maps     : the sampled workload with the spatial maps added (key masses, sink / recent / current
             spatial maps per head and per record, the 64 x 96 pooled map per head, one query's
             probabilities and its 99.5th-percentile clip); reports the maps' own time beside the
             statistics-only call.
* p2       : the fixed-budget residual-window protocol at head dimension 32 (18 inputs x R in
             {0, 16, 64}: pack, 4-bit attention, bf16 reference, comparison); launch-latency-bound.
* tiny     : the three 128 x 128 variants (clean, early_focus, recent_focus) with every statistic and
             O in one call, and the same rows in MXFP8 mode (pack + statistics): launch-latency-bound,
             reported as microseconds per call with no roofline claim.

Prints one JSON line (metric, value in rows/s, roofline of the row kernel, oracle CPU baseline).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "query-head rows/s at Sk=6240 (full stats) + % of bf16 MFMA / HBM roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="sampled", choices=["sampled", "full_rows", "decode", "decode_batch", "mx_sampled", "ablation", "tiny",
                                                         "maps", "p2"])
    ap.add_argument("--records", type=int, default=None)
    ap.add_argument("--kv", default="int4", choices=["int4", "bf16"], help="decode_batch: packed 4-bit or bf16 K/V")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-full-rows", action="store_true", help="skip the full-row sub-measurement of the default run")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time a plain 1 GiB device copy instead (counter calibration)")
    return ap.parse_args()


def video_inputs(n_records: int, sampled: bool, dev):
    import torch

    from quantized_kv_amd import inputs

    qs, ks = [], []
    for r in range(n_records):
        rec = inputs.video_record(r, with_v=False, sampled=sampled)
        qs.append(rec.q.to(dev))
        ks.append(rec.k.to(dev))
    return torch.stack(qs), torch.stack(ks)


KERNEL_SOURCES = ("quantized_kv_amd/csrc/rowstats_impl.h", "quantized_kv_amd/csrc/kvprof_device.h",
                  "quantized_kv_amd/csrc/kvprof_internal.h")
COUNTERS = os.path.join(ROOT, "profiles", "row_kernel_video_sampled_counters.json")


def measured_traffic():
    """HBM bytes per row-kernel launch from the committed FETCH_SIZE / WRITE_SIZE counter runs (scaled
    by a plain copy's reading), or None when the kernel sources changed since they were taken."""
    import hashlib

    if not os.path.exists(COUNTERS):
        return None
    rec = json.load(open(COUNTERS))
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return rec["traffic_bytes_per_dispatch"] if rec.get("kernel_sources_sha256") == h.hexdigest() else None


def time_it(fn, steps, warmup, stream):
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        fn()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps  # ms per call


def cpu_baseline_video(n_records: int, sampled: bool, threads=1, heads=None):
    """The oracle, as it stands, on the first n_records records (all heads, or the first `heads`), with
    `threads` BLAS threads (None: every core of the host)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import kvprof_oracle as O
    from quantized_kv_amd import inputs

    bias = inputs.video_key_bias().astype(np.float64)
    dt, rows = 0.0, 0
    for r in range(n_records):
        rec = inputs.video_record(r, with_v=False, sampled=sampled)
        q, k = inputs.bf16_values(rec.q), inputs.bf16_values(rec.k)
        with threadpool_limits(threads):
            t = time.perf_counter()
            for h in range(q.shape[0] if heads is None else heads):
                O.row_stats(q[h], k[h], scale=128 ** -0.5, key_bias=bias,
                            region_bounds=inputs.VIDEO_REGION_BOUNDS, frame_len=inputs.LF_TOKENS,
                            n_frames=inputs.N_KEY_FRAMES)
                rows += q.shape[1]
            dt += time.perf_counter() - t
    if threads is None:  # the BLAS thread count in effect (OMP / OpenBLAS settings of the host)
        from threadpoolctl import threadpool_info

        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    else:
        cores = threads
    return {"value": round(rows / dt, 1), "unit": "rows/s", "cores": cores, "kind": "oracle",
            "sample": f"records 0..{n_records - 1}, {q.shape[0] if heads is None else heads} heads x {q.shape[1]} "
                      f"queries x 6240 keys ({rows} rows, {dt:.1f} s of oracle time)",
            "cpu": cpu_model()}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def copy_calibration(args):
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    ms = time_it(lambda: dst.copy_(src), args.steps, args.warmup, stream)
    return {"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "ms": round(ms, 4),
            "gbs": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}


def achievable_hbm_gbs():
    """Bytes moved per second by a plain 1 GiB device copy (read + write), measured in the same run: the
    achievable HBM rate beside the published 8 TB/s."""
    import torch

    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    ms = time_it(lambda: dst.copy_(src), 10, 2, torch.cuda.current_stream())
    del src, dst
    return round(2 * nbytes / (ms * 1e-3) / 1e9, 1)


def run_video(args, sampled: bool):
    import torch

    from quantized_kv_amd import binding as B
    from quantized_kv_amd import inputs

    dev = torch.device("cuda:0")
    n_rec = args.records or inputs.N_RECORDS
    t_gen = time.time()
    Q, K = video_inputs(n_rec, sampled, dev)
    gen_s = time.time() - t_gen
    Bn, H, Mq, _ = Q.shape
    Sk = K.shape[2]
    rows = Bn * H * Mq
    bias = torch.from_numpy(inputs.video_key_bias()).to(dev)
    groups = torch.from_numpy(inputs.video_sample_groups() if sampled else
                              (torch.arange(Mq) // inputs.LF_TOKENS).numpy().astype("int32")).to(dev)
    kw = dict(scale=128 ** -0.5, key_bias=bias, region_bounds=inputs.VIDEO_REGION_BOUNDS,
              frame_len=inputs.LF_TOKENS, n_frames=inputs.N_KEY_FRAMES, row_group=groups, n_groups=6)
    want = ("support", "top_mass", "top32", "strict_zero", "region_mass", "frame_mass", "row_max", "row_lse")
    stream = torch.cuda.current_stream()
    # one allocation of outputs + workspace, then repeated calls on the same buffers
    res = B.run(Q, K, want=want, heatmap=True, hist=True, **kw)
    args_full = res["_keepalive"][0]
    # the row kernel alone (frame masses still written; no heatmap / histogram kernels)
    res_rows = B.run(Q, K, want=want, **kw)
    args_rows = res_rows["_keepalive"][0]
    step = lambda: B.kvprof_row_stats(args_full, stream)  # noqa: E731
    kern = lambda: B.kvprof_row_stats(args_rows, stream)  # noqa: E731
    ms = time_it(step, args.steps, args.warmup, stream)
    ms_kernel = time_it(kern, args.steps, 1, stream)
    # algorithmic bytes per launch: K once per (record, head), Q rows, bias, and every output
    out_bytes_row = 4 + 12 + 128 + 4 + 12 + 64 + 4 + 4
    nbytes = K.numel() * 2 + Q.numel() * 2 + Sk * 4 + rows * out_bytes_row
    flops = 2.0 * 128 * Sk * rows
    achieved_gbs = nbytes / (ms_kernel * 1e-3) / 1e9
    achieved_tfs = flops / (ms_kernel * 1e-3) / 1e12
    if sampled:
        ach = achievable_hbm_gbs()
        roof = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                "algorithmic_bytes": nbytes, "achievable_copy": ach,
                "frac_of_achievable": round(achieved_gbs / ach, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(achieved_tfs, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved_tfs / BF16_PEAK_TFLOPS, 4), "traffic": None}
    out = {
        "metric": METRIC, "value": round(rows / (ms * 1e-3), 1), "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": ("video steady chunk, sampled queries" if sampled else "video steady chunk, full rows"),
                   "records": Bn, "heads": H, "queries_per_head": Mq, "keys": Sk, "head_dim": 128,
                   "rows_per_step": rows, "outputs": list(want) + ["heatmap", "hist"]},
        "roofline": roof,
        "row_kernel_ms": round(ms_kernel, 4),
        "input_gen_s": round(gen_s, 1),
    }
    if not args.no_cpu_baseline:
        if sampled:
            out["cpu_baseline"] = cpu_baseline_video(6, True)
            # the same oracle with NumPy's BLAS on every host core (its per-row loops stay single-threaded)
            out["cpu_baseline_all_cores"] = cpu_baseline_video(3, True, threads=None)
        else:
            out["cpu_baseline"] = cpu_baseline_video(1, False, heads=4)
    return out


def run_mx(args):
    import torch

    from quantized_kv_amd import binding as B
    from quantized_kv_amd import inputs

    dev = torch.device("cuda:0")
    n_rec = args.records or inputs.N_RECORDS
    Q, K = video_inputs(n_rec, True, dev)
    Bn, H, Mq, _ = Q.shape
    Sk = K.shape[2]
    rows = Bn * H * Mq
    lib = B.load()
    signs = torch.from_numpy(inputs.hadamard_signs(4)).to(dev)
    qc = torch.empty(Q.shape, dtype=torch.uint8, device=dev)
    qs = torch.empty(Q.shape[:-1] + (4,), dtype=torch.uint8, device=dev)
    kc = torch.empty(K.shape, dtype=torch.uint8, device=dev)
    ks = torch.empty(K.shape[:-1] + (4,), dtype=torch.uint8, device=dev)
    bias = torch.from_numpy(inputs.video_key_bias()).to(dev)
    want = ("support", "top_mass", "top32", "strict_zero", "region_mass", "frame_mass", "tv_qk", "argmax",
            "argmax_ref", "p_zero_frac", "tv_p", "p_rowsum")
    res = B.run(Q, K, want=want, mode=B.MODE_MXFP8, q_codes=qc, q_scales=qs, k_codes=kc, k_scales=ks,
                scale=128 ** -0.5, key_bias=bias, region_bounds=inputs.VIDEO_REGION_BOUNDS,
                frame_len=inputs.LF_TOKENS, n_frames=inputs.N_KEY_FRAMES)
    a = res["_keepalive"][0]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def step():
        B._check("kvprof_pack_mxfp8", lib.kvprof_pack_mxfp8(Q.data_ptr(), rows, 128, signs.data_ptr(),
                                                            qc.data_ptr(), qs.data_ptr(), sp))
        B._check("kvprof_pack_mxfp8", lib.kvprof_pack_mxfp8(K.data_ptr(), K.numel() // 128, 128, signs.data_ptr(),
                                                            kc.data_ptr(), ks.data_ptr(), sp))
        B.kvprof_row_stats(a, stream)

    ms = time_it(step, args.steps, args.warmup, stream)
    ms_rows = time_it(lambda: B.kvprof_row_stats(a, stream), args.steps, 1, stream)
    # algorithmic bytes of the MX row statistics: K and Q codes + scales once, the bf16 reference K
    # and Q once, the bias, and the outputs
    out_row = 4 + 12 + 128 + 4 + 12 + 64 + 6 * 4
    nbytes = K.numel() * (1 + 2) + K.numel() // 32 + Q.numel() * (1 + 2) + Q.numel() // 32 + Sk * 4 + rows * out_row
    gbs = nbytes / (ms_rows * 1e-3) / 1e9
    return {"metric": METRIC, "value": round(rows / (ms * 1e-3), 1), "unit": "rows/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "video steady chunk, sampled queries, MXFP8 mode (pack + stats)",
                       "records": Bn, "heads": H, "queries_per_head": Mq, "keys": Sk, "head_dim": 128,
                       "rows_per_step": rows, "outputs": list(want)},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "algorithmic_bytes": nbytes},
            "row_kernel_ms": round(ms_rows, 4)}


def run_decode(args):
    import torch

    from quantized_kv_amd import binding as B
    from quantized_kv_amd import inputs

    dev = torch.device("cuda:0")
    Q, K, V = inputs.decode_inputs(5)
    L, Mq, R = inputs.DECODE_L, inputs.DECODE_MQ, 16
    Qd = Q[None].to(dev)
    packed = B.kvprof_pack_int4kv(K.to(dev), V.to(dev), R)
    stream = torch.cuda.current_stream()
    res = B.run(Qd, None, want=("top32", "o", "region_mass"), attend=True, mode=B.MODE_INT4KV, kv_packed=packed,
                r_window=R, n_k=L, n_heads_kv=2, causal=True, q_pos0=L - Mq, region_bounds=[0, L - R, L])
    a = res["_keepalive"][0]
    ms = time_it(lambda: B.kvprof_attend(a, stream), args.steps, args.warmup, stream)
    rows = Q.shape[0] * Mq
    vis = sum(L - Mq + i + 1 for i in range(Mq)) * Q.shape[0]
    flops = 4.0 * 128 * vis
    tfs = flops / (ms * 1e-3) / 1e12
    return {"metric": METRIC, "value": round(rows / (ms * 1e-3), 1), "unit": "rows/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
            "config": {"workload": "decode GQA over 4-bit KV, R=16", "q_heads": 16, "kv_heads": 2, "keys": L,
                       "positions": Mq},
            "roofline": {"bound": "mfma", "achieved": round(tfs, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tfs / BF16_PEAK_TFLOPS, 5), "traffic": None}}


def run_tiny(args):
    """The tiny three-variant workload: latency per call (bf16 mode with O; MXFP8 mode with packing)."""
    import torch

    from quantized_kv_amd import binding as B
    from quantized_kv_amd import inputs

    dev = torch.device("cuda:0")
    Q, K, V = (x.to(dev) for x in inputs.tiny_inputs(1))
    rb = [0, inputs.TINY_EARLY, inputs.TINY_N]
    stream = torch.cuda.current_stream()
    want = ("support", "top_mass", "top32", "strict_zero", "region_mass", "row_max", "row_lse", "o")
    a = B.run(Q, K, V, want=want, attend=True, region_bounds=rb)["_keepalive"][0]
    ms = time_it(lambda: B.kvprof_attend(a, stream), args.steps, args.warmup, stream)
    sg = torch.from_numpy(inputs.hadamard_signs(4)).to(dev)
    qc, qs = B.kvprof_pack_mxfp8(Q.reshape(-1, 128), sg)
    kc, ks = B.kvprof_pack_mxfp8(K.reshape(-1, 128), sg)
    want_mx = ("support", "top_mass", "top32", "strict_zero", "region_mass", "tv_qk", "argmax", "argmax_ref",
               "p_zero_frac", "tv_p", "p_rowsum")
    am = B.run(Q, K, want=want_mx, mode=B.MODE_MXFP8, q_codes=qc, q_scales=qs, k_codes=kc, k_scales=ks,
               region_bounds=rb)["_keepalive"][0]

    lib, sp = B.load(), stream.cuda_stream

    def mx_step():  # packs into the same code / scale buffers every call
        B._check("kvprof_pack_mxfp8", lib.kvprof_pack_mxfp8(Q.data_ptr(), Q.numel() // 128, 128, sg.data_ptr(),
                                                            qc.data_ptr(), qs.data_ptr(), sp))
        B._check("kvprof_pack_mxfp8", lib.kvprof_pack_mxfp8(K.data_ptr(), K.numel() // 128, 128, sg.data_ptr(),
                                                            kc.data_ptr(), ks.data_ptr(), sp))
        B.kvprof_row_stats(am, stream)

    ms_mx = time_it(mx_step, args.steps, args.warmup, stream)
    rows = Q.shape[0] * Q.shape[1] * Q.shape[2]
    return {"metric": METRIC, "value": round(rows / (ms * 1e-3), 1), "unit": "rows/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "tiny three variants, 128 queries x 128 keys, all statistics and O",
                       "variants": list(inputs.TINY_VARIANTS), "rows": rows},
            "roofline": None, "us_per_call": round(ms * 1e3, 1),
            "mxfp8": {"us_per_call": round(ms_mx * 1e3, 1), "note": "pack Q and K, then every statistic, TV, argmax and the P path"}}


DECODE_BATCH = 512  # sequences per launch, seeds 5000 + b
DECODE_BATCH_SEED0 = 5000


def decode_batch_inputs(n_seq: int, r_window: int, dev):
    """n_seq independent sequences, each one query position (the last, t = L - 1) for 16 query heads
    over 2 KV heads of L keys, seeds DECODE_BATCH_SEED0 + b. K/V are packed on the device in chunks,
    so the bf16 cache never has to be resident whole. Returns Q [n_seq, 16, 1, 128] and the blobs
    [n_seq * 2, blob_bytes]."""
    import torch

    from quantized_kv_amd import binding as B
    from quantized_kv_amd import inputs

    L, hkv, hq = inputs.DECODE_L, inputs.DECODE_HKV, inputs.DECODE_HQ
    blob = B.kvprof_int4kv_bytes(L, 128, r_window)
    packed = torch.empty((n_seq * hkv, blob), dtype=torch.uint8, device=dev)
    Q = torch.empty((n_seq, hq, 1, 128), dtype=torch.bfloat16, device=dev)
    chunk = 32
    for c0 in range(0, n_seq, chunk):
        seqs = range(c0, min(n_seq, c0 + chunk))
        qs, ks, vs = zip(*[inputs.decode_inputs(DECODE_BATCH_SEED0 + b, mq=1) for b in seqs])
        Q[c0:c0 + len(seqs)] = torch.stack(qs).to(dev)
        k = torch.cat(ks).to(dev)
        v = torch.cat(vs).to(dev)
        packed[c0 * hkv:(c0 + len(seqs)) * hkv] = B.kvprof_pack_int4kv(k, v, r_window)
    return Q, packed


def decode_batch_bf16_inputs(n_seq: int, dev):
    """The batched decode step's sequences with bf16 K/V (no packing): Q [n_seq, 16, 1, 128], K, V
    [n_seq, 2, L, 128]."""
    import torch

    from quantized_kv_amd import inputs

    L, hkv, hq = inputs.DECODE_L, inputs.DECODE_HKV, inputs.DECODE_HQ
    Q = torch.empty((n_seq, hq, 1, 128), dtype=torch.bfloat16, device=dev)
    K = torch.empty((n_seq, hkv, L, 128), dtype=torch.bfloat16, device=dev)
    V = torch.empty_like(K)
    for b in range(n_seq):
        q, k, v = inputs.decode_inputs(DECODE_BATCH_SEED0 + b, mq=1)
        Q[b], K[b], V[b] = q.to(dev), k.to(dev), v.to(dev)
    return Q, K, V


def run_decode_batch(args):
    """Decode-shaped attention over the packed 4-bit cache: one query position per sequence, many
    sequences per launch, so every byte of the packed K/V is read once per step (HBM-bound)."""
    import torch

    from quantized_kv_amd import binding as B
    from quantized_kv_amd import inputs

    dev = torch.device("cuda:0")
    L, R = inputs.DECODE_L, 16
    n_seq = args.records or DECODE_BATCH
    t_gen = time.time()
    if args.kv == "bf16":
        Q, K, V = decode_batch_bf16_inputs(n_seq, dev)
        packed = None
    else:
        Q, packed = decode_batch_inputs(n_seq, R, dev)
    gen_s = time.time() - t_gen
    stream = torch.cuda.current_stream()
    if args.kv == "bf16":
        res = B.run(Q, K, V, want=("top32", "o", "region_mass"), attend=True, causal=True, q_pos0=L - 1,
                    region_bounds=[0, L - R, L])
    else:
        res = B.run(Q, None, want=("top32", "o", "region_mass"), attend=True, mode=B.MODE_INT4KV, kv_packed=packed,
                    r_window=R, n_k=L, n_heads_kv=inputs.DECODE_HKV, causal=True, q_pos0=L - 1,
                    region_bounds=[0, L - R, L])
    a = res["_keepalive"][0]
    ms = time_it(lambda: B.kvprof_attend(a, stream), args.steps, args.warmup, stream)
    # the codec on its own: pack 32 sequences' K/V (bf16 in, blobs out)
    ks, vs = zip(*[inputs.decode_inputs(DECODE_BATCH_SEED0 + b, mq=1)[1:] for b in range(32)])
    kc, vc = torch.cat(ks).to(dev), torch.cat(vs).to(dev)
    ms_pack = time_it(lambda: B.kvprof_pack_int4kv(kc, vc, R), args.steps, args.warmup, stream)
    pack_bytes = kc.numel() * 2 * 2 + kc.shape[0] * B.kvprof_int4kv_bytes(L, 128, R)
    rows = Q.shape[0] * Q.shape[1]
    # algorithmic bytes: every packed blob (or bf16 K and V) once, the Q rows, and the outputs (O, top-32,
    # 2 region masses)
    kv_bytes = packed.numel() if packed is not None else (K.numel() + V.numel()) * 2
    nbytes = kv_bytes + Q.numel() * 2 + rows * (128 * 4 + 32 * 4 + 2 * 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"metric": METRIC, "value": round(rows / (ms * 1e-3), 1), "unit": "rows/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
            "config": {"workload": ("batched decode step over 4-bit KV, R=16" if args.kv == "int4" else
                                    "batched decode step over bf16 KV"), "sequences": n_seq,
                       "q_heads": inputs.DECODE_HQ, "kv_heads": inputs.DECODE_HKV, "keys": L, "positions": 1},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "algorithmic_bytes": nbytes},
            "pack_int4kv": {"kv_heads": kc.shape[0], "ms": round(ms_pack, 4),
                            "gbs": round(pack_bytes / (ms_pack * 1e-3) / 1e9, 1),
                            "frac": round(pack_bytes / (ms_pack * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            "input_gen_s": round(gen_s, 1)}


ABLATION_DROPS = {"drop_sink": (0, 1560), "drop_recent": (1560, 3900), "drop_history": (0, 3900)}


def cpu_baseline_ablation(n_records: int):
    """The oracle, as it stands, on the ablation of the first n_records sampled records, one BLAS thread."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import kvprof_oracle as O
    from quantized_kv_amd import inputs

    bias = inputs.video_key_bias().astype(np.float64)
    dt, rows = 0.0, 0
    for r in range(n_records):
        rec = inputs.video_record(r, with_v=True, sampled=True)
        q, k, v = inputs.bf16_values(rec.q), inputs.bf16_values(rec.k), inputs.bf16_values(rec.v)
        with threadpool_limits(1):
            t = time.perf_counter()
            for h in range(q.shape[0]):
                full = O.ablated_output(q[h], k[h], v[h], scale=128 ** -0.5, key_bias=bias)
                for drop in ABLATION_DROPS.values():
                    O.ablation_metrics(O.ablated_output(q[h], k[h], v[h], scale=128 ** -0.5, key_bias=bias,
                                                        drop=drop), full)
                rows += q.shape[1]
            dt += time.perf_counter() - t
    return {"value": round(rows / dt, 1), "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"records 0..{n_records - 1} of the ablation, {q.shape[0]} heads x {q.shape[1]} queries x "
                      f"6240 keys, full + 3 ablations ({rows} rows, {dt:.1f} s of oracle time)"}


def run_ablation(args):
    """Local output ablation over the sampled workload (42 records x 32 heads x 96 queries x 6,240 keys
    with V): one step = the full O, then for each of the three drops its key bias, O with P
    renormalised over the kept keys (plus region masses, which show the dropped mass is 0), and the
    per-row relative L2 and cosine against the full O."""
    import torch

    from quantized_kv_amd import binding as B
    from quantized_kv_amd import inputs

    dev = torch.device("cuda:0")
    n_rec = args.records or inputs.N_RECORDS
    t_gen = time.time()
    qs, ks, vs = [], [], []
    for r in range(n_rec):
        rec = inputs.video_record(r, with_v=True, sampled=True)
        qs.append(rec.q.to(dev))
        ks.append(rec.k.to(dev))
        vs.append(rec.v.to(dev))
    Q, K, V = torch.stack(qs), torch.stack(ks), torch.stack(vs)
    del qs, ks, vs
    gen_s = time.time() - t_gen
    Bn, H, Mq, _ = Q.shape
    Sk = K.shape[2]
    rows = Bn * H * Mq
    bias = torch.from_numpy(inputs.video_key_bias()).to(dev)
    kw = dict(scale=128 ** -0.5, region_bounds=inputs.VIDEO_REGION_BOUNDS)
    want = ("o", "region_mass")
    stream = torch.cuda.current_stream()
    full = B.run(Q, K, V, want=want, attend=True, key_bias=bias, **kw)
    biases = {n: B.kvprof_ablation_bias(Sk, d, key_bias=bias) for n, d in ABLATION_DROPS.items()}
    runs = {n: B.run(Q, K, V, want=want, attend=True, key_bias=b, **kw) for n, b in biases.items()}
    o_full = full["o"]
    rel = torch.empty(rows, dtype=torch.float32, device=dev)
    cos = torch.empty(rows, dtype=torch.float32, device=dev)
    rsums = torch.empty(2 + 2 * rows, dtype=torch.float64, device=dev)
    csums = torch.empty(3 + 3 * rows, dtype=torch.float64, device=dev)
    lib = B.load()
    sp = stream.cuda_stream

    def step():
        B.kvprof_attend(full["_keepalive"][0], stream)
        for n, d in ABLATION_DROPS.items():
            lib.kvprof_ablation_bias(bias.data_ptr(), Sk, d[0], d[1], biases[n].data_ptr(), sp)
            B.kvprof_attend(runs[n]["_keepalive"][0], stream)
            o = runs[n]["o"]
            lib.kvprof_compare(o.data_ptr(), o_full.data_ptr(), None, None, rows, 128, rel.data_ptr(), None,
                               rsums.data_ptr(), sp)
            lib.kvprof_cosine(o.data_ptr(), o_full.data_ptr(), rows, 128, cos.data_ptr(), csums.data_ptr(), sp)

    ms = time_it(step, args.steps, args.warmup, stream)
    kern = lambda: B.kvprof_attend(runs["drop_sink"]["_keepalive"][0], stream)  # noqa: E731
    ms_kernel = time_it(kern, args.steps, 1, stream)
    # one attend launch: K and V once per (record, head), Q, the bias, O and the region masses
    nbytes = K.numel() * 2 + V.numel() * 2 + Q.numel() * 2 + Sk * 4 + rows * (128 * 4 + 3 * 4)
    gbs = nbytes / (ms_kernel * 1e-3) / 1e9
    summary = {}
    for n in ABLATION_DROPS:
        o = runs[n]["o"]
        B.kvprof_compare(o, o_full)  # warm, unchecked
        r_row, _, rs = B.kvprof_compare(o, o_full)
        c_row, cs = B.kvprof_cosine(o, o_full)
        torch.cuda.synchronize()
        rs, cs = rs.cpu().tolist(), cs.cpu().tolist()
        summary[n] = {"rel_l2": round((rs[0] / rs[1]) ** 0.5, 5), "cos": round(cs[0] / (cs[1] * cs[2]) ** 0.5, 5),
                      "rel_l2_row_median": round(float(r_row.median()), 5),
                      "cos_row_median": round(float(c_row.median()), 5)}
    out = {"metric": METRIC, "value": round(rows / (ms * 1e-3), 1), "unit": "rows/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "local output ablation, video steady chunk, sampled queries", "records": Bn,
                      "heads": H, "queries_per_head": Mq, "keys": Sk, "head_dim": 128, "rows_per_step": rows,
                      "ablations": list(ABLATION_DROPS)},
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "algorithmic_bytes": nbytes},
           "attend_kernel_ms": round(ms_kernel, 4), "ablation": summary, "input_gen_s": round(gen_s, 1)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_ablation(3)
    return out


def run_maps(args):
    """The sampled workload's statistics with and without the spatial maps; the difference is the maps'
    second pass over K (maps_kernel) and their small reductions."""
    import torch

    from quantized_kv_amd import binding as B
    from quantized_kv_amd import inputs

    dev = torch.device("cuda:0")
    n_rec = args.records or inputs.N_RECORDS
    Q, K = video_inputs(n_rec, True, dev)
    Bn, H, Mq, _ = Q.shape
    Sk = K.shape[2]
    rows = Bn * H * Mq
    bias = torch.from_numpy(inputs.video_key_bias()).to(dev)
    kw = dict(scale=128 ** -0.5, key_bias=bias, region_bounds=inputs.VIDEO_REGION_BOUNDS, frame_len=inputs.LF_TOKENS,
              n_frames=inputs.N_KEY_FRAMES)
    want = ("support", "top_mass", "top32", "strict_zero", "region_mass", "frame_mass", "row_max", "row_lse")
    stream = torch.cuda.current_stream()
    plain = B.run(Q, K, want=want, **kw)["_keepalive"][0]
    res = B.run(Q, K, want=want, maps_want=("key_mass", "spatial", "spatial_mean"), pool=(64, 96), p_row=23 * 96 + 50,
                **kw)
    full = res["_keepalive"][0]
    p_row = res["p_row_out"][: inputs.N_KEY_FRAMES * inputs.LF_TOKENS]
    clip = torch.empty(1, dtype=torch.float32, device=dev)
    clipped = torch.empty_like(p_row)
    lib, sp = B.load(), stream.cuda_stream

    def step():
        B.kvprof_row_stats(full, stream)
        lib.kvprof_percentile_clip(p_row.data_ptr(), p_row.numel(), 99.5, B.QUANTILE_SAMPLE_CAP, clip.data_ptr(),
                                   clipped.data_ptr(), sp)

    ms = time_it(step, args.steps, args.warmup, stream)
    ms_plain = time_it(lambda: B.kvprof_row_stats(plain, stream), args.steps, 1, stream)
    ms_maps = ms - ms_plain
    # the maps pass: K once per (record, head) per 32-row block group of that head (read through L2), the
    # row lse, and the partial outputs written and reduced
    kbytes = K.numel() * 2 + Q.numel() * 2 + rows * 4
    gbs = kbytes / (ms_maps * 1e-3) / 1e9
    return {"metric": METRIC, "value": round(rows / (ms * 1e-3), 1), "unit": "rows/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "video steady chunk, sampled queries, statistics + spatial maps", "records": Bn,
                       "heads": H, "queries_per_head": Mq, "keys": Sk, "pool": [64, 96]},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "algorithmic_bytes": kbytes,
                         "kernel": "maps pass (call with maps minus call without)"},
            "maps_ms": round(ms_maps, 4), "statistics_ms": round(ms_plain, 4)}


def run_p2(args):
    """The residual-window protocol's 54 comparisons through the C ABI, timed as a whole."""
    import torch

    from quantized_kv_amd import inputs, p2

    dev = torch.device("cuda:0")
    keys = [(v, s) for v in inputs.TINY_VARIANTS for s in inputs.P2_SEEDS]
    data = []  # per length: the 9 inputs stacked in the batch dimension
    for n in inputs.P2_LENGTHS:
        qkv = [inputs.p2_inputs(s, n, v) for v, s in keys]
        data.append(tuple(torch.stack([t[j] for t in qkv]).to(dev) for j in range(3)))

    def step():
        return [(keys[i][0], r) for q, k, v in data for i, r in enumerate(p2.run_batch(q, k, v))]

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    recs = []
    for _ in range(args.steps):
        recs = step()
    dt = (time.perf_counter() - t0) / args.steps
    summary = {}
    for vv in inputs.TINY_VARIANTS:
        rs = [r for name, r in recs if name == vv]
        summary[vv] = {"rel_l2": {w: round(sum(r["rel_l2"][w] for r in rs) / len(rs), 5) for w in inputs.P2_WINDOWS},
                       "recent_mass": {w: round(sum(r["recent_mass"][w] for r in rs) / len(rs), 5)
                                       for w in inputs.P2_WINDOWS}}
    return {"metric": METRIC, "value": round(54 / dt, 1), "unit": "comparisons/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(dt * 1e3, 3), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "residual-window protocol, 18 inputs x R in {0, 16, 64}, head dim 32",
                       "lengths": list(inputs.P2_LENGTHS), "seeds": list(inputs.P2_SEEDS)},
            "roofline": None, "note": "launch-latency-bound (the 9 inputs of a length share each launch, one "
                                      "synchronisation per length); no roofline claimed",
            "summary": summary}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "kvprof runs on one GPU per process; --gpus must be 1"}))
        sys.exit(2)
    import torch

    from quantized_kv_amd import binding as B

    B.load()
    assert torch.cuda.is_available(), "needs a GPU"
    if args.copy_calibration:
        out = copy_calibration(args)
    elif args.workload == "decode":
        out = run_decode(args)
    elif args.workload == "decode_batch":
        out = run_decode_batch(args)
    elif args.workload == "tiny":
        out = run_tiny(args)
    elif args.workload == "mx_sampled":
        out = run_mx(args)
    elif args.workload == "ablation":
        out = run_ablation(args)
    elif args.workload == "maps":
        out = run_maps(args)
    elif args.workload == "p2":
        out = run_p2(args)
    else:
        out = run_video(args, sampled=args.workload == "sampled")
        if args.workload == "sampled" and not args.no_full_rows:
            # the full-row configuration (all 2,340 queries of each head, 42 records) on the same GPU,
            # reported beside the sampled line with its own MFMA roofline
            torch.cuda.empty_cache()
            print("bench: sampled done, measuring full rows", file=sys.stderr, flush=True)
            sub = argparse.Namespace(**{**vars(args), "steps": min(args.steps, 10), "warmup": min(args.warmup, 2),
                                        "records": None})
            fr = run_video(sub, sampled=False)
            out["full_rows"] = {k: fr[k] for k in ("value", "unit", "ms_per_step", "steps", "warmup", "config",
                                                   "roofline", "row_kernel_ms", "cpu_baseline") if k in fr}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
