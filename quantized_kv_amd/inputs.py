"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the benchmark.

This module builds inputs only. It holds none of the profiler's arithmetic (no scores, softmax,
statistics or codecs), so the oracle and the HIP path can both take their inputs from here without
sharing any of the method.

Every array is drawn with numpy's PCG64 generator from a stated seed, in float32, and then rounded
to bfloat16 (round-to-nearest-even) by torch's dtype cast. Both sides of every parity check use the
same bf16 values. The shapes follow the workloads the pages describe:

* "Catnip Week 10 KV Cache Attention Study", section "实验设计 / From production boundary to
  statistics" and the sink/recent/current banner: 16 key latent frames (LF) of 15x26 = 390 tokens,
  ordered [sink 4 LF | recent 6 LF | current 6 LF] = 6,240 keys; the query chunk is 6 LF (2,340
  tokens); 32 heads; 96 sampled queries per head from a 4x4 spatial grid per query LF; 42 records
  (7 layers x 3 chunks x 2 denoise positions).
* "KV residual window" (huhohoo.com), section on the fixed budget: early_focus / recent_focus inputs
  built from one random base by raising the first channel of Q and of the first or last 16 keys.
* The attention-predictor study (bjdmk.com.cn), section "0. 实验基线与评价指标": 16 query heads sharing
  2 KV heads, head_dim 128.

The temperature, bias and focus offsets are input construction choices for synthetic data; they are
not part of what the profiler computes.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

HEAD_DIM = 128

# Video layout (page 1): frames of 15x26 tokens, 16 key frames, 6 query frames.
LF_H, LF_W = 15, 26
LF_TOKENS = LF_H * LF_W  # 390
N_KEY_FRAMES = 16
N_QUERY_FRAMES = 6
SINK_FRAMES, RECENT_FRAMES, CURRENT_FRAMES = 4, 6, 6
VIDEO_SK = N_KEY_FRAMES * LF_TOKENS  # 6240
VIDEO_MQ = N_QUERY_FRAMES * LF_TOKENS  # 2340
VIDEO_HEADS = 32
VIDEO_REGION_BOUNDS = [0, SINK_FRAMES * LF_TOKENS, (SINK_FRAMES + RECENT_FRAMES) * LF_TOKENS, VIDEO_SK]
N_RECORDS = 42
RECORD_SEED0 = 3000
CURRENT_BIAS = 0.5
# Query sampling grid inside one 15x26 latent frame: 4x4 cell centres (rows of 15, cols of 26).
GRID_Y = (1, 5, 9, 13)
GRID_X = (3, 9, 16, 22)


def to_bf16(x_f32: np.ndarray):
    """float32 numpy array -> torch.bfloat16 CPU tensor (round to nearest even, by torch's cast)."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32)).to(torch.bfloat16)


def bf16_values(t) -> np.ndarray:
    """bf16 torch tensor -> float64 numpy array holding exactly the same values."""
    import torch

    return t.to(torch.float32).numpy().astype(np.float64)


def video_sample_rows() -> np.ndarray:
    """Indices (into the 2,340-token query chunk) of the 96 sampled queries, grouped by query LF.

    Per query LF l: token index 390*l + 26*y + x for y in GRID_Y, x in GRID_X, row-major.
    """
    rows = [LF_TOKENS * l + LF_W * y + x for l in range(N_QUERY_FRAMES) for y in GRID_Y for x in GRID_X]
    return np.asarray(rows, dtype=np.int64)


def video_sample_groups() -> np.ndarray:
    """Query-LF group (0..5) of each of the 96 sampled queries."""
    return np.repeat(np.arange(N_QUERY_FRAMES, dtype=np.int32), len(GRID_Y) * len(GRID_X))


def video_key_bias(sk: int = VIDEO_SK) -> np.ndarray:
    """Additive logit bias per key: +0.5 on the current-chunk keys, 0 elsewhere (float32)."""
    b = np.zeros(sk, dtype=np.float32)
    b[VIDEO_REGION_BOUNDS[2]:] = CURRENT_BIAS
    return b


@dataclass
class VideoRecord:
    seed: int
    tau: np.ndarray  # [H] float64 temperatures
    q: object  # torch bf16 [H, Mq, 128]
    k: object  # torch bf16 [H, Sk, 128]
    v: object | None  # torch bf16 [H, Sk, 128] or None


def video_record(r: int, *, heads: int = VIDEO_HEADS, mq: int = VIDEO_MQ, sk: int = VIDEO_SK,
                 with_v: bool = True, sampled: bool = False) -> VideoRecord:
    """Record r of the steady-chunk video workload.

    Draw order from default_rng(3000 + r): tau = lognormal(0, 0.75, heads); Q = N(0,1) [heads, mq, 128]
    scaled by tau per head; K = N(0,1) [heads, sk, 128]; V = N(0,1) [heads, sk, 128].
    With ``sampled`` the 96 grid queries are gathered from the full query chunk, so a sampled record
    holds exactly the rows of the full record at those positions.
    """
    rng = np.random.default_rng(RECORD_SEED0 + r)
    tau = rng.lognormal(0.0, 0.75, heads)
    q = rng.standard_normal((heads, mq, HEAD_DIM), dtype=np.float32)
    q *= tau.astype(np.float32)[:, None, None]
    k = rng.standard_normal((heads, sk, HEAD_DIM), dtype=np.float32)
    v = rng.standard_normal((heads, sk, HEAD_DIM), dtype=np.float32) if with_v else None
    if sampled:
        q = q[:, video_sample_rows(), :]
    return VideoRecord(seed=RECORD_SEED0 + r, tau=tau, q=to_bf16(q), k=to_bf16(k),
                       v=None if v is None else to_bf16(v))


TINY_N = 128
TINY_EARLY = 112  # regions: early [0,112), recent [112,128)
TINY_FOCUS = 3.0
TINY_VARIANTS = ("clean", "early_focus", "recent_focus")


def tiny_inputs(seed: int = 1):
    """The three tiny variants built from one seed.

    Q, K, V = standard_normal((128,128), float32) drawn in that order from default_rng(seed).
    early_focus adds +3.0 to channel 0 of every query and of the first 16 keys; recent_focus adds it to
    channel 0 of every query and of the last 16 keys. Returns bf16 tensors stacked as
    [3 variants, 1 head, 128, 128] for Q, K and V.
    """
    import torch

    rng = np.random.default_rng(seed)
    q = rng.standard_normal((TINY_N, HEAD_DIM), dtype=np.float32)
    k = rng.standard_normal((TINY_N, HEAD_DIM), dtype=np.float32)
    v = rng.standard_normal((TINY_N, HEAD_DIM), dtype=np.float32)
    qs, ks = [], []
    for name in TINY_VARIANTS:
        qv, kv = q.copy(), k.copy()
        if name == "early_focus":
            qv[:, 0] += TINY_FOCUS
            kv[:16, 0] += TINY_FOCUS
        elif name == "recent_focus":
            qv[:, 0] += TINY_FOCUS
            kv[TINY_N - 16:, 0] += TINY_FOCUS
        qs.append(qv)
        ks.append(kv)
    Q = torch.stack([to_bf16(x) for x in qs])[:, None]
    K = torch.stack([to_bf16(x) for x in ks])[:, None]
    V = torch.stack([to_bf16(v) for _ in TINY_VARIANTS])[:, None]
    return Q, K, V


P2_SEEDS = (1, 2, 3)
P2_LENGTHS = (128, 512)
P2_D = 32
P2_WINDOWS = (0, 16, 64)
P2_FOCUS = 4.85  # recent_focus then puts about 77 % of the reference mass on the last 16 tokens
P2_FOCUS_TOKENS = 16


def p2_inputs(seed: int, n: int, variant: str, d: int = P2_D):
    """One input of the fixed-budget residual-window protocol: Q, K, V = standard_normal((n, d), float32)
    drawn in that order from default_rng(seed). early_focus adds P2_FOCUS to channel 0 of every query and
    of the first 16 keys, recent_focus to channel 0 of every query and of the last 16 keys; both start
    from the same base arrays as clean. Returns bf16 tensors [n, d]."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n, d), dtype=np.float32)
    k = rng.standard_normal((n, d), dtype=np.float32)
    v = rng.standard_normal((n, d), dtype=np.float32)
    if variant == "early_focus":
        q[:, 0] += P2_FOCUS
        k[:P2_FOCUS_TOKENS, 0] += P2_FOCUS
    elif variant == "recent_focus":
        q[:, 0] += P2_FOCUS
        k[n - P2_FOCUS_TOKENS:, 0] += P2_FOCUS
    elif variant != "clean":
        raise ValueError(variant)
    return to_bf16(q), to_bf16(k), to_bf16(v)


def hadamard_signs(seed: int = 4, n: int = HEAD_DIM) -> np.ndarray:
    """Random signs for the signed Hadamard rotation: 2*default_rng(seed).integers(0,2,n)-1 (int8)."""
    return (2 * np.random.default_rng(seed).integers(0, 2, n) - 1).astype(np.int8)


DECODE_HQ, DECODE_HKV, DECODE_L, DECODE_MQ = 16, 2, 4096, 256


def decode_inputs(seed: int = 5, hq: int = DECODE_HQ, hkv: int = DECODE_HKV, L: int = DECODE_L,
                  mq: int = DECODE_MQ):
    """Decode-shaped GQA inputs: Q [hq, mq, 128], K, V [hkv, L, 128], N(0,1) from default_rng(seed),
    drawn in the order Q, K, V, rounded to bf16. Query i sits at absolute position L - mq + i."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((hq, mq, HEAD_DIM), dtype=np.float32)
    k = rng.standard_normal((hkv, L, HEAD_DIM), dtype=np.float32)
    v = rng.standard_normal((hkv, L, HEAD_DIM), dtype=np.float32)
    return to_bf16(q), to_bf16(k), to_bf16(v)


def generic_inputs(seed: int, shape_q, shape_kv, q_scale: float = 1.0):
    """Plain N(0,1) bf16 tensors for parity sweeps at arbitrary shapes (Q scaled by q_scale)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal(shape_q, dtype=np.float32) * np.float32(q_scale)
    k = rng.standard_normal(shape_kv, dtype=np.float32)
    v = rng.standard_normal(shape_kv, dtype=np.float32)
    return to_bf16(q), to_bf16(k), to_bf16(v)
