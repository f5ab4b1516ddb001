"""ctypes binding of libkvprof (include/kvprof.h). Argument marshalling only: every step of the
profiler runs in the library's HIP kernels. Tensors are torch tensors on the current HIP device; torch
provides device memory and the stream, nothing else.

The functions keep the C names (kvprof_pack_mxfp8, kvprof_pack_int4kv, kvprof_row_stats, ...). There
is no fallback: if the library is missing or a call fails, a KvprofError is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvprof.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "kvprof.h")

KVPROF_OK = 0
KVPROF_EINVAL = -1
KVPROF_ESHAPE = -2
KVPROF_EALIGN = -3
KVPROF_ESIZE = -4
KVPROF_EUNSUPPORTED = -6
KVPROF_ELAUNCH = -7
MODE_BF16, MODE_MXFP8, MODE_INT4KV = 0, 1, 2
HEAD_DIM = 128


class KvprofError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


_P = ctypes.c_void_p


class KvprofArgs(ctypes.Structure):
    """Mirror of struct kvprof_args (same field order; ctypes applies the C layout rules)."""

    _fields_ = [
        ("mode", ctypes.c_int32),
        ("n_batch", ctypes.c_int32), ("n_heads_q", ctypes.c_int32), ("n_heads_kv", ctypes.c_int32),
        ("n_q", ctypes.c_int32), ("n_k", ctypes.c_int32), ("d", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("q", _P), ("k", _P), ("v", _P),
        ("q_codes", _P), ("q_scales", _P), ("k_codes", _P), ("k_scales", _P),
        ("kv_packed", _P), ("r_window", ctypes.c_int32),
        ("key_bias", _P),
        ("causal", ctypes.c_int32), ("q_pos0", ctypes.c_int64),
        ("n_regions", ctypes.c_int32), ("region_bounds", ctypes.POINTER(ctypes.c_int32)),
        ("frame_len", ctypes.c_int32), ("n_frames", ctypes.c_int32),
        ("row_group", _P), ("n_groups", ctypes.c_int32),
        ("hist_bins", ctypes.c_int32),
        ("support", _P), ("top_mass", _P), ("top32", _P), ("strict_zero", _P),
        ("region_mass", _P), ("frame_mass", _P), ("row_max", _P), ("row_lse", _P), ("o", _P),
        ("tv_qk", _P), ("argmax", _P), ("argmax_ref", _P), ("p_zero_frac", _P), ("tv_p", _P),
        ("p_rowsum", _P),
        ("heatmap", _P), ("heatmap_mean", _P), ("hist", _P),
        ("key_mass", _P), ("spatial", _P), ("spatial_mean", _P),
        ("pool_h", ctypes.c_int32), ("pool_w", ctypes.c_int32), ("pooled", _P),
        ("p_row", ctypes.c_int64), ("p_row_out", _P),
        ("workspace", _P), ("workspace_bytes", ctypes.c_size_t),
    ]


_lib = None


def load(path: str = LIB_PATH):
    """Load libkvprof.so (built by quantized_kv_amd.build). Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise KvprofError("load", KVPROF_EUNSUPPORTED,
                          f"{path} not found: build it with `python -m quantized_kv_amd.build`")
    lib = ctypes.CDLL(path)
    lib.kvprof_abi_version.restype = ctypes.c_int
    lib.kvprof_last_error.restype = ctypes.c_char_p
    lib.kvprof_int4kv_bytes.restype = ctypes.c_size_t
    lib.kvprof_int4kv_bytes.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]
    lib.kvprof_pack_mxfp8.argtypes = [_P, ctypes.c_int64, ctypes.c_int32, _P, _P, _P, _P]
    lib.kvprof_unpack_mxfp8.argtypes = [_P, _P, ctypes.c_int64, ctypes.c_int32, _P, _P]
    lib.kvprof_pack_int4kv.argtypes = [_P, _P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                       ctypes.c_int32, _P, ctypes.c_size_t, _P]
    lib.kvprof_unpack_int4kv.argtypes = [_P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_int32, _P, _P, _P]
    lib.kvprof_workspace_bytes.restype = ctypes.c_size_t
    lib.kvprof_workspace_bytes.argtypes = [ctypes.POINTER(KvprofArgs)]
    lib.kvprof_row_stats.argtypes = [ctypes.POINTER(KvprofArgs), _P]
    lib.kvprof_attend.argtypes = [ctypes.POINTER(KvprofArgs), _P]
    lib.kvprof_row_stats_noalloc.argtypes = [ctypes.POINTER(KvprofArgs), _P]
    lib.kvprof_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.kvprof_noalloc_scratch_bytes.argtypes = []
    lib.kvprof_compare.argtypes = [_P, _P, _P, _P, ctypes.c_int64, ctypes.c_int32, _P, _P, _P, _P]
    lib.kvprof_ablation_bias.argtypes = [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P]
    lib.kvprof_cosine.argtypes = [_P, _P, ctypes.c_int64, ctypes.c_int32, _P, _P, _P]
    lib.kvprof_int4kv_append_window.restype = ctypes.c_int64
    lib.kvprof_int4kv_append_window.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32]
    lib.kvprof_int4kv_append.argtypes = [_P, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _P, _P,
                                         ctypes.c_int64, ctypes.c_int32, _P, ctypes.c_size_t, _P]
    lib.kvprof_percentile_clip.argtypes = [_P, ctypes.c_int64, ctypes.c_double, ctypes.c_int64, _P, _P, _P]
    for name in ("kvprof_pack_mxfp8", "kvprof_unpack_mxfp8", "kvprof_pack_int4kv",
                 "kvprof_unpack_int4kv", "kvprof_row_stats", "kvprof_attend", "kvprof_row_stats_noalloc",
                 "kvprof_compare",
                 "kvprof_ablation_bias", "kvprof_cosine", "kvprof_percentile_clip", "kvprof_int4kv_append"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def declared_functions(header: str = HEADER) -> list:
    """Names of the functions include/kvprof.h declares."""
    import re

    txt = open(header).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(kvprof_\w+)\s*\(", txt, re.M)))


def _check(fn: str, status: int):
    if status != KVPROF_OK:
        raise KvprofError(fn, status, load().kvprof_last_error().decode())


def _ptr(t) -> Optional[int]:
    """Device address of a tensor argument. The library reads and writes every array as dense memory
    on the GPU, so a host tensor or a strided view is refused here, before any call reaches it."""
    if t is None:
        return None
    if not t.is_cuda:
        raise KvprofError("binding", KVPROF_EINVAL, f"tensor on {t.device}: the library needs GPU memory")
    if not t.is_contiguous():
        raise KvprofError("binding", KVPROF_EINVAL,
                          f"tensor of shape {tuple(t.shape)} and strides {t.stride()} is not contiguous")
    return t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


# ---- codecs --------------------------------------------------------------------------------------

def kvprof_pack_mxfp8(x, signs=None, stream=None):
    """x: bf16 [rows, d] (contiguous, on the GPU); signs: int8 [d] of +-1 or None.
    Returns (codes uint8 [rows, d], scales uint8 [rows, d/32])."""
    import torch

    x = x.contiguous()
    rows, d = x.reshape(-1, x.shape[-1]).shape
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    scales = torch.empty(x.shape[:-1] + (d // 32,), dtype=torch.uint8, device=x.device)
    _check("kvprof_pack_mxfp8", load().kvprof_pack_mxfp8(_ptr(x), rows, d, _ptr(signs), _ptr(codes),
                                                         _ptr(scales), _stream(stream)))
    return codes, scales


def kvprof_unpack_mxfp8(codes, scales, stream=None):
    import torch

    d = codes.shape[-1]
    rows = codes.numel() // d
    out = torch.empty(codes.shape, dtype=torch.float32, device=codes.device)
    _check("kvprof_unpack_mxfp8", load().kvprof_unpack_mxfp8(_ptr(codes), _ptr(scales), rows, d,
                                                             _ptr(out), _stream(stream)))
    return out


def kvprof_int4kv_bytes(n_tokens: int, d: int, r_window: int) -> int:
    return int(load().kvprof_int4kv_bytes(n_tokens, d, r_window))


def kvprof_pack_int4kv(k, v, r_window: int, stream=None):
    """k, v: bf16 [heads, N, d]. Returns uint8 [heads, blob_bytes] holding one blob per KV head."""
    import torch

    heads, N, d = k.shape
    blob = kvprof_int4kv_bytes(N, d, r_window)
    out = torch.empty((heads, blob), dtype=torch.uint8, device=k.device)
    _check("kvprof_pack_int4kv", load().kvprof_pack_int4kv(_ptr(k.contiguous()), _ptr(v.contiguous()), heads,
                                                           N, d, r_window, _ptr(out), out.numel(),
                                                           _stream(stream)))
    return out


def kvprof_int4kv_append_window(r_in: int, n_new: int, r_window: int) -> int:
    return int(load().kvprof_int4kv_append_window(r_in, n_new, r_window))


def kvprof_int4kv_append(packed, n_tokens: int, d: int, r_in: int, k_new, v_new, r_window: int, stream=None):
    """Append bf16 tokens k_new, v_new [heads, t, d] to packed blobs uint8 [heads, bytes] (rolling float32
    window of nominal length r_window). Returns (new blobs uint8 [heads, bytes'], new window length)."""
    import torch

    heads, t = k_new.shape[0], k_new.shape[1]
    r_out = kvprof_int4kv_append_window(r_in, t, r_window)
    blob = kvprof_int4kv_bytes(n_tokens + t, d, r_out)
    out = torch.empty((heads, blob), dtype=torch.uint8, device=packed.device)
    _check("kvprof_int4kv_append", load().kvprof_int4kv_append(_ptr(packed), heads, n_tokens, d, r_in, _ptr(k_new),
                                                               _ptr(v_new), t, r_window, _ptr(out), out.numel(),
                                                               _stream(stream)))
    return out, r_out


def kvprof_unpack_int4kv(packed, n_tokens: int, d: int, r_window: int, stream=None):
    import torch

    heads = packed.shape[0]
    k = torch.empty((heads, n_tokens, d), dtype=torch.float32, device=packed.device)
    v = torch.empty_like(k)
    _check("kvprof_unpack_int4kv", load().kvprof_unpack_int4kv(_ptr(packed), heads, n_tokens, d, r_window,
                                                               _ptr(k), _ptr(v), _stream(stream)))
    return k, v


# ---- row statistics / attention ------------------------------------------------------------------

ROW_OUTPUTS = ("support", "top_mass", "top32", "strict_zero", "region_mass", "frame_mass", "row_max",
               "row_lse", "o", "tv_qk", "argmax", "argmax_ref", "p_zero_frac", "tv_p", "p_rowsum")


def _alloc_outputs(want: Sequence[str], rows: int, n_regions: int, n_frames: int, device, d: int = HEAD_DIM):
    import torch

    shapes = {"support": (rows,), "top_mass": (rows, 3), "top32": (rows, 32), "strict_zero": (rows,),
              "region_mass": (rows, n_regions), "frame_mass": (rows, n_frames), "row_max": (rows,),
              "row_lse": (rows,), "o": (rows, d), "tv_qk": (rows,), "argmax": (rows,),
              "argmax_ref": (rows,), "p_zero_frac": (rows,), "tv_p": (rows,), "p_rowsum": (rows,)}
    ints = {"top32", "strict_zero", "argmax", "argmax_ref"}
    return {n: torch.empty(shapes[n], dtype=torch.int32 if n in ints else torch.float32, device=device)
            for n in want}


def make_args(q, k=None, v=None, *, mode=MODE_BF16, scale=None, q_codes=None, q_scales=None,
              k_codes=None, k_scales=None, kv_packed=None, r_window=0, n_k=None, n_heads_kv=None,
              key_bias=None, causal=False, q_pos0=0, region_bounds=None, frame_len=0, n_frames=0,
              row_group=None, n_groups=0, hist_bins=0, outputs=None, heatmap=None, heatmap_mean=None,
              hist=None, workspace=None):
    """Fill a KvprofArgs from tensors. q: bf16 [B, Hq, Mq, 128]; k, v: bf16 [B, Hkv, Sk, 128]."""
    B, Hq, Mq, d = q.shape
    if k is not None:
        _, Hkv, Sk, _ = k.shape
    else:
        Hkv, Sk = n_heads_kv, n_k
    a = KvprofArgs()
    a.mode = mode
    a.n_batch, a.n_heads_q, a.n_heads_kv, a.n_q, a.n_k, a.d = B, Hq, Hkv, Mq, Sk, d
    a.scale = float(scale if scale is not None else d ** -0.5)
    a.q, a.k, a.v = _ptr(q), _ptr(k), _ptr(v)
    a.q_codes, a.q_scales, a.k_codes, a.k_scales = (_ptr(q_codes), _ptr(q_scales), _ptr(k_codes),
                                                    _ptr(k_scales))
    a.kv_packed, a.r_window = _ptr(kv_packed), int(r_window)
    a.key_bias = _ptr(key_bias)
    a.causal, a.q_pos0 = int(bool(causal)), int(q_pos0)
    if region_bounds is not None:
        rb = (ctypes.c_int32 * len(region_bounds))(*[int(x) for x in region_bounds])
        a._rb_keepalive = rb
        a.n_regions = len(region_bounds) - 1
        a.region_bounds = rb
    a.frame_len, a.n_frames = int(frame_len), int(n_frames)
    a.row_group, a.n_groups = _ptr(row_group), int(n_groups)
    a.hist_bins = int(hist_bins)
    for name, t in (outputs or {}).items():
        setattr(a, name, _ptr(t))
    a.heatmap, a.heatmap_mean, a.hist = _ptr(heatmap), _ptr(heatmap_mean), _ptr(hist)
    if workspace is not None:
        a.workspace, a.workspace_bytes = _ptr(workspace), workspace.numel()
    return a


def kvprof_workspace_bytes(args: KvprofArgs) -> int:
    return int(load().kvprof_workspace_bytes(ctypes.byref(args)))


def kvprof_row_stats(args: KvprofArgs, stream=None):
    _check("kvprof_row_stats", load().kvprof_row_stats(ctypes.byref(args), _stream(stream)))


def kvprof_attend(args: KvprofArgs, stream=None):
    _check("kvprof_attend", load().kvprof_attend(ctypes.byref(args), _stream(stream)))


def kvprof_row_stats_noalloc(args: KvprofArgs, stream=None):
    """kvprof_row_stats with the library's fixed device scratch instead of args.workspace."""
    _check("kvprof_row_stats_noalloc", load().kvprof_row_stats_noalloc(ctypes.byref(args), _stream(stream)))


def kvprof_noalloc_scratch_bytes() -> int:
    return int(load().kvprof_noalloc_scratch_bytes())


def kvprof_compare(o_q, o_ref, top32_q=None, top32_ref=None, stream=None):
    """Per-row relative L2 and recall@32, plus the two sums of the tensor-level relative L2."""
    import torch

    rows, d = o_q.shape
    rel = torch.empty(rows, dtype=torch.float32, device=o_q.device)
    rec = torch.empty(rows, dtype=torch.float32, device=o_q.device) if top32_q is not None else None
    sums = torch.empty(2 + 2 * rows, dtype=torch.float64, device=o_q.device)
    _check("kvprof_compare", load().kvprof_compare(_ptr(o_q), _ptr(o_ref), _ptr(top32_q), _ptr(top32_ref), rows, d,
                                                   _ptr(rel), _ptr(rec), _ptr(sums), _stream(stream)))
    return rel, rec, sums[:2]


def kvprof_ablation_bias(n_k: int, drop, key_bias=None, device=None, stream=None):
    """Key bias that drops keys [lo, hi) (local output ablation); returns a float32 [n_k] tensor."""
    import torch

    dev = key_bias.device if key_bias is not None else (device if device is not None else
                                                         torch.device("cuda", torch.cuda.current_device()))
    out = torch.empty(n_k, dtype=torch.float32, device=dev)
    _check("kvprof_ablation_bias", load().kvprof_ablation_bias(_ptr(key_bias), n_k, int(drop[0]), int(drop[1]),
                                                               _ptr(out), _stream(stream)))
    return out


def kvprof_cosine(a, b, stream=None):
    """Per-row cosine of two float32 [rows, d] tensors, plus the three sums of the tensor-level cosine."""
    import torch

    rows, d = a.shape
    cos = torch.empty(rows, dtype=torch.float32, device=a.device)
    sums = torch.empty(3 + 3 * rows, dtype=torch.float64, device=a.device)
    _check("kvprof_cosine", load().kvprof_cosine(_ptr(a), _ptr(b), rows, d, _ptr(cos), _ptr(sums), _stream(stream)))
    return cos, sums[:3]


QUANTILE_SAMPLE_CAP = 65536


def kvprof_percentile_clip(x, pct=99.5, cap=QUANTILE_SAMPLE_CAP, clipped=True, stream=None):
    """Percentile of a float32 tensor's values (over the capped sample) and, with clipped=True, the
    values clipped to it. Returns (clip float32 [1], y float32 like x or None)."""
    import torch

    clip = torch.empty(1, dtype=torch.float32, device=x.device)
    y = torch.empty_like(x) if clipped else None
    _check("kvprof_percentile_clip", load().kvprof_percentile_clip(_ptr(x), x.numel(), float(pct), int(cap),
                                                                   _ptr(clip), _ptr(y), _stream(stream)))
    return clip, y


def run(q, k=None, v=None, *, want=("support", "top_mass", "top32", "strict_zero", "row_max", "row_lse"),
        attend=False, heatmap=False, hist=False, noalloc=False, maps_want=(), pool=None, p_row=None,
        stream=None, **kw):
    """Allocate the requested outputs (and the workspace), call kvprof_row_stats (or kvprof_attend),
    and return the outputs as a dict of torch tensors (not synchronised). maps_want names the key-mass
    / spatial outputs, pool=(H, W) asks for the pooled map and p_row for one row's probabilities."""
    import torch

    B, Hq, Mq, _ = q.shape
    rows = B * Hq * Mq
    rb = kw.get("region_bounds")
    n_regions = 0 if rb is None else len(rb) - 1
    n_frames = kw.get("n_frames", 0)
    outs = _alloc_outputs(want, rows, n_regions, n_frames, q.device, q.shape[-1])
    hm = hm_mean = hs = None
    if heatmap:
        ng = kw["n_groups"]
        hm = torch.empty((B, Hq, ng, n_frames), dtype=torch.float32, device=q.device)
        hm_mean = torch.empty((B, ng, n_frames), dtype=torch.float32, device=q.device)
    if hist:
        kw.setdefault("hist_bins", 100)
        hs = torch.empty((B, 1 + n_regions, kw["hist_bins"]), dtype=torch.int32, device=q.device)
    maps = {}
    if maps_want:
        # probability maps: key_mass, spatial, spatial_mean, pooled (shape pool=(H, W)), p_row (index)
        n_k = k.shape[2] if k is not None else kw["n_k"]
        fl = kw.get("frame_len", 0)
        shapes = {"key_mass": (B, Hq, n_k), "spatial": (B, Hq, n_regions, fl), "spatial_mean": (B, n_regions, fl)}
        for name in maps_want:
            if name in shapes:
                maps[name] = torch.empty(shapes[name], dtype=torch.float32, device=q.device)
        if pool is not None:
            maps["pooled"] = torch.empty((B, Hq) + tuple(pool), dtype=torch.float32, device=q.device)
        if p_row is not None:
            maps["p_row_out"] = torch.empty(n_k, dtype=torch.float32, device=q.device)
    args = make_args(q, k, v, outputs=outs, heatmap=hm, heatmap_mean=hm_mean, hist=hs, **kw)
    for name, t in maps.items():
        setattr(args, name, _ptr(t))
    if pool is not None:
        args.pool_h, args.pool_w = int(pool[0]), int(pool[1])
    if p_row is not None:
        args.p_row = int(p_row)
    ws = None
    if noalloc:  # the library's own device scratch: no workspace tensor
        kvprof_row_stats_noalloc(args, stream)
    else:
        nws = kvprof_workspace_bytes(args)
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=q.device) if nws else None
        if ws is not None:
            args.workspace, args.workspace_bytes = ws.data_ptr(), ws.numel()
        (kvprof_attend if attend else kvprof_row_stats)(args, stream)
    res = dict(outs)
    res.update(maps)
    if hm is not None:
        res["heatmap"], res["heatmap_mean"] = hm, hm_mean
    if hs is not None:
        res["hist"] = hs
    res["_keepalive"] = (args, ws)
    return res
