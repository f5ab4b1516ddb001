"""GPU test of kvprof_row_stats_noalloc, the allocation-free variant of kvprof_row_stats: through the C
ABI, its outputs must equal those of kvprof_row_stats (same kernels, so bit for bit) on two calls in a
row, the second with a smaller input, including calls whose scratch holds per-row intermediates (heatmap
and histograms without their per-row outputs) and decoded MXFP8 operands."""
import numpy as np
import pytest
import torch

from quantized_kv_amd import binding as B
from quantized_kv_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
STATS = ("support", "top_mass", "top32", "strict_zero", "row_max", "row_lse", "region_mass", "frame_mass")


def _same(a, b):
    for k, v in a.items():
        if isinstance(v, torch.Tensor):
            assert torch.equal(v, b[k]), k


def _pair(Q, K, **kw):
    ref = B.run(Q, K, **kw)
    got = B.run(Q, K, noalloc=True, **kw)
    torch.cuda.synchronize()
    _same(ref, got)
    return got


def test_noalloc_matches_row_stats_two_calls(kvprof_lib):
    assert B.kvprof_noalloc_scratch_bytes() == 32 << 20
    for (Bn, Hq, Hkv, Mq, Sk, seed) in ((2, 4, 2, 53, 2100, 31), (1, 2, 1, 19, 700, 32)):
        Q, K, _ = inputs.generic_inputs(seed, (Bn, Hq, Mq, 128), (Bn, Hkv, Sk, 128), q_scale=1.3)
        rb = [0, Sk // 3, Sk // 2, Sk]
        groups = torch.from_numpy((np.arange(Mq) % 4).astype(np.int32)).to(DEV)
        kw = dict(scale=0.088, region_bounds=rb, frame_len=Sk // 7 + 1, n_frames=7, row_group=groups,
                  n_groups=4)
        print(f"noalloc case B={Bn} Hq={Hq} Hkv={Hkv} Mq={Mq} Sk={Sk}", flush=True)
        _pair(Q.to(DEV), K.to(DEV), want=STATS, heatmap=True, hist=True, **kw)
        # heatmap and histograms without their per-row inputs: those arrays live in the scratch
        _pair(Q.to(DEV), K.to(DEV), want=("top32",), heatmap=True, hist=True, **kw)


def test_noalloc_mxfp8_two_calls(kvprof_lib):
    signs = torch.from_numpy(inputs.hadamard_signs(4)).to(DEV)
    for (Mq, Sk, seed) in ((96, 600, 41), (40, 200, 42)):
        print(f"noalloc MXFP8 case Mq={Mq} Sk={Sk}", flush=True)
        Q, K, _ = inputs.generic_inputs(seed, (1, 2, Mq, 128), (1, 1, Sk, 128), q_scale=1.5)
        Q, K = Q.to(DEV), K.to(DEV)
        qc, qs = B.kvprof_pack_mxfp8(Q.reshape(-1, 128), signs)
        kc, ks = B.kvprof_pack_mxfp8(K.reshape(-1, 128), signs)
        _pair(Q, K, mode=B.MODE_MXFP8, q_codes=qc, q_scales=qs, k_codes=kc, k_scales=ks,
              want=STATS[:6] + ("tv_qk", "argmax", "argmax_ref", "p_zero_frac", "tv_p", "p_rowsum"),
              scale=0.088)
