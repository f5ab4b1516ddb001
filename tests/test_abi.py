"""CPU checks of the C ABI: the library loads, exports every function the header declares, computes
the host-side payload formula, and rejects invalid arguments before touching a device (every call
below fails validation, so no GPU is needed)."""
import ctypes
import json
import os

import pytest

from quantized_kv_amd import binding as B

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def lib():
    return B.load()


def test_exports_every_declared_symbol(lib):
    names = B.declared_functions()
    assert {"kvprof_pack_mxfp8", "kvprof_pack_int4kv", "kvprof_row_stats", "kvprof_attend",
            "kvprof_int4kv_bytes", "kvprof_compare", "kvprof_workspace_bytes", "kvprof_ablation_bias",
            "kvprof_cosine", "kvprof_percentile_clip", "kvprof_row_stats_noalloc"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.kvprof_abi_version() == 2


def test_args_struct_layout_matches_header():
    # offsets fixed by the C layout rules on x86-64 / LP64
    assert B.KvprofArgs.scale.offset == 28
    assert B.KvprofArgs.q.offset == 32
    assert B.KvprofArgs.workspace_bytes.offset + 8 == ctypes.sizeof(B.KvprofArgs)


def test_payload_pins_through_the_library(lib):
    g = json.load(open(os.path.join(GOLDEN, "p2_payload.json")))
    for row in g["rows"]:
        assert B.kvprof_int4kv_bytes(g["n_tokens"], 32, row["r_window"]) == row["payload_bytes"]
    # decode shape: N = 4096, d = 128
    assert [B.kvprof_int4kv_bytes(4096, 128, r) for r in (0, 16, 64)] == [655376, 670480, 710672]
    assert B.kvprof_int4kv_bytes(10, 32, 11) == 0  # R > N
    assert B.kvprof_int4kv_bytes(10, 33, 0) == 0  # d not a multiple of 32


def _err(lib):
    return lib.kvprof_last_error().decode()


def test_codec_validation(lib):
    fake = ctypes.c_void_p(0x1000)
    assert lib.kvprof_pack_mxfp8(fake, 4, 48, None, fake, fake, None) == B.KVPROF_ESHAPE
    assert "multiple of 32" in _err(lib)
    assert lib.kvprof_pack_mxfp8(fake, 4, 96, fake, fake, fake, None) == B.KVPROF_ESHAPE  # rotate, not 2^k
    assert lib.kvprof_pack_mxfp8(None, 4, 128, None, fake, fake, None) == B.KVPROF_EINVAL
    assert lib.kvprof_pack_mxfp8(fake, -1, 128, None, fake, fake, None) == B.KVPROF_EINVAL
    assert lib.kvprof_pack_int4kv(fake, fake, 2, 128, 32, 129, fake, 1 << 20, None) == B.KVPROF_EINVAL
    assert lib.kvprof_pack_int4kv(fake, fake, 2, 128, 32, 16, fake, 100, None) == B.KVPROF_ESIZE
    assert lib.kvprof_pack_int4kv(fake, fake, 2, 128, 32, 16, ctypes.c_void_p(0x1001), 1 << 20, None) == B.KVPROF_EALIGN
    assert lib.kvprof_pack_int4kv(fake, fake, 2, 128, 40, 16, fake, 1 << 20, None) == B.KVPROF_ESHAPE


def _args(**over):
    a = B.KvprofArgs()
    a.mode = B.MODE_BF16
    a.n_batch, a.n_heads_q, a.n_heads_kv, a.n_q, a.n_k, a.d = 1, 4, 2, 16, 256, 128
    a.scale = 0.088
    a.q = a.k = a.v = 0x10000
    a.support = 0x20000
    for k_, v_ in over.items():
        setattr(a, k_, v_)
    return a


@pytest.mark.parametrize("over,code,needle", [
    (dict(d=48), B.KVPROF_ESHAPE, "head dimension"),
    (dict(d=64, top32=0x30000), B.KVPROF_EUNSUPPORTED, "head dimension 64"),
    (dict(d=32, mode=B.MODE_MXFP8, q_codes=1, q_scales=1, k_codes=1, k_scales=1), B.KVPROF_EUNSUPPORTED, "MXFP8"),
    (dict(n_heads_q=3), B.KVPROF_ESHAPE, "multiple of n_heads_kv"),
    (dict(n_k=7000), B.KVPROF_EUNSUPPORTED, "exceeds"),
    (dict(n_k=0), B.KVPROF_ESHAPE, "n_k"),
    (dict(q=0), B.KVPROF_EINVAL, "q is null"),
    (dict(q=0x10008), B.KVPROF_EALIGN, "16-byte"),
    (dict(mode=7), B.KVPROF_EINVAL, "unknown mode"),
    (dict(mode=B.MODE_MXFP8), B.KVPROF_EINVAL, "q_codes"),
    (dict(mode=B.MODE_MXFP8, n_k=6401, q_codes=1, q_scales=1, k_codes=1, k_scales=1), B.KVPROF_EUNSUPPORTED, "exceeds"),
    (dict(mode=B.MODE_INT4KV), B.KVPROF_EINVAL, "kv_packed"),
    (dict(causal=2), B.KVPROF_EINVAL, "causal"),
    (dict(q_pos0=-1), B.KVPROF_EINVAL, "q_pos0"),
    (dict(o=0x30000, v=0), B.KVPROF_EINVAL, "o needs v"),
    (dict(frame_mass=0x30000), B.KVPROF_EINVAL, "n_frames"),
    (dict(tv_qk=0x30000), B.KVPROF_EINVAL, "MXFP8"),
    (dict(n_frames=65, frame_len=10), B.KVPROF_EUNSUPPORTED, "n_frames"),
    (dict(hist=0x30000), B.KVPROF_EINVAL, "hist_bins"),
    (dict(support=0x20002), B.KVPROF_EALIGN, "4-byte"),
])
def test_row_stats_validation(lib, over, code, needle):
    a = _args(**over)
    assert lib.kvprof_row_stats(ctypes.byref(a), None) == code
    assert needle in _err(lib)


def test_region_and_workspace_validation(lib):
    rb = (ctypes.c_int32 * 3)(0, 300, 256)
    a = _args(n_regions=2, region_bounds=rb)
    assert lib.kvprof_row_stats(ctypes.byref(a), None) == B.KVPROF_ESHAPE
    rb = (ctypes.c_int32 * 3)(0, 200, 100)
    a = _args(n_regions=2, region_bounds=rb)
    assert lib.kvprof_row_stats(ctypes.byref(a), None) == B.KVPROF_ESHAPE
    # every call with rows needs a workspace (the redo list of the row kernel)
    a = _args(n_frames=64, frame_len=2, frame_mass=0x30000)
    need = lib.kvprof_workspace_bytes(ctypes.byref(a))
    assert need >= 4 * (1 + 1)
    assert lib.kvprof_row_stats(ctypes.byref(a), None) == B.KVPROF_ESIZE
    # too many tiny segments inside one wave's key slice (validation never touches the workspace)
    a.workspace, a.workspace_bytes = 0x40000, need
    assert lib.kvprof_row_stats(ctypes.byref(a), None) == B.KVPROF_EUNSUPPORTED
    # MX mode needs a workspace for the decoded Q/K
    a = _args(mode=B.MODE_MXFP8, q_codes=1, q_scales=1, k_codes=1, k_scales=1)
    need = lib.kvprof_workspace_bytes(ctypes.byref(a))
    assert need >= (1 * 4 * 16 + 1 * 2 * 256) * 128 * 2
    assert lib.kvprof_row_stats(ctypes.byref(a), None) == B.KVPROF_ESIZE
    a = _args()
    assert lib.kvprof_attend(ctypes.byref(a), None) == B.KVPROF_EINVAL  # attend needs o
    assert lib.kvprof_compare(None, None, None, None, 4, 128, None, None, None, None) == B.KVPROF_EINVAL


def test_ablation_entry_points_validate(lib):
    """Local output ablation entry points reject bad ranges and pointers before any launch."""
    fake = ctypes.c_void_p(256)  # never dereferenced: every call below fails validation
    assert lib.kvprof_ablation_bias(None, 0, 0, 0, fake, None) == B.KVPROF_EINVAL
    assert lib.kvprof_ablation_bias(None, 100, 0, 0, None, None) == B.KVPROF_EINVAL
    assert lib.kvprof_ablation_bias(None, 100, 5, 4, fake, None) == B.KVPROF_EINVAL
    assert lib.kvprof_ablation_bias(None, 100, -1, 4, fake, None) == B.KVPROF_EINVAL
    assert lib.kvprof_ablation_bias(None, 100, 0, 101, fake, None) == B.KVPROF_EINVAL
    assert lib.kvprof_ablation_bias(None, 100, 0, 100, fake, None) == B.KVPROF_EINVAL
    assert b"keep at least one key" in lib.kvprof_last_error()
    assert lib.kvprof_ablation_bias(None, 100, 0, 10, ctypes.c_void_p(258), None) == B.KVPROF_EALIGN
    assert lib.kvprof_cosine(None, None, -1, 128, None, None, None) == B.KVPROF_EINVAL
    assert lib.kvprof_cosine(None, None, 4, 0, None, None, None) == B.KVPROF_EINVAL
    assert lib.kvprof_cosine(None, fake, 4, 128, fake, fake, None) == B.KVPROF_EINVAL
    assert lib.kvprof_cosine(fake, fake, 4, 128, fake, ctypes.c_void_p(260), None) == B.KVPROF_EALIGN


def test_binding_refuses_host_and_strided_tensors():
    """The binding passes device addresses only: a host tensor or a non-contiguous view is refused
    before any library call (the library would otherwise read or write it as dense GPU memory)."""
    import torch

    with pytest.raises(B.KvprofError, match="GPU memory"):
        B._ptr(torch.zeros(4))

    class _StridedDeviceView:  # stands in for a CUDA view on a machine without a GPU
        is_cuda = True
        shape = (4, 2)
        device = "cuda:0"

        def is_contiguous(self):
            return False

        def stride(self):
            return (4, 2)

        def data_ptr(self):
            raise AssertionError("address taken from a strided view")

    with pytest.raises(B.KvprofError, match="not contiguous"):
        B._ptr(_StridedDeviceView())
    q = torch.zeros((1, 1, 4, 128), dtype=torch.bfloat16)
    with pytest.raises(B.KvprofError, match="GPU memory"):
        B.run(q, q, want=("support",))


# The calls the boundary exports and their parameter types, as declared in include/kvprof.h. These are
# the survey's proposed calls with its two deliberate departures: bf16-only inputs (no dtype argument)
# and dense rows (no leading dimension), and the stream passed as void*.
_SIGNATURES = {
    "kvprof_abi_version": ("int", ["void"]),
    "kvprof_last_error": ("const char*", ["void"]),
    "kvprof_pack_mxfp8": ("int", ["const uint16_t*", "int64_t", "int32_t", "const int8_t*", "uint8_t*",
                                  "uint8_t*", "void*"]),
    "kvprof_unpack_mxfp8": ("int", ["const uint8_t*", "const uint8_t*", "int64_t", "int32_t", "float*",
                                    "void*"]),
    "kvprof_int4kv_bytes": ("size_t", ["int64_t", "int32_t", "int32_t"]),
    "kvprof_pack_int4kv": ("int", ["const uint16_t*", "const uint16_t*", "int32_t", "int64_t", "int32_t",
                                   "int32_t", "void*", "size_t", "void*"]),
    "kvprof_unpack_int4kv": ("int", ["const void*", "int32_t", "int64_t", "int32_t", "int32_t", "float*",
                                     "float*", "void*"]),
    "kvprof_workspace_bytes": ("size_t", ["const kvprof_args*"]),
    "kvprof_row_stats": ("int", ["const kvprof_args*", "void*"]),
    "kvprof_attend": ("int", ["const kvprof_args*", "void*"]),
    "kvprof_int4kv_append_window": ("int64_t", ["int64_t", "int64_t", "int32_t"]),
    "kvprof_int4kv_append": ("int", ["const void*", "int32_t", "int64_t", "int32_t", "int32_t", "const uint16_t*",
                                     "const uint16_t*", "int64_t", "int32_t", "void*", "size_t", "void*"]),
    "kvprof_percentile_clip": ("int", ["const float*", "int64_t", "double", "int64_t", "float*", "float*",
                                       "void*"]),
}


def _declarations():
    import re

    txt = open(B.HEADER).read()
    txt = re.sub(r"/\*.*?\*/", " ", txt, flags=re.S)
    out = {}
    for m in re.finditer(r"((?:const\s+)?\w+\s*\*?)\s*(kvprof_\w+)\s*\(([^)]*)\)\s*;", txt):
        ret = m.group(1).replace(" ", "").replace("constchar", "const char")
        params = []
        for p in m.group(3).split(","):
            p = " ".join(p.split())
            if p != "void":
                p = re.sub(r"\s*(\w+)$", "", p)  # drop the parameter name
            params.append(p.replace(" *", "*"))
        out[m.group(2)] = (ret, params)
    return out


def test_declared_signatures_match_the_boundary_list():
    decl = _declarations()
    for name, (ret, params) in _SIGNATURES.items():
        assert name in decl, name
        assert decl[name] == (ret, params), (name, decl[name])


def test_noalloc_rejects_oversized_scratch_before_device_work(lib):
    """The allocation-free entry point refuses arguments whose scratch exceeds its fixed array, before
    any device call (so this runs without a GPU), and validates like kvprof_row_stats."""
    assert lib.kvprof_noalloc_scratch_bytes() == 32 << 20
    a = _args(mode=B.MODE_MXFP8, n_batch=8, n_heads_q=32, n_heads_kv=32, n_q=96, n_k=6240,
              q_codes=1, q_scales=1, k_codes=1, k_scales=1)
    assert lib.kvprof_workspace_bytes(ctypes.byref(a)) > (32 << 20)
    assert lib.kvprof_row_stats_noalloc(ctypes.byref(a), None) == B.KVPROF_ESIZE
    assert "allocation-free" in _err(lib)
    assert lib.kvprof_row_stats_noalloc(None, None) == B.KVPROF_EINVAL
    a = _args(d=48)
    assert lib.kvprof_row_stats_noalloc(ctypes.byref(a), None) == B.KVPROF_ESHAPE


def test_maps_validation(lib):
    """Probability-map arguments are checked on the host before anything is enqueued."""
    fake = 0x10000
    a = _args(mode=B.MODE_MXFP8, q_codes=1, q_scales=1, k_codes=1, k_scales=1)
    a.key_mass = fake
    assert lib.kvprof_row_stats(ctypes.byref(a), None) == B.KVPROF_EUNSUPPORTED
    assert "BF16" in _err(lib)
    a = _args()
    a.spatial = fake
    assert lib.kvprof_row_stats(ctypes.byref(a), None) == B.KVPROF_EINVAL  # no regions / frame_len
    a = _args()
    a.pooled, a.pool_h, a.pool_w = fake, 64, 129
    assert lib.kvprof_row_stats(ctypes.byref(a), None) == B.KVPROF_EINVAL
    a.pool_w = 0
    assert lib.kvprof_row_stats(ctypes.byref(a), None) == B.KVPROF_EINVAL
    a = _args()
    a.p_row_out, a.p_row = fake, a.n_batch * a.n_heads_q * a.n_q
    assert lib.kvprof_row_stats(ctypes.byref(a), None) == B.KVPROF_EINVAL
    a.p_row = -1
    assert lib.kvprof_row_stats(ctypes.byref(a), None) == B.KVPROF_EINVAL


def test_maps_workspace_sizes(lib):
    a = _args(n_batch=1, n_heads_q=32, n_heads_kv=32, n_q=96, n_k=6240)
    base = lib.kvprof_workspace_bytes(ctypes.byref(a))
    a.key_mass = 0x10000
    blocks = 32 * 3  # 32-row blocks
    assert lib.kvprof_workspace_bytes(ctypes.byref(a)) == base + _r256(32 * 96 * 4) + _r256(blocks * 6240 * 4)
    a.pooled, a.pool_h, a.pool_w = 0x10000, 64, 96
    assert lib.kvprof_workspace_bytes(ctypes.byref(a)) == (base + _r256(32 * 96 * 4) + _r256(blocks * 6240 * 4)
                                                         + _r256(32 * 96 * 96 * 4))


def _r256(x):
    return (x + 255) // 256 * 256


def test_percentile_clip_validation(lib):
    fake = ctypes.c_void_p(0x10000)
    f = lib.kvprof_percentile_clip
    assert f(fake, 0, 99.5, 65536, fake, None, None) == B.KVPROF_EINVAL
    assert f(fake, 10, 100.5, 65536, fake, None, None) == B.KVPROF_EINVAL
    assert f(fake, 10, float("nan"), 65536, fake, None, None) == B.KVPROF_EINVAL
    assert f(fake, 10, 99.5, 0, fake, None, None) == B.KVPROF_EINVAL
    assert f(None, 10, 99.5, 8, fake, None, None) == B.KVPROF_EINVAL
    assert f(ctypes.c_void_p(0x10002), 10, 99.5, 8, fake, None, None) == B.KVPROF_EALIGN


def test_append_window_rule_matches_oracle(lib):
    from oracle import kvprof_oracle as O

    for r_in in range(0, 90, 5):
        for t in range(0, 130, 7):
            for R in (0, 16, 64):
                assert B.kvprof_int4kv_append_window(r_in, t, R) == O.rolled_window(r_in, t, R)
    assert B.kvprof_int4kv_append_window(-1, 0, 0) == -1


def test_append_validation(lib):
    fake = ctypes.c_void_p(0x10000)
    f = lib.kvprof_int4kv_append
    big = 1 << 30
    # 112 tokens in the 4-bit part: not whole groups
    assert f(fake, 2, 128, 32, 16, fake, fake, 1, 16, ctypes.c_void_p(0x10000000), big, None) == B.KVPROF_EINVAL
    assert "whole" in _err(lib)
    assert f(fake, 2, 128, 48, 0, fake, fake, 1, 16, ctypes.c_void_p(0x10000000), big, None) == B.KVPROF_ESHAPE
    assert f(fake, 2, 128, 32, 0, None, fake, 1, 16, ctypes.c_void_p(0x10000000), big, None) == B.KVPROF_EINVAL
    assert f(fake, 2, 128, 32, 0, fake, fake, 1, 16, ctypes.c_void_p(0x10000000), 100, None) == B.KVPROF_ESIZE
    assert f(fake, 2, 128, 32, 0, fake, fake, 1, 16, ctypes.c_void_p(0x10001), big, None) == B.KVPROF_EALIGN
    assert f(fake, 2, 128, 32, 0, fake, fake, 1, 16, ctypes.c_void_p(0x10100), big, None) == B.KVPROF_EINVAL  # overlap
    assert "overlaps" in _err(lib)
