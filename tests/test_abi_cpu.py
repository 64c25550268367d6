"""The C ABI without a GPU: the library loads, exports every declared entry
point, and rejects bad arguments on the host with the documented status before
anything is launched (these calls never reach HIP)."""
import ctypes
import os
import re

import pytest

import mla_latent_kv_09_amd as mla
from mla_latent_kv_09_amd import _Cache, _Dims, _QProj

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")

OK, NULL, SHAPE, DTYPE, UNSUP, WS, HIP, ALIGN = range(8)
P = 0x100000  # stands in for a device pointer; never dereferenced by these calls


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = mla.library()
    names = declared_functions()
    assert {"mla_rope_latent_project", "mla_decode", "mla_prefill"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert mla.mla_version() >= 100


def test_status_strings():
    for s in range(8):
        assert mla.mla_status_string(s)
    assert "unknown" in mla.mla_status_string(99)


def V3(dtype=1, **kw):
    d = dict(n_heads=128, d_c=512, d_rope=64, d_nope=128, d_v=128, softmax_scale=0.0, rope_base=10000.0, dtype=dtype)
    d.update(kw)
    return _Dims(**d)


def cache(**kw):
    c = dict(rows=P, num_blocks=128, block_size=64, block_table=P, max_blocks_per_seq=128, context_lens=P,
             max_context=8192)
    c.update(kw)
    return _Cache(**c)


def decode(d=None, batch=4, ptrs=(P, P, P, P), c=None, out=P, ws=P, wsb=1 << 30):
    lib = mla.library()
    d = V3() if d is None else d
    c = cache() if c is None else c
    return lib.mla_decode(ctypes.byref(d) if d is not None else None, batch, *ptrs, ctypes.byref(c), out, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=2), DTYPE), (dict(dtype=-1), DTYPE),
    (dict(n_heads=0), SHAPE), (dict(n_heads=257), SHAPE),
    (dict(d_c=0), SHAPE), (dict(d_c=12), SHAPE), (dict(d_c=2048), SHAPE),
    (dict(d_rope=3), SHAPE), (dict(d_rope=0), SHAPE), (dict(d_rope=130), SHAPE), (dict(d_rope=6), SHAPE),
    (dict(d_nope=0), SHAPE), (dict(d_v=300), SHAPE),
    (dict(rope_base=1.0), SHAPE), (dict(rope_base=float("nan")), SHAPE),
    (dict(softmax_scale=float("inf")), SHAPE),
])
def test_bad_dims_are_rejected(kw, status):
    assert decode(V3(**kw)) == status


def test_null_and_shape_errors_in_decode():
    lib = mla.library()
    assert lib.mla_decode(None, 4, P, P, P, P, ctypes.byref(cache()), P, P, 1 << 30, None) == NULL
    assert decode(batch=-1) == SHAPE
    assert decode(batch=0) == OK                       # empty batch: no-op
    for i in range(4):
        ptrs = [P] * 4
        ptrs[i] = None
        assert decode(ptrs=tuple(ptrs)) == NULL
    assert decode(out=None) == NULL
    assert decode(c=cache(rows=None)) == NULL
    assert decode(c=cache(context_lens=None)) == NULL
    assert decode(c=cache(max_context=0)) == SHAPE
    assert decode(c=cache(block_size=0)) == SHAPE
    assert decode(c=cache(max_blocks_per_seq=10)) == SHAPE   # 10 * 64 < 8192
    assert decode(c=cache(num_blocks=0)) == SHAPE


def test_alignment_errors():
    assert decode(ptrs=(P + 2, P, P, P)) == ALIGN
    assert decode(out=P + 8) == ALIGN
    assert decode(c=cache(rows=P + 4)) == ALIGN
    assert decode(c=cache(context_lens=P + 2)) == ALIGN


def test_workspace_errors():
    need = mla.mla_decode_workspace_size(V3(), 4, 8192)
    if need:
        assert decode(wsb=need - 1) == WS
        assert decode(ws=None, wsb=need) == NULL
        assert decode(ws=P + 16, wsb=need) == ALIGN


def test_prefill_errors():
    lib = mla.library()
    c = cache()

    def pf(batch=2, seq=100, cc=c, ptrs=(P, P, P, P), out=P):
        return lib.mla_prefill(ctypes.byref(V3()), batch, seq, *ptrs, ctypes.byref(cc), out, P, 1 << 30, None)
    assert pf(seq=-1) == SHAPE
    assert pf(batch=-3) == SHAPE
    assert pf(seq=0) == OK and pf(batch=0) == OK
    assert pf(seq=9000) == SHAPE                         # more queries than the context bound
    assert pf(ptrs=(P, None, P, P)) == NULL
    assert pf(out=None) == NULL


def test_decode_multi_errors():
    lib = mla.library()
    c = cache()

    def dm(batch=4, q_len=2, cc=c, ptrs=(P, P, P, P), out=P, ws=P, wsb=1 << 30):
        return lib.mla_decode_multi(ctypes.byref(V3()), batch, q_len, *ptrs, ctypes.byref(cc), out, ws, wsb, None)
    assert dm(q_len=0) == SHAPE and dm(q_len=-1) == SHAPE
    assert dm(q_len=65) == SHAPE                          # above the documented q_len bound
    assert dm(batch=-1) == SHAPE
    assert dm(batch=1100, q_len=60) == SHAPE              # 66,000 query rows
    assert dm(batch=0) == OK
    assert dm(q_len=8, cc=cache(max_context=4, max_blocks_per_seq=1)) == SHAPE  # q_len > max_context
    assert dm(ptrs=(P, P, None, P)) == NULL
    assert dm(out=None) == NULL
    assert dm(ptrs=(P, P + 2, P, P)) == ALIGN
    need = mla.mla_decode_multi_workspace_size(V3(), 4, 2, 8192)
    assert need > 0
    assert dm(wsb=need - 1) == WS
    assert dm(ws=None, wsb=need) == NULL
    # query rows are what the workspace scales with: 4 x 2 rows need what 8 x 1 rows do
    assert need == mla.mla_decode_workspace_size(V3(), 8, 8192)
    assert mla.mla_decode_multi_workspace_size(V3(), 4, 1, 8192) == mla.mla_decode_workspace_size(V3(), 4, 8192)
    with pytest.raises(mla.MLAError):
        mla.mla_decode_multi_workspace_size(V3(), 4, 0, 8192)


def test_fp8_entry_points_errors_and_sizes():
    lib = mla.library()
    assert mla.mla_fp8_page_bytes(V3(), 64) == 41024          # 64 x 640 + 64
    assert mla.mla_fp8_page_bytes(_Dims(4, 32, 8, 16, 16, 0.0, 10000.0, 1), 16) == 16 * 48 + 16
    assert mla.mla_fp8_page_bytes(_Dims(4, 40, 8, 16, 16, 0.0, 10000.0, 1), 3) == 176   # 3 x 56 + 3 -> 176
    with pytest.raises(mla.MLAError):
        mla.mla_fp8_page_bytes(V3(), 0)

    def q(n=8, rows=P, slots=P, bs=64, pool=P, d=None):
        d = V3() if d is None else d
        return lib.mla_quantize_fp8(ctypes.byref(d), n, rows, slots, bs, pool, None)
    assert q(n=0) == OK
    assert q(n=-1) == SHAPE and q(bs=0) == SHAPE and q(bs=5000) == SHAPE
    assert q(rows=None) == NULL and q(pool=None) == NULL
    assert q(rows=P + 8) == ALIGN and q(pool=P + 4) == ALIGN and q(slots=P + 2) == ALIGN
    assert q(d=V3(dtype=0)) == DTYPE                           # rows must be bf16

    def d8(batch=4, q_len=1, d=None, c=None, ptrs=(P, P, P, P), out=P, ws=P, wsb=1 << 30):
        d = V3() if d is None else d
        c = cache() if c is None else c
        return lib.mla_decode_fp8(ctypes.byref(d), batch, q_len, *ptrs, ctypes.byref(c), out, ws, wsb, None)
    assert d8(batch=0) == OK
    assert d8(q_len=0) == SHAPE and d8(q_len=65) == SHAPE and d8(batch=-2) == SHAPE
    assert d8(ptrs=(None, P, P, P)) == NULL and d8(out=None) == NULL
    assert d8(d=_Dims(4, 32, 8, 16, 16, 0.0, 10000.0, 1)) == UNSUP       # not the DeepSeek-V3 shape
    assert d8(c=cache(block_table=None)) == UNSUP                          # contiguous cache
    assert d8(d=V3(n_heads=129)) == UNSUP                                  # more heads than the FP8 kernel holds
    assert d8(d=V3(n_heads=257)) == SHAPE                                  # beyond any path
    need = mla.mla_decode_fp8_workspace_size(V3(), 4, 2, 8192)
    assert need > 0 and d8(q_len=2, wsb=need - 1) == WS
    assert mla.mla_decode_fp8_workspace_size(_Dims(4, 32, 8, 16, 16, 0.0, 10000.0, 1), 4, 1, 64) == 0


def test_project_errors():
    lib = mla.library()
    d = V3()
    c = cache()

    def pj(n=16, dm=7168, ptrs=(P, P, P, P, P), q=None, ws=P, wsb=1 << 30, dd=d):
        return lib.mla_rope_latent_project(ctypes.byref(dd), n, dm, *ptrs, ctypes.byref(c),
                                           ctypes.byref(q) if q is not None else None, ws, wsb, None)
    assert pj(n=-1) == SHAPE
    assert pj(n=0) == OK
    assert pj(dm=0) == SHAPE and pj(dm=20000) == SHAPE
    for i in range(5):
        ptrs = [P] * 5
        ptrs[i] = None
        assert pj(ptrs=tuple(ptrs)) == NULL
    assert pj(ptrs=(P + 2, P, P, P, P)) == ALIGN
    assert pj(ptrs=(P, P, P, P + 2, P)) == ALIGN
    q = _QProj(1536, P, P, P, P, P)
    assert pj(q=_QProj(1530, P, P, P, P, P)) == SHAPE
    assert pj(q=_QProj(1536, P, None, P, P, P)) == NULL
    need = mla.mla_project_workspace_size(d, 16, 1536)
    assert need == 16 * 1536 * 4
    assert pj(q=q, wsb=need - 1) == WS
    assert pj(q=q, ws=None, wsb=need) == NULL
    assert pj(dd=V3(dtype=5)) == DTYPE


def test_workspace_sizes_and_paths():
    assert mla.mla_project_workspace_size(V3(), 0, 0) == 0
    assert mla.mla_decode_workspace_size(V3(), 0, 8192) == 0
    tiny = _Dims(4, 32, 8, 16, 16, 0.0, 10000.0, 0)
    assert mla.mla_decode_workspace_size(tiny, 1, 64) == 0
    assert mla.mla_decode_path(tiny, 64, 0) == 0          # fp32 -> generic kernels
    assert mla.mla_decode_path(V3(dtype=9), 64, 1) == -1
    with pytest.raises(mla.MLAError):
        mla.mla_decode_workspace_size(V3(dtype=9), 1, 1)


def test_one_workspace_call_for_the_three_core_entry_points():
    d = V3()
    assert mla.mla_workspace_size(mla.MLA_OP_PROJECT, d, 16, 1536) == mla.mla_project_workspace_size(d, 16, 1536)
    assert mla.mla_workspace_size(mla.MLA_OP_DECODE, d, 64, 8192) == mla.mla_decode_workspace_size(d, 64, 8192)
    assert mla.mla_workspace_size(mla.MLA_OP_PREFILL, d, 4, 4096) == \
        mla.mla_prefill_workspace_size(d, 4, 4096, 4096)
    assert mla.mla_workspace_size(mla.MLA_OP_DECODE, d, 64, 8192) > 0
    lib = mla.library()
    n = ctypes.c_size_t(12345)
    assert lib.mla_workspace_size(7, ctypes.byref(d.c() if hasattr(d, "c") else d), 1, 1, ctypes.byref(n)) == 4
    assert n.value == 12345                               # untouched on an unknown op
    with pytest.raises(mla.MLAError):
        mla.mla_workspace_size(mla.MLA_OP_DECODE, d, -1, 8192)
