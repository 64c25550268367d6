"""The no-allocation decode entry point (mla_decode_noalloc) against
mla_decode_multi, through the C ABI: two calls in a row on the library's fixed
scratch array, the second smaller, each equal to the workspace entry point's
output bit for bit (same kernels, same launch plan); a call too large for the
array is refused before anything runs."""
import numpy as np
import pytest
import torch

import mla_latent_kv_09_amd as mla
from synth import Dims, from_torch, make_decode_case, to_torch

from gpu_helpers import assert_parity, device_cache

pytestmark = pytest.mark.gpu

V3 = dict(d_c=512, d_rope=64, d_nope=128, d_v=128)


def _both(case):
    c = device_cache(case.cache)
    qn, qp = to_torch(case.q_nope), to_torch(case.q_pe)
    if case.q_len == 1:
        qn, qp = qn.unsqueeze(1), qp.unsqueeze(1)
    wuk, wuv = to_torch(case.w_uk), to_torch(case.w_uv)
    ref = mla.mla_decode_multi(case.dims, qn, qp, wuk, wuv, c)
    out = torch.full_like(ref, float("nan"))
    mla.mla_decode_noalloc(case.dims, qn, qp, wuk, wuv, c, out)
    torch.cuda.synchronize()
    return from_torch(out), from_torch(ref)


def test_noalloc_decode_matches_the_workspace_entry_point_twice():
    print("noalloc decode: large call then a smaller one", flush=True)
    big = make_decode_case(71, 16, Dims(128, **V3), [8192] * 8 + [5000, 1, 64, 65, 2047, 300, 7000, 129],
                           shuffle=True)
    assert mla.mla_decode_multi_workspace_size(big.dims, 16, 1, 8192) <= mla.mla_noalloc_scratch_bytes()
    got, ref = _both(big)
    assert np.array_equal(got, ref)
    assert_parity(got, ref, "bf16", "noalloc large")
    small = make_decode_case(72, 3, Dims(32, **V3), [100, 1, 700], shuffle=True, q_len=2)
    got, ref = _both(small)
    assert np.array_equal(got, ref)
    assert_parity(got, ref, "bf16", "noalloc small")


def test_noalloc_decode_refuses_more_than_the_fixed_array():
    print("noalloc decode: oversize call refused", flush=True)
    d = Dims(128, **V3)
    B, L = 256, 16384
    need = mla.mla_decode_multi_workspace_size(d, B, 1, L)
    assert need > mla.mla_noalloc_scratch_bytes()
    case = make_decode_case(73, 2, d, [64, 64])
    rows = device_cache(case.cache).rows
    # only the sizes the host check reads matter: B sequences of up to L tokens
    # (block table of L / 64 pages each); the call is refused before any launch
    table = torch.zeros((B, L // 64), dtype=torch.int32, device="cuda")
    c = mla.Cache(rows, torch.full((B,), 64, dtype=torch.int32, device="cuda"), L, table)
    qn = torch.zeros((B, 1, 128, 128), dtype=torch.bfloat16, device="cuda")
    qp = torch.zeros((B, 1, 128, 64), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((B, 1, 128, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mla.MLAError) as e:
        mla.mla_decode_noalloc(d, qn, qp, to_torch(case.w_uk), to_torch(case.w_uv), c, out)
    assert e.value.status == 5   # MLA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
