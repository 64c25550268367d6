"""The attention layer's output side on the GPU, through the C ABI: W_O over
the per-head outputs (mla_output_project), W_UV folded into W_O
(mla_fold_output_weights, "DeepSeek-V2 paper digest" §2.2) and decode straight
to the layer output with the folded weights (mla_decode_folded), each against
the oracle's plain definition (W_O applied to the concatenated per-head
outputs of the explicit-K/V attention)."""
import numpy as np
import pytest
import torch

import mla_latent_kv_09_amd as mla
import oracle
from synth import Dims, draw_output_weights, f32_to_bf16_bits, from_torch, make_decode_case, to_torch

from gpu_helpers import assert_parity, device_cache, fails_bar

pytestmark = pytest.mark.gpu

V3 = dict(d_c=512, d_rope=64, d_nope=128, d_v=128)


def _log(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("n,H,dv,d_model,dtype", [
    (64, 128, 128, 7168, "bf16"),     # decode rows, the V3 output projection (row GEMM path)
    (7, 16, 128, 1000, "bf16"),       # few rows, d_model not a multiple of 64
    (300, 16, 128, 512, "bf16"),      # many rows (tiled MFMA GEMM)
    (5, 3, 5, 10, "bf16"),            # odd widths (generic kernel)
    (4, 4, 16, 24, "f32"),            # fp32 (generic kernel)
])
def test_output_project_matches_the_oracle(n, H, dv, d_model, dtype):
    _log(f"output projection n={n} H={H} d_v={dv} d_model={d_model} {dtype}")
    rng = np.random.default_rng(n + H + d_model)
    x = rng.standard_normal((n, H, dv)).astype(np.float32) * 0.05
    x = f32_to_bf16_bits(x) if dtype == "bf16" else x
    dims = Dims(H, 16, 8, 8, dv, dtype=dtype)
    w_o = draw_output_weights(77 + n, d_model, H, dv, dtype)
    got = from_torch(mla.mla_output_project(dims, to_torch(x), to_torch(w_o)))
    torch.cuda.synchronize()
    ref = oracle.output_projection(x, w_o)
    assert_parity(got, ref, dtype, "output projection")


@pytest.mark.parametrize("H,dv,dc,d_model,dtype", [(128, 128, 512, 256, "bf16"), (3, 5, 16, 10, "bf16"),
                                                   (4, 8, 16, 24, "f32")])
def test_fold_output_weights_matches_the_oracle(H, dv, dc, d_model, dtype):
    _log(f"fold W_UV into W_O H={H} d_v={dv} d_c={dc} d_model={d_model} {dtype}")
    dims = Dims(H, dc, 8, 16, dv, dtype=dtype)
    case = make_decode_case(90 + H, 1, dims, [1])
    w_o = draw_output_weights(91 + H, d_model, H, dv, dtype)
    got = from_torch(mla.mla_fold_output_weights(dims, to_torch(case.w_uv), to_torch(w_o)))
    torch.cuda.synchronize()
    ref = oracle.fold_output_weights(case.w_uv, w_o, H, dv)
    if dtype == "f32":
        assert np.allclose(got, ref, rtol=1e-5, atol=1e-6)
    else:
        # one bf16 rounding of an fp32 sum: within half a bf16 ulp plus accumulation slack
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6 * np.abs(ref).max())


def _folded_case(seed, B, H, lens, d_model, q_len=1):
    dims = Dims(H, **V3)
    case = make_decode_case(seed, B, dims, lens, shuffle=True, q_len=q_len)
    w_o = draw_output_weights(seed + 1, d_model, H, 128)
    return case, w_o


def _run_folded(case, w_o):
    c = device_cache(case.cache)
    qn, qp = to_torch(case.q_nope), to_torch(case.q_pe)
    if case.q_len == 1:
        qn, qp = qn.unsqueeze(1), qp.unsqueeze(1)
    w_ouv = mla.mla_fold_output_weights(case.dims, to_torch(case.w_uv), to_torch(w_o))
    out = mla.mla_decode_folded(case.dims, qn, qp, to_torch(case.w_uk), w_ouv, c)
    torch.cuda.synchronize()
    return from_torch(out)


def _oracle_out(case, w_o, seqs=None, w_uv=None):
    c = case.cache
    w_uv = case.w_uv if w_uv is None else w_uv
    if case.q_len == 1:
        return oracle.decode_output(case.dims, case.q_nope, case.q_pe, case.w_uk, w_uv, w_o, c.pool, c.block_table,
                                    c.context_lens, batch_rows=seqs)[:, None]
    seqs = list(range(case.batch)) if seqs is None else seqs
    out = np.empty((len(seqs), case.q_len, w_o.shape[0]))
    for j in range(case.q_len):
        out[:, j] = oracle.decode_output(case.dims, case.q_nope[:, j], case.q_pe[:, j], case.w_uk, w_uv, w_o,
                                         c.pool, c.block_table, c.context_lens - (case.q_len - 1 - j),
                                         batch_rows=seqs)
    return out


@pytest.mark.parametrize("name,B,H,lens,d_model,q_len", [
    ("H128 ragged", 4, 128, [1, 64, 700, 2049], 1024, 1),
    ("H16 d_model 7168", 3, 16, [129, 5000, 3], 7168, 1),
    ("H100 q2", 3, 100, [2, 300, 1500], 512, 2),
])
def test_decode_folded_matches_the_oracle(name, B, H, lens, d_model, q_len):
    _log(f"decode with W_UV folded into W_O: {name}")
    case, w_o = _folded_case(300 + H + q_len, B, H, lens, d_model, q_len)
    got = _run_folded(case, w_o)
    ref = _oracle_out(case, w_o)
    assert_parity(got, ref, "bf16", name)


def test_decode_folded_negative_controls_fail_the_bar():
    _log("decode folded: negative controls")
    case, w_o = _folded_case(310, 3, 128, [100, 700, 1], 1024)
    got = _run_folded(case, w_o)
    assert_parity(got, _oracle_out(case, w_o), "bf16", "control")
    H, dv = 128, 128
    reversed_heads = w_o.reshape(-1, H, dv)[:, ::-1].reshape(w_o.shape).copy()
    assert fails_bar(got, _oracle_out(case, reversed_heads), "bf16")
    assert fails_bar(got, _oracle_out(case, w_o, w_uv=np.roll(case.w_uv, 128, axis=0)), "bf16")


def test_decode_then_output_project_equals_the_folded_decode():
    """The two orders of the output side (per-head W_UV then W_O, or the folded
    weights on o_c) agree within the bar on the same inputs."""
    _log("decode + W_O vs folded decode")
    case, w_o = _folded_case(320, 8, 128, [8192, 1, 3000, 64, 65, 4097, 129, 7000], 2048)
    c = device_cache(case.cache)
    per_head = mla.mla_decode(case.dims, to_torch(case.q_nope), to_torch(case.q_pe), to_torch(case.w_uk),
                              to_torch(case.w_uv), c)
    plain = from_torch(mla.mla_output_project(case.dims, per_head, to_torch(w_o)))
    folded = _run_folded(case, w_o)[:, 0]
    assert_parity(folded, plain, "bf16", "folded vs W_O after W_UV")
    ref = _oracle_out(case, w_o, seqs=[0, 2, 7])[:, 0]
    assert_parity(plain[[0, 2, 7]], ref, "bf16", "W_O after W_UV vs oracle")


def test_decode_folded_refuses_shapes_outside_the_mfma_path():
    dims = Dims(4, 32, 8, 16, 16, dtype="f32")
    case = make_decode_case(330, 2, dims, [10, 20])
    c = device_cache(case.cache)
    w_ouv = torch.zeros((64, 4 * 32), dtype=torch.float32, device="cuda")
    with pytest.raises(mla.MLAError) as e:
        mla.mla_decode_folded(dims, to_torch(case.q_nope).unsqueeze(1), to_torch(case.q_pe).unsqueeze(1),
                              to_torch(case.w_uk), w_ouv, c)
    assert e.value.status == 4
