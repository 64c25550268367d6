"""The entry points under HIP graph capture (torch.cuda.CUDAGraph).

Every kernel the library launches goes on the caller's stream, with the
caller's workspace and no allocation, synchronisation or memset of its own, so
a decode or prefill step can be captured once and replayed. Each graph is
replayed several times, with eager work and synchronisations between the
replays and new inputs copied into the captured buffers, and every replay must
equal the eager call on the same inputs bit for bit.
"""
import numpy as np
import pytest
import torch

import mla_latent_kv_09_amd as mla
from synth import Dims, from_torch, make_decode_case, to_torch

from gpu_helpers import device_cache

pytestmark = pytest.mark.gpu

V3 = dict(d_c=512, d_rope=64, d_nope=128, d_v=128)


def _log(msg):
    print(msg, flush=True)


def _replays_match(capture_fn, eager_fn, set_inputs, n_inputs=3):
    """capture_fn() records the step into the graph; eager_fn() returns a
    fresh eager result for the current inputs; set_inputs(k) writes input set
    k into the captured buffers."""
    set_inputs(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        capture_fn()          # warm-up outside the graph, on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        out = capture_fn()
    torch.cuda.synchronize()
    for k in list(range(n_inputs)) + [0]:
        set_inputs(k)
        torch.cuda.synchronize()
        ref = from_torch(eager_fn())
        scratch = torch.randn(1 << 20, device="cuda")      # unrelated eager work between replays
        scratch.mul_(2.0).sum().item()
        g.replay()
        torch.cuda.synchronize()
        got = from_torch(out)
        assert np.array_equal(got, ref), f"replay with inputs {k} differs from the eager call"


def _query_sets(case, n):
    rng = np.random.default_rng(7)
    from synth import f32_to_bf16_bits
    sets = [(case.q_nope, case.q_pe)]
    for _ in range(n - 1):
        sets.append((f32_to_bf16_bits(rng.standard_normal(case.q_nope.shape).astype(np.float32)),
                     f32_to_bf16_bits(rng.standard_normal(case.q_pe.shape).astype(np.float32))))
    return sets


def test_decode_replays_in_a_graph():
    _log("graph: mla_decode")
    case = make_decode_case(61, 6, Dims(128, **V3), [1, 64, 65, 700, 2048, 3000], shuffle=True)
    c = device_cache(case.cache)
    d = case.dims
    qn, qp = to_torch(case.q_nope), to_torch(case.q_pe)
    wk, wv = to_torch(case.w_uk), to_torch(case.w_uv)
    ws = torch.empty(mla.mla_decode_workspace_size(d, case.batch, c.max_context), dtype=torch.uint8, device="cuda")
    out = torch.empty((case.batch, d.n_heads, d.d_v), dtype=torch.bfloat16, device="cuda")
    sets = _query_sets(case, 3)

    def set_inputs(k):
        qn.copy_(to_torch(sets[k][0]))
        qp.copy_(to_torch(sets[k][1]))

    _replays_match(lambda: mla.mla_decode(d, qn, qp, wk, wv, c, out=out, workspace=ws),
                   lambda: mla.mla_decode(d, qn, qp, wk, wv, c), set_inputs)


def test_multi_token_decode_replays_in_a_graph():
    _log("graph: mla_decode_multi")
    case = make_decode_case(62, 8, Dims(64, **V3), [2, 3, 64, 65, 129, 700, 1500, 2047], shuffle=True, q_len=2)
    c = device_cache(case.cache)
    d = case.dims
    qn, qp = to_torch(case.q_nope), to_torch(case.q_pe)
    wk, wv = to_torch(case.w_uk), to_torch(case.w_uv)
    ws = torch.empty(mla.mla_decode_multi_workspace_size(d, case.batch, 2, c.max_context), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((case.batch, 2, d.n_heads, d.d_v), dtype=torch.bfloat16, device="cuda")
    sets = _query_sets(case, 3)

    def set_inputs(k):
        qn.copy_(to_torch(sets[k][0]))
        qp.copy_(to_torch(sets[k][1]))

    _replays_match(lambda: mla.mla_decode_multi(d, qn, qp, wk, wv, c, out=out, workspace=ws),
                   lambda: mla.mla_decode_multi(d, qn, qp, wk, wv, c), set_inputs)


def test_fp8_decode_replays_in_a_graph():
    _log("graph: mla_decode_fp8")
    case = make_decode_case(63, 5, Dims(128, **V3), [1, 100, 640, 1000, 4097], shuffle=True)
    cc = case.cache
    d = case.dims
    nb, P, R = cc.pool.shape
    pages = torch.zeros((nb, mla.mla_fp8_page_bytes(d, P)), dtype=torch.uint8, device="cuda")
    mla.mla_quantize_fp8(d, to_torch(cc.pool).view(nb * P, R), pages, None, P)
    c = mla.Fp8Cache(pages, to_torch(cc.context_lens.astype(np.int32)), int(cc.context_lens.max()),
                     to_torch(cc.block_table.astype(np.int32)))
    qn, qp = to_torch(case.q_nope), to_torch(case.q_pe)
    wk, wv = to_torch(case.w_uk), to_torch(case.w_uv)
    ws = torch.empty(mla.mla_decode_fp8_workspace_size(d, case.batch, 1, c.max_context), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((case.batch, d.n_heads, d.d_v), dtype=torch.bfloat16, device="cuda")
    sets = _query_sets(case, 3)

    def set_inputs(k):
        qn.copy_(to_torch(sets[k][0]))
        qp.copy_(to_torch(sets[k][1]))

    _replays_match(lambda: mla.mla_decode_fp8(d, qn, qp, wk, wv, c, out=out, workspace=ws),
                   lambda: mla.mla_decode_fp8(d, qn, qp, wk, wv, c), set_inputs)


def test_chunked_prefill_replays_in_a_graph():
    _log("graph: mla_prefill")
    d = Dims(16, **V3)
    case = make_decode_case(64, 2, d, [300, 200], shuffle=True)
    c = device_cache(case.cache)
    S = 70
    rng = np.random.default_rng(5)
    from synth import f32_to_bf16_bits
    sets = [(f32_to_bf16_bits(rng.standard_normal((2, S, 16, 128)).astype(np.float32)),
             f32_to_bf16_bits(rng.standard_normal((2, S, 16, 64)).astype(np.float32))) for _ in range(3)]
    qn, qp = to_torch(sets[0][0]), to_torch(sets[0][1])
    wk, wv = to_torch(case.w_uk), to_torch(case.w_uv)
    ws = torch.empty(max(mla.mla_prefill_workspace_size(d, 2, S, c.max_context), 1), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((2, S, 16, 128), dtype=torch.bfloat16, device="cuda")

    def set_inputs(k):
        qn.copy_(to_torch(sets[k][0]))
        qp.copy_(to_torch(sets[k][1]))

    _replays_match(lambda: mla.mla_prefill(d, qn, qp, wk, wv, c, out=out, workspace=ws),
                   lambda: mla.mla_prefill(d, qn, qp, wk, wv, c), set_inputs)


def test_output_projection_and_folded_decode_replay_in_a_graph():
    _log("graph: mla_output_project, mla_decode_folded")
    from synth import draw_output_weights
    case = make_decode_case(65, 4, Dims(128, **V3), [1, 129, 1000, 3000], shuffle=True)
    c = device_cache(case.cache)
    d = case.dims
    d_model = 1024
    qn, qp = to_torch(case.q_nope).unsqueeze(1), to_torch(case.q_pe).unsqueeze(1)
    wk, wv = to_torch(case.w_uk), to_torch(case.w_uv)
    w_o = to_torch(draw_output_weights(66, d_model, 128, 128))
    w_ouv = mla.mla_fold_output_weights(d, wv, w_o)
    ws_f = torch.empty(mla.mla_decode_folded_workspace_size(d, case.batch, 1, c.max_context, d_model),
                       dtype=torch.uint8, device="cuda")
    y = torch.empty((case.batch, 1, d_model), dtype=torch.bfloat16, device="cuda")
    sets = _query_sets(case, 3)

    def set_inputs(k):
        qn.copy_(to_torch(sets[k][0]).unsqueeze(1))
        qp.copy_(to_torch(sets[k][1]).unsqueeze(1))

    _replays_match(lambda: mla.mla_decode_folded(d, qn, qp, wk, w_ouv, c, out=y, workspace=ws_f),
                   lambda: mla.mla_decode_folded(d, qn, qp, wk, w_ouv, c), set_inputs)

    x = torch.empty((case.batch, 128, 128), dtype=torch.bfloat16, device="cuda")
    ws_o = torch.empty(max(mla.mla_output_workspace_size(d, case.batch, d_model), 1), dtype=torch.uint8,
                       device="cuda")
    yo = torch.empty((case.batch, d_model), dtype=torch.bfloat16, device="cuda")
    rng = np.random.default_rng(9)
    from synth import f32_to_bf16_bits
    xs = [f32_to_bf16_bits(rng.standard_normal((case.batch, 128, 128)).astype(np.float32) * 0.05) for _ in range(3)]

    def set_x(k):
        x.copy_(to_torch(xs[k]))

    _replays_match(lambda: mla.mla_output_project(d, x, w_o, out=yo, workspace=ws_o),
                   lambda: mla.mla_output_project(d, x, w_o), set_x)


def test_fp8_projection_replays_in_a_graph():
    _log("graph: mla_rope_latent_project_fp8")
    from synth import f32_to_bf16_bits, make_project_case
    d = Dims(128, **V3)
    case = make_project_case(67, batch=2, seq_len=130, d_model=512, dims=d, shuffle=True)
    T, nb = case.n_tokens, case.num_blocks
    pb = mla.mla_fp8_page_bytes(d, 64)
    h = to_torch(case.h)
    wd, wr = to_torch(case.w_dkv), to_torch(case.w_kr)
    pos, slots = to_torch(case.positions), to_torch(case.slots)
    pages = torch.zeros((nb, pb), dtype=torch.uint8, device="cuda")
    ws = torch.empty(max(mla.mla_project_fp8_workspace_size(d, T), 1), dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(11)
    hs = [case.h] + [f32_to_bf16_bits(rng.standard_normal(case.h.shape).astype(np.float32)) for _ in range(2)]

    def set_inputs(k):
        h.copy_(to_torch(hs[k]))

    def capture():
        mla.mla_rope_latent_project_fp8(d, h, wd, wr, pos, slots, pages, 64, workspace=ws)
        return pages

    def eager():
        fresh = torch.zeros_like(pages)
        mla.mla_rope_latent_project_fp8(d, h, wd, wr, pos, slots, fresh, 64)
        torch.cuda.synchronize()
        return fresh

    _replays_match(capture, eager, set_inputs)
