"""Pins of the CPU oracle to facts outside itself (no GPU needed).

Each test checks the oracle against something the pages or mathematics fix:
printed worked numbers (tests/golden), closed forms, invariants, special cases
that reduce to a textbook result, a library routine (torch's scaled dot-product
attention on the CPU) and pure-Python brute force on tiny shapes. The last
group plants typical mistakes into the oracle and checks that the pins catch
every one of them.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.mla as om
from synth import Dims, make_decode_case, make_project_case, paged_layout

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].split()
            if line:
                vals[line[0]] = (float(line[1]), float(line[2]))
    return vals


def _close_to_page(value, key, g):
    ref, tol = g[key]
    assert abs(value - ref) <= tol * abs(ref) + 1e-12, (key, value, ref)


# ------------------------------------------------------------ golden values --

def test_golden_cache_sizes_nlpx():
    g = _golden("cache_arithmetic.txt")
    mha = oracle.mha_cache_values_per_token(32, 128)
    mla = oracle.mla_cache_values_per_token(512, 64)
    _close_to_page(mha, "nlpx_mha_values_per_token", g)
    _close_to_page(mla, "nlpx_mla_values_per_token", g)
    _close_to_page(mha / mla, "nlpx_ratio", g)


def test_golden_cache_bytes_sheraton():
    g = _golden("cache_arithmetic.txt")
    vals = oracle.mha_cache_values_per_token(40, 128)
    _close_to_page(vals, "shq_values_per_token", g)
    b = vals * 2  # fp16
    _close_to_page(b / 1024, "shq_bytes_per_token_kib", g)
    _close_to_page(b * 10_000 / 1e6, "shq_bytes_10k_tokens_mb", g)
    # the page multiplies its rounded 200 MB by 32
    _close_to_page(b * 10_000 * 32 / 1e9, "shq_bytes_batch32_gb", g)


def test_golden_score_count_intelliparadigm():
    g = _golden("cache_arithmetic.txt")
    _close_to_page(oracle.attention_score_macs(2048, 2048, 1), "ip_scores_2048", g)
    _close_to_page(oracle.attention_score_macs(2048, 2048, 128), "ip_macs_2048_d128", g)


def test_cache_sizes_of_the_measured_shapes():
    # DeepSeek-V3 shape: 1152 bytes per token in bf16; MHA K/V at 128 heads of
    # (128 + 64) key and 128 value dims would be 40960 values.
    assert oracle.mla_cache_values_per_token(512, 64) * 2 == 1152
    assert 128 * (192 + 128) / oracle.mla_cache_values_per_token(512, 64) == pytest.approx(71.11, abs=0.01)
    assert oracle.mla_cache_values_per_token(32, 8) == 40


# ------------------------------------------------------------------- RoPE ---

def test_rope_identity_at_position_zero():
    x = np.random.default_rng(0).standard_normal((5, 8))
    assert np.array_equal(oracle.rope(x, 0), x)


def test_rope_two_dims_is_a_plane_rotation():
    # d_rope = 2: the single pair has frequency base^0 = 1, so position p turns
    # the plane by p radians, counter-clockwise.
    for p in (0.0, 1.0, 2.5, 37.0, 4095.0):
        assert np.allclose(oracle.rope(np.array([1.0, 0.0]), p), [math.cos(p), math.sin(p)], atol=1e-12)
        assert np.allclose(oracle.rope(np.array([0.0, 1.0]), p), [-math.sin(p), math.cos(p)], atol=1e-12)


def test_rope_preserves_norm_and_composes():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 64))
    a, b = 123, 4567
    ra = oracle.rope(x, a)
    assert np.allclose(np.linalg.norm(ra, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    assert np.allclose(oracle.rope(ra, b), oracle.rope(x, a + b), atol=1e-9)


def test_rope_scores_depend_on_relative_position_only():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for m, n in ((10, 3), (8191, 0), (5000, 4999)):
        lhs = oracle.rope(q, m) @ oracle.rope(k, n)
        rhs = oracle.rope(q, m - n) @ k
        assert lhs == pytest.approx(rhs, rel=1e-9, abs=1e-9)


def test_rope_touches_only_the_rotary_slice_of_cache_rows():
    case = make_project_case(3, 1, 16, 24, Dims(4, 12, 6, 5, 7, dtype="f32"), draw_query=False)
    r0 = oracle.latent_rows(case.h, case.w_dkv, case.w_kr, case.positions)
    r1 = oracle.latent_rows(case.h, case.w_dkv, case.w_kr, case.positions + 1000)
    assert np.array_equal(r0[:, :12], r1[:, :12])          # c_KV bit-identical
    assert np.all(np.abs(r0[:, 12:] - r1[:, 12:]).max(axis=1) > 1e-6)  # k_pe moved
    assert np.allclose(np.linalg.norm(r0[:, 12:], axis=1), np.linalg.norm(r1[:, 12:], axis=1))


# --------------------------------------------------------- brute force -----

def _w(a):
    """float64 copy of an input array, widened with torch's own bfloat16 type
    (uint16 bit patterns) rather than the oracle's widening, so that the pins
    do not share that conversion with the oracle."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    return a.astype(np.float64)


def _bf_rope(x, pos, base):
    out = []
    d = len(x)
    for i in range(d // 2):
        ang = pos * base ** (-2.0 * i / d)
        c, s = math.cos(ang), math.sin(ang)
        out += [x[2 * i] * c - x[2 * i + 1] * s, x[2 * i] * s + x[2 * i + 1] * c]
    return out


def _bf_attend_one(dims, qn, qp_rot, rows, wuk, wuv, h):
    """One head, one query, by loops: explicit K and V, then softmax."""
    dc, dn, dv = dims.d_c, dims.d_nope, dims.d_v
    scores = []
    for r in rows:
        c, kpe = r[:dc], r[dc:]
        k = [sum(wuk[h * dn + j][m] * c[m] for m in range(dc)) for j in range(dn)] + list(kpe)
        q = list(qn) + list(qp_rot)
        scores.append(dims.scale * sum(a * b for a, b in zip(q, k)))
    mx = max(scores)
    e = [math.exp(s - mx) for s in scores]
    z = sum(e)
    out = []
    for j in range(dv):
        acc = 0.0
        for t, r in enumerate(rows):
            v = sum(wuv[h * dv + j][m] * r[m] for m in range(dc))
            acc += e[t] / z * v
        out.append(acc)
    return out


def bruteforce_decode(case):
    d = case.dims
    qn, qp = _w(case.q_nope).tolist(), _w(case.q_pe).tolist()
    wuk, wuv = _w(case.w_uk).tolist(), _w(case.w_uv).tolist()
    out = np.zeros((case.batch, d.n_heads, d.d_v))
    pool, table = _w(case.cache.pool), case.cache.block_table
    for b in range(case.batch):
        L = int(case.cache.context_lens[b])
        rows = [pool[table[b][t // 64], t % 64].tolist() for t in range(L)]
        for h in range(d.n_heads):
            qr = _bf_rope(qp[b][h], L - 1, d.rope_base)
            out[b, h] = _bf_attend_one(d, qn[b][h], qr, rows, wuk, wuv, h)
    return out


def bruteforce_prefill(dims, qn, qp, wuk, wuv, rows):
    qn, qp, wuk, wuv, rows = (_w(a).tolist() for a in (qn, qp, wuk, wuv, rows))
    B, S = len(qn), len(qn[0])
    out = np.zeros((B, S, dims.n_heads, dims.d_v))
    for b in range(B):
        for s in range(S):
            for h in range(dims.n_heads):
                qr = _bf_rope(qp[b][s][h], s, dims.rope_base)
                out[b, s, h] = _bf_attend_one(dims, qn[b][s][h], qr, rows[b][:s + 1], wuk, wuv, h)
    return out


TINY = [
    (Dims(3, 8, 4, 5, 6, dtype="f32"), [1, 2, 7]),
    (Dims(2, 16, 8, 4, 4, dtype="f32"), [65, 3]),
    (Dims(1, 8, 2, 3, 5, dtype="bf16"), [64, 129]),
]


def _oracle_decode(case):
    c = case.cache
    return oracle.decode(case.dims, case.q_nope, case.q_pe, case.w_uk, case.w_uv,
                         c.pool, c.block_table, c.context_lens)


@pytest.mark.parametrize("dims,lens", TINY)
def test_decode_matches_bruteforce(dims, lens):
    case = make_decode_case(11, len(lens), dims, lens, shuffle=True, w_std=0.5)
    assert np.allclose(_oracle_decode(case), bruteforce_decode(case), rtol=1e-11, atol=1e-12)


def test_prefill_matches_bruteforce():
    dims = Dims(2, 8, 4, 3, 5, dtype="f32")
    case = make_project_case(12, 2, 9, 6, dims, draw_query=False)
    rows = oracle.latent_rows(case.h, case.w_dkv, case.w_kr, case.positions).reshape(2, 9, -1)
    rng = np.random.default_rng(5)
    qn, qp = rng.standard_normal((2, 9, 2, 3)), rng.standard_normal((2, 9, 2, 4))
    got = oracle.prefill(dims, qn, qp, case.w_uk, case.w_uv, rows)
    assert np.allclose(got, bruteforce_prefill(dims, qn, qp, case.w_uk, case.w_uv, rows), rtol=1e-11, atol=1e-12)
    sub = oracle.prefill(dims, qn, qp, case.w_uk, case.w_uv, rows, queries=[(1, 0), (0, 8), (1, 4)])
    assert np.allclose(sub, got[[1, 0, 1], [0, 8, 4]], rtol=1e-12, atol=1e-13)


def bruteforce_latent_rows(h, w_dkv, w_kr, positions, base):
    """[V2] §2.1: c_t[i] = sum_j W_DKV[i, j] h_t[j]; [V2] §2.3: the rotary key
    is W_KR h_t rotated at the token's own position. Plain loops."""
    H, Wd, Wr = _w(h).tolist(), _w(w_dkv).tolist(), _w(w_kr).tolist()
    rows = []
    for t, ht in enumerate(H):
        c = [sum(Wd[i][j] * ht[j] for j in range(len(ht))) for i in range(len(Wd))]
        k = [sum(Wr[i][j] * ht[j] for j in range(len(ht))) for i in range(len(Wr))]
        rows.append(c + _bf_rope(k, int(positions[t]), base))
    return np.array(rows)


def bruteforce_query_projection(h, w_dq, w_uq, w_qr, n_heads, d_nope, d_rope):
    """[V2] §4.3: c_Q = W_DQ h; head hh's q_nope is rows hh*d_nope .. of
    W_UQ times c_Q and its q_pe rows hh*d_rope .. of W_QR times c_Q. Loops."""
    H, Wd, Wu, Wr = _w(h).tolist(), _w(w_dq).tolist(), _w(w_uq).tolist(), _w(w_qr).tolist()
    T = len(H)
    qn = np.zeros((T, n_heads, d_nope))
    qp = np.zeros((T, n_heads, d_rope))
    for t, ht in enumerate(H):
        cq = [sum(Wd[i][j] * ht[j] for j in range(len(ht))) for i in range(len(Wd))]
        for hh in range(n_heads):
            for j in range(d_nope):
                qn[t, hh, j] = sum(Wu[hh * d_nope + j][i] * cq[i] for i in range(len(cq)))
            for j in range(d_rope):
                qp[t, hh, j] = sum(Wr[hh * d_rope + j][i] * cq[i] for i in range(len(cq)))
    return qn, qp


# projection cases: positions far from 0 and not in token order, so that a
# rotation at the wrong position or no rotation shows; d_nope == d_rope and
# d_q == d_model so that the planted mistakes below keep valid shapes
PROJ_CASES = [
    (Dims(3, 8, 4, 4, 5, dtype="f32"), 7, 12, 12),
    (Dims(2, 16, 8, 8, 4, dtype="bf16"), 5, 16, 16),
]


def _projection_case(dims, n_tok, d_model, d_q, seed=31):
    case = make_project_case(seed, 1, n_tok, d_model, dims, d_q=d_q)
    pos = np.random.default_rng(seed).integers(0, 5000, size=n_tok).astype(np.int32)
    return case, pos


@pytest.mark.parametrize("dims,n_tok,d_model,d_q", PROJ_CASES)
def test_latent_rows_match_bruteforce(dims, n_tok, d_model, d_q):
    case, pos = _projection_case(dims, n_tok, d_model, d_q)
    got = oracle.latent_rows(case.h, case.w_dkv, case.w_kr, pos, dims.rope_base)
    assert np.allclose(got, bruteforce_latent_rows(case.h, case.w_dkv, case.w_kr, pos, dims.rope_base),
                       rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("dims,n_tok,d_model,d_q", PROJ_CASES)
def test_query_projection_matches_bruteforce(dims, n_tok, d_model, d_q):
    case, _ = _projection_case(dims, n_tok, d_model, d_q)
    qn, qp = oracle.query_projection(case.h, case.w_dq, case.w_uq, case.w_qr, dims.n_heads, dims.d_nope,
                                     dims.d_rope)
    bn, bp = bruteforce_query_projection(case.h, case.w_dq, case.w_uq, case.w_qr, dims.n_heads, dims.d_nope,
                                         dims.d_rope)
    assert qn.shape == bn.shape and qp.shape == bp.shape
    assert np.allclose(qn, bn, rtol=1e-11, atol=1e-12) and np.allclose(qp, bp, rtol=1e-11, atol=1e-12)


def test_projection_store_rounds_to_bf16():
    dims, n_tok, d_model, d_q = PROJ_CASES[1]
    case, pos = _projection_case(dims, n_tok, d_model, d_q)
    exact = bruteforce_latent_rows(case.h, case.w_dkv, case.w_kr, pos, dims.rope_base)
    got = oracle.latent_rows(case.h, case.w_dkv, case.w_kr, pos, dims.rope_base, store="bf16")
    # every stored value is a bf16 number within half a bf16 ulp of the exact row
    bits = torch.from_numpy(got.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bits, got)
    assert np.all(np.abs(got - exact) <= np.abs(exact) * 2.0 ** -8 + 1e-30)


def _projection_pins_pass():
    ok = True
    for dims, n_tok, d_model, d_q in PROJ_CASES:
        case, pos = _projection_case(dims, n_tok, d_model, d_q)
        rows = oracle.latent_rows(case.h, case.w_dkv, case.w_kr, pos, dims.rope_base)
        ok &= np.allclose(rows, bruteforce_latent_rows(case.h, case.w_dkv, case.w_kr, pos, dims.rope_base),
                          rtol=1e-9, atol=1e-11)
        qn, qp = oracle.query_projection(case.h, case.w_dq, case.w_uq, case.w_qr, dims.n_heads, dims.d_nope,
                                         dims.d_rope)
        bn, bp = bruteforce_query_projection(case.h, case.w_dq, case.w_uq, case.w_qr, dims.n_heads,
                                             dims.d_nope, dims.d_rope)
        ok &= np.allclose(qn, bn, rtol=1e-9, atol=1e-11) and np.allclose(qp, bp, rtol=1e-9, atol=1e-11)
    return bool(ok)


_ORIG_QP = om.query_projection
_ORIG_ROPE = om.rope


def _plant_q_heads_transposed(h, w_dq, w_uq, w_qr, n_heads, d_nope, d_rope, store=None):
    # per-head split read as [d, n_heads] instead of [n_heads, d]
    qn, qp = _ORIG_QP(h, w_dq, w_uq, w_qr, n_heads, d_nope, d_rope, store)
    T = qn.shape[0]
    return (qn.reshape(T, -1).reshape(T, d_nope, n_heads).transpose(0, 2, 1),
            qp.reshape(T, -1).reshape(T, d_rope, n_heads).transpose(0, 2, 1))


def _plant_uq_qr_swapped(h, w_dq, w_uq, w_qr, n_heads, d_nope, d_rope, store=None):
    # the cases use d_nope == d_rope, so swapped weights still have the right shapes
    return _ORIG_QP(h, w_dq, w_qr, w_uq, n_heads, d_nope, d_rope, store)


def _plant_cq_skipped(h, w_dq, w_uq, w_qr, n_heads, d_nope, d_rope, store=None):
    # up-projections applied to h directly (d_q == d_model in the cases)
    eye = np.eye(np.asarray(w_dq).shape[0])
    return _ORIG_QP(h, eye, w_uq, w_qr, n_heads, d_nope, d_rope, store)


PROJECTION_PLANTS = {
    "query head axis transposed": ("query_projection", _plant_q_heads_transposed),
    "W_UQ and W_QR swapped": ("query_projection", _plant_uq_qr_swapped),
    "c_Q skipped": ("query_projection", _plant_cq_skipped),
    "key RoPE at position + 1": ("rope", lambda x, pos, base=10000.0: _ORIG_ROPE(x, np.asarray(pos) + 1, base)),
    "key RoPE skipped": ("rope", lambda x, pos, base=10000.0: np.asarray(x, dtype=np.float64)),
}


def test_projection_pins_pass_on_the_true_oracle():
    assert _projection_pins_pass()


@pytest.mark.parametrize("name", sorted(PROJECTION_PLANTS))
def test_projection_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = PROJECTION_PLANTS[name]
    monkeypatch.setattr(om, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    assert not _projection_pins_pass(), name


# ------------------------------------------------------- library routine ---

def _sdpa_decode(case):
    """torch's CPU scaled_dot_product_attention on K/V built here with torch."""
    d = case.dims
    H, dn, dv, dc = d.n_heads, d.d_nope, d.d_v, d.d_c
    wuk = torch.from_numpy(_w(case.w_uk)).view(H, dn, dc)
    wuv = torch.from_numpy(_w(case.w_uv)).view(H, dv, dc)
    pool = torch.from_numpy(_w(case.cache.pool))
    outs = []
    for b in range(case.batch):
        L = int(case.cache.context_lens[b])
        idx = torch.arange(L)
        rows = pool[torch.from_numpy(case.cache.block_table[b])[idx // 64].long(), idx % 64]
        c, kpe = rows[:, :dc], rows[:, dc:]
        k = torch.cat([torch.einsum("hnc,tc->htn", wuk, c), kpe.expand(H, L, d.d_rope)], dim=-1)
        v = torch.einsum("hvc,tc->htv", wuv, c)
        ang = (L - 1) * d.rope_base ** (-torch.arange(0, d.d_rope, 2, dtype=torch.float64) / d.d_rope)
        qp = torch.from_numpy(_w(case.q_pe[b]))
        rot = torch.view_as_real(torch.view_as_complex(qp.view(H, -1, 2).contiguous())
                                 * torch.polar(torch.ones_like(ang), ang)).view(H, -1)
        q = torch.cat([torch.from_numpy(_w(case.q_nope[b])), rot], dim=-1)[:, None, :]
        outs.append(torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=d.scale)[:, 0])
    return torch.stack(outs).numpy()


@pytest.mark.parametrize("shuffle", [False, True])
def test_decode_matches_torch_sdpa(shuffle):
    dims = Dims(8, 64, 16, 32, 24, dtype="bf16")
    case = make_decode_case(13, 3, dims, [1, 100, 300], shuffle=shuffle)
    assert np.allclose(_oracle_decode(case), _sdpa_decode(case), rtol=1e-10, atol=1e-12)


def test_prefill_matches_torch_sdpa_causal():
    dims = Dims(4, 32, 8, 16, 16, dtype="f32")
    case = make_project_case(14, 2, 40, 48, dims, draw_query=False)
    rows = oracle.latent_rows(case.h, case.w_dkv, case.w_kr, case.positions).reshape(2, 40, -1)
    rng = np.random.default_rng(6)
    qn, qp = rng.standard_normal((2, 40, 4, 16)), rng.standard_normal((2, 40, 4, 8))
    got = oracle.prefill(dims, qn, qp, case.w_uk, case.w_uv, rows)
    H = 4
    wuk = torch.from_numpy(_w(case.w_uk)).view(H, 16, 32)
    wuv = torch.from_numpy(_w(case.w_uv)).view(H, 16, 32)
    for b in range(2):
        r = torch.from_numpy(rows[b])
        k = torch.cat([torch.einsum("hnc,tc->htn", wuk, r[:, :32]), r[:, 32:].expand(H, 40, 8)], -1)
        v = torch.einsum("hvc,tc->htv", wuv, r[:, :32])
        pos = torch.arange(40, dtype=torch.float64)[:, None] * 10000.0 ** (-torch.arange(0, 8, 2, dtype=torch.float64) / 8)
        qpc = torch.view_as_complex(torch.from_numpy(qp[b]).view(40, H, 4, 2).contiguous())
        rot = torch.view_as_real(qpc * torch.polar(torch.ones_like(pos), pos)[:, None, :]).view(40, H, 8)
        q = torch.cat([torch.from_numpy(qn[b]), rot], -1).transpose(0, 1)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=dims.scale)
        assert np.allclose(got[b], ref.transpose(0, 1).numpy(), rtol=1e-10, atol=1e-12)


# -------------------------------------------------- closed-form special cases

def _wuv_c(case, h, c):
    d = case.dims
    return _w(case.w_uv)[h * d.d_v:(h + 1) * d.d_v] @ c


def test_single_token_context_returns_its_value():
    case = make_decode_case(15, 2, Dims(4, 16, 4, 8, 8, dtype="f32"), [1, 1])
    out = _oracle_decode(case)
    for b in range(2):
        c0 = _w(case.cache.pool[case.cache.block_table[b, 0], 0])[:16]
        for h in range(4):
            assert np.allclose(out[b, h], _wuv_c(case, h, c0), rtol=1e-13, atol=1e-14)


def test_identical_rows_return_their_value():
    case = make_decode_case(16, 1, Dims(4, 16, 4, 8, 8, dtype="f32"), [77])
    pool = case.cache.pool
    pool[:] = pool[0, 0]
    out = _oracle_decode(case)
    for h in range(4):
        assert np.allclose(out[0, h], _wuv_c(case, h, _w(pool[0, 0, :16])), rtol=1e-12, atol=1e-13)


def test_zero_query_gives_uniform_average():
    case = make_decode_case(17, 2, Dims(4, 16, 4, 8, 8, dtype="f32"), [70, 130], shuffle=True)
    case.q_nope[:] = 0
    case.q_pe[:] = 0
    out = _oracle_decode(case)
    for b in range(2):
        rows = oracle.gather_rows(case.cache.pool, case.cache.block_table, case.cache.context_lens, b)
        mean_c = rows[:, :16].mean(axis=0)
        for h in range(4):
            assert np.allclose(out[b, h], _wuv_c(case, h, mean_c), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- invariants

def test_token_order_and_page_placement_do_not_matter():
    dims = Dims(4, 16, 4, 8, 8, dtype="f32")
    a = make_decode_case(18, 2, dims, [100, 64], shuffle=False)
    ref = _oracle_decode(a)
    # same logical rows, pages placed at shuffled physical blocks
    table, nb = paged_layout(a.cache.context_lens, np.random.default_rng(3))
    pool = np.zeros_like(a.cache.pool)
    for b in range(2):
        for p in range((int(a.cache.context_lens[b]) + 63) // 64):
            pool[table[b, p]] = a.cache.pool[a.cache.block_table[b, p]]
    moved = oracle.decode(dims, a.q_nope, a.q_pe, a.w_uk, a.w_uv, pool, table, a.cache.context_lens)
    assert np.allclose(moved, ref, rtol=1e-13, atol=1e-14)
    # tokens permuted within the context (k_pe already rotated, so no position moves)
    perm_pool = a.cache.pool.copy()
    rows = oracle.gather_rows(a.cache.pool, a.cache.block_table, a.cache.context_lens, 0)
    rows = rows[np.random.default_rng(4).permutation(100)]
    for t in range(100):
        perm_pool[a.cache.block_table[0, t // 64], t % 64] = rows[t]
    perm = oracle.decode(dims, a.q_nope, a.q_pe, a.w_uk, a.w_uv, perm_pool, a.cache.block_table, a.cache.context_lens)
    assert np.allclose(perm, ref, rtol=1e-12, atol=1e-13)


def test_shifting_every_position_leaves_decode_unchanged():
    dims = Dims(4, 16, 8, 8, 8, dtype="f32")
    case = make_project_case(19, 1, 50, 32, dims, paged=False)
    lens = np.array([50], dtype=np.int32)
    outs = []
    for delta in (0, 777, 30000):
        rows = oracle.latent_rows(case.h, case.w_dkv, case.w_kr, case.positions + delta)
        qpe = oracle.rope(_w(case.q_pe), delta)        # query moved by the same delta
        outs.append(oracle.decode(dims, case.q_nope, qpe, case.w_uk, case.w_uv, rows[None], None, lens))
    assert np.allclose(outs[1], outs[0], rtol=1e-9, atol=1e-11)
    assert np.allclose(outs[2], outs[0], rtol=1e-9, atol=1e-11)


def test_absorbed_form_equals_explicit_form():
    rng = np.random.default_rng(20)
    for H in (1, 3, 4):
        for dc, dr in ((8, 2), (32, 8)):
            lens = rng.integers(1, 130, size=2)
            case = make_decode_case(int(rng.integers(1 << 30)), 2, Dims(H, dc, dr, 5, 7, dtype="f32"), lens,
                                    shuffle=True, w_std=0.7)
            c = case.cache
            a = oracle.absorbed_decode(case.dims, case.q_nope, case.q_pe, case.w_uk, case.w_uv,
                                       c.pool, c.block_table, c.context_lens)
            e = _oracle_decode(case)
            assert np.linalg.norm(a - e) <= 1e-12 * np.linalg.norm(e)


def test_prefill_row_equals_decode_over_its_prefix():
    dims = Dims(4, 16, 8, 8, 8, dtype="f32")
    case = make_project_case(21, 1, 70, 32, dims, draw_query=False)
    rows = oracle.latent_rows(case.h, case.w_dkv, case.w_kr, case.positions)
    rng = np.random.default_rng(7)
    qn, qp = rng.standard_normal((1, 70, 4, 8)), rng.standard_normal((1, 70, 4, 8))
    pre = oracle.prefill(dims, qn, qp, case.w_uk, case.w_uv, rows[None])
    for s in (0, 1, 63, 64, 69):
        dec = oracle.decode(dims, qn[:, s], qp[:, s], case.w_uk, case.w_uv, rows[None], None,
                            np.array([s + 1], dtype=np.int32))
        assert np.allclose(pre[0, s], dec[0], rtol=1e-12, atol=1e-13)


def _split_combine_model(scores, values, bounds):
    """Split-context softmax: per split (m, l, o) partials, then an LSE merge."""
    parts = []
    for lo, hi in bounds:
        s = scores[lo:hi]
        m = s.max()
        p = np.exp(s - m)
        parts.append((m, p.sum(), p @ values[lo:hi]))
    m = max(p[0] for p in parts)
    l = sum(p[1] * math.exp(p[0] - m) for p in parts)
    o = sum(p[2] * math.exp(p[0] - m) for p in parts)
    return o / l


def test_split_context_combine_equals_one_pass_softmax():
    rng = np.random.default_rng(8)
    for L in (1, 2, 63, 64, 65, 1000):
        s = rng.standard_normal(L) * 3
        v = rng.standard_normal((L, 5))
        ref = oracle.attend(np.ones((1, 1)), s[:, None], v, 1.0)[0]
        for n in (1, 2, 3, 7):
            cuts = sorted(set([0, L] + list(rng.integers(0, L + 1, size=n))))
            bounds = [(a, b) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
            assert np.allclose(_split_combine_model(s, v, bounds), ref, rtol=1e-12, atol=1e-14)


def test_round_to_bf16_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.0e38])
    r = oracle.round_to(x, "bf16")
    assert r[0] == 1.0 and r[1] == 1.0            # tie rounds to even (down)
    assert r[2] == 1.0 + 2 ** -6                  # tie rounds to even (up)
    assert r[3] == 1.0 and r[4] == -2.5
    assert r[5] == pytest.approx(3.0e38, rel=2 ** -8)


# ------------------------------------------------------ output projection --

def bruteforce_output_projection(attn, w_o):
    """out[n][j] = sum over heads h and value dims v of W_O[j][h*d_v + v] *
    attn[n][h][v], by loops."""
    A, W = _w(attn).tolist(), _w(w_o).tolist()
    out = np.zeros((len(A), len(W)))
    for n, an in enumerate(A):
        dv = len(an[0])
        for j, wj in enumerate(W):
            out[n, j] = sum(wj[h * dv + v] * an[h][v] for h in range(len(an)) for v in range(dv))
    return out


def _wo_case(seed, H, dv, d_model, dtype="f32"):
    from synth import draw_output_weights
    dims = Dims(H, 16, 4, 8, dv, dtype=dtype)
    case = make_decode_case(seed, 3, dims, [1, 70, 130], shuffle=True, w_std=0.6)
    return case, draw_output_weights(seed + 1, d_model, H, dv, dtype)


def _output_pins_pass():
    ok = True
    for seed, H, dv, d_model, dtype in ((40, 3, 5, 7, "f32"), (41, 2, 4, 8, "bf16"), (42, 4, 6, 24, "f32")):
        case, w_o = _wo_case(seed, H, dv, d_model, dtype)
        c = case.cache
        attn = _oracle_decode(case)
        plain = oracle.output_projection(attn, w_o)
        ok &= np.allclose(plain, bruteforce_output_projection(attn, w_o), rtol=1e-11, atol=1e-12)
        ok &= np.allclose(oracle.decode_output(case.dims, case.q_nope, case.q_pe, case.w_uk, case.w_uv, w_o, c.pool,
                                               c.block_table, c.context_lens), plain, rtol=1e-12, atol=1e-13)
        w_ouv = oracle.fold_output_weights(case.w_uv, w_o, H, dv)
        folded = oracle.folded_decode_output(case.dims, case.q_nope, case.q_pe, case.w_uk, w_ouv, c.pool,
                                             c.block_table, c.context_lens)
        ok &= np.linalg.norm(folded - plain) <= 1e-12 * np.linalg.norm(plain)
    return bool(ok)


def test_output_projection_matches_bruteforce_and_the_fold():
    """[V2] §2.2: W_UV absorbed into W_O gives the same layer output as W_O
    applied to the per-head outputs (an exact rewrite, checked in fp64)."""
    assert _output_pins_pass()


def test_output_projection_of_one_head_with_identity_weights_is_its_output():
    case, _ = _wo_case(43, 1, 8, 8)
    attn = _oracle_decode(case)
    assert np.array_equal(oracle.output_projection(attn, np.eye(8)), attn[:, 0])


def test_fold_of_identity_output_weights_is_w_uv():
    """With W_O the identity (d_model = n_h d_v) the folded weight of head h is
    W_UV,h laid out as column block h."""
    H, dv, dc = 3, 4, 16
    case, _ = _wo_case(44, H, dv, H * dv)
    f = oracle.fold_output_weights(case.w_uv, np.eye(H * dv), H, dv)
    wuv = _w(case.w_uv)
    for h in range(H):
        assert np.array_equal(f[h * dv:(h + 1) * dv, h * dc:(h + 1) * dc], wuv[h * dv:(h + 1) * dv])
        for g in range(H):
            if g != h:
                assert not np.any(f[g * dv:(g + 1) * dv, h * dc:(h + 1) * dc])


_ORIG_OP = om.output_projection


def _plant_heads_interleaved(attn, w_o):
    # concatenation in [d_v, n_h] order instead of [n_h, d_v]
    a = om.widen(attn)
    return _ORIG_OP(np.swapaxes(a, -1, -2).reshape(a.shape), w_o)


def _plant_head_blocks_reversed(attn, w_o):
    return _ORIG_OP(om.widen(attn)[..., ::-1, :], w_o)


OUTPUT_PLANTS = {
    "heads interleaved in the concatenation": _plant_heads_interleaved,
    "head blocks of W_O reversed": _plant_head_blocks_reversed,
    "one head dropped": lambda attn, w_o: _ORIG_OP(np.concatenate([om.widen(attn)[..., :-1, :],
                                                                   0 * om.widen(attn)[..., -1:, :]], axis=-2), w_o),
}


@pytest.mark.parametrize("name", sorted(OUTPUT_PLANTS))
def test_output_pins_catch_planted_mistake(name, monkeypatch):
    monkeypatch.setattr(om, "output_projection", OUTPUT_PLANTS[name])
    monkeypatch.setattr(oracle, "output_projection", OUTPUT_PLANTS[name])
    assert not _output_pins_pass(), name


# ------------------------------------------------------ planted mistakes ----

def _pins_pass():
    """The brute-force and library pins on one tiny case."""
    dims = Dims(3, 8, 4, 4, 4, dtype="f32")
    case = make_decode_case(22, 2, dims, [5, 70], shuffle=True, w_std=0.6)
    o = _oracle_decode(case)
    ok_bf = np.allclose(o, bruteforce_decode(case), rtol=1e-9, atol=1e-11)
    ok_lib = np.allclose(o, _sdpa_decode(case), rtol=1e-9, atol=1e-11)
    return ok_bf and ok_lib


def _plant_no_kpe(rows, wk, wv, dc):
    k, v = _ORIG_KV(rows, wk, wv, dc)
    k[:, wk.shape[0]:] = 0
    return k, v


def _plant_swap_kv(rows, wk, wv, dc):
    return _ORIG_KV(rows, wv, wk, dc)


_ORIG_KV = om._explicit_kv
_ORIG_ROT = om._rotate_pairs
PLANTS = {
    "dropped k_pe term": ("_explicit_kv", _plant_no_kpe),
    "key and value weights swapped": ("_explicit_kv", _plant_swap_kv),
    "rotation sign flipped": ("_rotate_pairs", lambda x, a: _ORIG_ROT(x, -a)),
    "next head's weights": ("_head_rows", lambda w, h, d: w[((h + 1) % 3) * d:((h + 1) % 3 + 1) * d]),
    # rows of head h read as h, h+H, h+2H, ... ([d, H] instead of [H, d] order)
    "head axis transposed": ("_head_rows", lambda w, h, d: w[h::w.shape[0] // d]),
    "softmax without normalisation": ("_softmax", lambda s: np.exp(s - s.max(axis=-1, keepdims=True))),
}


def test_pins_pass_on_the_true_oracle():
    assert _pins_pass()


@pytest.mark.parametrize("name", sorted(PLANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = PLANTS[name]
    monkeypatch.setattr(om, attr, fn)
    assert not _pins_pass(), name


def test_query_position_off_by_one_is_caught(monkeypatch):
    orig = om.rope
    monkeypatch.setattr(om, "rope", lambda x, pos, base=10000.0: orig(x, np.asarray(pos) + 1, base))
    assert not _pins_pass()
