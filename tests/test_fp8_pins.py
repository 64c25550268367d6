"""Pins of the FP8 cache oracle (oracle/fp8.py) to things other than itself:
torch's float8_e4m3fn conversion (a library routine), brute force over all
256 codes, the format's definition on hand-worked values, and the bounds and
invariants the quantiser must satisfy. Planted mistakes must fail them."""
import numpy as np
import pytest
import torch

from oracle import fp8


def _torch_codes(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _torch_values(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _test_values():
    rng = np.random.default_rng(7)
    finite = _torch_values(np.arange(256, dtype=np.uint8))
    finite = np.unique(finite[np.isfinite(finite)])
    mids = (finite[:-1] + finite[1:]) / 2          # every tie
    x = np.concatenate([finite, mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf),
                        rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 0.01,
                        rng.standard_normal(5000) * 1e-3, [0.0, -0.0, 448.0, -448.0, 2.0 ** -10, -(2.0 ** -10)]])
    x = x.astype(np.float32).astype(np.float64)      # the same inputs for both sides
    return x[np.abs(x) <= 448]


def test_e4m3_rounding_matches_torch_float8():
    x = _test_values()
    assert np.array_equal(fp8.e4m3_encode(fp8.e4m3_round(x)), _torch_codes(x))


def test_e4m3_decode_matches_torch_on_all_codes():
    c = np.arange(256, dtype=np.uint8)
    a, b = fp8.e4m3_decode(c), _torch_values(c)
    assert np.array_equal(np.isnan(a), np.isnan(b))
    ok = ~np.isnan(a)
    assert np.array_equal(a[ok], b[ok]) and np.array_equal(np.signbit(a[ok]), np.signbit(b[ok]))


def test_e4m3_rounding_is_nearest_even_by_brute_force():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = _torch_values(codes)
    rng = np.random.default_rng(8)
    x = np.concatenate([rng.uniform(-448, 448, 3000), rng.standard_normal(2000) * 0.02,
                        (vals[:-1] + vals[1:]) / 2])
    x = x[np.abs(x) <= 448]
    got = fp8.e4m3_round(x)
    for xi, gi in zip(x, got):
        d = np.abs(vals - xi)
        best = vals[d == d.min()]
        if len(np.unique(best)) == 1:
            assert gi == best[0]
        else:   # a tie: the candidate whose code has an even mantissa
            cand = codes[d == d.min()]
            even = [v for v, c in zip(vals[d == d.min()], cand) if (c & 1) == 0]
            assert gi in even


def test_e4m3_encoding_of_hand_worked_values():
    # 1.0 = 2^0: exponent field 7, mantissa 0 -> 0 0111 000
    # -2.5 = -1.25 * 2^1: field 8, mantissa 2 -> 1 1000 010
    # 448 = 1.75 * 2^8: field 15, mantissa 6 -> 0 1111 110
    # 2^-9: smallest subnormal -> 0 0000 001; 2^-6: smallest normal -> 0 0001 000
    # 0.1875 = 1.5 * 2^-3: field 4, mantissa 4 -> 0 0100 100
    vals = np.array([1.0, -2.5, 448.0, 2.0 ** -9, 2.0 ** -6, 0.1875, -0.0])
    want = np.array([0x38, 0xC2, 0x7E, 0x01, 0x08, 0x24, 0x80], dtype=np.uint8)
    assert np.array_equal(fp8.e4m3_encode(vals), want)
    # ties go to the even mantissa: 1.0625 lies between 1.0 and 1.125 -> 1.0;
    # 1.1875 between 1.125 and 1.25 -> 1.25 (mantissa 2)
    assert fp8.e4m3_round(np.array([1.0625, 1.1875])).tolist() == [1.0, 1.25]


def test_e4m3_rejects_values_outside_the_format():
    with pytest.raises(ValueError):
        fp8.e4m3_round(np.array([449.0]))
    with pytest.raises(ValueError):
        fp8.e4m3_encode(np.array([1.1]))


@pytest.mark.parametrize("amax", [0.0, 1e-45, 2.0 ** -140, 1e-3, 0.5, 1.0, 3.5, 447.9, 448.0, 448.5, 896.0,
                                  897.0, 7e4, 3.3e38])
def test_scale_exponent_is_the_smallest_that_fits(amax):
    e = fp8.scale_exponent(amax)
    assert amax <= 448.0 * 2.0 ** e
    assert e == -127 or amax > 448.0 * 2.0 ** (e - 1)


def _bf16_rows(n, width, seed, spread=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, width)).astype(np.float32)
    if spread:   # rows of very different magnitude: the reason for per-block scales
        x *= (2.0 ** rng.integers(-20, 20, size=(n, 1))).astype(np.float32)
    u = x.view(np.uint32)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def test_quantised_rows_are_within_half_a_step():
    rows = _bf16_rows(64, 576, 9)
    codes, kbits, E = fp8.quantize_rows(rows, 512)
    back = fp8.dequantize_rows(codes, kbits, E)
    s = 2.0 ** (E.astype(np.float64) - 127)[:, None]
    c, cb = rows[:, :512], back[:, :512]
    normal = np.abs(c) >= 2.0 ** -6 * s
    assert np.all(np.abs(cb - c)[normal] <= 2.0 ** -4 * np.abs(c)[normal])
    assert np.all(np.abs(cb - c)[~normal] <= 2.0 ** -10 * np.broadcast_to(s, c.shape)[~normal])
    assert np.array_equal(back[:, 512:], rows[:, 512:])          # k_pe kept exactly
    # the minimal scale puts every row's largest magnitude in (224, 448]
    top = np.abs(c).max(axis=1) / s[:, 0]
    assert np.all((top > 224) & (top <= 448))


def test_quantisation_is_idempotent_and_zero_rows_stay_zero():
    """Quantising the dequantised rows again gives the same values (the codes
    may differ: a row whose largest code rounded down to 224 re-encodes one
    binade up with half the scale)."""
    rows = _bf16_rows(32, 576, 10)
    rows[3, :512] = 0.0
    q = fp8.quantize_rows(rows, 512)
    v = fp8.dequantize_rows(*q)
    assert np.array_equal(fp8.dequantize_rows(*fp8.quantize_rows(v, 512)), v)
    assert np.all(q[0][3] == 0) and q[2][3] == 0      # e = -127 for an all-zero block


def test_one_global_scale_would_lose_the_small_rows():
    """Per-token scales keep every row's relative error at fp8's; one scale
    for all rows flushes the small rows to zero ([HDU] §5)."""
    rows = _bf16_rows(16, 576, 11)
    codes, kbits, E = fp8.quantize_rows(rows, 512)
    back = fp8.dequantize_rows(codes, kbits, E)[:, :512]
    err = np.linalg.norm(back - rows[:, :512], axis=1) / np.linalg.norm(rows[:, :512], axis=1)
    assert err.max() < 0.05
    e = fp8.scale_exponent(np.abs(rows[:, :512]).max())
    glob = fp8.e4m3_round(rows[:, :512] * 2.0 ** -e) * 2.0 ** e
    gerr = np.linalg.norm(glob - rows[:, :512], axis=1) / np.linalg.norm(rows[:, :512], axis=1)
    assert gerr.max() > 0.5


def test_page_layout_round_trip():
    rows = _bf16_rows(128, 576, 12, spread=False)
    pages = fp8.quantize_pool(rows.reshape(2, 64, 576), 512)
    assert pages.shape == (2, fp8.page_bytes(64, 512, 64)) and pages.shape[1] == 41024
    # row r of page p starts at 640 r; its k_pe bytes are the bf16 bits; scales after the rows
    codes, kbits, E = fp8.quantize_rows(rows, 512)
    assert np.array_equal(pages[1, 640 * 5:640 * 5 + 512], codes[64 + 5])
    assert np.array_equal(pages[1, 640 * 5 + 512:640 * 6].view("<u2"), kbits[64 + 5])
    assert np.array_equal(pages[0, 40960:41024], E[:64])
    back = fp8.dequantize_pool(pages, 64, 512, 64)
    assert np.array_equal(back.reshape(128, 576), fp8.dequantize_rows(codes, kbits, E))


# ------------------------------------------------ planted mistakes -----------

def _pins_pass():
    try:
        test_e4m3_rounding_matches_torch_float8()
        test_e4m3_encoding_of_hand_worked_values()
        test_quantised_rows_are_within_half_a_step()
        for a in (1e-3, 448.0, 448.5):
            test_scale_exponent_is_the_smallest_that_fits(a)
    except (AssertionError, ValueError):
        return False
    return True


def test_pins_pass_on_the_true_fp8_oracle():
    assert _pins_pass()


def _round_truncating(x):
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    k = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    step = np.where(a >= 2.0 ** -6, 2.0 ** (k - 3), 2.0 ** -9)
    return np.copysign(np.floor(a / step) * step, x)


def _round_half_up(x):
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    k = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    step = np.where(a >= 2.0 ** -6, 2.0 ** (k - 3), 2.0 ** -9)
    return np.copysign(np.floor(a / step + 0.5) * step, x)


def _scale_one_low(amax):
    e = -127
    while amax > 448.0 * 2.0 ** e:
        e += 1
    return e - 1


@pytest.mark.parametrize("name,attr,fake", [
    ("truncation", "e4m3_round", _round_truncating),
    ("ties away from zero", "e4m3_round", _round_half_up),
    ("scale one binade low", "scale_exponent", _scale_one_low),
])
def test_fp8_pins_catch_planted_mistake(name, attr, fake, monkeypatch):
    monkeypatch.setattr(fp8, attr, fake)
    assert not _pins_pass(), name


# ----------------------------------------------- decode with an FP8 query ---
# fp8_query_decode is the oracle's decode with the absorbed query rounded the
# way the FP8 decode feeds it to the FP8 product. Its pins: with a query that
# every rounding keeps exact it is the plain decode; on a realistic case its
# distance from the plain decode is that of an E4M3 rounding of the query;
# dropping a page with a position-free query is the decode of the other pages.

def _exact_query_case(seed, n_pages, L, H=2):
    """lam = softmax scale * log2(e) = 1 and an absorbed query of integers
    |.| <= 8 (exact in bf16 and in E4M3 at the per-head scale), rotary query 0
    (so the score does not depend on the position)."""
    from synth import Dims
    import oracle
    dims = Dims(H, 16, 8, 4, 4, softmax_scale=1.0 / np.log2(np.e))
    rng = np.random.default_rng(seed)
    w_uk = rng.integers(0, 2, size=(H * 4, 16)).astype(np.float64)
    q_nope = rng.integers(-2, 3, size=(1, H, 4)).astype(np.float64)
    q_pe = np.zeros((1, H, 8))
    w_uv = oracle.round_to(rng.standard_normal((H * 4, 16)) * 0.25, "bf16")
    pool = oracle.round_to(rng.standard_normal((n_pages, 64, 24)), "bf16")
    table = rng.permutation(n_pages).astype(np.int32)[None, :]
    lens = np.array([L], dtype=np.int32)
    return dims, q_nope, q_pe, w_uk, w_uv, pool, table, lens


def _fp8_query_pins_pass():
    import oracle
    from synth import Dims, make_decode_case
    try:
        # 1. exact query: equals the plain decode
        dims, qn, qp, wuk, wuv, pool, table, lens = _exact_query_case(3, 3, 150)
        lam = dims.scale * np.log2(np.e)
        assert abs(lam - 1.0) < 1e-15
        q_abs = np.stack([wuk[h * 4:(h + 1) * 4].T @ qn[0, h] for h in range(2)])
        assert np.all(q_abs == np.round(q_abs)) and np.abs(q_abs).max() <= 8
        got = fp8.fp8_query_decode(dims, qn, qp, wuk, wuv, pool, table, lens)
        ref = oracle.decode(dims, qn, qp, wuk, wuv, pool, table, lens)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-14), float(np.abs(got - ref).max())
        # 2. dropping logical page 1 of 3 (query without a rotary part) is the
        # decode over logical pages 0 and 2
        got = fp8.fp8_query_decode(dims, qn, qp, wuk, wuv, pool, table, lens, drop_page=(0, 1))
        t2 = table[:, [0, 2]]
        ref = oracle.decode(dims, qn, qp, wuk, wuv, pool, t2, np.array([150 - 64], dtype=np.int32))
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-14), float(np.abs(got - ref).max())
        # 3. a realistic query (V3 head widths): the rounding moves the output
        # by an E4M3-sized amount (unit roundoff 2^-4; about 2 % here), far
        # more than the bf16 rounding alone (about 0.15 %) and far less than
        # 2^-3
        case = make_decode_case(7, 1, Dims(8, 512, 64, 128, 128), [300], shuffle=True)
        c = case.cache
        a = fp8.fp8_query_decode(case.dims, case.q_nope, case.q_pe, case.w_uk, case.w_uv, c.pool, c.block_table,
                                 c.context_lens)
        b = oracle.decode(case.dims, case.q_nope, case.q_pe, case.w_uk, case.w_uv, c.pool, c.block_table,
                          c.context_lens)
        rel = np.linalg.norm(a - b) / np.linalg.norm(b)
        assert 2.0 ** -7 < rel < 2.0 ** -3, rel
    except (AssertionError, ValueError):
        return False
    return True


def test_fp8_query_decode_pins_pass():
    assert _fp8_query_pins_pass()


def _round_nothing(x):
    return np.asarray(x, dtype=np.float64)


@pytest.mark.parametrize("name,attr,fake", [
    ("query not rounded to E4M3", "e4m3_round", _round_nothing),
    ("query scale one binade low", "scale_exponent", _scale_one_low),
])
def test_fp8_query_pins_catch_planted_mistake(name, attr, fake, monkeypatch):
    monkeypatch.setattr(fp8, attr, fake)
    assert not _fp8_query_pins_pass(), name
