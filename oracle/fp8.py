"""CPU oracle for the FP8 latent cache: quantisation of cache rows and its
inverse.

TEST INFRASTRUCTURE, NOT PART OF THE LIBRARY. Only the tests, the smoke check
and the benchmark's CPU-baseline leg may import or call this module. It shares
no code with the HIP library and imports nothing from it.

Sources (sections as the pages number them):

* [IP] "DeepSeek core techniques: MoE and MLA attention"
  (intelliparadigm.com/article/weixin_29047545/2249442), §6.3: for
  deployment the KV cache is quantised to FP8 dynamically (scales taken from
  the data as it is written).
* [HDU] "8.1 DeepSeek architecture: MLA, DeepSeekMoE and FP8 training"
  (www.hdu-wiki.cn/courses/deepseek-architecture), §5 and exercise Q4 of §7:
  FP8's range and precision are small, so the scale is chosen per tile or
  block, not once globally; one global scale would let blocks of very
  different magnitude underflow or overflow.

Readings taken where the pages are silent (each a choice, stated once):

* FP8 is the OCP E4M3 format ("fn"): sign, 4 exponent bits with bias 7, 3
  mantissa bits; largest finite value 448; subnormals below 2^-6 with spacing
  2^-9; no infinities; S.1111.111 is NaN. Rounding is to nearest, ties to
  even.
* The block is one token's latent vector c_KV (d_c values). Its scale is a
  power of two, 2^e, with e the smallest integer >= -127 such that
  max|c| <= 448 * 2^e: no code saturates, and the largest magnitude lands
  in (224, 448] times the scale. The codes are RNE(c / 2^e). The scale is stored as the byte
  E = e + 127 (value 2^(E - 127)).
* The rotary key k_pe stays bfloat16: it carries position and is d_rope of
  the d_c + d_rope values of a row.
* Page layout, for pages of P tokens: P rows of [d_c code bytes || d_rope
  bfloat16 k_pe values], then the P scale bytes, then zero bytes up to a
  multiple of 16.
* fp8_query_decode: the pages say nothing of the query of an FP8 decode; this
  reference takes the library's declared query arithmetic (the absorbed
  query scaled by softmax scale * log2(e), rounded to bfloat16, its latent
  part then quantised like a cache row with one scale per head) so that a
  tighter bar can be set on what is left. Its pins are in
  tests/test_fp8_pins.py.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_SUBNORMAL_STEP = 2.0 ** -9
SCALE_BIAS = 127
SCALE_MIN_EXP = -127


def e4m3_round(x) -> np.ndarray:
    """Nearest E4M3 value (ties to even) of each element, as float64.

    Normal binade [2^k, 2^(k+1)), k >= -6, holds 8 values spaced 2^(k-3);
    below 2^-6 the spacing is 2^-9. Magnitudes above 448 are outside the
    format's finite range and are rejected (the quantiser never produces them).
    """
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("magnitude above the largest E4M3 value")
    a = np.abs(x)
    k = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    # log2 may round across a binade edge: settle k so that 2^k <= a < 2^(k+1)
    k = np.where((a > 0) & (2.0 ** k > a), k - 1, k)
    k = np.where((a > 0) & (2.0 ** (k + 1) <= a), k + 1, k)
    step = np.where(a >= E4M3_MIN_NORMAL, 2.0 ** (k - 3), E4M3_SUBNORMAL_STEP)
    r = np.rint(a / step) * step          # np.rint rounds half to even
    return np.copysign(r, x)


def e4m3_encode(v) -> np.ndarray:
    """Byte codes of values that are exact E4M3 values (as e4m3_round returns).

    Normal: sign << 7 | (k + 7) << 3 | (v / 2^k * 8 - 8); subnormal: sign << 7 |
    v / 2^-9. Negative zero keeps its sign bit.
    """
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.uint8) << 7
    a = np.abs(v)
    code = np.zeros(v.shape, dtype=np.int64)
    sub = a < E4M3_MIN_NORMAL
    code[sub] = np.rint(a[sub] / E4M3_SUBNORMAL_STEP).astype(np.int64)
    nrm = ~sub
    if np.any(nrm):
        m, ex = np.frexp(a[nrm])             # a = m * 2^ex, m in [0.5, 1)
        k = ex - 1
        mant = m * 16 - 8                    # a / 2^k * 8 - 8, an integer 0..7
        if not np.all(mant == np.rint(mant)):
            raise ValueError("value is not an E4M3 value")
        code[nrm] = (k + 7) * 8 + mant.astype(np.int64)
    if np.any(code > 0x7E):
        raise ValueError("value is not a finite E4M3 value")
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    """Values of E4M3 byte codes (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 7
    val = np.where(e == 0, m * E4M3_SUBNORMAL_STEP, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return s * val


def scale_exponent(amax: float) -> int:
    """Smallest integer e >= -127 with amax <= 448 * 2^e (see the module
    docstring); found by stepping, with exact float64 comparisons."""
    amax = float(amax)
    if not np.isfinite(amax) or amax < 0:
        raise ValueError("amax must be finite and non-negative")
    e = SCALE_MIN_EXP
    while amax > E4M3_MAX * 2.0 ** e:
        e += 1
    return e


def quantize_rows(rows, d_c: int):
    """FP8 form of cache rows [n, d_c + d_rope] (float64 values that are
    bfloat16 numbers, e.g. ``widen`` of a bf16 pool).

    Returns (codes [n, d_c] uint8, kpe [n, d_rope] uint16 bfloat16 bits,
    scale bytes [n] uint8).
    """
    rows = np.asarray(rows, dtype=np.float64)
    c, kpe = rows[:, :d_c], rows[:, d_c:]
    n = rows.shape[0]
    codes = np.empty((n, d_c), dtype=np.uint8)
    E = np.empty(n, dtype=np.uint8)
    for i in range(n):
        e = scale_exponent(np.abs(c[i]).max() if d_c else 0.0)
        codes[i] = e4m3_encode(e4m3_round(c[i] * 2.0 ** (-e)))
        E[i] = e + SCALE_BIAS
    kpe32 = kpe.astype(np.float32)
    if not np.array_equal(kpe32.astype(np.float64), kpe):
        raise ValueError("k_pe values must be exact float32 numbers")
    kbits = (kpe32.view(np.uint32) >> 16).astype(np.uint16)
    if not np.array_equal((kbits.astype(np.uint32) << 16).view(np.float32), kpe32):
        raise ValueError("k_pe values must be bfloat16 numbers")
    return codes, kbits, E


def dequantize_rows(codes, kpe_bits, E) -> np.ndarray:
    """float64 rows [n, d_c + d_rope]: c = code value * 2^(E - 127), k_pe as stored."""
    c = e4m3_decode(codes) * 2.0 ** (np.asarray(E, dtype=np.float64)[:, None] - SCALE_BIAS)
    k = (np.asarray(kpe_bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.concatenate([c, k], axis=1)


def page_bytes(page: int, d_c: int, d_rope: int) -> int:
    """Bytes of one FP8 page: rows, scale bytes, zero padding to 16."""
    raw = page * (d_c + 2 * d_rope) + page
    return (raw + 15) // 16 * 16


def pack_pages(codes, kpe_bits, E, page: int) -> np.ndarray:
    """Lays quantised rows (row r = page r // P, offset r % P) out as pages
    [n / P, page_bytes] of uint8, per the layout in the module docstring."""
    n, d_c = codes.shape
    d_rope = kpe_bits.shape[1]
    if n % page:
        raise ValueError("row count must be a whole number of pages")
    rb = d_c + 2 * d_rope
    out = np.zeros((n // page, page_bytes(page, d_c, d_rope)), dtype=np.uint8)
    rows = np.concatenate([codes, kpe_bits.astype("<u2").view(np.uint8).reshape(n, 2 * d_rope)], axis=1)
    out[:, :page * rb] = rows.reshape(n // page, page * rb)
    out[:, page * rb:page * rb + page] = np.asarray(E, dtype=np.uint8).reshape(n // page, page)
    return out


def unpack_pages(pages, page: int, d_c: int, d_rope: int):
    """Inverse of pack_pages: (codes, kpe_bits, E) of every row slot."""
    pages = np.asarray(pages, dtype=np.uint8)
    nb = pages.shape[0]
    rb = d_c + 2 * d_rope
    rows = pages[:, :page * rb].reshape(nb * page, rb)
    codes = rows[:, :d_c].copy()
    kpe_bits = rows[:, d_c:].copy().view("<u2").astype(np.uint16)
    E = pages[:, page * rb:page * rb + page].reshape(nb * page).copy()
    return codes, kpe_bits, E


def quantize_pool(pool_rows, d_c: int) -> np.ndarray:
    """FP8 pages of a pool of cache rows [num_blocks, P, d_c + d_rope]."""
    nb, P, R = pool_rows.shape
    codes, kbits, E = quantize_rows(np.asarray(pool_rows, dtype=np.float64).reshape(nb * P, R), d_c)
    return pack_pages(codes, kbits, E, P)


def dequantize_pool(pages, page: int, d_c: int, d_rope: int) -> np.ndarray:
    """float64 cache rows [num_blocks, P, d_c + d_rope] held by FP8 pages:
    the rows the attention over an FP8 cache reads."""
    codes, kbits, E = unpack_pages(pages, page, d_c, d_rope)
    return dequantize_rows(codes, kbits, E).reshape(np.asarray(pages).shape[0], page, d_c + d_rope)


# ------------------------------------------------ decode with an FP8 query --
def fp8_query_decode(dims, q_nope, q_pe, w_uk, w_uv, pool, block_table, context_lens, drop_page=None):
    """Decode over a (dequantised) cache with the absorbed query in the form
    an FP8 decode feeds it to an FP8 product, for one query per sequence.

    The decode itself is "DeepSeek-V2 paper digest" §2.2-2.3 in its absorbed
    form (scores c_t . q_abs + k_pe,t . RoPE(q_pe), values W_UV,h sum_t p_t c_t);
    the FP8 cache is [IP] §6.3. What this adds is the query rounding that the
    library's FP8 decode declares: with lam = softmax scale * log2(e), the
    latent part lam * W_UK,h^T q_nope and the rotary part lam * RoPE(q_pe) are
    each rounded to bfloat16, and the latent part is then quantised like a
    cache row (one power-of-two scale per head, codes RNE to E4M3). Scores are
    then base-2 logits of the rounded query; everything else is exact (fp64).

    drop_page = (b, j) leaves logical page j (64 tokens) of sequence b out of
    the attention while the query keeps its position (a negative control)."""
    from .mla import _head_rows, gather_rows, rope, round_to, widen
    H, dn, dv, dc = dims.n_heads, dims.d_nope, dims.d_v, dims.d_c
    lam = dims.scale * np.log2(np.e)
    wuk, wuv = widen(w_uk), widen(w_uv)
    qn_all, qp_all = widen(q_nope), widen(q_pe)
    B = qn_all.shape[0]
    out = np.empty((B, H, dv))
    for b in range(B):
        rows = gather_rows(pool, block_table, context_lens, b)
        L = rows.shape[0]
        keep = np.ones(L, dtype=bool)
        if drop_page is not None and drop_page[0] == b:
            keep[64 * drop_page[1]:64 * (drop_page[1] + 1)] = False
        c, kpe = rows[keep, :dc], rows[keep, dc:]
        qpe = rope(qp_all[b], L - 1, dims.rope_base)
        for h in range(H):
            q_c = round_to(lam * (_head_rows(wuk, h, dn).T @ qn_all[b, h]), "bf16")
            e = scale_exponent(np.abs(q_c).max())
            q_c8 = e4m3_round(q_c * 2.0 ** (-e)) * 2.0 ** e
            q_r = round_to(lam * qpe[h], "bf16")
            s2 = c @ q_c8 + kpe @ q_r
            p = np.exp2(s2 - s2.max())
            out[b, h] = _head_rows(wuv, h, dv) @ (p @ c) / p.sum()
    return out
