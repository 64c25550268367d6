"""CPU oracle for Multi-head Latent Attention over a compressed latent KV cache.

TEST INFRASTRUCTURE, NOT PART OF THE LIBRARY. Only the tests, the smoke check
and the benchmark's CPU-baseline leg may import or call this module. It shares
no code with the HIP library and imports nothing from it.

It computes the plain definition of the method, in float64, with numpy:
explicit per-head key and value up-projection followed by ordinary two-pass
softmax attention. The matrix-absorbed form that the GPU path uses is written
out separately (``absorbed_decode``) only so that the tests can pin the two
forms to each other.

Sources (web pages on DeepSeek's architecture; sections as the pages number
them):

* [V2] "DeepSeek-V2 paper digest" (www.hncyxsy.com/news/273095):
  §1.1 the MHA cache size 2*n_h*d_h*l; §2.1 joint low-rank KV compression
  c_KV = W_DKV h, k_C = W_UK c_KV, v_C = W_UV c_KV with W_DKV [d_c, d] and
  W_UK, W_UV [n_h*d_h, d_c]; §2.2 absorption of W_UK into the query and of
  W_UV on the output side; §2.3 decoupled RoPE: the head dimension splits into
  a rotary part and a non-rotary part, RoPE acts only on the rotary part, and
  the cache holds the latent vector plus one small positional key; §4.3 the
  low-rank query path.
* [HDU] "8.1 DeepSeek architecture: MLA, DeepSeekMoE and FP8 training"
  (www.hdu-wiki.cn/courses/deepseek-architecture), §2: c_t = W^{DKV} h_t,
  k_t = W^{UK} c_t, v_t = W^{UV} c_t; the query side is compressed likewise.
* [NLPX] "DeepSeek 2025 technical report walkthrough: MoE and MLA"
  (m.nlpx.cn/news/79410), §3.3: worked per-token cache example (MHA
  2*32*128 = 8192 values against MLA 512 + 64 = 576, ratio about 14.2).
* [SHQ] "From MLA to DeepSeekMoE" (www.sheratonhq.com/news/177126), §2.1:
  MHA cache at hidden size 5120 in fp16 (about 20 KB per token).
* [IP] "DeepSeek core techniques: MoE and MLA attention"
  (intelliparadigm.com/article/weixin_29047545/2249442), §3.1: score count
  of a 2048-token sequence and its multiply-add count at dimension 128.

The output projection W_O (the attention layer's last step, which the pages'
§2.2 of [V2] names when it says W_UV can be absorbed into it) is written here
in its plain form, W_O applied to the concatenated per-head outputs, with
the fused weight W_O,h W_UV,h written out separately (``fold_output_weights``
and ``folded_decode_output``) only so that the tests can pin the two forms to
each other.

Readings taken where the pages are silent (each is a choice, stated once):

* RoPE pairs elements (2i, 2i+1) and rotates pair i by pos * base^(-2i/d_rope)
  with base 10000 (the pages name RoPE but give no formula; the pairing
  convention is parity unpinned by the pages; the tests pin its invariants).
* One positional key k_pe per token, shared by all heads; q_pe is per head.
* Cached token t sits at position t. A decode query sits at position L-1 and
  attends to all L cached tokens; prefill query s attends to keys 0..s.
* Softmax scale 1/sqrt(d_nope + d_rope) unless a scale is given.
* Weights use the pages' [out, in] orientation; head h owns rows
  h*d .. h*d + d - 1 of W_UK (d = d_nope) and of W_UV (d = d_v).
* W_O is [d_model, n_h*d_v]; head h's output goes into columns
  h*d_v .. h*d_v + d_v - 1, the order in which the heads' outputs are
  concatenated.
"""
from __future__ import annotations

import math

import numpy as np

# --------------------------------------------------------------- precision --

def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the storage type ("f32" or "bf16"), back in f64.

    bf16 rounding goes through float32 (both steps round to nearest even).
    """
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return x32.astype(np.float64)
    if dtype != "bf16":
        raise ValueError(dtype)
    u = x32.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def widen(a: np.ndarray) -> np.ndarray:
    """float64 view of an input array: float32 as is, uint16 as bfloat16 bits."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


# ------------------------------------------------------ cache-size formulas --

def mha_cache_values_per_token(n_heads: int, d_head: int, layers: int = 1) -> int:
    """[V2] §1.1: standard MHA caches keys and values, 2*n_h*d_h per layer."""
    return 2 * n_heads * d_head * layers


def mla_cache_values_per_token(d_c: int, d_rope: int, layers: int = 1) -> int:
    """[V2] §2.1 + §2.3, [NLPX] §3.3: the latent vector plus one positional key."""
    return (d_c + d_rope) * layers


def attention_score_macs(n_query: int, n_key: int, d: int) -> int:
    """[IP] §3.1: each score is a d-long dot product (d multiply-adds)."""
    return n_query * n_key * d


# ---------------------------------------------------------------- RoPE -----

def rope_angles(pos: np.ndarray, d_rope: int, base: float) -> np.ndarray:
    """Angle of pair i at position pos: pos * base^(-2i/d_rope) (reading above)."""
    i = np.arange(d_rope // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / d_rope)
    return np.asarray(pos, dtype=np.float64)[..., None] * theta


def _rotate_pairs(x: np.ndarray, ang: np.ndarray) -> np.ndarray:
    x0, x1 = x[..., 0::2], x[..., 1::2]
    c, s = np.cos(ang), np.sin(ang)
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def rope(x: np.ndarray, pos, base: float = 10000.0) -> np.ndarray:
    """Rotate the last axis (the d_rope slice only) of x at positions pos.

    [V2] §2.3: the rotary part carries position; nothing else is rotated.
    ``pos`` broadcasts against x.shape[:-1].
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % 2:
        raise ValueError("d_rope must be even")
    ang = rope_angles(np.broadcast_to(np.asarray(pos), x.shape[:-1]), d, base)
    return _rotate_pairs(x, ang)


# ----------------------------------------------------------- projections ---

def latent_rows(h, w_dkv, w_kr, positions, base: float = 10000.0, store: str | None = None):
    """Cache rows [c_KV || k_pe] of tokens h [T, d_model].

    [V2] §2.1 / [HDU] §2: c_KV = W_DKV h_t (W_DKV [d_c, d_model]).
    [V2] §2.3: the decoupled key is k_pe = RoPE(W_KR h_t) at the token's
    position; it is shared by all heads and cached beside c_KV.
    ``store`` rounds the rows to the cache's storage type.
    """
    h = widen(h)
    c = h @ widen(w_dkv).T
    k = rope(h @ widen(w_kr).T, np.asarray(positions), base)
    rows = np.concatenate([c, k], axis=-1)
    return round_to(rows, store) if store else rows


def query_projection(h, w_dq, w_uq, w_qr, n_heads: int, d_nope: int, d_rope: int,
                     store: str | None = None):
    """Low-rank query path ([V2] §4.3, [HDU] §2): c_Q = W_DQ h, then
    q_nope = W_UQ c_Q and q_pe = W_QR c_Q, split per head. q_pe is unrotated."""
    cq = widen(h) @ widen(w_dq).T
    qn = (cq @ widen(w_uq).T).reshape(-1, n_heads, d_nope)
    qp = (cq @ widen(w_qr).T).reshape(-1, n_heads, d_rope)
    if store:
        qn, qp = round_to(qn, store), round_to(qp, store)
    return qn, qp


# ------------------------------------------------------------ the cache ----

def gather_rows(pool, block_table, context_lens, b: int) -> np.ndarray:
    """Cached rows 0..L-1 of sequence b, in token order, as float64.

    Paged layout: token t lives in page block_table[b][t // bs] at offset
    t % bs. Contiguous layout (block_table None): pool[b, t].
    """
    L = int(context_lens[b])
    if block_table is None:
        return widen(pool[b, :L])
    bs = pool.shape[1]
    t = np.arange(L)
    return widen(pool[np.asarray(block_table)[b, t // bs], t % bs])


# ------------------------------------------------------------- attention ---

def _head_rows(w: np.ndarray, h: int, d: int) -> np.ndarray:
    """Rows h*d .. h*d+d-1 of a [n_heads*d, d_c] up-projection."""
    return w[h * d:(h + 1) * d]


def _softmax(s: np.ndarray) -> np.ndarray:
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def _explicit_kv(rows, w_uk_h, w_uv_h, d_c: int):
    """Per-head keys and values, up-projected explicitly ([V2] §2.1).

    K_h[t] = [W_UK,h c_t || k_pe_t]   (d_nope + d_rope wide; k_pe shared)
    V_h[t] = W_UV,h c_t               (d_v wide)
    """
    c, kpe = rows[:, :d_c], rows[:, d_c:]
    k = np.concatenate([c @ w_uk_h.T, kpe], axis=1)
    v = c @ w_uv_h.T
    return k, v


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, causal_offset=None):
    """Standard softmax attention of queries q [S, dk] over keys k [L, dk].

    With ``causal_offset`` o, query s sees keys 0..o+s only.
    """
    s = scale * (q @ k.T)
    if causal_offset is not None:
        qi = np.arange(q.shape[0])[:, None] + causal_offset
        s = np.where(np.arange(k.shape[0])[None, :] <= qi, s, -np.inf)
    return _softmax(s) @ v


def decode(dims, q_nope, q_pe, w_uk, w_uv, pool, block_table, context_lens, batch_rows=None):
    """Decode output [len(batch_rows), H, d_v]: one query per sequence.

    The query of sequence b sits at position L_b - 1 and attends to all L_b
    cached rows. Its rotary part is rotated there ([V2] §2.3); then each head
    runs attention over explicitly up-projected keys and values.
    """
    H, dn, dv, dc = dims.n_heads, dims.d_nope, dims.d_v, dims.d_c
    wuk, wuv = widen(w_uk), widen(w_uv)
    qn_all, qp_all = widen(q_nope), widen(q_pe)
    rows_b = range(qn_all.shape[0]) if batch_rows is None else batch_rows
    out = np.empty((len(rows_b), H, dv))
    for i, b in enumerate(rows_b):
        rows = gather_rows(pool, block_table, context_lens, b)
        L = rows.shape[0]
        qpe = rope(qp_all[b], L - 1, dims.rope_base)
        for h in range(H):
            k, v = _explicit_kv(rows, _head_rows(wuk, h, dn), _head_rows(wuv, h, dv), dc)
            q = np.concatenate([qn_all[b, h], qpe[h]])[None, :]
            out[i, h] = attend(q, k, v, dims.scale)[0]
    return out


def prefill(dims, q_nope, q_pe, w_uk, w_uv, rows, queries=None):
    """Causal prefill output.

    q_nope [B, S, H, d_nope], q_pe [B, S, H, d_rope] (unrotated, query s at
    position s), rows [B, S, d_c + d_rope] (the cache rows of the same tokens).
    Returns [B, S, H, d_v], or, with ``queries`` a list of (b, s), an array
    [len(queries), H, d_v] for just those queries.
    """
    H, dn, dv, dc = dims.n_heads, dims.d_nope, dims.d_v, dims.d_c
    wuk, wuv = widen(w_uk), widen(w_uv)
    qn, qp = widen(q_nope), widen(q_pe)
    rows = widen(rows)
    B, S = qn.shape[:2]
    if queries is None:
        out = np.empty((B, S, H, dv))
        for b in range(B):
            qpe = rope(qp[b], np.arange(S)[:, None], dims.rope_base)   # [S, H, dr]
            for h in range(H):
                k, v = _explicit_kv(rows[b], _head_rows(wuk, h, dn), _head_rows(wuv, h, dv), dc)
                q = np.concatenate([qn[b, :, h], qpe[:, h]], axis=1)
                out[b, :, h] = attend(q, k, v, dims.scale, causal_offset=0)
        return out
    out = np.empty((len(queries), H, dv))
    for i, (b, s) in enumerate(queries):
        r = rows[b, :s + 1]
        qpe = rope(qp[b, s], s, dims.rope_base)
        for h in range(H):
            k, v = _explicit_kv(r, _head_rows(wuk, h, dn), _head_rows(wuv, h, dv), dc)
            q = np.concatenate([qn[b, s, h], qpe[h]])[None, :]
            out[i, h] = attend(q, k, v, dims.scale)[0]
    return out


def absorbed_decode(dims, q_nope, q_pe, w_uk, w_uv, pool, block_table, context_lens):
    """The absorbed form of ``decode`` ([V2] §2.2), for pinning only.

    q_abs = W_UK,h^T q_nope: scores are q_abs . c_KV + RoPE(q_pe) . k_pe; the
    latent output o_c = sum_t p_t c_t; W_UV,h is applied to o_c afterwards.
    Keys and values are never formed.
    """
    H, dn, dv, dc = dims.n_heads, dims.d_nope, dims.d_v, dims.d_c
    wuk, wuv = widen(w_uk), widen(w_uv)
    qn_all, qp_all = widen(q_nope), widen(q_pe)
    B = qn_all.shape[0]
    out = np.empty((B, H, dv))
    for b in range(B):
        rows = gather_rows(pool, block_table, context_lens, b)
        c, kpe = rows[:, :dc], rows[:, dc:]
        qpe = rope(qp_all[b], rows.shape[0] - 1, dims.rope_base)
        for h in range(H):
            q_abs = _head_rows(wuk, h, dn).T @ qn_all[b, h]
            s = dims.scale * (c @ q_abs + kpe @ qpe[h])
            p = _softmax(s)
            out[b, h] = _head_rows(wuv, h, dv) @ (p @ c)
    return out


# ----------------------------------------------------- output projection ---

def output_projection(attn_out, w_o) -> np.ndarray:
    """Attention layer output: W_O applied to the concatenation of the
    per-head outputs. attn_out [..., n_h, d_v], w_o [d_model, n_h*d_v];
    returns [..., d_model]."""
    a = widen(attn_out)
    lead = a.shape[:-2]
    x = a.reshape(lead + (a.shape[-2] * a.shape[-1],))
    return x @ widen(w_o).T


def decode_output(dims, q_nope, q_pe, w_uk, w_uv, w_o, pool, block_table, context_lens, batch_rows=None):
    """Decode followed by the output projection: [len(rows), d_model]."""
    return output_projection(decode(dims, q_nope, q_pe, w_uk, w_uv, pool, block_table, context_lens,
                                    batch_rows), w_o)


def fold_output_weights(w_uv, w_o, n_heads: int, d_v: int) -> np.ndarray:
    """[V2] §2.2: W_UV absorbed into the output projection. Block h of the
    result, columns h*d_c .. of [d_model, n_h*d_c], is W_O,h W_UV,h, with
    W_O,h the columns of W_O that take head h's output. For pinning only."""
    wuv, wo = widen(w_uv), widen(w_o)
    return np.concatenate([wo[:, h * d_v:(h + 1) * d_v] @ _head_rows(wuv, h, d_v) for h in range(n_heads)],
                          axis=1)


def folded_decode_output(dims, q_nope, q_pe, w_uk, w_ouv, pool, block_table, context_lens):
    """The absorbed form of ``decode_output`` ([V2] §2.2 on both sides), for
    pinning only: scores and the latent output o_c as in ``absorbed_decode``,
    then out = sum_h W_OUV,h o_c,h with the folded weights [d_model, n_h*d_c];
    neither keys, values nor per-head outputs are formed."""
    H, dn, dc = dims.n_heads, dims.d_nope, dims.d_c
    wuk, wouv = widen(w_uk), widen(w_ouv)
    qn_all, qp_all = widen(q_nope), widen(q_pe)
    B = qn_all.shape[0]
    out = np.zeros((B, wouv.shape[0]))
    for b in range(B):
        rows = gather_rows(pool, block_table, context_lens, b)
        c, kpe = rows[:, :dc], rows[:, dc:]
        qpe = rope(qp_all[b], rows.shape[0] - 1, dims.rope_base)
        for h in range(H):
            q_abs = _head_rows(wuk, h, dn).T @ qn_all[b, h]
            p = _softmax(dims.scale * (c @ q_abs + kpe @ qpe[h]))
            out[b] += wouv[:, h * dc:(h + 1) * dc] @ (p @ c)
    return out
