"""Seeded synthetic inputs for MLA decode and prefill.

This module draws random inputs and lays them out in memory (paged latent
cache pools, block tables, slot numbers). It holds none of the attention
arithmetic: no projection, rotation, softmax or contraction happens here.
Both the CPU oracle and the GPU path read the arrays it returns.

Representation
--------------
Every floating-point array is drawn as float32 from numpy's PCG64 generator.
For bfloat16 workloads it is rounded once, to nearest-even, and returned as a
``uint16`` array of bfloat16 bit patterns (numpy has no bfloat16 type). For
float32 workloads it is returned as float32. ``as_f64`` widens either kind
exactly.

Named workloads
---------------
``WORKLOADS`` holds the six shapes the library is measured on: a tiny fp32
case, three decode shapes (uniform 4K, DeepSeek-V3-shaped 8K, ragged long
context), a prefill with the latent and query projections, and a two-token
decode (a draft token per sequence) of the 8K shape.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

PAGE = 64  # tokens per cache page (block)


# ---------------------------------------------------------------- bf16 bits --
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    # NaN stays NaN (never produced by normal draws, kept for completeness)
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def as_f64(a: np.ndarray) -> np.ndarray:
    """Exact widening of a float32 array or a uint16 bfloat16-bit array."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


# ------------------------------------------------------------------- shapes --
@dataclasses.dataclass(frozen=True)
class Dims:
    n_heads: int
    d_c: int
    d_rope: int
    d_nope: int
    d_v: int
    dtype: str = "bf16"          # "bf16" or "f32"
    rope_base: float = 10000.0
    softmax_scale: float = 0.0   # <= 0: 1/sqrt(d_nope + d_rope)

    @property
    def row(self) -> int:
        return self.d_c + self.d_rope

    @property
    def scale(self) -> float:
        return self.softmax_scale if self.softmax_scale > 0 else 1.0 / math.sqrt(self.d_nope + self.d_rope)


class _Draw:
    """Draws N(0, std^2) float32 arrays in a fixed order, rounded to the dtype."""

    def __init__(self, seed: int, dtype: str):
        self.rng = np.random.Generator(np.random.PCG64(seed))
        self.dtype = dtype

    def normal(self, shape, std: float = 1.0) -> np.ndarray:
        x = self.rng.standard_normal(size=shape, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        return f32_to_bf16_bits(x) if self.dtype == "bf16" else x


# ------------------------------------------------------------ paged layout --
@dataclasses.dataclass
class PagedCache:
    """A pool of pages [num_blocks, block_size, row] plus its block table.

    ``block_table`` is None for the contiguous layout [batch, max_context, row]
    (then ``pool`` has that shape).
    """
    pool: np.ndarray                 # uint16 bf16 bits or float32
    block_table: Optional[np.ndarray]  # int32 [batch, max_blocks] (-1 = unused) or None
    context_lens: np.ndarray         # int32 [batch]
    block_size: int

    @property
    def max_context(self) -> int:
        return int(self.context_lens.max()) if self.context_lens.size else 0


def paged_layout(lens: np.ndarray, shuffle_rng: Optional[np.random.Generator]):
    """Block table for sequences of the given lengths.

    Identity placement puts sequence b's logical page p at physical block
    (pages of sequences < b) + p. With ``shuffle_rng`` the physical blocks are
    a seeded random permutation of the pool. Unused entries are -1.
    """
    pages = [(int(L) + PAGE - 1) // PAGE for L in lens]
    num_blocks = int(sum(pages))
    max_blocks = max(pages) if pages else 0
    table = np.full((len(lens), max(max_blocks, 1)), -1, dtype=np.int32)
    phys = np.arange(num_blocks, dtype=np.int32)
    if shuffle_rng is not None:
        phys = shuffle_rng.permutation(num_blocks).astype(np.int32)
    g = 0
    for b, n in enumerate(pages):
        table[b, :n] = phys[g:g + n]
        g += n
    return table, num_blocks


# --------------------------------------------------------------- workloads --
@dataclasses.dataclass
class DecodeCase:
    dims: Dims
    q_nope: np.ndarray     # [B, H, d_nope], or [B, q_len, H, d_nope] for q_len > 1
    q_pe: np.ndarray       # [B, H, d_rope] / [B, q_len, H, d_rope] (unrotated)
    w_uk: np.ndarray       # [H*d_nope, d_c]
    w_uv: np.ndarray       # [H*d_v, d_c]
    cache: PagedCache      # rows already hold rotated k_pe
    seed: int

    @property
    def batch(self) -> int:
        return self.q_nope.shape[0]

    @property
    def q_len(self) -> int:
        return 1 if self.q_nope.ndim == 3 else self.q_nope.shape[1]


@dataclasses.dataclass
class ProjectCase:
    """Inputs of the latent (and optionally query) projection + attention."""
    dims: Dims
    batch: int
    seq_len: int
    d_model: int
    h: np.ndarray          # [batch*seq_len, d_model]
    w_dkv: np.ndarray      # [d_c, d_model]
    w_kr: np.ndarray       # [d_rope, d_model]
    w_dq: Optional[np.ndarray]   # [d_q, d_model]
    w_uq: Optional[np.ndarray]   # [H*d_nope, d_q]
    w_qr: Optional[np.ndarray]   # [H*d_rope, d_q]
    w_uk: np.ndarray       # [H*d_nope, d_c]
    w_uv: np.ndarray       # [H*d_v, d_c]
    q_nope: Optional[np.ndarray]  # [batch, H, d_nope] when drawn (no query projection)
    q_pe: Optional[np.ndarray]
    positions: np.ndarray  # int32 [batch*seq_len]
    slots: np.ndarray      # int32 [batch*seq_len]
    block_table: Optional[np.ndarray]
    num_blocks: int
    seed: int

    @property
    def n_tokens(self) -> int:
        return self.batch * self.seq_len


def make_decode_case(seed: int, batch: int, dims: Dims, lens, paged: bool = True,
                     shuffle: bool = False, w_std: Optional[float] = None, q_len: int = 1) -> DecodeCase:
    """Decode inputs: q drawn N(0,1); W_UK, W_UV std 1/sqrt(d_c) (unless given);
    cache rows (c_KV || k_pe) drawn N(0,1), k_pe taken as already rotated.
    With q_len > 1 there are q_len queries per sequence (the last q_len tokens
    of its context) and the query arrays gain a q_len axis after the batch."""
    d = _Draw(seed, dims.dtype)
    H = dims.n_heads
    std = (1.0 / math.sqrt(dims.d_c)) if w_std is None else w_std
    w_uk = d.normal((H * dims.d_nope, dims.d_c), std)
    w_uv = d.normal((H * dims.d_v, dims.d_c), std)
    qshape = (batch,) if q_len == 1 else (batch, q_len)
    q_nope = d.normal(qshape + (H, dims.d_nope))
    q_pe = d.normal(qshape + (H, dims.d_rope))
    lens = np.asarray(lens, dtype=np.int64)
    if lens.ndim == 0:
        lens = np.full(batch, int(lens), dtype=np.int64)
    lens = lens.astype(np.int32)
    if paged:
        table, nb = paged_layout(lens, d.rng if shuffle else None)
        pool = d.normal((nb, PAGE, dims.row))
        cache = PagedCache(pool, table, lens, PAGE)
    else:
        maxc = int(lens.max())
        pool = d.normal((batch, maxc, dims.row))
        cache = PagedCache(pool, None, lens, maxc)
    return DecodeCase(dims, q_nope, q_pe, w_uk, w_uv, cache, seed)


def make_ragged_lens(seed: int, batch: int, lo: int, hi: int) -> np.ndarray:
    """Context lengths uniform on the integers [lo, hi], from their own stream."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(lo, hi, size=batch, endpoint=True).astype(np.int32)


def make_project_case(seed: int, batch: int, seq_len: int, d_model: int, dims: Dims,
                      d_q: int = 0, paged: bool = True, shuffle: bool = False,
                      draw_query: bool = True) -> ProjectCase:
    """Projection / prefill inputs: h ~ N(0,1); every weight std 1/sqrt(fan_in).

    Token t of sequence b sits at position t and is written to the cache slot
    block_table[b][t // 64] * 64 + t % 64 (paged) or b*seq_len + t (contiguous).
    With d_q > 0 the query comes from the low-rank query projection; otherwise,
    if ``draw_query``, one decode query per sequence is drawn N(0,1).
    """
    d = _Draw(seed, dims.dtype)
    H = dims.n_heads
    T = batch * seq_len
    h = d.normal((T, d_model))
    w_dkv = d.normal((dims.d_c, d_model), 1.0 / math.sqrt(d_model))
    w_kr = d.normal((dims.d_rope, d_model), 1.0 / math.sqrt(d_model))
    w_dq = w_uq = w_qr = None
    if d_q > 0:
        w_dq = d.normal((d_q, d_model), 1.0 / math.sqrt(d_model))
        w_uq = d.normal((H * dims.d_nope, d_q), 1.0 / math.sqrt(d_q))
        w_qr = d.normal((H * dims.d_rope, d_q), 1.0 / math.sqrt(d_q))
    w_uk = d.normal((H * dims.d_nope, dims.d_c), 1.0 / math.sqrt(dims.d_c))
    w_uv = d.normal((H * dims.d_v, dims.d_c), 1.0 / math.sqrt(dims.d_c))
    q_nope = q_pe = None
    if d_q == 0 and draw_query:
        q_nope = d.normal((batch, H, dims.d_nope))
        q_pe = d.normal((batch, H, dims.d_rope))
    positions = np.tile(np.arange(seq_len, dtype=np.int32), batch)
    lens = np.full(batch, seq_len, dtype=np.int32)
    if paged:
        table, nb = paged_layout(lens, d.rng if shuffle else None)
        t = np.arange(seq_len)
        slots = np.concatenate([table[b, t // PAGE] * PAGE + t % PAGE for b in range(batch)]).astype(np.int32)
    else:
        table, nb = None, batch
        slots = np.arange(T, dtype=np.int32)
    return ProjectCase(dims, batch, seq_len, d_model, h, w_dkv, w_kr, w_dq, w_uq, w_qr,
                       w_uk, w_uv, q_nope, q_pe, positions, slots, table, nb, seed)


def draw_output_weights(seed: int, d_model: int, n_heads: int, d_v: int, dtype: str = "bf16") -> np.ndarray:
    """The output projection W_O [d_model, n_heads*d_v], std 1/sqrt(fan_in),
    drawn from its own seeded stream (so no other draw of a workload moves)."""
    return _Draw(seed, dtype).normal((d_model, n_heads * d_v), 1.0 / math.sqrt(n_heads * d_v))


# The five measured shapes. Each entry builds its inputs from seed 1000 + k.
V3 = dict(d_c=512, d_rope=64, d_nope=128, d_v=128)


def workload(k: int):
    """Inputs of named workload k (1..6)."""
    seed = 1000 + k
    if k == 1:   # tiny fp32, contiguous cache, rows made by the projection
        dims = Dims(n_heads=4, d_c=32, d_rope=8, d_nope=16, d_v=16, dtype="f32")
        return make_project_case(seed, batch=1, seq_len=64, d_model=64, dims=dims, paged=False)
    if k == 2:   # uniform 4K-context decode, 16 heads
        return make_decode_case(seed, 16, Dims(n_heads=16, **V3), 4096)
    if k == 3:   # DeepSeek-V3-shaped decode, all 128 heads
        return make_decode_case(seed, 64, Dims(n_heads=128, **V3, softmax_scale=1.0 / math.sqrt(192.0)), 8192)
    if k == 4:   # ragged long-context decode, shuffled pages
        lens = make_ragged_lens(seed + 500, 32, 1024, 32768)
        return make_decode_case(seed, 32, Dims(n_heads=128, **V3), lens, shuffle=True)
    if k == 5:   # causal prefill with latent and query projections
        return make_project_case(seed, batch=4, seq_len=4096, d_model=7168,
                                 dims=Dims(n_heads=128, **V3), d_q=1536)
    if k == 6:   # two-token decode (one draft token per sequence), DeepSeek-V3 shape
        return make_decode_case(seed, 64, Dims(n_heads=128, **V3, softmax_scale=1.0 / math.sqrt(192.0)), 8192,
                                q_len=2)
    raise ValueError(k)


WORKLOADS = {
    1: "tiny fp32 MLA: B=1 H=4 d_model=64 d_c=32 d_rope=8 d_nope=d_v=16 L=64, contiguous",
    2: "bf16 decode: B=16 H=16 d_c=512 d_rope=64 L=4096, 64-token pages",
    3: "bf16 decode, DeepSeek-V3 shape: B=64 H=128 d_c=512 d_rope=64 L=8192, 64-token pages",
    4: "bf16 ragged decode: B=32 H=128 L~U[1024,32768], shuffled 64-token pages",
    5: "bf16 causal prefill: B=4 S=4096 d_model=7168 d_q=1536 H=128, projections + attention",
    6: "bf16 two-token decode, DeepSeek-V3 shape: B=64 q_len=2 H=128 d_c=512 d_rope=64 L=8192, 64-token pages",
}


# ----------------------------------------------------------- device copies --
def to_torch(a: np.ndarray, device="cuda"):
    """Device tensor of a generated array: uint16 bf16 bits -> torch.bfloat16,
    float32 -> torch.float32, int32 stays int32. Bits are copied unchanged."""
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def from_torch(t) -> np.ndarray:
    """Host float64 copy of a device tensor (bf16 widened exactly)."""
    import torch
    return t.detach().to("cpu", torch.float64).numpy()
