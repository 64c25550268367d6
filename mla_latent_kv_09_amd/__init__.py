"""Python binding of libmla, the MI355X (gfx950) MLA library.

Argument marshalling only: torch tensors are checked against the dims (shape,
dtype, device, contiguity) so that no kernel is launched on mismatched
buffers, and are handed to the C ABI in include/mla.h as raw device pointers
on the current torch stream. Every step of the computation runs in the HIP
kernels of libmla.so; there is no fallback. If the library is not built the
first call raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional

import torch

__all__ = [
    "Dims", "Cache", "QProj", "MLAError", "library", "library_path",
    "mla_rope_latent_project", "mla_decode", "mla_decode_multi", "mla_prefill",
    "mla_project_workspace_size", "mla_decode_workspace_size", "mla_decode_multi_workspace_size",
    "mla_prefill_workspace_size", "Fp8Cache", "mla_fp8_page_bytes", "mla_quantize_fp8", "mla_decode_fp8",
    "mla_decode_fp8_workspace_size", "mla_decode_noalloc", "mla_noalloc_scratch_bytes",
    "mla_rope_latent_project_fp8", "mla_project_fp8_workspace_size",
    "mla_output_project", "mla_output_workspace_size", "mla_fold_output_weights", "mla_decode_folded",
    "mla_decode_folded_workspace_size", "mla_workspace_size", "MLA_OP_PROJECT", "MLA_OP_DECODE", "MLA_OP_PREFILL",
    "mla_status_string", "mla_decode_path", "mla_prefill_path", "mla_version",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libmla.so")

MLA_F32, MLA_BF16 = 0, 1
MLA_OP_PROJECT, MLA_OP_DECODE, MLA_OP_PREFILL = 0, 1, 2
_TORCH_DTYPE = {MLA_F32: torch.float32, MLA_BF16: torch.bfloat16}


class MLAError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: status {status} ({mla_status_string(status)})")
        self.status = status


# ------------------------------------------------------------- C structs ---
class _Dims(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("d_c", ctypes.c_int32), ("d_rope", ctypes.c_int32),
                ("d_nope", ctypes.c_int32), ("d_v", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("rope_base", ctypes.c_float), ("dtype", ctypes.c_int32)]


class _Cache(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_void_p), ("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("block_table", ctypes.c_void_p), ("max_blocks_per_seq", ctypes.c_int32),
                ("context_lens", ctypes.c_void_p), ("max_context", ctypes.c_int32)]


class _QProj(ctypes.Structure):
    _fields_ = [("d_q", ctypes.c_int32), ("w_dq", ctypes.c_void_p), ("w_uq", ctypes.c_void_p),
                ("w_qr", ctypes.c_void_p), ("q_nope", ctypes.c_void_p), ("q_pe", ctypes.c_void_p)]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def library():
    """The loaded libmla.so (ctypes), loading it on first use."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m mla_latent_kv_09_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        pd, pc, pq = ctypes.POINTER(_Dims), ctypes.POINTER(_Cache), ctypes.POINTER(_QProj)
        lib.mla_rope_latent_project.argtypes = [pd, i32, i32, vp, vp, vp, vp, vp, pc, pq, vp, sz, vp]
        lib.mla_decode.argtypes = [pd, i32, vp, vp, vp, vp, pc, vp, vp, sz, vp]
        lib.mla_decode_multi.argtypes = [pd, i32, i32, vp, vp, vp, vp, pc, vp, vp, sz, vp]
        lib.mla_prefill.argtypes = [pd, i32, i32, vp, vp, vp, vp, pc, vp, vp, sz, vp]
        lib.mla_decode_fp8.argtypes = [pd, i32, i32, vp, vp, vp, vp, pc, vp, vp, sz, vp]
        lib.mla_rope_latent_project_fp8.argtypes = [pd, i32, i32, vp, vp, vp, vp, vp, vp, i32, pq, vp, sz, vp]
        lib.mla_rope_latent_project_fp8.restype = ctypes.c_int
        lib.mla_project_fp8_workspace_size.argtypes = [pd, i32, i32, ctypes.POINTER(sz)]
        lib.mla_project_fp8_workspace_size.restype = ctypes.c_int
        lib.mla_output_project.argtypes = [pd, i32, i32, vp, vp, vp, vp, sz, vp]
        lib.mla_fold_output_weights.argtypes = [pd, i32, vp, vp, vp, vp]
        lib.mla_decode_folded.argtypes = [pd, i32, i32, vp, vp, vp, vp, i32, pc, vp, vp, sz, vp]
        lib.mla_output_workspace_size.argtypes = [pd, i32, i32, i32, ctypes.POINTER(sz)]
        lib.mla_decode_folded_workspace_size.argtypes = [pd, i32, i32, i32, i32, ctypes.POINTER(sz)]
        for f in ("mla_output_project", "mla_fold_output_weights", "mla_decode_folded", "mla_output_workspace_size",
                  "mla_decode_folded_workspace_size"):
            getattr(lib, f).restype = ctypes.c_int
        lib.mla_decode_noalloc.argtypes = [pd, i32, i32, vp, vp, vp, vp, pc, vp, vp]
        lib.mla_decode_noalloc.restype = ctypes.c_int
        lib.mla_noalloc_scratch_bytes.argtypes = []
        lib.mla_noalloc_scratch_bytes.restype = sz
        lib.mla_quantize_fp8.argtypes = [pd, i32, vp, vp, i32, vp, vp]
        lib.mla_fp8_page_bytes.argtypes = [pd, i32, ctypes.POINTER(sz)]
        lib.mla_decode_fp8_workspace_size.argtypes = [pd, i32, i32, i32, ctypes.POINTER(sz)]
        lib.mla_project_workspace_size.argtypes = [pd, i32, i32, ctypes.POINTER(sz)]
        lib.mla_decode_workspace_size.argtypes = [pd, i32, i32, ctypes.POINTER(sz)]
        lib.mla_decode_multi_workspace_size.argtypes = [pd, i32, i32, i32, ctypes.POINTER(sz)]
        lib.mla_prefill_workspace_size.argtypes = [pd, i32, i32, i32, ctypes.POINTER(sz)]
        lib.mla_workspace_size.argtypes = [i32, pd, i32, i32, ctypes.POINTER(sz)]
        lib.mla_status_string.argtypes = [ctypes.c_int]
        lib.mla_status_string.restype = ctypes.c_char_p
        lib.mla_decode_path.argtypes = [pd, i32, i32]
        lib.mla_prefill_path.argtypes = [pd, i32, i32]
        lib.mla_profile_begin.argtypes = []
        lib.mla_profile_only.argtypes = [ctypes.c_char_p]
        for f in ("mla_rope_latent_project", "mla_decode", "mla_decode_multi", "mla_prefill",
                  "mla_project_workspace_size", "mla_decode_workspace_size", "mla_decode_multi_workspace_size",
                  "mla_prefill_workspace_size", "mla_profile_begin", "mla_profile_only", "mla_decode_fp8",
                  "mla_quantize_fp8", "mla_fp8_page_bytes", "mla_decode_fp8_workspace_size",
                  "mla_workspace_size"):
            getattr(lib, f).restype = ctypes.c_int
        for f in ("mla_decode_path", "mla_prefill_path", "mla_version"):
            getattr(lib, f).restype = ctypes.c_int32
        _lib = lib
    return _lib


# ------------------------------------------------------------ Python side ---
@dataclasses.dataclass(frozen=True)
class Dims:
    n_heads: int
    d_c: int
    d_rope: int
    d_nope: int
    d_v: int
    dtype: str = "bf16"            # "bf16" or "f32"
    softmax_scale: float = 0.0     # <= 0: 1/sqrt(d_nope + d_rope)
    rope_base: float = 10000.0

    @classmethod
    def of(cls, d) -> "Dims":
        if isinstance(d, cls):
            return d
        if isinstance(d, _Dims):
            return cls(d.n_heads, d.d_c, d.d_rope, d.d_nope, d.d_v,
                       {MLA_F32: "f32", MLA_BF16: "bf16"}.get(d.dtype, d.dtype), d.softmax_scale, d.rope_base)
        return cls(d.n_heads, d.d_c, d.d_rope, d.d_nope, d.d_v, getattr(d, "dtype", "bf16"),
                   getattr(d, "softmax_scale", 0.0), getattr(d, "rope_base", 10000.0))

    @property
    def code(self) -> int:
        return {"f32": MLA_F32, "bf16": MLA_BF16}.get(self.dtype, self.dtype)

    @property
    def torch_dtype(self):
        return _TORCH_DTYPE[self.code]

    @property
    def row(self) -> int:
        return self.d_c + self.d_rope

    def c(self) -> _Dims:
        return _Dims(self.n_heads, self.d_c, self.d_rope, self.d_nope, self.d_v, self.softmax_scale,
                     self.rope_base, self.code)


@dataclasses.dataclass
class Cache:
    """Latent cache on the device.

    rows: [num_blocks, block_size, d_c + d_rope] with a block table [batch,
    max_blocks] (int32), or [batch, max_context, d_c + d_rope] with none.
    context_lens: int32 [batch]. max_context: host-side bound of context_lens.
    """
    rows: torch.Tensor
    context_lens: torch.Tensor
    max_context: int
    block_table: Optional[torch.Tensor] = None

    @property
    def batch(self) -> int:
        return self.context_lens.shape[0]

    def c(self) -> _Cache:
        if self.block_table is None:
            return _Cache(self.rows.data_ptr(), 0, 0, None, 0, self.context_lens.data_ptr(), int(self.max_context))
        return _Cache(self.rows.data_ptr(), self.rows.shape[0], self.rows.shape[1], self.block_table.data_ptr(),
                      self.block_table.shape[1], self.context_lens.data_ptr(), int(self.max_context))


@dataclasses.dataclass
class Fp8Cache:
    """FP8 latent cache on the device (format in include/mla.h).

    pages: uint8 [num_blocks, mla_fp8_page_bytes(dims, block_size)];
    block_table: int32 [batch, max_blocks]; context_lens: int32 [batch].
    """
    pages: torch.Tensor
    context_lens: torch.Tensor
    max_context: int
    block_table: torch.Tensor
    block_size: int = 64

    @property
    def batch(self) -> int:
        return self.context_lens.shape[0]

    def c(self) -> _Cache:
        return _Cache(self.pages.data_ptr(), self.pages.shape[0], self.block_size, self.block_table.data_ptr(),
                      self.block_table.shape[1], self.context_lens.data_ptr(), int(self.max_context))


@dataclasses.dataclass
class QProj:
    """Optional query path of mla_rope_latent_project (outputs q_nope, q_pe)."""
    w_dq: torch.Tensor      # [d_q, d_model]
    w_uq: torch.Tensor      # [H*d_nope, d_q]
    w_qr: torch.Tensor      # [H*d_rope, d_q]
    q_nope: torch.Tensor    # out [n_tokens, H, d_nope]
    q_pe: torch.Tensor      # out [n_tokens, H, d_rope]

    @property
    def d_q(self) -> int:
        return self.w_dq.shape[0]


def _need(t: torch.Tensor, name: str, shape, dtype):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_cache(cache: Cache, d: Dims, batch: int):
    _need(cache.context_lens, "context_lens", (batch,), torch.int32)
    if cache.block_table is None:
        _need(cache.rows, "cache rows", (batch, cache.max_context, d.row), d.torch_dtype)
    else:
        r = cache.rows
        if r.dim() != 3:
            raise ValueError("paged cache rows must be [num_blocks, block_size, row]")
        _need(r, "cache rows", (r.shape[0], r.shape[1], d.row), d.torch_dtype)
        _need(cache.block_table, "block_table", (batch, cache.block_table.shape[1]), torch.int32)


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream) if hasattr(s, "cuda_stream") else int(s)


def _workspace(nbytes: int, device, workspace):
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace has {workspace.numel() * workspace.element_size()} bytes, needs {nbytes}")
    return workspace, workspace.numel() * workspace.element_size()


def _ok(status: int, where: str):
    if status != 0:
        raise MLAError(status, where)


def mla_status_string(status: int) -> str:
    return library().mla_status_string(int(status)).decode()


def mla_version() -> int:
    return library().mla_version()


def mla_project_workspace_size(dims, n_tokens: int, d_q: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _ok(library().mla_project_workspace_size(ctypes.byref(Dims.of(dims).c()), n_tokens, d_q, ctypes.byref(n)),
        "mla_project_workspace_size")
    return n.value


def mla_decode_workspace_size(dims, batch: int, max_context: int) -> int:
    n = ctypes.c_size_t(0)
    _ok(library().mla_decode_workspace_size(ctypes.byref(Dims.of(dims).c()), batch, max_context, ctypes.byref(n)),
        "mla_decode_workspace_size")
    return n.value


def mla_decode_multi_workspace_size(dims, batch: int, q_len: int, max_context: int) -> int:
    n = ctypes.c_size_t(0)
    _ok(library().mla_decode_multi_workspace_size(ctypes.byref(Dims.of(dims).c()), batch, q_len, max_context,
                                                  ctypes.byref(n)), "mla_decode_multi_workspace_size")
    return n.value


def mla_prefill_workspace_size(dims, batch: int, seq_len: int, max_context: int) -> int:
    n = ctypes.c_size_t(0)
    _ok(library().mla_prefill_workspace_size(ctypes.byref(Dims.of(dims).c()), batch, seq_len, max_context,
                                             ctypes.byref(n)), "mla_prefill_workspace_size")
    return n.value


def mla_workspace_size(op: int, dims, size_a: int, size_b: int) -> int:
    """Workspace of MLA_OP_PROJECT (n_tokens, d_q), MLA_OP_DECODE (batch,
    max_context) or MLA_OP_PREFILL (batch, seq_len) (see include/mla.h)."""
    n = ctypes.c_size_t(0)
    _ok(library().mla_workspace_size(op, ctypes.byref(Dims.of(dims).c()), size_a, size_b, ctypes.byref(n)),
        "mla_workspace_size")
    return n.value


def mla_decode_path(dims, block_size: int = 64, paged: bool = True) -> int:
    return library().mla_decode_path(ctypes.byref(Dims.of(dims).c()), block_size, int(paged))


def mla_prefill_path(dims, block_size: int = 64, paged: bool = True) -> int:
    return library().mla_prefill_path(ctypes.byref(Dims.of(dims).c()), block_size, int(paged))


def mla_rope_latent_project(dims, h, w_dkv, w_kr, positions, slots, cache: Cache, qproj: Optional[QProj] = None,
                            workspace=None, stream=None):
    """Write [c_KV || RoPE(k)] of each token of h into its cache slot (see include/mla.h)."""
    d = Dims.of(dims)
    T, d_model = h.shape
    dt = d.torch_dtype
    _need(h, "h", (T, d_model), dt)
    _need(w_dkv, "w_dkv", (d.d_c, d_model), dt)
    _need(w_kr, "w_kr", (d.d_rope, d_model), dt)
    _need(positions, "positions", (T,), torch.int32)
    _need(slots, "slots", (T,), torch.int32)
    rows = cache.rows
    if rows.shape[-1] != d.row or rows.dtype != dt or not rows.is_contiguous():
        raise ValueError("cache rows do not match dims")
    qp = None
    d_q = 0
    if qproj is not None:
        d_q = qproj.d_q
        _need(qproj.w_dq, "w_dq", (d_q, d_model), dt)
        _need(qproj.w_uq, "w_uq", (d.n_heads * d.d_nope, d_q), dt)
        _need(qproj.w_qr, "w_qr", (d.n_heads * d.d_rope, d_q), dt)
        _need(qproj.q_nope, "q_nope", (T, d.n_heads, d.d_nope), dt)
        _need(qproj.q_pe, "q_pe", (T, d.n_heads, d.d_rope), dt)
        qp = _QProj(d_q, qproj.w_dq.data_ptr(), qproj.w_uq.data_ptr(), qproj.w_qr.data_ptr(),
                    qproj.q_nope.data_ptr(), qproj.q_pe.data_ptr())
    ws, nbytes = _workspace(mla_project_workspace_size(d, T, d_q), h.device, workspace)
    cc = cache.c()
    _ok(library().mla_rope_latent_project(ctypes.byref(d.c()), T, d_model, h.data_ptr(), w_dkv.data_ptr(),
                                          w_kr.data_ptr(), positions.data_ptr(), slots.data_ptr(), ctypes.byref(cc),
                                          ctypes.byref(qp) if qp is not None else None,
                                          ws.data_ptr() if ws is not None else None, nbytes, _stream(stream)),
        "mla_rope_latent_project")


def mla_project_fp8_workspace_size(dims, n_tokens: int, d_q: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _ok(library().mla_project_fp8_workspace_size(ctypes.byref(Dims.of(dims).c()), n_tokens, d_q, ctypes.byref(n)),
        "mla_project_fp8_workspace_size")
    return n.value


def mla_rope_latent_project_fp8(dims, h, w_dkv, w_kr, positions, slots, pages, block_size: int = 64,
                                qproj: Optional[QProj] = None, workspace=None, stream=None):
    """The latent rows of each token of h, RoPE'd and quantised straight into
    the FP8 pages [num_blocks, page_bytes] at slots (see include/mla.h)."""
    d = Dims.of(dims)
    T, d_model = h.shape
    dt = d.torch_dtype
    _need(h, "h", (T, d_model), dt)
    _need(w_dkv, "w_dkv", (d.d_c, d_model), dt)
    _need(w_kr, "w_kr", (d.d_rope, d_model), dt)
    _need(positions, "positions", (T,), torch.int32)
    _need(slots, "slots", (T,), torch.int32)
    if pages.dtype != torch.uint8 or pages.dim() != 2 or not pages.is_contiguous() or \
            pages.shape[1] != mla_fp8_page_bytes(d, block_size):
        raise ValueError("pages must be contiguous uint8 [num_blocks, mla_fp8_page_bytes]")
    qp = None
    d_q = 0
    if qproj is not None:
        d_q = qproj.d_q
        _need(qproj.w_dq, "w_dq", (d_q, d_model), dt)
        _need(qproj.w_uq, "w_uq", (d.n_heads * d.d_nope, d_q), dt)
        _need(qproj.w_qr, "w_qr", (d.n_heads * d.d_rope, d_q), dt)
        _need(qproj.q_nope, "q_nope", (T, d.n_heads, d.d_nope), dt)
        _need(qproj.q_pe, "q_pe", (T, d.n_heads, d.d_rope), dt)
        qp = _QProj(d_q, qproj.w_dq.data_ptr(), qproj.w_uq.data_ptr(), qproj.w_qr.data_ptr(),
                    qproj.q_nope.data_ptr(), qproj.q_pe.data_ptr())
    ws, nbytes = _workspace(mla_project_fp8_workspace_size(d, T, d_q), h.device, workspace)
    _ok(library().mla_rope_latent_project_fp8(ctypes.byref(d.c()), T, d_model, h.data_ptr(), w_dkv.data_ptr(),
                                              w_kr.data_ptr(), positions.data_ptr(), slots.data_ptr(),
                                              pages.data_ptr(), block_size,
                                              ctypes.byref(qp) if qp is not None else None,
                                              ws.data_ptr() if ws is not None else None, nbytes, _stream(stream)),
        "mla_rope_latent_project_fp8")


def mla_decode(dims, q_nope, q_pe, w_uk, w_uv, cache: Cache, out=None, workspace=None, stream=None):
    """One query per sequence over its whole cached context; returns out [B, H, d_v]."""
    d = Dims.of(dims)
    B = q_nope.shape[0]
    dt = d.torch_dtype
    _need(q_nope, "q_nope", (B, d.n_heads, d.d_nope), dt)
    _need(q_pe, "q_pe", (B, d.n_heads, d.d_rope), dt)
    _need(w_uk, "w_uk", (d.n_heads * d.d_nope, d.d_c), dt)
    _need(w_uv, "w_uv", (d.n_heads * d.d_v, d.d_c), dt)
    _check_cache(cache, d, B)
    if out is None:
        out = torch.empty((B, d.n_heads, d.d_v), dtype=dt, device=q_nope.device)
    _need(out, "out", (B, d.n_heads, d.d_v), dt)
    ws, nbytes = _workspace(mla_decode_workspace_size(d, B, cache.max_context), q_nope.device, workspace)
    cc = cache.c()
    _ok(library().mla_decode(ctypes.byref(d.c()), B, q_nope.data_ptr(), q_pe.data_ptr(), w_uk.data_ptr(),
                             w_uv.data_ptr(), ctypes.byref(cc), out.data_ptr(),
                             ws.data_ptr() if ws is not None else None, nbytes, _stream(stream)), "mla_decode")
    return out


def mla_decode_multi(dims, q_nope, q_pe, w_uk, w_uv, cache: Cache, out=None, workspace=None, stream=None):
    """q_len new queries per sequence (the last q_len tokens of its context),
    absorbed form; q_nope is [B, q_len, H, d_nope]; returns out [B, q_len, H, d_v]."""
    d = Dims.of(dims)
    B, Q = q_nope.shape[:2]
    dt = d.torch_dtype
    _need(q_nope, "q_nope", (B, Q, d.n_heads, d.d_nope), dt)
    _need(q_pe, "q_pe", (B, Q, d.n_heads, d.d_rope), dt)
    _need(w_uk, "w_uk", (d.n_heads * d.d_nope, d.d_c), dt)
    _need(w_uv, "w_uv", (d.n_heads * d.d_v, d.d_c), dt)
    _check_cache(cache, d, B)
    if out is None:
        out = torch.empty((B, Q, d.n_heads, d.d_v), dtype=dt, device=q_nope.device)
    _need(out, "out", (B, Q, d.n_heads, d.d_v), dt)
    ws, nbytes = _workspace(mla_decode_multi_workspace_size(d, B, Q, cache.max_context), q_nope.device, workspace)
    cc = cache.c()
    _ok(library().mla_decode_multi(ctypes.byref(d.c()), B, Q, q_nope.data_ptr(), q_pe.data_ptr(), w_uk.data_ptr(),
                                   w_uv.data_ptr(), ctypes.byref(cc), out.data_ptr(),
                                   ws.data_ptr() if ws is not None else None, nbytes, _stream(stream)),
        "mla_decode_multi")
    return out


def mla_output_workspace_size(dims, n_rows: int, d_model: int, folded: bool = False) -> int:
    n = ctypes.c_size_t(0)
    _ok(library().mla_output_workspace_size(ctypes.byref(Dims.of(dims).c()), n_rows, d_model, int(folded),
                                            ctypes.byref(n)), "mla_output_workspace_size")
    return n.value


def mla_output_project(dims, attn_out, w_o, out=None, workspace=None, stream=None):
    """W_O applied to the concatenated per-head outputs: attn_out [n, H, d_v],
    w_o [d_model, H*d_v]; returns out [n, d_model]."""
    d = Dims.of(dims)
    n = attn_out.shape[0]
    d_model = w_o.shape[0]
    dt = d.torch_dtype
    _need(attn_out, "attn_out", (n, d.n_heads, d.d_v), dt)
    _need(w_o, "w_o", (d_model, d.n_heads * d.d_v), dt)
    if out is None:
        out = torch.empty((n, d_model), dtype=dt, device=attn_out.device)
    _need(out, "out", (n, d_model), dt)
    ws, nbytes = _workspace(mla_output_workspace_size(d, n, d_model), attn_out.device, workspace)
    _ok(library().mla_output_project(ctypes.byref(d.c()), n, d_model, attn_out.data_ptr(), w_o.data_ptr(),
                                     out.data_ptr(), ws.data_ptr() if ws is not None else None, nbytes,
                                     _stream(stream)), "mla_output_project")
    return out


def mla_fold_output_weights(dims, w_uv, w_o, w_ouv=None, stream=None):
    """W_OUV [d_model, H*d_c] with column block h = W_O,h W_UV,h."""
    d = Dims.of(dims)
    d_model = w_o.shape[0]
    dt = d.torch_dtype
    _need(w_uv, "w_uv", (d.n_heads * d.d_v, d.d_c), dt)
    _need(w_o, "w_o", (d_model, d.n_heads * d.d_v), dt)
    if w_ouv is None:
        w_ouv = torch.empty((d_model, d.n_heads * d.d_c), dtype=dt, device=w_o.device)
    _need(w_ouv, "w_ouv", (d_model, d.n_heads * d.d_c), dt)
    _ok(library().mla_fold_output_weights(ctypes.byref(d.c()), d_model, w_uv.data_ptr(), w_o.data_ptr(),
                                          w_ouv.data_ptr(), _stream(stream)), "mla_fold_output_weights")
    return w_ouv


def mla_decode_folded_workspace_size(dims, batch: int, q_len: int, max_context: int, d_model: int) -> int:
    n = ctypes.c_size_t(0)
    _ok(library().mla_decode_folded_workspace_size(ctypes.byref(Dims.of(dims).c()), batch, q_len, max_context,
                                                   d_model, ctypes.byref(n)), "mla_decode_folded_workspace_size")
    return n.value


def mla_decode_folded(dims, q_nope, q_pe, w_uk, w_ouv, cache: Cache, out=None, workspace=None, stream=None):
    """Decode whose output is the layer output through the folded weights:
    q_nope [B, q_len, H, d_nope]; returns out [B, q_len, d_model]."""
    d = Dims.of(dims)
    B, Q = q_nope.shape[:2]
    d_model = w_ouv.shape[0]
    dt = d.torch_dtype
    _need(q_nope, "q_nope", (B, Q, d.n_heads, d.d_nope), dt)
    _need(q_pe, "q_pe", (B, Q, d.n_heads, d.d_rope), dt)
    _need(w_uk, "w_uk", (d.n_heads * d.d_nope, d.d_c), dt)
    _need(w_ouv, "w_ouv", (d_model, d.n_heads * d.d_c), dt)
    _check_cache(cache, d, B)
    if out is None:
        out = torch.empty((B, Q, d_model), dtype=dt, device=q_nope.device)
    _need(out, "out", (B, Q, d_model), dt)
    ws, nbytes = _workspace(mla_decode_folded_workspace_size(d, B, Q, cache.max_context, d_model), q_nope.device,
                            workspace)
    cc = cache.c()
    _ok(library().mla_decode_folded(ctypes.byref(d.c()), B, Q, q_nope.data_ptr(), q_pe.data_ptr(), w_uk.data_ptr(),
                                    w_ouv.data_ptr(), d_model, ctypes.byref(cc), out.data_ptr(),
                                    ws.data_ptr() if ws is not None else None, nbytes, _stream(stream)),
        "mla_decode_folded")
    return out


def mla_decode_noalloc(dims, q_nope, q_pe, w_uk, w_uv, cache: Cache, out, stream=None):
    """mla_decode_multi without a workspace: the library's fixed scratch array
    is used instead (see include/mla.h). q_nope is [B, q_len, H, d_nope]; out
    [B, q_len, H, d_v] must be given (this call allocates nothing)."""
    d = Dims.of(dims)
    B, Q = q_nope.shape[:2]
    dt = d.torch_dtype
    _need(q_nope, "q_nope", (B, Q, d.n_heads, d.d_nope), dt)
    _need(q_pe, "q_pe", (B, Q, d.n_heads, d.d_rope), dt)
    _need(w_uk, "w_uk", (d.n_heads * d.d_nope, d.d_c), dt)
    _need(w_uv, "w_uv", (d.n_heads * d.d_v, d.d_c), dt)
    _check_cache(cache, d, B)
    _need(out, "out", (B, Q, d.n_heads, d.d_v), dt)
    cc = cache.c()
    _ok(library().mla_decode_noalloc(ctypes.byref(d.c()), B, Q, q_nope.data_ptr(), q_pe.data_ptr(), w_uk.data_ptr(),
                                     w_uv.data_ptr(), ctypes.byref(cc), out.data_ptr(), _stream(stream)),
        "mla_decode_noalloc")
    return out


def mla_noalloc_scratch_bytes() -> int:
    return int(library().mla_noalloc_scratch_bytes())


def mla_fp8_page_bytes(dims, block_size: int = 64) -> int:
    n = ctypes.c_size_t(0)
    _ok(library().mla_fp8_page_bytes(ctypes.byref(Dims.of(dims).c()), block_size, ctypes.byref(n)),
        "mla_fp8_page_bytes")
    return n.value


def mla_quantize_fp8(dims, rows, pages, slots=None, block_size: int = 64, stream=None):
    """Quantises bf16 cache rows [n, d_c + d_rope] into the FP8 pages at
    slots (int32 [n]; row r to slot r when None)."""
    d = Dims.of(dims)
    n = rows.shape[0]
    _need(rows, "rows", (n, d.row), torch.bfloat16)
    pb = mla_fp8_page_bytes(d, block_size)
    _need(pages, "pages", (pages.shape[0], pb), torch.uint8)
    if slots is not None:
        _need(slots, "slots", (n,), torch.int32)
    _ok(library().mla_quantize_fp8(ctypes.byref(d.c()), n, rows.data_ptr(),
                                   slots.data_ptr() if slots is not None else None, block_size, pages.data_ptr(),
                                   _stream(stream)), "mla_quantize_fp8")
    return pages


def mla_decode_fp8_workspace_size(dims, batch: int, q_len: int, max_context: int) -> int:
    n = ctypes.c_size_t(0)
    _ok(library().mla_decode_fp8_workspace_size(ctypes.byref(Dims.of(dims).c()), batch, q_len, max_context,
                                                ctypes.byref(n)), "mla_decode_fp8_workspace_size")
    return n.value


def mla_decode_fp8(dims, q_nope, q_pe, w_uk, w_uv, cache: Fp8Cache, out=None, workspace=None, stream=None):
    """Decode over an FP8 cache. q_nope [B, H, d_nope] (one new token per
    sequence) or [B, q_len, H, d_nope]; out has the same leading shape."""
    d = Dims.of(dims)
    multi = q_nope.dim() == 4
    B = q_nope.shape[0]
    Q = q_nope.shape[1] if multi else 1
    lead = (B, Q) if multi else (B,)
    dt = d.torch_dtype
    _need(q_nope, "q_nope", lead + (d.n_heads, d.d_nope), dt)
    _need(q_pe, "q_pe", lead + (d.n_heads, d.d_rope), dt)
    _need(w_uk, "w_uk", (d.n_heads * d.d_nope, d.d_c), dt)
    _need(w_uv, "w_uv", (d.n_heads * d.d_v, d.d_c), dt)
    _need(cache.context_lens, "context_lens", (B,), torch.int32)
    _need(cache.pages, "pages", (cache.pages.shape[0], mla_fp8_page_bytes(d, cache.block_size)), torch.uint8)
    _need(cache.block_table, "block_table", (B, cache.block_table.shape[1]), torch.int32)
    if out is None:
        out = torch.empty(lead + (d.n_heads, d.d_v), dtype=dt, device=q_nope.device)
    _need(out, "out", lead + (d.n_heads, d.d_v), dt)
    ws, nbytes = _workspace(mla_decode_fp8_workspace_size(d, B, Q, cache.max_context), q_nope.device, workspace)
    cc = cache.c()
    _ok(library().mla_decode_fp8(ctypes.byref(d.c()), B, Q, q_nope.data_ptr(), q_pe.data_ptr(), w_uk.data_ptr(),
                                 w_uv.data_ptr(), ctypes.byref(cc), out.data_ptr(),
                                 ws.data_ptr() if ws is not None else None, nbytes, _stream(stream)),
        "mla_decode_fp8")
    return out


def mla_prefill(dims, q_nope, q_pe, w_uk, w_uv, cache: Cache, out=None, workspace=None, stream=None):
    """Causal attention of the last S tokens of each sequence; returns out [B, S, H, d_v]."""
    d = Dims.of(dims)
    B, S = q_nope.shape[:2]
    dt = d.torch_dtype
    _need(q_nope, "q_nope", (B, S, d.n_heads, d.d_nope), dt)
    _need(q_pe, "q_pe", (B, S, d.n_heads, d.d_rope), dt)
    _need(w_uk, "w_uk", (d.n_heads * d.d_nope, d.d_c), dt)
    _need(w_uv, "w_uv", (d.n_heads * d.d_v, d.d_c), dt)
    _check_cache(cache, d, B)
    if out is None:
        out = torch.empty((B, S, d.n_heads, d.d_v), dtype=dt, device=q_nope.device)
    _need(out, "out", (B, S, d.n_heads, d.d_v), dt)
    ws, nbytes = _workspace(mla_prefill_workspace_size(d, B, S, cache.max_context), q_nope.device, workspace)
    cc = cache.c()
    _ok(library().mla_prefill(ctypes.byref(d.c()), B, S, q_nope.data_ptr(), q_pe.data_ptr(), w_uk.data_ptr(),
                              w_uv.data_ptr(), ctypes.byref(cc), out.data_ptr(),
                              ws.data_ptr() if ws is not None else None, nbytes, _stream(stream)), "mla_prefill")
    return out
