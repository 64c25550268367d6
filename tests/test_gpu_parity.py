"""Parity of the HIP library with the CPU oracle, through the C ABI.

Inputs are the seeded synthetic workloads; the oracle computes the plain
definition (explicit K/V up-projection, two-pass softmax) in float64. Bars:
fp32 max|d| <= 1e-4; bf16 max|d| <= 2e-2 plus normwise relative error <= 1e-2
and max|d| <= 5% of max|ref|.
"""
import numpy as np
import pytest
import torch

import mla_latent_kv_09_amd as mla
import oracle
from synth import Dims, from_torch, make_decode_case, make_project_case, to_torch, workload

from gpu_helpers import (assert_parity, assert_projection_parity, device_cache, fails_bar, host_run_pages,
                         one_round_run_pages, run_decode)

pytestmark = pytest.mark.gpu

V3 = dict(d_c=512, d_rope=64, d_nope=128, d_v=128)


def oracle_decode(case, rows=None):
    c = case.cache
    return oracle.decode(case.dims, case.q_nope, case.q_pe, case.w_uk, case.w_uv, c.pool, c.block_table,
                         c.context_lens, batch_rows=rows)


def _log(msg):
    print(msg, flush=True)


# ------------------------------------------------------------ tiny fp32 ----

def test_workload1_tiny_fp32_project_then_decode():
    _log("workload 1: tiny fp32 projection + decode")
    case = workload(1)
    d = case.dims
    rows = torch.zeros((1, 64, d.row), dtype=torch.float32, device="cuda")
    lens = torch.tensor([64], dtype=torch.int32, device="cuda")
    cache = mla.Cache(rows, lens, 64, None)
    mla.mla_rope_latent_project(d, to_torch(case.h), to_torch(case.w_dkv), to_torch(case.w_kr),
                                to_torch(case.positions), to_torch(case.slots), cache)
    out = mla.mla_decode(d, to_torch(case.q_nope), to_torch(case.q_pe), to_torch(case.w_uk),
                         to_torch(case.w_uv), cache)
    torch.cuda.synchronize()
    ref_rows = oracle.latent_rows(case.h, case.w_dkv, case.w_kr, case.positions, store="f32")
    assert np.abs(from_torch(rows)[0] - ref_rows).max() <= 1e-5
    ref = oracle.decode(d, case.q_nope, case.q_pe, case.w_uk, case.w_uv, ref_rows[None], None,
                        np.array([64], dtype=np.int32))
    assert_parity(from_torch(out), ref, "f32", "workload 1")


# --------------------------------------------------------- bf16 decode -----

SMALL = [
    ("H16 ragged tails", 16, [1, 63, 64, 65, 700], True),
    ("H128 ragged tails", 128, [1, 129, 1000], True),
    ("H128 identity pages", 128, [64, 2047], False),
    ("H32 long", 32, [5000, 3], True),
    # 8 rows of ragged length, up to 17 splits each (some past the context)
    ("H128 eight rows", 128, [1, 64, 65, 700, 2000, 4097, 130, 3000], True),
]


@pytest.mark.parametrize("name,H,lens,shuffle", SMALL, ids=[s[0] for s in SMALL])
def test_decode_small_bf16(name, H, lens, shuffle):
    _log(f"decode {name}")
    case = make_decode_case(100 + H, len(lens), Dims(H, **V3), lens, shuffle=shuffle)
    assert_parity(run_decode(case), oracle_decode(case), "bf16", name)


def test_decode_tiny_dims_bf16_and_f32():
    for dt in ("bf16", "f32"):
        for H, dc, dr, dn, dv, lens in ((3, 8, 8, 5, 7, [1, 9]), (5, 40, 16, 24, 8, [130, 64, 65])):
            _log(f"decode tiny dims {dt} H={H} dc={dc}")
            case = make_decode_case(7, len(lens), Dims(H, dc, dr, dn, dv, dtype=dt), lens, shuffle=True,
                                    w_std=0.5)
            assert_parity(run_decode(case), oracle_decode(case), dt, f"tiny {dt}")


def test_decode_contiguous_layout_bf16():
    _log("decode contiguous layout")
    case = make_decode_case(8, 3, Dims(16, **V3), [100, 1, 77], paged=False)
    assert_parity(run_decode(case), oracle_decode(case), "bf16", "contiguous")


def test_decode_negative_controls_fail_the_bar():
    """Mistakes planted in the oracle (on the CPU) must fail the bar against
    the GPU output, which proves the bar can fail."""
    _log("negative controls")
    lens = [300, 129]
    case = make_decode_case(9, 2, Dims(16, **V3), lens, shuffle=True)
    got = run_decode(case)
    ref = oracle_decode(case)
    assert_parity(got, ref, "bf16", "control")
    c = case.cache
    # k_pe dropped
    pool = c.pool.copy()
    pool[..., 512:] = 0
    bad = oracle.decode(case.dims, case.q_nope, case.q_pe, case.w_uk, case.w_uv, pool, c.block_table,
                        c.context_lens)
    assert fails_bar(got, bad, "bf16")
    # last page skipped
    short = (c.context_lens - (c.context_lens - 1) % 64 - 1).astype(np.int32)
    short = np.maximum(short, 1)
    bad = oracle.decode(case.dims, case.q_nope, case.q_pe, case.w_uk, case.w_uv, c.pool, c.block_table, short)
    assert fails_bar(got, bad, "bf16")
    # block table ignored (identity placement)
    ident = np.zeros_like(c.block_table)
    g = 0
    for b, L in enumerate(c.context_lens):
        n = (int(L) + 63) // 64
        ident[b, :n] = np.arange(g, g + n)
        g += n
    bad = oracle.decode(case.dims, case.q_nope, case.q_pe, case.w_uk, case.w_uv, c.pool, ident, c.context_lens)
    assert fails_bar(got, bad, "bf16")
    # query rotated at L instead of L-1: shift q_pe by one more position
    qpe = oracle.rope(oracle.widen(case.q_pe), 1)
    bad = oracle.decode(case.dims, case.q_nope, qpe, case.w_uk, case.w_uv, c.pool, c.block_table, c.context_lens)
    assert fails_bar(got, bad, "bf16")
    # W_UV of the wrong head
    wuv = np.roll(case.w_uv, 128, axis=0)
    bad = oracle.decode(case.dims, case.q_nope, case.q_pe, case.w_uk, wuv, c.pool, c.block_table, c.context_lens)
    assert fails_bar(got, bad, "bf16")


def test_decode_is_deterministic():
    _log("determinism")
    case = make_decode_case(10, 4, Dims(128, **V3), [3000, 64, 1, 4097], shuffle=True)
    a = run_decode(case)
    b = run_decode(case)
    assert np.array_equal(a, b)


# ------------------------------------------------------- projection --------

def test_project_with_query_path_then_prefill_small():
    _log("projection + query path + prefill (small)")
    dims = Dims(16, **V3)
    case = make_project_case(11, batch=2, seq_len=100, d_model=256, dims=dims, d_q=96, shuffle=True)
    T = case.n_tokens
    nb = case.num_blocks
    rows = torch.zeros((nb, 64, dims.row), dtype=torch.bfloat16, device="cuda")
    lens = torch.full((2,), 100, dtype=torch.int32, device="cuda")
    cache = mla.Cache(rows, lens, 100, to_torch(case.block_table))
    qn = torch.empty((T, 16, 128), dtype=torch.bfloat16, device="cuda")
    qp = torch.empty((T, 16, 64), dtype=torch.bfloat16, device="cuda")
    qproj = mla.QProj(to_torch(case.w_dq), to_torch(case.w_uq), to_torch(case.w_qr), qn, qp)
    mla.mla_rope_latent_project(dims, to_torch(case.h), to_torch(case.w_dkv), to_torch(case.w_kr),
                                to_torch(case.positions), to_torch(case.slots), cache, qproj)
    out = mla.mla_prefill(dims, qn.view(2, 100, 16, 128), qp.view(2, 100, 16, 64), to_torch(case.w_uk),
                          to_torch(case.w_uv), cache)
    torch.cuda.synchronize()
    ref_rows = oracle.latent_rows(case.h, case.w_dkv, case.w_kr, case.positions)
    got_rows = from_torch(rows)[case.slots // 64, case.slots % 64]
    # rows are stored in bf16: allow one bf16 rounding step of the fp64 value
    assert np.all(np.abs(got_rows - ref_rows) <= 2 ** -7 * np.abs(ref_rows) + 1e-3)
    ref_qn, ref_qp = oracle.query_projection(case.h, case.w_dq, case.w_uq, case.w_qr, 16, 128, 64)
    assert_projection_parity(from_torch(qn), ref_qn, "q_nope")
    assert_projection_parity(from_torch(qp), ref_qp, "q_pe")
    ref = oracle.prefill(dims, ref_qn.reshape(2, 100, 16, 128), ref_qp.reshape(2, 100, 16, 64), case.w_uk,
                         case.w_uv, oracle.round_to(ref_rows, "bf16").reshape(2, 100, -1))
    assert_parity(from_torch(out), ref, "bf16", "prefill")


@pytest.mark.parametrize("H", [16, 256])
def test_chunked_prefill_over_a_cached_prefix(H):
    """Queries that are the last S tokens of a longer context see the prefix
    (256: the largest head count the library accepts)."""
    _log(f"chunked prefill H={H}")
    dims = Dims(H, **V3)
    L, S = 300, 70
    case = make_decode_case(12, 2, dims, [L, L], shuffle=True)
    rng = np.random.default_rng(3)
    from synth import f32_to_bf16_bits
    qn = f32_to_bf16_bits(rng.standard_normal((2, S, H, 128)).astype(np.float32))
    qp = f32_to_bf16_bits(rng.standard_normal((2, S, H, 64)).astype(np.float32))
    c = device_cache(case.cache)
    out = mla.mla_prefill(dims, to_torch(qn), to_torch(qp), to_torch(case.w_uk), to_torch(case.w_uv), c)
    torch.cuda.synchronize()
    got = from_torch(out)
    for s in (0, 1, 63, 64, 69):
        lens = np.array([L - S + s + 1] * 2, dtype=np.int32)
        ref = oracle.decode(dims, qn[:, s], qp[:, s], case.w_uk, case.w_uv, case.cache.pool,
                            case.cache.block_table, lens)
        assert_parity(got[:, s], ref, "bf16", f"chunked query {s}")


# ------------------------------------------------- measured workloads ------

def test_workload2_full():
    _log("workload 2 (B=16 H=16 L=4096), all sequences")
    case = workload(2)
    assert_parity(run_decode(case), oracle_decode(case), "bf16", "workload 2")


@pytest.mark.parametrize("k", [3, 4])
def test_workload_3_4_full_size_sampled(k):
    _log(f"workload {k}: full size on the GPU, oracle on sampled sequences")
    case = workload(k)
    got = run_decode(case)
    lens = case.cache.context_lens
    sample = sorted({0, int(np.argmax(lens)), int(np.argmin(lens)), case.batch - 1})
    assert_parity(got[sample], oracle_decode(case, rows=sample), "bf16", f"workload {k}")


# ------------------------------------------------- MFMA path specifics -----

def test_mfma_path_is_selected_for_the_v3_shape():
    assert mla.mla_decode_path(Dims(128, **V3)) == 1
    assert mla.mla_decode_path(Dims(16, **V3)) == 1
    assert mla.mla_decode_path(Dims(16, **V3), paged=False) == 0
    assert mla.mla_decode_path(Dims(4, 32, 8, 16, 16, dtype="f32")) == 0


def test_decode_at_the_longest_context_of_the_fast_path():
    """One sequence of 2^20 - 5 tokens: 16384 pages, the most the MFMA decode
    takes (runs of 64 pages, one page number per lane; 256 splits, the most
    the combine merges), with a ragged last page and shuffled pages. Checked
    against the oracle's absorbed form (pinned equal to the explicit one),
    which never forms the 2^20 x 128 keys per head."""
    _log("decode at the longest fast-path context: B=1 H=16 L=2^20-5")
    case = make_decode_case(61, 1, Dims(16, **V3), [(1 << 20) - 5], shuffle=True)
    assert mla.mla_decode_path(case.dims) == 1
    # a workspace is needed only on the MFMA path (the generic kernel takes none)
    assert mla.mla_decode_workspace_size(mla.Dims.of(case.dims), 1, (1 << 20) - 5) > 0
    got = run_decode(case)
    _log("  GPU done, oracle (absorbed form)")
    c = case.cache
    ref = oracle.absorbed_decode(case.dims, case.q_nope, case.q_pe, case.w_uk, case.w_uv, c.pool, c.block_table,
                                 c.context_lens)
    assert_parity(got, ref, "bf16", "L = 2^20 - 5")


def _ragged_lens(seed, n, hi, exact=()):
    lens = np.random.default_rng(seed).integers(1, hi + 1, n)
    for i, v in enumerate(exact):
        lens[7 * i + 3] = v
    return [int(x) for x in lens]


# With one new token per row and at most 256 rows, the split kernels take a
# step's runs longest first: every full run (row by row), then the rows'
# shorter last runs by decreasing length. The order is worked out from the
# context lengths in passes of 64 rows; these batches need several passes,
# mix rows with full runs only (a context that is a whole number of runs),
# last runs only and both, and take more than one round of the chip. Every
# row is checked (against the absorbed oracle, pinned equal to the explicit
# one): a run taken twice or never would show in some row. Runs are of
# pps * 64 tokens, with pps = clamp(ceil(rows * max_pages / 256), 4, 32).
RUN_ORDER = [
    # rows, H, contexts: 130 rows, pps 13 (runs of 832 tokens)
    ("130 rows H128", 130, 128, _ragged_lens(71, 130, 1600, exact=(832, 1600, 831))),
    # 200 rows, pps 32 (runs of 2048 tokens)
    ("200 rows H16", 200, 16, _ragged_lens(72, 200, 4000, exact=(2048, 4000, 1))),
    # 256 rows, the most in this order; pps 32 (runs of 2048 tokens)
    ("256 rows H48", 256, 48, _ragged_lens(73, 256, 3000, exact=(2048, 3000, 2047, 2049))),
    # 300 rows: plain row order (pps 13, one run per row)
    ("300 rows H16 plain order", 300, 16, _ragged_lens(74, 300, 700, exact=(256, 700))),
]


@pytest.mark.parametrize("name,rows,H,lens", RUN_ORDER, ids=[r[0] for r in RUN_ORDER])
def test_decode_run_order_covers_every_run_once(name, rows, H, lens):
    _log(f"decode, run order: {name}")
    case = make_decode_case(80 + rows, rows, Dims(H, **V3), lens, shuffle=True)
    assert mla.mla_decode_path(case.dims) == 1
    got = run_decode(case)
    c = case.cache
    ref = oracle.absorbed_decode(case.dims, case.q_nope, case.q_pe, case.w_uk, case.w_uv, c.pool, c.block_table,
                                 c.context_lens)
    assert_parity(got, ref, "bf16", name)


# Runs a little longer than the host's choice. The host sets pps from the
# longest context alone; when the actual contexts then cut into a few more
# runs than the chip has compute units (one split workgroup each), the split
# kernel lengthens the runs by up to a quarter so that they fit one round,
# and the combine reads the length it used (from the workspace's last 256
# bytes). These batches take that path on a 256-CU device.
LONGER_RUNS = [
    # 230 rows: pps 28 gives 257 runs, 29 gives 246
    ("230 rows H16", 230, 16, _ragged_lens(214, 230, 2000)),
    # 256 rows: pps 32 (the cap) gives 267 runs, 34 gives 256
    ("256 rows H32", 256, 32, _ragged_lens(120, 256, 2200)),
    # two head groups (128 + 72 heads), so a round is half the CUs per group:
    # pps 4 gives 129 runs, 5 gives 108
    ("51 rows H200", 51, 200, _ragged_lens(1875, 51, 1000)),
]


@pytest.mark.parametrize("name,rows,H,lens", LONGER_RUNS, ids=[r[0] for r in LONGER_RUNS])
def test_decode_lengthens_runs_to_fit_one_round(name, rows, H, lens):
    _log(f"decode with runs lengthened to fit one round: {name}")
    case = make_decode_case(81, rows, Dims(H, **V3), lens, shuffle=True)
    n = mla.mla_decode_workspace_size(mla.Dims.of(case.dims), rows, max(lens))
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    got = run_decode(case, workspace=ws)
    used = int(ws[n - 256:n - 252].view(torch.int32).item())
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    pps = host_run_pages(rows, max(lens))
    assert used == one_round_run_pages(lens, pps, cus // ((H + 127) // 128))  # a round per head group
    if cus == 256:
        assert used > pps
    c = case.cache
    ref = oracle.absorbed_decode(case.dims, case.q_nope, case.q_pe, case.w_uk, case.w_uv, c.pool, c.block_table,
                                 c.context_lens)
    assert_parity(got, ref, "bf16", name)


@pytest.mark.parametrize("H", [1, 48, 100, 129, 256])
def test_decode_odd_head_counts(H):
    """Every head count the library accepts (1 .. 256) runs on the MFMA path;
    above 128 the split kernel runs head groups of 128 (129: a second group
    of one head; 256: two full groups)."""
    _log(f"decode H={H}")
    case = make_decode_case(200 + H, 3, Dims(H, **V3), [129, 1, 640], shuffle=True)
    assert mla.mla_decode_path(case.dims) == 1
    assert_parity(run_decode(case), oracle_decode(case), "bf16", f"H={H}")


def test_decode_large_score_growth_takes_the_rescale_branch():
    """The k_pe slice of later pages is scaled up (1x -> 6x along the context),
    so the running max of the scores grows far beyond the lazy-rescale
    threshold inside one page run, while the values (c_KV) keep their scale."""
    _log("decode rescale branch")
    from synth import bf16_bits_to_f32, f32_to_bf16_bits
    case = make_decode_case(13, 2, Dims(128, **V3), [700, 1500], shuffle=True)
    pool = bf16_bits_to_f32(case.cache.pool)
    table = case.cache.block_table
    for b, L in enumerate(case.cache.context_lens):
        n = (int(L) + 63) // 64
        for p in range(n):
            pool[table[b, p], :, 512:] *= 1.0 + 5.0 * p / n
    case.cache.pool = f32_to_bf16_bits(pool)
    assert_parity(run_decode(case), oracle_decode(case), "bf16", "rescale")


@pytest.mark.parametrize("jump", [300.0, 600.0])
def test_decode_score_jump_beyond_the_shift_field(jump):
    """Scores that jump by more than 255 log2 units inside one page run: the
    first pages of each sequence score about `jump` below the rest, so the
    lazy reference is reset to the new max instead of moved by k."""
    _log(f"decode with a score jump of {jump} log2 units inside a run")
    from gpu_helpers import score_jump_case
    case = score_jump_case(make_decode_case(14, 3, Dims(128, **V3), [300, 700, 1500], shuffle=True), jump)
    got = run_decode(case)
    assert np.all(np.isfinite(got))
    assert_parity(got, oracle_decode(case), "bf16", f"jump {jump}")


def _poison_tails(case):
    """Fills every cache row past a sequence's context in its last page with
    NaN or infinity bit patterns, as a reused page may hold."""
    c = case.cache
    for b, L in enumerate(c.context_lens):
        L = int(L)
        if L % 64:
            page = c.block_table[b, (L - 1) // 64]
            c.pool[page, L % 64:, :] = (0x7FC0, 0x7F80, 0xFF80)[b % 3]


def test_decode_ignores_non_finite_rows_past_the_context():
    _log("decode with NaN/Inf rows past the context")
    case = make_decode_case(44, 4, Dims(128, **V3), [1, 33, 100, 1000], shuffle=True)
    _poison_tails(case)
    got = run_decode(case)
    assert np.all(np.isfinite(got))
    assert_parity(got, oracle_decode(case), "bf16", "poisoned tails")


# rows with fewer page runs than the launch has splits, with one or several
# groups of splits in the combine, at 4 and 16 query rows per combine block
NAN_WS = [
    ("H16 ragged tails", 16, [1, 63, 64, 65, 700]),
    ("H128 ragged tails", 128, [1, 129, 1000]),
    ("H32 long", 32, [5000, 3]),
    ("H128 eight rows", 128, [1, 64, 65, 700, 2000, 4097, 130, 3000]),
]


@pytest.mark.parametrize("name,H,lens", NAN_WS, ids=[c[0] for c in NAN_WS])
def test_decode_with_a_nan_filled_workspace(name, H, lens):
    """The split partials of runs past a row's context are never written, so
    they hold whatever the workspace held before; filled with NaN bytes here,
    they must not reach the output."""
    _log(f"decode over a NaN-filled workspace: {name}")
    case = make_decode_case(46, len(lens), Dims(H, **V3), lens, shuffle=True)
    n = mla.mla_decode_workspace_size(mla.Dims.of(case.dims), len(lens), max(lens))
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")
    got = run_decode(case, workspace=ws)
    assert np.all(np.isfinite(got))
    assert_parity(got, oracle_decode(case), "bf16", name)


def test_chunked_prefill_ignores_non_finite_rows_past_the_context():
    _log("chunked prefill with NaN/Inf rows past the context")
    dims = Dims(16, **V3)
    case = make_decode_case(45, 3, dims, [70, 129, 200], shuffle=True)
    _poison_tails(case)
    S = 70
    rng = np.random.default_rng(4)
    from synth import f32_to_bf16_bits
    qn = f32_to_bf16_bits(rng.standard_normal((3, S, 16, 128)).astype(np.float32))
    qp = f32_to_bf16_bits(rng.standard_normal((3, S, 16, 64)).astype(np.float32))
    out = mla.mla_prefill(dims, to_torch(qn), to_torch(qp), to_torch(case.w_uk), to_torch(case.w_uv),
                          device_cache(case.cache))
    torch.cuda.synchronize()
    got = from_torch(out)
    assert np.all(np.isfinite(got))
    lens0 = case.cache.context_lens
    for s in (0, 37, 69):
        lens = lens0 - (S - 1 - s)
        ref = oracle.decode(dims, qn[:, s], qp[:, s], case.w_uk, case.w_uv, case.cache.pool, case.cache.block_table,
                            lens)
        assert_parity(got[:, s], ref, "bf16", f"poisoned tails, query {s}")


# ---------------------------------------------------- multi-token decode --

def oracle_multi(case, seqs=None):
    """Query j of q_len sits at position L - q_len + j: the oracle's decode of
    that single query over the first L - (q_len - 1 - j) cached tokens."""
    c = case.cache
    Q = case.q_len
    seqs = list(range(case.batch)) if seqs is None else seqs
    out = np.empty((len(seqs), Q, case.dims.n_heads, case.dims.d_v))
    for j in range(Q):
        lens = c.context_lens - (Q - 1 - j)
        out[:, j] = oracle.decode(case.dims, case.q_nope[:, j], case.q_pe[:, j], case.w_uk, case.w_uv, c.pool,
                                  c.block_table, lens, batch_rows=seqs)
    return out


def run_multi(case):
    c = device_cache(case.cache)
    out = mla.mla_decode_multi(case.dims, to_torch(case.q_nope), to_torch(case.q_pe), to_torch(case.w_uk),
                               to_torch(case.w_uv), c)
    torch.cuda.synchronize()
    return from_torch(out)


MULTI = [
    # 8 sequences: (sequence, split) units a multiple of 8, so the q_len rows of a unit share an XCD
    ("H16 q2 ragged", 16, 2, [2, 3, 63, 64, 65, 130, 700, 1000], True),
    ("H128 q4 ragged", 128, 4, [4, 64, 65, 127, 128, 129, 1500, 2047], True),
    # 3 sequences of at most 11 pages: 3 splits, 9 units, plain block order
    ("H128 q3 few units", 128, 3, [3, 129, 700], True),
    ("H32 q7 long", 32, 7, [5000, 7], True),
    ("H128 q2 identity pages", 128, 2, [64, 2047], False),
    # the largest q_len the library accepts; 8 sequences, so paired XCD order
    ("H8 q64 max", 8, 64, [64, 65, 100, 300, 700, 64, 1000, 129], True),
    # two head groups of the split kernel, the second one partial
    ("H200 q2 head groups", 200, 2, [2, 64, 700, 1500], True),
]


@pytest.mark.parametrize("name,H,Q,lens,shuffle", MULTI, ids=[m[0] for m in MULTI])
def test_decode_multi_small_bf16(name, H, Q, lens, shuffle):
    _log(f"multi-token decode {name}")
    case = make_decode_case(300 + H + Q, len(lens), Dims(H, **V3), lens, shuffle=shuffle, q_len=Q)
    assert_parity(run_multi(case), oracle_multi(case), "bf16", name)


def test_decode_multi_ignores_non_finite_rows_past_the_context():
    _log("multi-token decode with NaN/Inf rows past the context")
    case = make_decode_case(46, 8, Dims(32, **V3), [3, 40, 64, 65, 97, 200, 513, 1000], shuffle=True, q_len=3)
    _poison_tails(case)
    got = run_multi(case)
    assert np.all(np.isfinite(got))
    assert_parity(got, oracle_multi(case), "bf16", "poisoned tails")


def test_decode_multi_q1_matches_decode_bitwise():
    _log("multi-token decode with q_len 1 is mla_decode")
    case = make_decode_case(41, 5, Dims(64, **V3), [1, 64, 300, 999, 4000], shuffle=True)
    got = run_decode(case)
    c = device_cache(case.cache)
    multi = mla.mla_decode_multi(case.dims, to_torch(case.q_nope)[:, None], to_torch(case.q_pe)[:, None],
                                 to_torch(case.w_uk), to_torch(case.w_uv), c)
    torch.cuda.synchronize()
    assert np.array_equal(from_torch(multi)[:, 0], got)


def test_decode_multi_fp32_generic_path():
    _log("multi-token decode, fp32 generic kernels")
    dims = Dims(4, 32, 8, 16, 16, dtype="f32")
    case = make_decode_case(42, 3, dims, [3, 70, 200], shuffle=True, q_len=3)
    assert mla.mla_decode_path(dims) == 0
    assert_parity(run_multi(case), oracle_multi(case), "f32", "fp32 q_len 3")


def test_decode_multi_short_context_gives_zeros():
    """A context shorter than q_len leaves the earliest queries with no
    visible token: their outputs are zero, the others are normal."""
    _log("multi-token decode, context shorter than q_len")
    case = make_decode_case(43, 2, Dims(16, **V3), [2, 300], shuffle=True, q_len=4)
    got = run_multi(case)
    assert np.all(got[0, :2] == 0.0)
    ref = oracle_multi(case, seqs=[1])
    assert_parity(got[1:], ref, "bf16", "normal sequence")
    c = case.cache
    for j in (2, 3):
        lens = c.context_lens - (3 - j)
        r = oracle.decode(case.dims, case.q_nope[:, j], case.q_pe[:, j], case.w_uk, case.w_uv, c.pool,
                          c.block_table, lens, batch_rows=[0])
        assert_parity(got[0, j][None], r, "bf16", f"short sequence, query {j}")


def test_workload6_two_token_decode_full_size_sampled():
    _log("workload 6 (B=64 q_len=2 H=128 L=8192): full size on the GPU, oracle on sampled sequences")
    case = workload(6)
    got = run_multi(case)
    sample = [0, 37, case.batch - 1]
    assert_parity(got[sample], oracle_multi(case, seqs=sample), "bf16", "workload 6")


# ------------------------------------------------ MFMA projection/prefill --

def _project_and_prefill(case, dims, d_q):
    """Runs the latent + query projection and causal prefill on the GPU;
    returns (rows gathered in token order, q_nope, q_pe, out) as float64."""
    B, S, T = case.batch, case.seq_len, case.n_tokens
    H = dims.n_heads
    rows = torch.zeros((case.num_blocks, 64, dims.row), dtype=torch.bfloat16, device="cuda")
    lens = torch.full((B,), S, dtype=torch.int32, device="cuda")
    cache = mla.Cache(rows, lens, S, to_torch(case.block_table))
    qn = torch.empty((T, H, dims.d_nope), dtype=torch.bfloat16, device="cuda")
    qp = torch.empty((T, H, dims.d_rope), dtype=torch.bfloat16, device="cuda")
    qproj = mla.QProj(to_torch(case.w_dq), to_torch(case.w_uq), to_torch(case.w_qr), qn, qp)
    mla.mla_rope_latent_project(dims, to_torch(case.h), to_torch(case.w_dkv), to_torch(case.w_kr),
                                to_torch(case.positions), to_torch(case.slots), cache, qproj)
    out = mla.mla_prefill(dims, qn.view(B, S, H, dims.d_nope), qp.view(B, S, H, dims.d_rope),
                          to_torch(case.w_uk), to_torch(case.w_uv), cache)
    torch.cuda.synchronize()
    got_rows = from_torch(rows)[case.slots // 64, case.slots % 64]
    return got_rows, from_torch(qn), from_torch(qp), from_torch(out)


def _check_rows(got_rows, ref_rows):
    # one bf16 rounding of the fp64 value, plus accumulation-order slack
    assert np.all(np.abs(got_rows - ref_rows) <= 2 ** -7 * np.abs(ref_rows) + 2e-3), \
        float(np.abs(got_rows - ref_rows).max())


@pytest.mark.parametrize("batch,seq_len", [(2, 7000), (2, 8192)])
def test_latent_projection_192_wide_tiles(batch, seq_len):
    """Latent projection over 14,000 and 16,384 tokens (N = 576): these take
    the 256 x 192 GEMM tiles (one round of 55 or 64 row tiles x 3 column tiles
    instead of two rounds of 128-wide tiles), the first with a ragged last row
    tile in plain order, the second with the column tiles of each row tile on
    one XCD. Every cache row is compared with the oracle, RoPE at positions up
    to 8191 included."""
    _log(f"latent projection, 256 x 192 tiles, B={batch} S={seq_len}")
    dims = Dims(128, **V3)
    case = make_project_case(60 + seq_len % 7, batch=batch, seq_len=seq_len, d_model=256, dims=dims,
                             shuffle=True, draw_query=False)
    rows = torch.full((case.num_blocks, 64, dims.row), 3.0, dtype=torch.bfloat16, device="cuda")
    lens = torch.full((batch,), seq_len, dtype=torch.int32, device="cuda")
    cache = mla.Cache(rows, lens, seq_len, to_torch(case.block_table))
    mla.mla_rope_latent_project(dims, to_torch(case.h), to_torch(case.w_dkv), to_torch(case.w_kr),
                                to_torch(case.positions), to_torch(case.slots), cache)
    torch.cuda.synchronize()
    got_rows = from_torch(rows)[case.slots // 64, case.slots % 64]
    _check_rows(got_rows, oracle.latent_rows(case.h, case.w_dkv, case.w_kr, case.positions))


def test_mfma_projection_and_prefill_ragged():
    _log("MFMA projection + prefill, B=2 S=300 H=128")
    dims = Dims(128, **V3)
    assert mla.mla_prefill_path(dims) == 1
    case = make_project_case(31, batch=2, seq_len=300, d_model=512, dims=dims, d_q=256, shuffle=True)
    got_rows, qn, qp, out = _project_and_prefill(case, dims, 256)
    ref_rows = oracle.latent_rows(case.h, case.w_dkv, case.w_kr, case.positions)
    _check_rows(got_rows, ref_rows)
    ref_qn, ref_qp = oracle.query_projection(case.h, case.w_dq, case.w_uq, case.w_qr, 128, 128, 64)
    assert_projection_parity(qn, ref_qn, "q_nope")
    assert_projection_parity(qp, ref_qp, "q_pe")
    queries = [(0, 0), (0, 1), (0, 63), (0, 64), (0, 127), (0, 128), (1, 200), (1, 255), (1, 256), (1, 299)]
    ref = oracle.prefill(dims, oracle.round_to(ref_qn, "bf16").reshape(2, 300, 128, 128),
                         oracle.round_to(ref_qp, "bf16").reshape(2, 300, 128, 64), case.w_uk, case.w_uv,
                         oracle.round_to(ref_rows, "bf16").reshape(2, 300, -1), queries=queries)
    got = out.reshape(2, 300, 128, 128)[[b for b, _ in queries], [s for _, s in queries]]
    assert_parity(got, ref, "bf16", "prefill")


def test_wide_gemm_tiles_projection_and_prefill():
    """4200 tokens at H = 128: the query up-projection (N = 24576, 17 x 96
    tiles of 256 x 256) and the K/V up-projections of prefill (N = 16384, 17 x
    64 tiles) take the 256 x 256 GEMM tiles, with a ragged last row tile.
    q_nope and q_pe are compared element by element; the prefill output on
    sampled queries whose keys span every row tile."""
    _log("wide GEMM tiles: projection + prefill, B=1 S=4200 H=128")
    dims = Dims(128, **V3)
    S = 4200
    case = make_project_case(32, batch=1, seq_len=S, d_model=512, dims=dims, d_q=256, shuffle=True)
    got_rows, qn, qp, out = _project_and_prefill(case, dims, 256)
    ref_rows = oracle.latent_rows(case.h, case.w_dkv, case.w_kr, case.positions)
    _check_rows(got_rows, ref_rows)
    ref_qn, ref_qp = oracle.query_projection(case.h, case.w_dq, case.w_uq, case.w_qr, 128, 128, 64)
    assert_projection_parity(qn, ref_qn, "q_nope")
    assert_projection_parity(qp, ref_qp, "q_pe")
    picks = [0, 255, 256, 2047, 4096, S - 1]
    ref = oracle.prefill(dims, oracle.round_to(ref_qn, "bf16").reshape(1, S, 128, 128),
                         oracle.round_to(ref_qp, "bf16").reshape(1, S, 128, 64), case.w_uk, case.w_uv,
                         oracle.round_to(ref_rows, "bf16").reshape(1, S, -1), queries=[(0, s) for s in picks])
    got = out.reshape(1, S, 128, 128)[0, picks]
    assert_parity(got, ref, "bf16", "prefill")


@pytest.mark.parametrize("H,d_nope,d_rope", [(3, 10, 8), (8, 5, 8), (5, 12, 8), (5, 8, 16)])
def test_projection_with_odd_head_widths(H, d_nope, d_rope):
    """Query path with per-head widths whose column groups do not line up with
    the MFMA epilogue's 4- and 8-column stores: H*d_nope not a multiple of 8
    takes the generic kernels; (8, 5, 8) and (5, 8, 16) take the MFMA path
    with odd per-head widths or head counts."""
    _log(f"projection H={H} d_nope={d_nope} d_rope={d_rope}")
    dims = Dims(H, 64, d_rope, d_nope, 16)
    case = make_project_case(41 + H, batch=2, seq_len=70, d_model=128, dims=dims, d_q=64, shuffle=True)
    T, nb = case.n_tokens, case.num_blocks
    rows = torch.zeros((nb, 64, dims.row), dtype=torch.bfloat16, device="cuda")
    cache = mla.Cache(rows, torch.full((2,), 70, dtype=torch.int32, device="cuda"), 70, to_torch(case.block_table))
    # one guard row past each output, which no call may touch
    qn = torch.full((T * H * d_nope + 64,), 7.0, dtype=torch.bfloat16, device="cuda")
    qp = torch.full((T * H * d_rope + 64,), 7.0, dtype=torch.bfloat16, device="cuda")
    qproj = mla.QProj(to_torch(case.w_dq), to_torch(case.w_uq), to_torch(case.w_qr),
                      qn[:T * H * d_nope].view(T, H, d_nope), qp[:T * H * d_rope].view(T, H, d_rope))
    mla.mla_rope_latent_project(dims, to_torch(case.h), to_torch(case.w_dkv), to_torch(case.w_kr),
                                to_torch(case.positions), to_torch(case.slots), cache, qproj)
    torch.cuda.synchronize()
    got_n, got_p = from_torch(qn), from_torch(qp)
    assert np.all(got_n[T * H * d_nope:] == 7.0) and np.all(got_p[T * H * d_rope:] == 7.0)
    ref_qn, ref_qp = oracle.query_projection(case.h, case.w_dq, case.w_uq, case.w_qr, H, d_nope, d_rope)
    assert_projection_parity(got_n[:T * H * d_nope].reshape(T, H, d_nope), ref_qn, "q_nope")
    assert_projection_parity(got_p[:T * H * d_rope].reshape(T, H, d_rope), ref_qp, "q_pe")
    ref_rows = oracle.latent_rows(case.h, case.w_dkv, case.w_kr, case.positions)
    _check_rows(from_torch(rows)[case.slots // 64, case.slots % 64], ref_rows)


def test_workload5_full_size_sampled():
    _log("workload 5: B=4 S=4096 d_model=7168 projection + prefill, oracle on sampled queries")
    case = workload(5)
    dims = case.dims
    got_rows, qn, qp, out = _project_and_prefill(case, dims, 1536)
    S = case.seq_len
    sample_b = 2
    tok = slice(sample_b * S, (sample_b + 1) * S)
    ref_rows = oracle.latent_rows(case.h[tok], case.w_dkv, case.w_kr, case.positions[tok])
    _check_rows(got_rows[tok], ref_rows)
    picks = [0, 1, 777, 2048, S - 1]
    ids = [sample_b * S + s for s in picks]
    ref_qn, ref_qp = oracle.query_projection(case.h[ids], case.w_dq, case.w_uq, case.w_qr, 128, 128, 64)
    assert_projection_parity(qn[ids], ref_qn, "q_nope")
    assert_projection_parity(qp[ids], ref_qp, "q_pe")
    qn_full = np.zeros((1, S, 128, 128))
    qp_full = np.zeros((1, S, 128, 64))
    qn_full[0, picks] = oracle.round_to(ref_qn, "bf16")
    qp_full[0, picks] = oracle.round_to(ref_qp, "bf16")
    ref = oracle.prefill(dims, qn_full, qp_full, case.w_uk, case.w_uv, oracle.round_to(ref_rows, "bf16")[None],
                         queries=[(0, s) for s in picks])
    got = out.reshape(4, S, 128, 128)[sample_b, picks]
    assert_parity(got, ref, "bf16", "workload 5 prefill")
