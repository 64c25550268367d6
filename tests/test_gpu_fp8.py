"""FP8 latent cache on the GPU, through the C ABI.

The quantiser (mla_quantize_fp8) must reproduce the oracle's FP8 pages byte
for byte. Decode over the FP8 cache (mla_decode_fp8) is compared with the
oracle's decode over the dequantised cache, the same rows the kernel reads,
within the FP8 bar of gpu_helpers.bar("fp8"); mistakes planted in the oracle
must fail that bar.
"""
import numpy as np
import pytest
import torch

import mla_latent_kv_09_amd as mla
import oracle
from oracle import fp8
from synth import Dims, f32_to_bf16_bits, from_torch, make_decode_case, to_torch, workload

from gpu_helpers import assert_parity, fails_bar, host_run_pages, one_round_run_pages

pytestmark = pytest.mark.gpu

V3 = dict(d_c=512, d_rope=64, d_nope=128, d_v=128)


def _log(msg):
    print(msg, flush=True)


def _expected_pool(rows_bits, slots, nb, bs, d_c, d_rope):
    """The oracle's FP8 pages holding rows at slots (unwritten bytes zero)."""
    codes, kbits, E = fp8.quantize_rows(oracle.widen(rows_bits), d_c)
    rb = d_c + 2 * d_rope
    pool = np.zeros((nb, fp8.page_bytes(bs, d_c, d_rope)), dtype=np.uint8)
    for r, sl in enumerate(slots):
        p, o = divmod(int(sl), bs)
        pool[p, o * rb:o * rb + d_c] = codes[r]
        pool[p, o * rb + d_c:(o + 1) * rb] = kbits[r].astype("<u2").view(np.uint8)
        pool[p, bs * rb + o] = E[r]
    return pool


def _gpu_quantize(dims, rows_bits, slots, nb, bs):
    pool = torch.zeros((nb, mla.mla_fp8_page_bytes(dims, bs)), dtype=torch.uint8, device="cuda")
    mla.mla_quantize_fp8(dims, to_torch(rows_bits), pool, to_torch(np.asarray(slots, dtype=np.int32)), bs)
    torch.cuda.synchronize()
    return pool.cpu().numpy()


@pytest.mark.parametrize("d_c,d_rope,bs,n,nb", [(512, 64, 64, 300, 6), (40, 8, 3, 50, 20), (32, 8, 16, 64, 4)])
def test_quantize_fp8_is_bit_exact_against_the_oracle(d_c, d_rope, bs, n, nb):
    _log(f"quantize fp8 d_c={d_c} d_rope={d_rope} block={bs} rows={n}")
    dims = Dims(4, d_c, d_rope, 16, 16)
    rng = np.random.default_rng(d_c + bs)
    x = rng.standard_normal((n, d_c + d_rope)).astype(np.float32)
    x *= (2.0 ** rng.integers(-30, 30, size=(n, 1))).astype(np.float32)   # very different row magnitudes
    x[0, :d_c] = 0.0                                   # all-zero block
    x[1, :d_c] = np.float32(1e-39)                     # subnormal magnitudes
    x[2, :d_c] = -0.0
    x[3, :d_c] = 448.0 * np.sign(x[3, :d_c])           # exactly the top value
    x[4, :d_c] *= np.float32(2.0 ** 100)               # large scales
    bits = f32_to_bf16_bits(x)
    slots = rng.permutation(nb * bs)[:n].astype(np.int32)
    got = _gpu_quantize(dims, bits, slots, nb, bs)
    want = _expected_pool(bits, slots, nb, bs, d_c, d_rope)
    bad = np.argwhere(got != want)
    assert len(bad) == 0, f"{len(bad)} bytes differ, first at {bad[:5].tolist()}"


def _fp8_case(case):
    """GPU FP8 pages of the case's bf16 pool, which must equal the oracle's
    pages byte for byte, and the oracle's dequantised pool (made from its own
    pages, never from the kernel's) that the oracle decodes over."""
    c = case.cache
    nb, P, R = c.pool.shape
    dims = case.dims
    slots = np.arange(nb * P, dtype=np.int32)
    got = _gpu_quantize(dims, c.pool.reshape(nb * P, R), slots, nb, P)
    want = fp8.quantize_pool(oracle.widen(c.pool), dims.d_c)
    bad = np.argwhere(got != want)
    assert len(bad) == 0, f"{len(bad)} page bytes differ from the oracle's, first at {bad[:5].tolist()}"
    return got, fp8.dequantize_pool(want, P, dims.d_c, dims.d_rope)


def _run_fp8(case, pages):
    c = case.cache
    cache = mla.Fp8Cache(to_torch(pages), to_torch(c.context_lens.astype(np.int32)), int(c.context_lens.max()),
                         to_torch(c.block_table.astype(np.int32)))
    out = mla.mla_decode_fp8(case.dims, to_torch(case.q_nope), to_torch(case.q_pe), to_torch(case.w_uk),
                             to_torch(case.w_uv), cache)
    torch.cuda.synchronize()
    return from_torch(out)


def _oracle_fp8(case, deq, seqs=None, w_uv=None, table=None, lens=None, q_pe=None):
    """Oracle decode over the dequantised pool; q_len queries per sequence as
    in multi-token decode (query j sees L - (q_len - 1 - j) rows)."""
    c = case.cache
    Q = case.q_len
    table = c.block_table if table is None else table
    lens = c.context_lens if lens is None else lens
    w_uv = case.w_uv if w_uv is None else w_uv
    qp_all = case.q_pe if q_pe is None else q_pe
    seqs = list(range(case.batch)) if seqs is None else seqs
    if Q == 1:
        return oracle.decode(case.dims, case.q_nope, qp_all, case.w_uk, w_uv, deq, table, lens, batch_rows=seqs)
    out = np.empty((len(seqs), Q, case.dims.n_heads, case.dims.d_v))
    for j in range(Q):
        out[:, j] = oracle.decode(case.dims, case.q_nope[:, j], qp_all[:, j], case.w_uk, w_uv, deq, table,
                                  lens - (Q - 1 - j), batch_rows=seqs)
    return out


SMALL = [
    ("H16 q1 ragged", 16, 1, [1, 63, 64, 65, 700], True),
    ("H128 q1 ragged", 128, 1, [1, 129, 1000], True),
    ("H128 q1 identity pages", 128, 1, [64, 2047], False),
    ("H32 q1 long", 32, 1, [5000, 3], True),
    ("H128 q1 eight rows", 128, 1, [1, 64, 65, 700, 2000, 4097, 130, 3000], True),
    ("H1", 1, 1, [129, 1, 640], True),
    ("H100", 100, 1, [129, 1, 640], True),
    ("H128 q2 pairs", 128, 2, [2, 64, 65, 127, 128, 129, 1500, 2047], True),
    ("H32 q3 few units", 32, 3, [3, 129, 700], True),
    ("H8 q64 max", 8, 64, [64, 65, 100, 300, 700, 64, 1000, 129], True),
    # more than 64 rows of one token each: the split kernel's longest-first
    # run order over several passes of 64 rows (runs of 640 tokens here)
    ("H32 q1 130 rows", 32, 1, [int(x) for x in np.random.default_rng(9).integers(1, 1100, 130)] , True),
]


@pytest.mark.parametrize("name,H,Q,lens,shuffle", SMALL, ids=[s[0] for s in SMALL])
def test_decode_fp8_small(name, H, Q, lens, shuffle):
    _log(f"decode fp8 {name}")
    case = make_decode_case(500 + H + Q, len(lens), Dims(H, **V3), lens, shuffle=shuffle, q_len=Q)
    pages, deq = _fp8_case(case)
    got = _run_fp8(case, pages)
    assert_parity(got, _oracle_fp8(case, deq), "fp8", name)
    if Q == 1:
        # with the query rounded as the kernel rounds it, only the rounding
        # of the probabilities is left: a bar twice as tight
        c = case.cache
        ref_q = fp8.fp8_query_decode(case.dims, case.q_nope, case.q_pe, case.w_uk, case.w_uv, deq, c.block_table,
                                     c.context_lens)
        assert_parity(got, ref_q, "fp8q", name + " (FP8 query)")


def test_decode_fp8_tight_bar_catches_a_skipped_page():
    """A page left out in the middle of a 3000-token context (the query keeping
    its position) moves the output by several percent: within the loose bar
    against the plain oracle (8 %) such a mistake could hide behind the
    query's E4M3 rounding, so the tight bar against the FP8-query oracle must
    reject it while the kernel passes."""
    _log("decode fp8: skipped page against the FP8-query oracle")
    case = make_decode_case(503, 2, Dims(32, **V3), [3000, 2100], shuffle=True)
    pages, deq = _fp8_case(case)
    got = _run_fp8(case, pages)
    c = case.cache
    args = (case.dims, case.q_nope, case.q_pe, case.w_uk, case.w_uv, deq, c.block_table, c.context_lens)
    assert_parity(got, fp8.fp8_query_decode(*args), "fp8q", "3000 / 2100 tokens")
    for b, page in ((0, 23), (1, 16)):
        assert fails_bar(got, fp8.fp8_query_decode(*args, drop_page=(b, page)), "fp8q"), (b, page)


def test_decode_fp8_negative_controls_fail_the_bar():
    _log("decode fp8 negative controls")
    case = make_decode_case(501, 2, Dims(16, **V3), [300, 129], shuffle=True)
    pages, deq = _fp8_case(case)
    got = _run_fp8(case, pages)
    assert_parity(got, _oracle_fp8(case, deq), "fp8", "control")
    c = case.cache
    no_kpe = deq.copy()
    no_kpe[..., 512:] = 0
    assert fails_bar(got, _oracle_fp8(case, no_kpe), "fp8")
    short = np.maximum(c.context_lens - (c.context_lens - 1) % 64 - 1, 1).astype(np.int32)
    assert fails_bar(got, _oracle_fp8(case, deq, lens=short), "fp8")
    ident = np.zeros_like(c.block_table)
    g = 0
    for b, L in enumerate(c.context_lens):
        n = (int(L) + 63) // 64
        ident[b, :n] = np.arange(g, g + n)
        g += n
    assert fails_bar(got, _oracle_fp8(case, deq, table=ident), "fp8")
    assert fails_bar(got, _oracle_fp8(case, deq, w_uv=np.roll(case.w_uv, 128, axis=0)), "fp8")
    # codes read without their token scales (every scale taken as 1)
    codes, kbits, E = fp8.unpack_pages(pages, 64, 512, 64)
    unscaled = fp8.dequantize_rows(codes, kbits, np.full_like(E, 127)).reshape(deq.shape)
    assert fails_bar(got, _oracle_fp8(case, unscaled), "fp8")


def test_decode_fp8_large_score_growth_takes_the_rescale_branch():
    _log("decode fp8 rescale branch")
    from synth import bf16_bits_to_f32
    case = make_decode_case(502, 2, Dims(128, **V3), [700, 1500], shuffle=True)
    pool = bf16_bits_to_f32(case.cache.pool)
    table = case.cache.block_table
    for b, L in enumerate(case.cache.context_lens):
        n = (int(L) + 63) // 64
        for p in range(n):
            pool[table[b, p], :, 512:] *= 1.0 + 5.0 * p / n
    case.cache.pool = f32_to_bf16_bits(pool)
    pages, deq = _fp8_case(case)
    assert_parity(_run_fp8(case, pages), _oracle_fp8(case, deq), "fp8", "rescale")


@pytest.mark.parametrize("jump", [300.0, 600.0])
def test_decode_fp8_score_jump_beyond_the_shift_field(jump):
    _log(f"decode fp8 with a score jump of {jump} log2 units inside a run")
    from gpu_helpers import score_jump_case
    case = score_jump_case(make_decode_case(505, 3, Dims(128, **V3), [300, 700, 1500], shuffle=True), jump)
    pages, deq = _fp8_case(case)
    got = _run_fp8(case, pages)
    assert np.all(np.isfinite(got))
    assert_parity(got, _oracle_fp8(case, deq), "fp8", f"jump {jump}")


def test_decode_fp8_ignores_non_finite_bytes_past_the_context():
    _log("decode fp8 with NaN codes and scales past the context")
    case = make_decode_case(503, 4, Dims(64, **V3), [1, 33, 100, 1000], shuffle=True, q_len=1)
    pages, deq = _fp8_case(case)
    poisoned = pages.copy()
    c = case.cache
    for b, L in enumerate(c.context_lens):
        L = int(L)
        if L % 64:
            p = c.block_table[b, (L - 1) // 64]
            for o in range(L % 64, 64):
                poisoned[p, o * 640:o * 640 + 512] = 0x7F          # NaN codes
                poisoned[p, o * 640 + 512:(o + 1) * 640] = 0xFF    # NaN k_pe (bf16 0xFFFF)
                poisoned[p, 64 * 640 + o] = 0xFF                   # NaN scale
    got = _run_fp8(case, poisoned)
    assert np.all(np.isfinite(got))
    assert_parity(got, _oracle_fp8(case, deq), "fp8", "poisoned tails")


def test_decode_fp8_is_deterministic():
    _log("decode fp8 determinism")
    case = make_decode_case(504, 4, Dims(128, **V3), [3000, 64, 1, 4097], shuffle=True)
    pages, _ = _fp8_case(case)
    assert np.array_equal(_run_fp8(case, pages), _run_fp8(case, pages))


def test_workload3_fp8_full_size_sampled():
    """The DeepSeek-V3 decode shape (B=64, H=128, L=8192) over an FP8 copy of
    its cache: every page quantised on the GPU, the pages of the sampled
    sequences checked against the oracle's, their outputs against the oracle."""
    _log("workload 3 over an FP8 cache: full size on the GPU, oracle on sampled sequences")
    case = workload(3)
    c = case.cache
    nb, P, R = c.pool.shape
    pages = _gpu_quantize(case.dims, c.pool.reshape(nb * P, R), np.arange(nb * P, dtype=np.int32), nb, P)
    got = _run_fp8(case, pages)
    sample = [0, 33, case.batch - 1]
    used = np.unique(np.concatenate([c.block_table[b, :(int(c.context_lens[b]) + 63) // 64] for b in sample]))
    want = fp8.quantize_pool(oracle.widen(c.pool[used]), 512)
    assert np.array_equal(pages[used], want)
    deq = np.zeros((nb, P, R))
    deq[used] = fp8.dequantize_pool(want, P, 512, 64)
    assert_parity(got[sample], _oracle_fp8(case, deq, seqs=sample), "fp8", "workload 3, fp8 cache")


def test_fp8_decode_lengthens_runs_to_fit_one_round():
    """256 rows of up to 2200 tokens: runs of 32 pages (the host's choice)
    would take 267 workgroups, so the FP8 split kernel takes runs of 34 pages
    (one round on a 256-CU device) and the combine reads that length back.
    Rows with 33 or 34 pages (one run now, two at 32) and the longest and
    shortest rows against the oracle over the oracle's own pages."""
    _log("fp8 decode with runs lengthened to fit one round")
    lens = [int(x) for x in np.random.default_rng(120).integers(1, 2201, 256)]
    case = make_decode_case(82, 256, Dims(32, **V3), lens, shuffle=True)
    c = case.cache
    nb, P, R = c.pool.shape
    pages = _gpu_quantize(case.dims, c.pool.reshape(nb * P, R), np.arange(nb * P, dtype=np.int32), nb, P)
    cache = mla.Fp8Cache(to_torch(pages), to_torch(c.context_lens.astype(np.int32)), max(lens),
                         to_torch(c.block_table.astype(np.int32)))
    n = mla.mla_decode_fp8_workspace_size(mla.Dims.of(case.dims), 256, 1, max(lens))
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    out = mla.mla_decode_fp8(case.dims, to_torch(case.q_nope), to_torch(case.q_pe), to_torch(case.w_uk),
                             to_torch(case.w_uv), cache, workspace=ws)
    torch.cuda.synchronize()
    got = from_torch(out)
    used = int(ws[n - 256:n - 252].view(torch.int32).item())
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    pps = host_run_pages(256, max(lens))
    assert used == one_round_run_pages(lens, pps, cus)
    if cus == 256:
        assert used > pps
    n_pages = [(L + 63) // 64 for L in lens]
    joined = [b for b in range(256) if pps < n_pages[b] <= used][:4]
    sample = sorted(set(joined) | {int(np.argmax(lens)), int(np.argmin(lens)), 0, 255})
    used_pages = np.unique(np.concatenate([c.block_table[b, :n_pages[b]] for b in sample]))
    want = fp8.quantize_pool(oracle.widen(c.pool[used_pages]), 512)
    assert np.array_equal(pages[used_pages], want)
    deq = np.zeros((nb, P, R))
    deq[used_pages] = fp8.dequantize_pool(want, P, 512, 64)
    assert_parity(got[sample], _oracle_fp8(case, deq, seqs=sample), "fp8", "runs lengthened to one round")


def _decode_fp8_bytes(pages, bs, d_c, d_rope):
    """Rows [n_pages * bs, d_c + d_rope] held by FP8 pages, decoded here with
    torch's float8_e4m3fn type and the scale bytes (2^(E - 127)); independent of
    the oracle's decoder."""
    t = torch.from_numpy(np.ascontiguousarray(pages))
    nb = t.shape[0]
    rb = d_c + 2 * d_rope
    body = t[:, :bs * rb].reshape(nb * bs, rb)
    codes = body[:, :d_c].contiguous().view(torch.float8_e4m3fn).to(torch.float64)
    kpe = body[:, d_c:].contiguous().view(torch.bfloat16).to(torch.float64)
    E = t[:, bs * rb:bs * rb + bs].reshape(nb * bs).to(torch.float64)
    return torch.cat([codes * torch.exp2(E - 127.0)[:, None], kpe], dim=1).numpy()


@pytest.mark.parametrize("d_model,d_q", [(512, 0), (256, 128)])
def test_project_fp8_writes_the_quantised_rows(d_model, d_q):
    """mla_rope_latent_project_fp8 gives the pages of the bf16 projection
    followed by mla_quantize_fp8, byte for byte; the rows it holds are the
    oracle's latent rows within E4M3 rounding (c_KV, relative 2^-4 of each
    token's scale) and the bf16 bar (k_pe); decode over it matches the oracle's
    decode over its own quantised rows."""
    from synth import make_project_case
    _log(f"projection into an FP8 cache d_model={d_model} d_q={d_q}")
    dims = Dims(128, **V3)
    case = make_project_case(61 + d_q, batch=2, seq_len=150, d_model=d_model, dims=dims, d_q=d_q, shuffle=True)
    T, nb = case.n_tokens, case.num_blocks
    pb = mla.mla_fp8_page_bytes(dims, 64)
    h, wd, wr = to_torch(case.h), to_torch(case.w_dkv), to_torch(case.w_kr)
    pos, slots = to_torch(case.positions), to_torch(case.slots)
    qp = None
    if d_q:
        qn = torch.empty((T, 128, 128), dtype=torch.bfloat16, device="cuda")
        qpe = torch.empty((T, 128, 64), dtype=torch.bfloat16, device="cuda")
        qp = mla.QProj(to_torch(case.w_dq), to_torch(case.w_uq), to_torch(case.w_qr), qn, qpe)
    fused = torch.zeros((nb, pb), dtype=torch.uint8, device="cuda")
    mla.mla_rope_latent_project_fp8(dims, h, wd, wr, pos, slots, fused, 64, qp)
    rows = torch.zeros((nb, 64, dims.row), dtype=torch.bfloat16, device="cuda")
    lens = torch.full((2,), 150, dtype=torch.int32, device="cuda")
    mla.mla_rope_latent_project(dims, h, wd, wr, pos, slots, mla.Cache(rows, lens, 150, to_torch(case.block_table)))
    two_step = torch.zeros((nb, pb), dtype=torch.uint8, device="cuda")
    mla.mla_quantize_fp8(dims, rows.view(nb * 64, dims.row)[slots.long()].contiguous(), two_step, slots, 64)
    torch.cuda.synchronize()
    got = fused.cpu().numpy()
    assert np.array_equal(got, two_step.cpu().numpy())
    sl = case.slots
    deq = _decode_fp8_bytes(got, 64, 512, 64)[sl]
    ref = oracle.latent_rows(case.h, case.w_dkv, case.w_kr, case.positions)
    scale = 2.0 ** (np.ceil(np.log2(np.abs(ref[:, :512]).max(axis=1) / 448.0)))[:, None]
    # E4M3 rounding (half an ulp: 2^-4 relative, 2^-10 of the scale below the
    # normal range) of a bf16 row that is itself within 2^-7 of the exact value
    assert np.all(np.abs(deq[:, :512] - ref[:, :512]) <= (2.0 ** -4 + 2.0 ** -7) * np.abs(ref[:, :512]) + 2.0 ** -9 * scale)
    assert np.all(np.abs(deq[:, 512:] - ref[:, 512:]) <= 2 ** -7 * np.abs(ref[:, 512:]) + 2e-3)
    # decode over the fused pool against the oracle's decode over its own pages
    rng = np.random.default_rng(5)
    q_nope = f32_to_bf16_bits(rng.standard_normal((2, 128, 128)).astype(np.float32))
    q_pe = f32_to_bf16_bits(rng.standard_normal((2, 128, 64)).astype(np.float32))
    dcase = make_decode_case(62, 2, dims, [150, 150])
    dcase.q_nope, dcase.q_pe = q_nope, q_pe
    dcase.cache.block_table = case.block_table
    dcase.cache.context_lens = np.array([150, 150], dtype=np.int32)
    own = np.zeros((nb, 64, dims.row))
    own.reshape(nb * 64, dims.row)[sl] = oracle.round_to(ref, "bf16")
    own_pages = fp8.quantize_pool(own, 512)
    want = _oracle_fp8(dcase, fp8.dequantize_pool(own_pages, 64, 512, 64))
    assert_parity(_run_fp8(dcase, got), want, "fp8", "decode over the projected FP8 cache")
