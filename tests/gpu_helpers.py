"""Shared helpers of the GPU tests: device copies of generated cases, calls
through the binding, and the acceptance bars."""
import numpy as np
import torch

import mla_latent_kv_09_amd as mla
from synth import from_torch, to_torch


def device_cache(cache, device="cuda"):
    rows = to_torch(cache.pool, device)
    lens = to_torch(cache.context_lens.astype(np.int32), device)
    table = None if cache.block_table is None else to_torch(cache.block_table.astype(np.int32), device)
    return mla.Cache(rows, lens, int(cache.context_lens.max()), table)


def run_decode(case, device="cuda", workspace=None):
    c = device_cache(case.cache, device)
    out = mla.mla_decode(case.dims, to_torch(case.q_nope, device), to_torch(case.q_pe, device),
                         to_torch(case.w_uk, device), to_torch(case.w_uv, device), c, workspace=workspace)
    torch.cuda.synchronize()
    return from_torch(out)


def bar(dtype):
    """(max-abs, normwise-relative, max-abs relative to max|ref|) bars.

    "fp8" is decode over an FP8 cache against the oracle's decode over the
    same (dequantised) cache: the kernel also rounds the absorbed query and
    the probabilities to E4M3, whose unit roundoff is 2^-4. Each score then
    carries a relative error of about 2^-4 / sqrt(3) of its spread and each
    weight the same again, so the output's normwise error sits near 3 %
    (measured 2-4 % on the oracle with those roundings); the bar allows
    8 % = 1.3 * 2^-4, and 15 % of max|ref| for the largest element. There is
    no absolute bar: short contexts have outputs near 1.

    "fp8q" is the same decode against the oracle's decode with the query
    rounded as the FP8 decode rounds it (fp8.fp8_query_decode), so only the
    kernel's E4M3 rounding of the probabilities is left (a relative 2^-4 per
    weight; 1-3 % normwise when simulated with the exact row max as the
    reference): normwise 4 %, 10 % of max|ref| for the largest element."""
    if dtype == "f32":
        return 1e-4, 1e-4, 1e-4
    if dtype == "fp8":
        return float("inf"), 8e-2, 0.15
    if dtype == "fp8q":
        return float("inf"), 4e-2, 0.10
    return 2e-2, 1e-2, 5e-2


def assert_parity(got, ref, dtype, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    d = np.abs(got - ref)
    max_abs, rel_bar, peak_bar = bar(dtype)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    msg = f"{what}: max|d|={d.max():.3e} rel={rel:.3e} max|ref|={np.abs(ref).max():.3e}"
    print(f"[parity] {msg}", flush=True)
    assert d.max() <= max_abs, msg
    assert rel <= rel_bar, msg
    assert d.max() <= peak_bar * np.abs(ref).max(), msg
    return d.max(), rel


def assert_projection_parity(got, ref, what=""):
    """Bar of a bf16 projection output (q_nope, q_pe) against the oracle's
    fp64 value: element-wise |d| <= 2e-2 + 2^-8 |ref|, normwise <= 1e-2.

    The output is stored in bf16 (relative rounding up to 2^-9) from an
    intermediate c_Q that is itself stored in bf16 (another 2^-9 of each input
    of the second product). The fixed 2e-2 of the attention outputs suits
    values of unit scale; projection outputs reach 6 sigma over millions of
    elements, where one bf16 rounding alone is 1.6e-2, so the element bar
    grows with the value by two roundings' worth."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    d = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    excess = float((d - (2e-2 + 2.0 ** -8 * np.abs(ref))).max())
    msg = f"{what}: max|d|={d.max():.3e} rel={rel:.3e} max|ref|={np.abs(ref).max():.3e} worst excess={excess:.3e}"
    print(f"[parity] {msg}", flush=True)
    assert excess <= 0.0, msg
    assert rel <= 1e-2, msg
    return d.max(), rel


def fails_bar(got, ref, dtype):
    try:
        assert_parity(got, ref, dtype)
    except AssertionError:
        return True
    return False


def score_jump_case(case, jump_log2, low_pages=2):
    """Makes the scores of every sequence's first `low_pages` pages about
    `jump_log2` log2 units below those of the rest, for every head, so that the
    running max of a page run jumps by that much inside the run.

    All heads of a sequence get head 0's rotary query v; the low pages' k_pe is
    set to -lam * R(L-1) v (R the oracle's rotation at the query's position),
    which adds -lam |v|^2 * scale to every head's score there. The values
    (c_KV) keep their scale, so the output is set by the high pages, whose
    scores are ordinary."""
    import oracle
    from synth import bf16_bits_to_f32, f32_to_bf16_bits
    d = case.dims
    pool = bf16_bits_to_f32(case.cache.pool)
    q_pe = bf16_bits_to_f32(case.q_pe)
    table = case.cache.block_table
    for b, L in enumerate(case.cache.context_lens):
        L = int(L)
        v = q_pe[b, 0].astype(np.float64)
        q_pe[b, :] = q_pe[b, 0]
        u = oracle.rope(v, L - 1, d.rope_base)
        lam = jump_log2 / (float(u @ u) * d.scale * np.log2(np.e))
        n_low = min(low_pages, (L + 63) // 64)
        for p in range(n_low):
            pool[table[b, p], :, d.d_c:] = (-lam * u).astype(np.float32)
    case.cache.pool = f32_to_bf16_bits(pool)
    case.q_pe = f32_to_bf16_bits(q_pe)
    return case


def host_run_pages(rows, max_context):
    """Pages per run as the library's host side plans a decode step with one
    new token per row: about one run per compute unit over rows x the
    longest context's pages, clamped to 4..32."""
    max_pages = -(-max_context // 64)
    return max(4, min(32, -(-rows * max_pages // 256)))


def one_round_run_pages(lens, pps, budget):
    """The run length the split kernels take over contexts `lens`: the
    smallest length in (pps, min(64, 5 pps / 4)] whose runs fit in one round
    of `budget` workgroups when the runs of pps need a second round (but not
    a third), else pps."""
    runs = lambda q: sum(-(-int(L) // (64 * q)) for L in lens)
    if runs(pps) <= budget or runs(pps) > 2 * budget:
        return pps
    for q in range(pps + 1, min(64, pps + pps // 4) + 1):
        if runs(q) <= budget:
            return q
    return pps
