"""The seeded input generator: determinism, rounding and paged layout."""
import hashlib

import numpy as np

from synth import Dims, PAGE, bf16_bits_to_f32, f32_to_bf16_bits, make_decode_case, make_ragged_lens, paged_layout


def _digest(*arrays):
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_same_seed_same_arrays_other_seed_other_arrays():
    dims = Dims(8, 64, 16, 32, 32)
    a = make_decode_case(5, 3, dims, [10, 70, 200], shuffle=True)
    b = make_decode_case(5, 3, dims, [10, 70, 200], shuffle=True)
    c = make_decode_case(6, 3, dims, [10, 70, 200], shuffle=True)
    da = _digest(a.q_nope, a.q_pe, a.w_uk, a.w_uv, a.cache.pool, a.cache.block_table)
    assert da == _digest(b.q_nope, b.q_pe, b.w_uk, b.w_uv, b.cache.pool, b.cache.block_table)
    assert da != _digest(c.q_nope, c.q_pe, c.w_uk, c.w_uv, c.cache.pool, c.cache.block_table)


def test_bf16_rounding_is_nearest_even_and_exact_on_bf16_values():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 65504.0, 1e-40], dtype=np.float32)
    b = f32_to_bf16_bits(x)
    assert b[0] == 0x3F80 and b[1] == 0x3F80 and b[2] == 0x3F82 and b[3] == 0x8000
    r = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    once = f32_to_bf16_bits(r)
    assert np.array_equal(f32_to_bf16_bits(bf16_bits_to_f32(once)), once)
    assert np.max(np.abs(bf16_bits_to_f32(once) - r) / np.abs(r)) <= 2 ** -8


def test_block_table_is_a_permutation_of_the_pool():
    lens = make_ragged_lens(1, 32, 1024, 32768)
    assert lens.min() >= 1024 and lens.max() <= 32768
    for rng in (None, np.random.default_rng(2)):
        table, nb = paged_layout(lens, rng)
        used = np.concatenate([table[b, :(int(L) + PAGE - 1) // PAGE] for b, L in enumerate(lens)])
        assert sorted(used.tolist()) == list(range(nb))
        for b, L in enumerate(lens):
            assert np.all(table[b, (int(L) + PAGE - 1) // PAGE:] == -1)


def test_weight_scale_follows_fan_in():
    case = make_decode_case(7, 2, Dims(16, 512, 64, 128, 128), 64)
    w = bf16_bits_to_f32(case.w_uk)
    assert abs(w.std() - 1 / np.sqrt(512)) < 0.002
