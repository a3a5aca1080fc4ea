"""The seeded input generator: sub-range regeneration, symmetry, needles."""
import numpy as np

import gen


def test_subrange_regenerates_bit_identically():
    full = gen.normal(5, 2, (10000,))
    part = gen.normal(5, 2, (777,), e0=1234)
    assert np.array_equal(full[1234:1234 + 777], part)
    k_full = gen.idx_keys(9, 3, 8192, 0, 8192, 64, 512, 4)
    k_part = gen.idx_keys(9, 3, 8192, 4000, 100, 64, 512, 4)
    assert np.array_equal(k_full[4000:4100], k_part)


def test_normal_table_is_symmetric_and_standard():
    t = gen.ntab().astype(np.float64)
    assert np.array_equal(t, -t[::-1])
    assert abs(t.mean()) < 1e-6 and abs(t.var() - 1.0) < 2e-3
    x = gen.bf16_to_f64(gen.normal(1, 1, (1 << 20,)))
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1.0) < 5e-3


def test_streams_and_seeds_differ():
    a = gen.normal(1, 1, (4096,))
    assert not np.array_equal(a, gen.normal(1, 2, (4096,)))
    assert not np.array_equal(a, gen.normal(2, 1, (4096,)))


def test_one_needle_block_per_window():
    seed, L, W, r, d = 1002, 32768, 512, 4, 64
    keys = gen.bf16_to_f64(gen.idx_keys(seed, 0, L, 0, L, d, W, r))
    plain = gen.bf16_to_f64(gen.idx_keys(seed, 0, L, 0, L, d, 0, r))
    u = gen.needle_dir(seed, d)
    assert abs(np.linalg.norm(u) - 1) < 1e-12
    moved = np.abs(keys - plain).sum(1) > 0
    tok = np.nonzero(moved)[0]
    assert len(tok) == (L // W) * r
    blocks = np.unique(tok // r)
    assert len(blocks) == L // W
    assert (np.bincount(blocks * r // W, minlength=L // W) == 1).all()
    # the planted shift is +3u along the needle direction
    shift = ((keys - plain)[moved] @ u)
    assert np.allclose(shift, 3.0, atol=0.15)
