"""The seeded input generator: published SplitMix64 outputs, grid values, reproducibility."""
import numpy as np

import tdb_inputs as ti


def test_splitmix64_published_outputs():
    # First outputs of SplitMix64 seeded with 1234567, as published with common
    # SplitMix64 implementations (state advanced by GAMMA before each mix).
    got = ti.splitmix64(1234567, np.arange(3, dtype=np.uint64))
    assert [int(x) for x in got] == [6457827717110365317, 3203168211198807973,
                                     9817491932198370423]


def test_index_addressable():
    s0 = ti.stream_state(42, 1)
    full = ti.splitmix64(s0, np.arange(1000, dtype=np.uint64))
    part = ti.splitmix64(s0, np.arange(500, 1000, dtype=np.uint64))
    assert np.array_equal(full[500:], part)
    assert np.array_equal(ti.grid_ints(42, 1, 100, start=900), ti.grid_ints(42, 1, 1000)[900:])


def test_grid_values_exact_and_in_range():
    A = ti.grid_matrix(1001, ti.STREAM_A, 128, 128)
    ia = ti.grid_matrix_ints(1001, ti.STREAM_A, 128, 128)
    assert A.dtype == np.float32
    assert np.array_equal(A.astype(np.float64), ia.astype(np.float64) * 2.0 ** -23)
    assert A.min() >= -1.0 and A.max() <= 1.0 - 2.0 ** -23
    assert ia.min() >= -(1 << 23) and ia.max() < (1 << 23)
    # roughly uniform: mean ~ 0, variance ~ 1/3
    assert abs(float(A.mean())) < 0.02
    assert abs(float(A.var()) - 1.0 / 3.0) < 0.02


def test_streams_and_seeds_differ():
    a = ti.grid_matrix(1, ti.STREAM_A, 8, 8)
    b = ti.grid_matrix(1, ti.STREAM_B, 8, 8)
    c = ti.grid_matrix(2, ti.STREAM_A, 8, 8)
    assert not np.array_equal(a, b) and not np.array_equal(a, c)


def test_padding_and_chunking():
    buf = ti.grid_matrix(7, 1, 5, 6, ld=9)
    assert buf.shape == (5, 9) and np.all(np.isnan(buf[:, 6:]))
    assert np.array_equal(buf[:, :6], ti.grid_matrix(7, 1, 5, 6))
    n = (1 << 23) + 17   # crosses the internal chunk boundary
    v = ti.grid_ints(3, 2, n)
    assert np.array_equal(v[-40:], ti.grid_ints(3, 2, 40, start=n - 40))


def test_sample_positions():
    i, j = ti.sample_positions(5001, 8192, 8192, 4096)
    assert i.shape == (4096,) and j.shape == (4096,)
    assert i.min() >= 0 and i.max() < 8192 and j.min() >= 0 and j.max() < 8192
    i2, j2 = ti.sample_positions(5001, 8192, 8192, 4096)
    assert np.array_equal(i, i2) and np.array_equal(j, j2)
