"""The seeded input generators: shapes, determinism and the recipe's statistics."""
import numpy as np

import workloads


def test_determinism_and_row_ranges():
    a = workloads.config(2, 0, 700)
    b = workloads.config(2, 600, 700)
    assert np.array_equal(a[600:700], b)
    assert np.array_equal(workloads.config(1), workloads.config(1))


def test_config2_recipe():
    x = workloads.config(2)
    assert x.shape == (4096, 32000) and x.dtype == np.float32
    n = x.size
    assert abs((x == 80).sum() / n - 0.5e-3) < 0.05e-3
    assert abs((x == -80).sum() / n - 0.5e-3) < 0.05e-3
    assert abs(np.isneginf(x).sum() / n - 1e-4) < 0.1e-4
    assert not np.isneginf(x).all(axis=1).any()
    assert np.isfinite(x[~np.isneginf(x)]).all()


def test_config3_bf16_rounding():
    b = workloads.config(3, 0, 256)
    assert b.dtype == np.uint16 and b.shape == (256, 2048)
    f = workloads.bf16_bits_to_f32(b)
    assert abs(float(f.std()) - 1.0 / np.sqrt(128)) < 2e-3
    # nearest-even rounding of a known halfway case and a near-halfway case
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20], dtype=np.float32)
    assert workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(x)).tolist() == [1.0, 1.015625, 1.0078125]


def test_config5_duplicated_maxima():
    x = workloads.config(5)
    picked = workloads.dup_rows_cfg5()
    assert len(picked) == 13
    for r in range(x.shape[0]):
        count = int((x[r] == x[r].max()).sum())
        if r in picked:
            assert 2 <= count <= 4
            first = int(np.argmax(x[r]))
            assert first < np.flatnonzero(x[r] == x[r].max())[-1]
        else:
            assert count == 1


def test_shapes_of_every_config():
    for n, (rows, cols) in workloads.SHAPES.items():
        x = workloads.config(n, 0, 2)
        assert x.shape == (2, cols)


def test_row_range_is_clamped_to_the_workload():
    x = workloads.config(1, 0, 256)
    assert x.shape == (64, 1024)
    assert np.array_equal(x, workloads.config(1))
    assert workloads.config(5, 250, 400).shape == (6, 128256)
