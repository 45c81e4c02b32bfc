"""Pins for the reduction oracle: exact integer sums, split == full, P = 1,
and the N(0,1) variance law."""
import numpy as np
import pytest

from oracle import reduce as R
from oracle.layout import OracleLayoutError


def test_integer_partials_exact():
    rng = np.random.default_rng(1)
    P, rows, cols = 5, 7, 9
    ints = rng.integers(-1024, 1025, size=(P, rows, cols))
    parts = [ints[p].astype(np.float32) for p in range(P)]
    got = R.reduce_full(parts)
    for i in range(rows):
        for j in range(cols):
            assert got[i, j] == sum(int(ints[p, i, j]) for p in range(P))


def test_split_blocks_concatenate_to_full():
    rng = np.random.default_rng(2)
    parts = [rng.standard_normal((12, 5)).astype(np.float32) for _ in range(3)]
    blocks = R.reduce_split(parts, 4)
    assert [b.shape for b in blocks] == [(3, 5)] * 4
    assert np.array_equal(np.concatenate(blocks, axis=0), R.reduce_full(parts))


def test_single_partial_is_identity():
    rng = np.random.default_rng(3)
    p = rng.standard_normal((6, 4)).astype(np.float32)
    assert np.array_equal(R.reduce_full([p]), p.astype(np.float64))
    assert np.array_equal(R.reduce_split([p], 1)[0], p.astype(np.float64))


def test_sum_of_normals_has_std_sqrt_p():
    rng = np.random.default_rng(4)
    P = 8
    parts = [rng.standard_normal((512, 512)).astype(np.float32) for _ in range(P)]
    s = R.reduce_full(parts)
    assert abs(s.std() / np.sqrt(P) - 1.0) < 0.02
    assert abs(s.mean()) < 0.05


def test_split_rejections():
    p = np.zeros((6, 2), np.float32)
    with pytest.raises(OracleLayoutError) as e:
        R.reduce_split([p, p], 4)
    assert e.value.kind == "indivisible"
    with pytest.raises(OracleLayoutError):
        R.reduce_split([p], 0)
    with pytest.raises(OracleLayoutError):
        R.reduce_full([])
    with pytest.raises(OracleLayoutError):
        R.reduce_full([p, np.zeros((2, 6), np.float32)])
