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


# ---- partial max / min and the row-parallel bias ----------------------------

def test_max_min_brute_force():
    """Element by element with Python's own max / min over the P values."""
    rng = np.random.default_rng(5)
    parts = [rng.integers(-9, 10, size=(3, 4)).astype(np.float32) for _ in range(5)]
    mx, mn = R.reduce_full(parts, "max"), R.reduce_full(parts, "min")
    for i in range(3):
        for j in range(4):
            vals = [float(p[i, j]) for p in parts]
            assert mx[i, j] == max(vals) and mn[i, j] == min(vals)


def test_max_min_invariants():
    rng = np.random.default_rng(6)
    parts = [rng.standard_normal((16, 8)) for _ in range(7)]
    mx, mn = R.reduce_full(parts, "max"), R.reduce_full(parts, "min")
    st = np.stack(parts)
    assert (st <= mx).all() and (st >= mn).all()
    assert ((st == mx).any(axis=0)).all() and ((st == mn).any(axis=0)).all()   # attained by some partial
    # max(a) = -min(-a)
    assert np.array_equal(mx, -R.reduce_full([-p for p in parts], "min"))
    assert np.array_equal(R.reduce_full(parts[:1], "max"), parts[0])
    # max(x, -x) = |x| and min(x, -x) = -|x|
    assert np.array_equal(R.reduce_full([parts[0], -parts[0]], "max"), np.abs(parts[0]))
    assert np.array_equal(R.reduce_full([parts[0], -parts[0]], "min"), -np.abs(parts[0]))


def test_max_ignores_nan_against_a_number():
    a = np.array([[np.nan, 1.0]])
    b = np.array([[2.0, np.nan]])
    assert np.array_equal(R.reduce_full([a, b], "max"), np.array([[2.0, 1.0]]))
    assert np.array_equal(R.reduce_full([a, b], "min"), np.array([[2.0, 1.0]]))


def test_bias_is_added_once_after_the_sum():
    """[CAI] section 5.2: the row-parallel layer's output with bias b is
    Y B + b for the full Y B; the ranks' partials sum to Y B, so b is added
    to the reduced value once (adding it per partial would count it P times)."""
    rng = np.random.default_rng(8)
    M, H, F, P = 5, 6, 3, 4
    Y = rng.standard_normal((M, P * F))
    B = rng.standard_normal((P * F, H))
    b = rng.standard_normal(H)
    parts = [Y[:, i * F:(i + 1) * F] @ B[i * F:(i + 1) * F, :] for i in range(P)]
    # the unsharded linear layer, row by row
    ref = np.array([[sum(Y[m, k] * B[k, h] for k in range(P * F)) + b[h] for h in range(H)] for m in range(M)])
    assert np.allclose(R.reduce_full(parts, "sum", b), ref, atol=1e-12)
    blocks = R.reduce_split(parts, 5, "sum", b)
    assert np.allclose(np.concatenate(blocks), ref, atol=1e-12)


def test_op_rejections():
    with pytest.raises(OracleLayoutError) as e:
        R.reduce_full([np.zeros((2, 2))], "prod")
    assert e.value.kind == "arg"
    with pytest.raises(OracleLayoutError):
        R.reduce_full([np.zeros((2, 2))], "sum", np.zeros(3))
