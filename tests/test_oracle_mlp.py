"""Pins for the MLP oracle: GeLU closed forms, the column/row split identity
in float64, and brute force against pure-Python loops on tiny shapes."""
import itertools
import math

import numpy as np
import pytest

from oracle import layout as L
from oracle import mlp as O

PHI_1 = 0.8413447460685429   # standard normal CDF at 1 (textbook table value)


def test_gelu_closed_forms():
    assert O.gelu(0.0) == 0.0
    assert abs(O.gelu(1.0) - PHI_1) < 1e-15
    assert abs(O.gelu(-1.0) - (PHI_1 - 1.0)) < 1e-15
    xs = np.linspace(-6, 6, 1001)
    # Phi(-x) = 1 - Phi(x)  =>  GeLU(-x) = GeLU(x) - x
    assert np.allclose(O.gelu(-xs), O.gelu(xs) - xs, rtol=0, atol=1e-14)
    assert abs(O.gelu(12.0) - 12.0) < 1e-14
    assert abs(O.gelu(-12.0)) < 1e-14
    # a second, independent erf: the standard library's
    ref = np.array([0.5 * x * (1.0 + math.erf(x / math.sqrt(2.0))) for x in xs])
    assert np.allclose(O.gelu(xs), ref, rtol=1e-14, atol=1e-15)


def _loops_hidden(X, A, act):
    M, H, F = len(X), len(X[0]), len(A[0])
    Y = [[0.0] * F for _ in range(M)]
    for m in range(M):
        for f in range(F):
            s = 0.0
            for h in range(H):
                s += X[m][h] * A[h][f]
            Y[m][f] = 0.5 * s * (1.0 + math.erf(s / math.sqrt(2.0))) if act else s
    return np.array(Y)


def _loops(X, A, B, act):
    M, H = len(X), len(X[0])
    F = len(A[0])
    N = len(B[0])
    Y = [[0.0] * F for _ in range(M)]
    for m in range(M):
        for f in range(F):
            s = 0.0
            for h in range(H):
                s += X[m][h] * A[h][f]
            Y[m][f] = 0.5 * s * (1.0 + math.erf(s / math.sqrt(2.0))) if act else s
    Z = [[0.0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            s = 0.0
            for f in range(F):
                s += Y[m][f] * B[f][n]
            Z[m][n] = s
    return np.array(Z)


@pytest.mark.parametrize("act", [O.GELU_NONE, O.GELU_ERF])
def test_brute_force_tiny_shapes(act):
    rng = np.random.default_rng(21)
    sizes = [1, 2, 3, 5, 8]
    for M, H, F in itertools.product(sizes, repeat=3):
        X = rng.standard_normal((M, H))
        A = rng.standard_normal((H, F))
        B = rng.standard_normal((F, H + 1))   # output width != H catches a transposed B
        got = O.mlp_rank(X, A, B, act)
        ref = _loops(X.tolist(), A.tolist(), B.tolist(), act)
        assert got.shape == (M, H + 1)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
        y = O.hidden(X, A, act)
        assert y.shape == (M, F)
        assert np.allclose(y, _loops_hidden(X.tolist(), A.tolist(), act), rtol=1e-12, atol=1e-12)


def test_worked_integer_example():
    # X = [1 2], A = [[1 0 2], [0 1 -1]] -> XA = [1 2 0]; B = [[1],[10],[100]] -> 21.
    X = np.array([[1.0, 2.0]])
    A = np.array([[1.0, 0.0, 2.0], [0.0, 1.0, -1.0]])
    B = np.array([[1.0], [10.0], [100.0]])
    assert O.mlp_rank(X, A, B, O.GELU_NONE)[0, 0] == 21.0
    # with GeLU: GeLU(1) + 10 GeLU(2) + 100 GeLU(0)
    g = lambda x: 0.5 * x * (1 + math.erf(x / math.sqrt(2)))
    assert abs(O.mlp_rank(X, A, B)[0, 0] - (g(1.0) + 10 * g(2.0))) < 1e-13


@pytest.mark.parametrize("P", [1, 2, 4])
@pytest.mark.parametrize("act", [O.GELU_NONE, O.GELU_ERF])
def test_sum_of_rank_shares_equals_unsharded(P, act):
    # ColossalAI 1D TP, sections 2 and 2.1: sum_i act(X A_i) B_i = act(X A) B
    # when A is cut by columns and B by rows into matching pieces.
    rng = np.random.default_rng(100 + P)
    M, H, Fall = 17, 24, 32
    X = rng.standard_normal((M, H))
    A = rng.standard_normal((H, Fall)) / math.sqrt(H)
    B = rng.standard_normal((Fall, H)) / math.sqrt(Fall)
    A_sh = L.split(A, {"device": list(range(P)), "sharded_dim": [{"axis": 1, "num_shards": P}]})
    B_sh = L.split(B, {"device": list(range(P)), "sharded_dim": [{"axis": 0, "num_shards": P}]})
    got = O.mlp_all_ranks(X, [A_sh[i] for i in range(P)], [B_sh[i] for i in range(P)], act)
    ref = O.mlp_unsharded(X, A, B, act)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))
    if P > 1:
        # a mismatched pairing (A_i with B_{i+1}) must not give the same answer
        bad = O.mlp_all_ranks(X, [A_sh[i] for i in range(P)], [B_sh[(i + 1) % P] for i in range(P)], act)
        assert np.max(np.abs(bad - ref)) > 1e-3 * np.max(np.abs(ref))


def test_row_sample_is_exact():
    rng = np.random.default_rng(8)
    X = rng.standard_normal((10, 6))
    A = rng.standard_normal((6, 5))
    B = rng.standard_normal((5, 6))
    rows = [0, 3, 9]
    assert np.array_equal(O.mlp_rank_rows(X, A, B, rows), O.mlp_rank(X, A, B)[rows])


def test_bf16_inputs_are_read_exactly():
    import torch
    x = torch.tensor([[1.0 + 2 ** -7, -3.0]], dtype=torch.bfloat16)
    a = torch.tensor([[1.0], [2 ** -8]], dtype=torch.bfloat16)
    b = torch.tensor([[1.0]], dtype=torch.bfloat16)
    z = O.mlp_rank(x, a, b, O.GELU_NONE)
    assert z[0, 0] == (1.0 + 2 ** -7) - 3.0 * 2 ** -8
