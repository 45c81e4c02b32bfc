"""Pins of the oracle's backward (ColossalAI 1D tensor parallelism, section
2.2; DeepSpeed-Domino, "backward").

The gradients are checked against central finite differences of the forward
loss <dZ, Z> (the forward oracle is pinned on its own), against a tabulated
value and identities of GeLU', and against the unsharded model's gradient, so
a dropped activation derivative, a transposed operand or a wrong rank sum
fails here rather than being restated.
"""
import math

import numpy as np
import pytest

from oracle import mlp as O

# Standard normal table: Phi(1) and phi(1) = exp(-1/2) / sqrt(2 pi).
PHI_1 = 0.8413447460685429
PDF_1 = 0.24197072451914337


def test_gelu_deriv_closed_forms():
    assert O.gelu_deriv(0.0) == 0.5
    assert abs(O.gelu_deriv(1.0) - (PHI_1 + PDF_1)) < 1e-15
    assert abs(O.gelu_deriv(12.0) - 1.0) < 1e-15
    assert abs(O.gelu_deriv(-12.0)) < 1e-15
    x = np.linspace(-7, 7, 141)
    # Phi(x) + Phi(-x) = 1 and x phi(x) is odd, so GeLU'(x) + GeLU'(-x) = 1.
    assert np.max(np.abs(O.gelu_deriv(x) + O.gelu_deriv(-x) - 1.0)) < 1e-14


def test_gelu_deriv_matches_finite_difference():
    x = np.linspace(-6, 6, 241)
    h = 1e-5
    fd = (O.gelu(x + h) - O.gelu(x - h)) / (2 * h)
    assert np.max(np.abs(fd - O.gelu_deriv(x))) < 1e-9


def _loss(X, A, B, dZ, act):
    return float(np.sum(dZ * O.mlp_rank(X, A, B, act)))


def _fd_grad(f, T, eps=1e-6):
    g = np.zeros_like(T)
    it = np.nditer(T, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = T[i]
        T[i] = old + eps
        up = f()
        T[i] = old - eps
        down = f()
        T[i] = old
        g[i] = (up - down) / (2 * eps)
    return g


@pytest.mark.parametrize("act", [O.GELU_NONE, O.GELU_ERF])
@pytest.mark.parametrize("M,H,F", [(3, 4, 5), (2, 6, 3)])
def test_backward_matches_finite_differences(act, M, H, F):
    rng = np.random.default_rng(7 + M + act)
    X, A, B, dZ = (rng.standard_normal(s) for s in [(M, H), (H, F), (F, H), (M, H)])
    g = O.backward_rank(X, A, B, dZ, act)
    assert np.allclose(_fd_grad(lambda: _loss(X, A, B, dZ, act), X), g["dX_i"], atol=1e-7, rtol=0)
    assert np.allclose(_fd_grad(lambda: _loss(X, A, B, dZ, act), A), g["dA_i"], atol=1e-7, rtol=0)
    assert np.allclose(_fd_grad(lambda: _loss(X, A, B, dZ, act), B), g["dB_i"], atol=1e-7, rtol=0)
    # dH is the gradient with respect to the pre-activation X A.
    pre = X @ A
    act_fn = O.gelu if act == O.GELU_ERF else (lambda t: t)
    dH_fd = _fd_grad(lambda: float(np.sum(dZ * (act_fn(pre) @ B))), pre)
    assert np.allclose(dH_fd, g["dH"], atol=1e-7, rtol=0)


@pytest.mark.parametrize("P", [2, 3])
def test_sum_of_rank_gradients_is_the_unsharded_gradient(P):
    rng = np.random.default_rng(11 + P)
    M, H, F = 3, 4, 2
    X, dZ = rng.standard_normal((M, H)), rng.standard_normal((M, H))
    A = rng.standard_normal((H, P * F))
    B = rng.standard_normal((P * F, H))
    A_sh = [A[:, i * F:(i + 1) * F] for i in range(P)]
    B_sh = [B[i * F:(i + 1) * F, :] for i in range(P)]
    dX, dA, dB = O.backward_all_ranks(X, A_sh, B_sh, dZ)
    loss = lambda: float(np.sum(dZ * O.mlp_unsharded(X, A, B)))
    assert np.allclose(_fd_grad(loss, X), dX, atol=1e-7, rtol=0)
    # Column shards of A and row shards of B: the per-rank weight gradients
    # tile the unsharded ones.
    assert np.allclose(_fd_grad(loss, A), np.concatenate(dA, axis=1), atol=1e-7, rtol=0)
    assert np.allclose(_fd_grad(loss, B), np.concatenate(dB, axis=0), atol=1e-7, rtol=0)


def test_row_chunks_split_input_gradients_and_sum_weight_gradients():
    """Domino's row chunks: dH and dX of a chunk come from that chunk's rows
    alone, and the weight gradients are sums over chunks."""
    rng = np.random.default_rng(3)
    M, H, F, R = 8, 5, 3, 4
    X, A, B, dZ = (rng.standard_normal(s) for s in [(M, H), (H, F), (F, H), (M, H)])
    full = O.backward_rank(X, A, B, dZ)
    rows = M // R
    parts = [O.backward_rank(X[r * rows:(r + 1) * rows], A, B, dZ[r * rows:(r + 1) * rows]) for r in range(R)]
    assert np.allclose(np.concatenate([p["dX_i"] for p in parts]), full["dX_i"], atol=1e-12)
    assert np.allclose(np.concatenate([p["dH"] for p in parts]), full["dH"], atol=1e-12)
    assert np.allclose(sum(p["dA_i"] for p in parts), full["dA_i"], atol=1e-12)
    assert np.allclose(sum(p["dB_i"] for p in parts), full["dB_i"], atol=1e-12)
