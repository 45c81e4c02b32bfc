"""Pins for the oracle's layer stack and its bf16 rounding: torch's own
float32 -> bfloat16 conversion (round to nearest even) on exactly
representable inputs, hand-worked ties, and the sharded stack against the
unsharded network it stands for."""
import numpy as np
import pytest
import torch

from oracle import mlp as O


def test_round_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200000) * np.exp(rng.uniform(-100, 85, 200000))
    x = x.astype(np.float32)
    specials = np.array([0.0, -0.0, np.inf, -np.inf, 3.3895313892515355e38, 3.4e38, 1e-40, -1e-41, 1.17549435e-38],
                        dtype=np.float32)
    x = np.concatenate([x, specials])
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    got = O.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)
    assert np.isnan(O.round_bf16(np.array([np.nan]))[0])


@pytest.mark.parametrize("x,expect", [
    (1 + 2 ** -8, 1.0),                   # halfway between 1 and 1 + 2**-7: to the even one, 1
    (1 + 3 * 2 ** -8, 1 + 2 ** -6),       # halfway between 1 + 2**-7 and 1 + 2**-6: to the even one
    (257.0, 256.0), (259.0, 260.0), (258.0, 258.0),
    (-257.0, -256.0),
    (2.0 ** -133, 2.0 ** -133),           # the smallest bf16 subnormal
    (2.0 ** -134, 0.0),                   # halfway to zero: ties to even (zero)
    (1.5 * 2.0 ** -133, 2.0 ** -132),
])
def test_round_bf16_hand_worked(x, expect):
    assert O.round_bf16(np.array([x]))[0] == expect


def _network(X, As, Bs, biases, act):
    x = np.asarray(X, np.float64)
    for A, B, b in zip(As, Bs, biases):
        x = O.mlp_unsharded(x, A, B, act) + (b[None, :] if b is not None else 0.0)
    return x


@pytest.mark.parametrize("act", [O.GELU_NONE, O.GELU_ERF])
def test_sharded_stack_is_the_unsharded_network(act):
    """Each layer's peers are the other ranks' partials of that layer's input;
    without rounding (f64) the stack is the unsharded 3-layer network."""
    rng = np.random.default_rng(5)
    M, H, F, P, L = 6, 8, 4, 3, 3
    X = rng.standard_normal((M, H))
    As = [rng.standard_normal((H, P * F)) * 0.3 for _ in range(L)]
    Bs = [rng.standard_normal((P * F, H)) * 0.3 for _ in range(L)]
    bs = [rng.standard_normal(H), None, rng.standard_normal(H)]
    x, layers = X, []
    for A, B, b in zip(As, Bs, bs):
        A_sh = [A[:, i * F:(i + 1) * F] for i in range(P)]
        B_sh = [B[i * F:(i + 1) * F, :] for i in range(P)]
        peers = [O.mlp_rank(x, A_sh[i], B_sh[i], act) for i in range(1, P)]
        layers.append({"A_i": A_sh[0], "B_i": B_sh[0], "peers": peers, "bias": b, "act": act})
        x = sum(O.mlp_rank(x, A_sh[i], B_sh[i], act) for i in range(P)) + (b if b is not None else 0.0)
    out = O.mlp_stack(X, layers, dtype="f64")
    assert np.allclose(out[-1][0], _network(X, As, Bs, bs, act), atol=1e-10, rtol=0)


def test_linear_stack_closed_form_with_rounding():
    """act NONE, A = I, B = c I (c a power of two), no peers: each layer scales
    by c, exactly representable, so the bf16 stack gives X * prod(c)."""
    rng = np.random.default_rng(2)
    H = 8
    X = O.round_bf16(rng.standard_normal((5, H)))
    cs = [2.0, 0.5, 4.0]
    layers = [{"A_i": np.eye(H), "B_i": c * np.eye(H), "act": O.GELU_NONE} for c in cs]
    out = O.mlp_stack(X, layers, dtype="bf16")
    assert np.array_equal(out[-1][1], X * 4.0)
    assert np.array_equal(out[0][0], X * 2.0)


def test_row_chunks_are_independent_across_layers():
    """The premise of the inter-layer overlap: rows of the stack's output depend
    on the same rows of the input only."""
    rng = np.random.default_rng(9)
    M, H, F = 8, 6, 5
    X = O.round_bf16(rng.standard_normal((M, H)))
    layers = [{"A_i": rng.standard_normal((H, F)), "B_i": rng.standard_normal((F, H)),
               "peers": [rng.standard_normal((M, H))], "bias": rng.standard_normal(H)} for _ in range(2)]
    full = O.mlp_stack(X, layers)
    rows = np.array([1, 2, 6])
    sub = O.mlp_stack(X[rows], [dict(l, peers=[p[rows] for p in l["peers"]]) for l in layers])
    for (zf, xf), (zs, xs) in zip(full, sub):
        assert np.array_equal(zf[rows], zs) and np.array_equal(xf[rows], xs)
