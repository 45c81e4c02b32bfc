"""Oracle for one rank's column->row MLP share (test infrastructure only).

Sources:
* ColossalAI 1D tensor parallelism, section 2: with A cut by columns into
  [A_1 ... A_P], rank i computes Y_i = X A_i and the Y_i side by side form XA.
* Same page, section 2.1: the second linear layer cuts B by rows into
  [B_1; ...; B_P]; rank i computes Y_i B_i and the sum over ranks (one
  all-reduce) is Z = Y B.
* DeepSpeed-Domino article, "forward" under implementation: each micro-batch
  runs GeMM, GeLU, GeMM; the row chunks of X are independent.
* ONNX multi-device proposal, operator-group rules: unary elementwise ops
  (Erf among them) accept any input sharding, so GeLU commutes with the column
  split; MatMul with a sharded K axis yields a partial sum.
* DeepSpeed-Domino article, design of the row-wise split of X: no dependency
  across row chunks within a layer or between layers, so a stack of layers
  consumes each layer's reduced output chunk by chunk (inter_layer_overlap).
* ColossalAI 1D tensor parallelism, section 2.2, and the DeepSpeed-Domino
  article, "backward": the column-parallel layer's input gradient is a partial
  per rank that an all-reduce sums; each gradient matmul splits into an
  input-gradient GEMM and an independent weight-gradient GEMM.

GeLU is never written out on the pages; the reading taken is the exact form
x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)).  Everything is evaluated in float64
on the exact values of the (bf16 or fp32) inputs; Y is not rounded.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf as _erf

from .layout import _as_numpy

GELU_NONE = 0
GELU_ERF = 1


def gelu(x):
    """x * Phi(x) with Phi the standard normal CDF, in float64."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + _erf(x / math.sqrt(2.0)))


def _f64(t):
    return _as_numpy(t).astype(np.float64)


def hidden(X, A_i, act=GELU_ERF):
    """Y_i = act(X A_i): the column-parallel output of one rank, fp64 [M, F]."""
    x, a = _f64(X), _f64(A_i)
    if x.shape[1] != a.shape[0]:
        raise ValueError("shape mismatch")
    y = x @ a
    return gelu(y) if act == GELU_ERF else y


def mlp_rank(X, A_i, B_i, act=GELU_ERF):
    """Z_i = act(X A_i) B_i: one rank's fp64 partial output [M, H]."""
    b = _f64(B_i)
    y = hidden(X, A_i, act)
    if y.shape[1] != b.shape[0]:
        raise ValueError("shape mismatch")
    return y @ b


def mlp_all_ranks(X, A_shards, B_shards, act=GELU_ERF):
    """Z = sum over ranks i of act(X A_i) B_i (the all-reduced output)."""
    if len(A_shards) != len(B_shards):
        raise ValueError("need one B_i per A_i")
    acc = None
    for a, b in zip(A_shards, B_shards):
        z = mlp_rank(X, a, b, act)
        acc = z if acc is None else acc + z
    return acc


def mlp_unsharded(X, A, B, act=GELU_ERF):
    """act(X A) B with the full weights: what the sharded sum must equal."""
    return mlp_rank(X, A, B, act)


def mlp_rank_rows(X, A_i, B_i, rows, act=GELU_ERF):
    """Rows ``rows`` of mlp_rank, computed from those rows of X only.

    Each output row depends on its own row of X alone (the row-chunk
    independence the Domino article relies on), so a row sample of a large
    problem is exact, not an approximation.
    """
    x = _f64(X)[np.asarray(rows, dtype=np.int64)]
    return mlp_rank(x, A_i, B_i, act)


# ---- a stack of layers ([DOM] "row-wise split of inputs X", inter-layer) ----
#
# Layer l+1 reads layer l's full output: the all-reduced sum of the ranks'
# partials plus the row layer's bias, stored in the input precision (rounded
# to nearest even for bf16), which is what the next GEMM consumes.


def round_bf16(x):
    """Round float64 values to the nearest bfloat16 (8 significant bits, ties to
    even; bf16 has float32's exponent range, subnormal step 2**-133), returned
    as float64.  NaN stays NaN; beyond the largest finite bf16 gives inf."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    _, e = np.frexp(x[fin])                          # |x| = m 2**e, 0.5 <= m < 1
    step = np.ldexp(1.0, np.maximum(e - 8, -133))    # spacing of bf16 values near x
    r = np.rint(x[fin] / step) * step                # np.rint rounds half to even
    big = np.ldexp(1.0, 128) - np.ldexp(1.0, 128 - 9)  # halfway past the largest finite bf16
    r = np.where(np.abs(x[fin]) >= big, np.copysign(np.inf, x[fin]), r)
    out[fin] = r
    return out


def round_to(x, dtype):
    """The stored value of x in ``dtype`` ("bf16", "f32", or "f64": unrounded), float64."""
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def mlp_stack(X, layers, dtype="bf16"):
    """Forward through a stack of layers; ``layers`` is a list of dicts with
    A_i, B_i, peers (the other ranks' partials of that layer, list), bias
    (or None) and act.  Returns (Z_l, X_{l+1}) per layer: the full output in
    float64 and the next layer's input, that output stored in ``dtype``."""
    x = _f64(X)
    out = []
    for layer in layers:
        z = mlp_rank(x, layer["A_i"], layer["B_i"], layer.get("act", GELU_ERF))
        for p in layer.get("peers", []):
            z = z + _f64(p)
        if layer.get("bias") is not None:
            z = z + _f64(layer["bias"])[None, :]
        x = round_to(z, dtype)
        out.append((z, x))
    return out


# ---- backward ([CAI] section 2.2; Domino article, "backward") --------------
#
# The loss is reached through Z, with dZ = dL/dZ given.  Since the forward is
# Z = sum_i act(X A_i) B_i, rank i's share of the chain rule is
#   dY_i = dZ B_i^T                  (row-parallel layer: no communication)
#   dH_i = dY_i * act'(X A_i)        (elementwise through the activation)
#   dX_i = dH_i A_i^T                (a partial: dX is the sum over ranks, the
#                                     all-reduce of the column-parallel layer)
#   dA_i = X^T dH_i,  dB_i = Y_i^T dZ   (weight gradients, no communication)


def gelu_deriv(x):
    """d/dx [x Phi(x)] = Phi(x) + x phi(x), phi the standard normal density, float64."""
    x = np.asarray(x, dtype=np.float64)
    cdf = 0.5 * (1.0 + _erf(x / math.sqrt(2.0)))
    pdf = np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)
    return cdf + x * pdf


def backward_rank(X, A_i, B_i, dZ, act=GELU_ERF):
    """Gradients of one rank's share, float64.

    Returns a dict with dH (gradient at the pre-activation X A_i, [M, F]),
    dX_i (this rank's partial input gradient, [M, H]), dA_i ([H, F]) and
    dB_i ([F, H]).
    """
    x, a, b, dz = _f64(X), _f64(A_i), _f64(B_i), _f64(dZ)
    if x.shape[1] != a.shape[0] or a.shape[1] != b.shape[0] or b.shape[1] != x.shape[1] or dz.shape != (x.shape[0], b.shape[1]):
        raise ValueError("shape mismatch")
    h = x @ a
    y = gelu(h) if act == GELU_ERF else h
    dy = dz @ b.T
    dh = dy * gelu_deriv(h) if act == GELU_ERF else dy
    return {"dH": dh, "dX_i": dh @ a.T, "dA_i": x.T @ dh, "dB_i": y.T @ dz}


def backward_all_ranks(X, A_shards, B_shards, dZ, act=GELU_ERF):
    """dX = sum over ranks of dX_i (the all-reduced input gradient), with the
    per-rank weight gradients."""
    outs = [backward_rank(X, a, b, dZ, act) for a, b in zip(A_shards, B_shards)]
    dX = outs[0]["dX_i"].copy()
    for o in outs[1:]:
        dX += o["dX_i"]
    return dX, [o["dA_i"] for o in outs], [o["dB_i"] for o in outs]
