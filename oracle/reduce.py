"""Oracle for partial-sum reduction (test infrastructure only; see the package header).

Sources:
* OneFlow global tensor article, section "SBP": under ``partial`` every device
  holds a tensor of the global shape, and adding them position by position
  gives the global tensor.
* ONNX multi-device proposal, operator-group rules, "reduction ops": a reduce
  over a sharded axis is a local reduce followed by a reduce across shards,
  whose default output is available to every participant.
* Same article, same section: besides sum, min and max also apply to
  ``partial``: the global tensor is the elementwise min / max over devices.
* ColossalAI 1D tensor parallelism, sections 2.1 (the row-parallel output is
  summed over ranks by one all-reduce), 3 and 5.3 (an all-reduce is a
  reduce-scatter followed by an all-gather; the reduce-scatter leaves rank j
  with block j of the sum), 5.2 (the row-parallel layer's bias acts on the
  full output: it is added once, after the sum).

Reading for the split form: block j of the sum along axis 0 (rows), for
``j < num_splits``; ``num_splits`` must divide the row count ("indivisible"
otherwise).  Sums are taken in float64.
"""
from __future__ import annotations

import numpy as np

from .layout import OracleLayoutError, _as_numpy


OPS = ("sum", "max", "min")


def reduce_full(partials, op="sum", bias=None):
    """out = op over p of partial_p, elementwise (sum accumulated in float64;
    max / min ignore a NaN against a number), then + bias along the last axis."""
    parts = [_as_numpy(p) for p in partials]
    if len(parts) < 1:
        raise OracleLayoutError("arg", "need at least one partial")
    if op not in OPS:
        raise OracleLayoutError("arg", f"unknown op {op}")
    shape = parts[0].shape
    acc = None
    for p in parts:
        if p.shape != shape:
            raise OracleLayoutError("arg", "partials differ in shape")
        v = p.astype(np.float64)
        if acc is None:
            acc = v.copy()
        elif op == "sum":
            acc += v
        elif op == "max":
            acc = np.fmax(acc, v)
        else:
            acc = np.fmin(acc, v)
    if bias is not None:
        b = _as_numpy(bias).astype(np.float64)
        if b.shape != (shape[-1],):
            raise OracleLayoutError("arg", "bias must have one value per column")
        acc = acc + b
    return acc


def reduce_split(partials, num_splits, op="sum", bias=None):
    """[out_0, ..., out_{S-1}]: out_j = rows [j*N/S, (j+1)*N/S) of the full reduction."""
    full = reduce_full(partials, op, bias)
    rows = full.shape[0]
    s = int(num_splits)
    if s < 1:
        raise OracleLayoutError("arg", "num_splits must be >= 1")
    if rows % s != 0:
        raise OracleLayoutError("indivisible", f"{rows} rows not divisible by {s}")
    h = rows // s
    return [full[j * h:(j + 1) * h].copy() for j in range(s)]
