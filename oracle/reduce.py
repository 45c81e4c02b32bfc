"""Oracle for partial-sum reduction (test infrastructure only; see the package header).

Sources:
* OneFlow global tensor article, section "SBP": under ``partial`` every device
  holds a tensor of the global shape, and adding them position by position
  gives the global tensor.
* ONNX multi-device proposal, operator-group rules, "reduction ops": a reduce
  over a sharded axis is a local reduce followed by a reduce across shards,
  whose default output is available to every participant.
* ColossalAI 1D tensor parallelism, sections 2.1 (the row-parallel output is
  summed over ranks by one all-reduce), 3 and 5.3 (an all-reduce is a
  reduce-scatter followed by an all-gather; the reduce-scatter leaves rank j
  with block j of the sum).

Reading for the split form: block j of the sum along axis 0 (rows), for
``j < num_splits``; ``num_splits`` must divide the row count ("indivisible"
otherwise).  Sums are taken in float64.
"""
from __future__ import annotations

import numpy as np

from .layout import OracleLayoutError, _as_numpy


def reduce_full(partials):
    """out = sum over p of partial_p, elementwise, accumulated in float64."""
    parts = [_as_numpy(p) for p in partials]
    if len(parts) < 1:
        raise OracleLayoutError("arg", "need at least one partial")
    shape = parts[0].shape
    acc = np.zeros(shape, dtype=np.float64)
    for p in parts:
        if p.shape != shape:
            raise OracleLayoutError("arg", "partials differ in shape")
        acc += p.astype(np.float64)
    return acc


def reduce_split(partials, num_splits):
    """[out_0, ..., out_{S-1}]: out_j = rows [j*N/S, (j+1)*N/S) of the full sum."""
    full = reduce_full(partials)
    rows = full.shape[0]
    s = int(num_splits)
    if s < 1:
        raise OracleLayoutError("arg", "num_splits must be >= 1")
    if rows % s != 0:
        raise OracleLayoutError("indivisible", f"{rows} rows not divisible by {s}")
    h = rows // s
    return [full[j * h:(j + 1) * h].copy() for j in range(s)]
