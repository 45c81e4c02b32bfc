"""Oracle for the host sharding checker (test infrastructure only).

Sources, cited by page title and section:

* ONNX multi-device execution proposal, sharding formalism: "validity check"
  (an implementation should say why a spec is unsupported), the group of
  broadcasting n-ary elementwise operators (non-broadcast axes must be
  sharded identically in every input; with broadcast axes the output shard's
  devices are the intersection of the device sets of the input shards it is
  computed from, and an empty intersection makes the specs incompatible) and
  the composition example Add([M,1], [1,N]) that follows it.
* Paddle "SPMD 推导规则与 Pipeline 调度", the rules for computing operators:
  write the einsum notation, merge the inputs' dims_mapping per einsum axis
  (equal values, or -1 against a value; different values need a reshard), then
  read the output's dims_mapping off the merged axes; the worked
  matmul [0,-1] x [-1,1] -> [0,1].

Readings taken where the pages leave a step open:
  * inputs of different rank align on their trailing axes (the usual
    broadcasting convention; the pages' examples have equal ranks);
  * output shards are listed row-major over the output axes (axis 0 outermost);
  * a contracted einsum axis that is sharded leaves the output partial over
    that mesh dim (the ONNX page's reduction group: a local reduction and then
    a collective one);
  * one mesh dim may cut at most one einsum axis (as within one tensor).
"""
from __future__ import annotations

import itertools

from .layout import OracleLayoutError, shard_boxes


def _counts(shape, spec):
    """num_shards per axis of one input under its spec (1 where not sharded)."""
    r = len(shape)
    n = [1] * r
    for d in spec.get("sharded_dim", []):
        a = d["axis"] + r if d["axis"] < 0 else d["axis"]
        k = d.get("num_shards")
        if k is None:
            k = d["simple_sharding"][0]["num_shards"]
        n[a] = int(k)
    return n


def broadcast_binary(shape1, spec1, shape2, spec2):
    """Output sharding of a broadcasting binary elementwise operator.

    Returns ``(out_shape, shards)``: ``shards`` lists, row-major over the output
    axes, ``(box, devices)`` with ``box`` a tuple of ``(start, stop)`` per output
    axis and ``devices`` the sorted device ids that hold every input element the
    shard is computed from.
    """
    s1, s2 = [int(d) for d in shape1], [int(d) for d in shape2]
    r = max(len(s1), len(s2))
    p1, p2 = [1] * (r - len(s1)) + s1, [1] * (r - len(s2)) + s2
    out_shape = []
    for a in range(r):
        if p1[a] != p2[a] and 1 not in (p1[a], p2[a]):
            raise OracleLayoutError("arg", f"dims {p1[a]} and {p2[a]} of axis {a} do not broadcast")
        out_shape.append(max(p1[a], p2[a]))
    boxes1, groups1 = shard_boxes(s1, spec1)
    boxes2, groups2 = shard_boxes(s2, spec2)
    n1 = [1] * (r - len(s1)) + _counts(s1, spec1)
    n2 = [1] * (r - len(s2)) + _counts(s2, spec2)
    nout = []
    for a in range(r):
        carriers = [n for n, p in ((n1[a], p1[a]), (n2[a], p2[a])) if p != 1]
        if len(carriers) == 2 and carriers[0] != carriers[1]:
            raise OracleLayoutError("spec", f"axis {a} is not broadcast and the inputs cut it differently")
        nout.append(carriers[0] if carriers else 1)
    # Device sets of each input's shards, keyed by the shard's box padded to rank r.
    def by_box(shape, boxes, groups):
        pad = r - len(shape)
        return {tuple([(0, 1)] * pad + list(b)): set(g) for b, g in zip(boxes, groups)}
    d1, d2 = by_box(s1, boxes1, groups1), by_box(s2, boxes2, groups2)
    shards = []
    for idx in itertools.product(*[range(n) for n in nout]):
        box = tuple((i * (out_shape[a] // nout[a]), (i + 1) * (out_shape[a] // nout[a])) for a, i in enumerate(idx))
        # The piece of each input this shard reads: its own box on carried axes, [0, 1) on broadcast ones.
        need1 = tuple(box[a] if p1[a] != 1 else (0, 1) for a in range(r))
        need2 = tuple(box[a] if p2[a] != 1 else (0, 1) for a in range(r))
        devs = d1[need1] & d2[need2]
        if not devs:
            raise OracleLayoutError("spec", f"output shard {idx}: no device holds both input shards")
        shards.append((box, sorted(devs)))
    return out_shape, shards


def einsum_dims_mapping(notation, maps, mesh_ndim):
    """Paddle's three steps for a computing operator.

    ``notation`` like ``"mk,kn->mn"``; ``maps`` one dims_mapping per input.
    Returns ``(out_map, partial_mesh_dims)``: the output's dims_mapping and the
    sorted mesh dims over which the output is a partial sum (contracted axes
    that are cut).
    """
    lhs, out = notation.replace(" ", "").split("->")
    ins = lhs.split(",")
    if len(ins) != len(maps):
        raise OracleLayoutError("arg", "one dims_mapping per input")
    merged = {}
    for letters, m in zip(ins, maps):
        if len(letters) != len(m):
            raise OracleLayoutError("arg", f"dims_mapping {m} does not match {letters}")
        used = [j for j in m if j >= 0]
        if any(j < -1 or j >= mesh_ndim for j in m) or len(used) != len(set(used)):
            raise OracleLayoutError("spec", f"invalid dims_mapping {m}")
        for ax, j in zip(letters, m):
            cur = merged.get(ax, -1)
            if cur != -1 and j != -1 and cur != j:
                raise OracleLayoutError("spec", f"axis {ax} is cut by mesh dims {cur} and {j}: needs a reshard")
            merged[ax] = j if j != -1 else cur
    cut = [j for j in merged.values() if j >= 0]
    if len(cut) != len(set(cut)):
        raise OracleLayoutError("spec", "one mesh dim cuts two einsum axes")
    out_map = [merged[ax] for ax in out]
    partial = sorted(merged[ax] for ax in merged if ax not in out and merged[ax] >= 0)
    return out_map, partial


def matmul_dims_mapping(x_map, y_map, mesh_ndim):
    """matmul(X[..., M, K], Y[..., K, N]) with equal ranks (leading batch axes)."""
    r = len(x_map)
    if r < 2 or len(y_map) != r:
        raise OracleLayoutError("arg", "X and Y need the same rank >= 2")
    batch = "abcdefgh"[:r - 2]
    return einsum_dims_mapping(f"{batch}mk,{batch}kn->{batch}mn", [list(x_map), list(y_map)], mesh_ndim)
