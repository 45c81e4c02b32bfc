"""Oracle for shard layouts (test infrastructure only; see the package header).

Sources, cited by page title and section:

* ONNX multi-device execution proposal ("ONNX 多设备执行提案解析：基于 ShardingSpec
  ..."), sections "Proto definitions" (ShardingSpecProto / ShardedDimProto /
  SimpleShardedDimProto field meaning), "Sharding as a Split", "index rule for
  multi-axis sharding", "note on divisibility", "Sharding as a Broadcast" and
  "mixing split and broadcast".
* OneFlow global tensor article, section "SBP" (split: concatenating the
  physical pieces restores the logical tensor; broadcast: every device holds a
  full copy) and section "2D SBP" (ranks matrix, placement.hierarchy).
* Paddle "SPMD 推导规则与 Pipeline 调度", sections "ProcessMesh" and
  "dims_mapping".
* ColossalAI 1D tensor parallelism, sections 5.1 (``gather_output``: the
  column layer's split outputs all-gathered along the last axis) and 5.3
  (sequence parallelism: the input all-gathered along the sequence axis); the
  gather functions below assemble that all-gathered tensor.

A spec is a plain dict::

    {"device": [ids or negative keys],
     "device_map": {negative key: [device ids]},          # optional
     "sharded_dim": [{"axis": a, "num_shards": n,          # shorthand, or
                      "dim_value": d},                     # d optional
                     {"axis": a, "simple_sharding": [{"num_shards": n, "dim_value": d}]}]}

Readings taken where the pages leave a step open (each also listed in the
design notes):
  * shards are enumerated with the first listed sharded_dim outermost (the
    page's a-outer / b-inner order for ascending axes);
  * a dim that num_shards does not divide is rejected ("indivisible"), as
    ColossalAI's Linear1D_Col does for out_features % tp_size != 0;
  * a physical device may receive at most one shard of one tensor;
  * more than one simple_sharding entry per axis is "unsupported".
"""
from __future__ import annotations

import itertools

import numpy as np


class OracleLayoutError(ValueError):
    """Rejected layout.  ``kind`` is one of "arg", "spec", "indivisible", "unsupported"."""

    def __init__(self, kind: str, msg: str):
        super().__init__(f"{kind}: {msg}")
        self.kind = kind


def _as_numpy(t):
    if isinstance(t, np.ndarray):
        return t
    try:  # torch tensor (bf16 has no numpy dtype: widen exactly to float32)
        import torch
        if isinstance(t, torch.Tensor):
            if t.dtype == torch.bfloat16:
                t = t.float()
            return t.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(t)


def _sharded_dims(spec):
    """(axis, num_shards, dim_value or None) per listed sharded_dim, as written."""
    out = []
    for sd in spec.get("sharded_dim", []):
        if "simple_sharding" in sd:
            ss = list(sd["simple_sharding"])
            if len(ss) != 1:
                # ShardedDimProto: the common case is a single SimpleShardedDimProto.
                raise OracleLayoutError("unsupported", "exactly one simple_sharding entry per axis")
            out.append((int(sd["axis"]), int(ss[0]["num_shards"]), ss[0].get("dim_value")))
        else:
            out.append((int(sd["axis"]), int(sd["num_shards"]), sd.get("dim_value")))
    return out


def expand_devices(spec):
    """Per shard k, the list of physical devices that receive it.

    A non-negative entry of ``device`` is a device; a negative one is a key
    into the device map and stands for every device of that group, in map
    order (ONNX proposal, "Sharding as a Broadcast").
    """
    dmap = {int(k): [int(d) for d in v] for k, v in spec.get("device_map", {}).items()}
    for k, grp in dmap.items():
        if k >= 0:
            raise OracleLayoutError("spec", f"device_map key {k} must be negative")
        if len(grp) == 0 or any(d < 0 for d in grp):
            raise OracleLayoutError("spec", f"device group {k} must list non-negative ids")
    groups = []
    for entry in spec["device"]:
        entry = int(entry)
        if entry >= 0:
            groups.append([entry])
        elif entry in dmap:
            groups.append(list(dmap[entry]))
        else:
            raise OracleLayoutError("spec", f"device key {entry} not in device_map")
    seen = set()
    for grp in groups:
        for d in grp:
            if d in seen:
                raise OracleLayoutError("spec", f"device {d} receives more than one shard")
            seen.add(d)
    return groups


def shard_boxes(shape, spec):
    """Normalise a spec and list the box of every shard.

    Returns ``(boxes, groups)``: ``boxes[k]`` is a tuple of ``(start, stop)``
    per tensor axis and ``groups[k]`` the devices that receive shard k.
    """
    shape = [int(d) for d in shape]
    r = len(shape)
    dims = _sharded_dims(spec)
    axes, counts = [], []
    for axis, n, dim_value in dims:
        # ShardedDimProto.axis lies in [-r, r-1]; a negative axis counts from the back.
        if not -r <= axis <= r - 1:
            raise OracleLayoutError("spec", f"axis {axis} out of range for rank {r}")
        a = axis + r if axis < 0 else axis
        if a in axes:
            raise OracleLayoutError("spec", f"axis {a} sharded twice")
        if n < 1:
            raise OracleLayoutError("spec", f"num_shards {n} < 1")
        if dim_value is not None and int(dim_value) != 0 and int(dim_value) != shape[a]:
            raise OracleLayoutError("spec", f"dim_value {dim_value} != dim {shape[a]}")
        if shape[a] % n != 0:
            raise OracleLayoutError("indivisible", f"dim {shape[a]} of axis {a} not divisible by {n}")
        axes.append(a)
        counts.append(n)
    total = 1
    for n in counts:
        total *= n
    if len(spec["device"]) != total:
        raise OracleLayoutError("spec", f"{len(spec['device'])} device entries for {total} shards")
    groups = expand_devices(spec)

    boxes = []
    # Shard k <-> digits (s_1, ..., s_m) of k in mixed radix (n_1, ..., n_m),
    # first listed axis most significant: the page's nested loops with the
    # first axis outermost, appending one slice per innermost iteration.
    for digits in itertools.product(*[range(n) for n in counts]):
        box = [(0, d) for d in shape]
        for a, n, s in zip(axes, counts, digits):
            w = shape[a] // n
            box[a] = (s * w, (s + 1) * w)
        boxes.append(tuple(box))
    return boxes, groups


def split(tensor, spec):
    """Materialise a ShardingSpec: ``{device id: its shard}`` (row-major copies).

    Each shard is the source restricted to its box (ONNX proposal, "index rule
    for multi-axis sharding"); each device of the shard's group gets a copy.
    """
    t = _as_numpy(tensor)
    boxes, groups = shard_boxes(t.shape, spec)
    out = {}
    for box, grp in zip(boxes, groups):
        piece = t[tuple(slice(a, b) for a, b in box)]
        for d in grp:
            out[d] = np.ascontiguousarray(piece).copy()
    return out


def _place(out, box, piece, who):
    piece = _as_numpy(piece)
    ext = tuple(b - a for a, b in box)
    if piece.shape != ext:
        raise OracleLayoutError("arg", f"piece of {who} has shape {piece.shape}, the layout gives {ext}")
    out[tuple(slice(a, b) for a, b in box)] = piece


def gather(pieces, shape, spec):
    """The inverse of ``split``: the logical tensor assembled from its pieces.

    ``pieces`` maps device id -> that device's shard.  OneFlow's SBP section
    defines split pieces as blocks that concatenate back to the logical tensor
    and broadcast pieces as full copies, so the logical tensor is every
    distinct shard written into its box.  ColossalAI's ``gather_output`` and
    the all-gather of sequence parallelism (sections 5.1 and 5.3) produce this
    tensor on every rank.  Replicas of a shard are equal by definition; the
    copy taken is the one on the first device the shard's group lists.
    """
    boxes, groups = shard_boxes(shape, spec)
    shape = tuple(int(d) for d in shape)
    first = None
    for grp in groups:
        if grp[0] not in pieces:
            raise OracleLayoutError("arg", f"no piece for device {grp[0]}")
        first = _as_numpy(pieces[grp[0]]) if first is None else first
    out = np.zeros(shape, dtype=first.dtype if first is not None else np.float32)
    for box, grp in zip(boxes, groups):
        _place(out, box, pieces[grp[0]], f"device {grp[0]}")
    return out


# --------------------------------------------------------------------------
# ProcessMesh + dims_mapping (Paddle SPMD-rules page; OneFlow 2D SBP)
# --------------------------------------------------------------------------

def mesh_shape(ranks):
    """Shape of a nested ranks list: the OneFlow placement ``hierarchy``.

    ``[0, 1, 2, 3, 4, 5]`` -> ``[6]``; ``[[0, 1, 2], [3, 4, 5]]`` -> ``[2, 3]``.
    """
    shape = []
    level = ranks
    while isinstance(level, (list, tuple)):
        shape.append(len(level))
        level = level[0] if len(level) else None
    return shape


def _check_mesh(shape, mesh_dims, process_ids, dims_mapping):
    q = len(mesh_dims)
    if any(m < 1 for m in mesh_dims):
        raise OracleLayoutError("spec", "mesh dims must be >= 1")
    count = 1
    for m in mesh_dims:
        count *= m
    if len(process_ids) != count:
        raise OracleLayoutError("spec", "process id count != mesh size")
    if len(set(process_ids)) != len(process_ids) or any(p < 0 for p in process_ids):
        raise OracleLayoutError("spec", "process ids must be distinct and >= 0")
    if len(dims_mapping) != len(shape):
        raise OracleLayoutError("spec", "dims_mapping length != tensor rank")
    used = set()
    for i, j in enumerate(dims_mapping):
        if not -1 <= j <= q - 1:
            raise OracleLayoutError("spec", f"dims_mapping[{i}] = {j} out of range")
        if j >= 0:
            if j in used:
                raise OracleLayoutError("spec", f"mesh dim {j} used by two tensor axes")
            used.add(j)
            if shape[i] % mesh_dims[j] != 0:
                raise OracleLayoutError("indivisible", f"dim {shape[i]} not divisible by mesh dim {mesh_dims[j]}")


def split_dims_mapping(tensor, mesh_dims, process_ids, dims_mapping):
    """``{process id: its local tensor}`` under a ProcessMesh and dims_mapping.

    Directly from the definition: ``dims_mapping[i] = j >= 0`` cuts tensor axis
    i into ``mesh_dims[j]`` equal blocks and the process at mesh coordinate
    ``c`` holds block ``c[j]``; ``-1`` leaves axis i whole (replicated).
    Process ids are laid out row-major over the mesh.
    """
    t = _as_numpy(tensor)
    shape = list(t.shape)
    mesh_dims = [int(m) for m in mesh_dims]
    process_ids = [int(p) for p in process_ids]
    dims_mapping = [int(j) for j in dims_mapping]
    _check_mesh(shape, mesh_dims, process_ids, dims_mapping)
    out = {}
    for linear, coord in enumerate(itertools.product(*[range(m) for m in mesh_dims])):
        sl = []
        for i, j in enumerate(dims_mapping):
            if j < 0:
                sl.append(slice(0, shape[i]))
            else:
                w = shape[i] // mesh_dims[j]
                sl.append(slice(coord[j] * w, (coord[j] + 1) * w))
        out[process_ids[linear]] = np.ascontiguousarray(t[tuple(sl)]).copy()
    return out


def gather_dims_mapping(pieces, shape, mesh_dims, process_ids, dims_mapping):
    """The inverse of ``split_dims_mapping``: the logical tensor from
    ``{process id: local tensor}``.  Processes whose mesh coordinates differ
    only along mesh dims no tensor axis uses hold the same block; the block is
    taken from the first of them in row-major mesh order."""
    shape = [int(d) for d in shape]
    mesh_dims = [int(m) for m in mesh_dims]
    process_ids = [int(p) for p in process_ids]
    dims_mapping = [int(j) for j in dims_mapping]
    _check_mesh(shape, mesh_dims, process_ids, dims_mapping)
    out = None
    done = set()
    for linear, coord in enumerate(itertools.product(*[range(m) for m in mesh_dims])):
        block = tuple(coord[j] if j >= 0 else 0 for j in dims_mapping)
        if block in done:
            continue
        done.add(block)
        pid = process_ids[linear]
        if pid not in pieces:
            raise OracleLayoutError("arg", f"no piece for process {pid}")
        if out is None:
            out = np.zeros(shape, dtype=_as_numpy(pieces[pid]).dtype)
        box = []
        for i, j in enumerate(dims_mapping):
            w = shape[i] // mesh_dims[j] if j >= 0 else shape[i]
            box.append((block[i] * w, block[i] * w + w) if j >= 0 else (0, shape[i]))
        _place(out, box, pieces[pid], f"process {pid}")
    return out
