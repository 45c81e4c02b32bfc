"""ctypes binding of libtpshard.so: argument marshalling only.

The functions here carry the C ABI's names (``tp_shard_materialize``,
``tp_colrow_mlp``, ``tp_partial_reduce``, ``tp_layout_plan``) and do nothing
but turn Python/torch arguments into the C structures and pointers the
library takes.  Every step of the path runs in the library's HIP kernels; if
the library is missing this module raises rather than falling back to
anything.
"""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libtpshard.so")

TP_OK = 0
TP_ERR_ARG = -1
TP_ERR_SPEC = -2
TP_ERR_INDIVISIBLE = -3
TP_ERR_UNSUPPORTED = -4
TP_ERR_HIP = -5
ERROR_NAMES = {TP_ERR_ARG: "arg", TP_ERR_SPEC: "spec", TP_ERR_INDIVISIBLE: "indivisible",
               TP_ERR_UNSUPPORTED: "unsupported", TP_ERR_HIP: "hip"}

TP_F32 = 0
TP_BF16 = 1
TP_LAYOUT_SPEC = 0
TP_LAYOUT_DIMS_MAPPING = 1
TP_REDUCE_FULL = 0
TP_REDUCE_SPLIT = 1
TP_ACT_NONE = 0
TP_ACT_GELU_ERF = 1
TP_REDUCE_OP_SUM = 0
TP_REDUCE_OP_MAX = 1
TP_REDUCE_OP_MIN = 2

# Every symbol include/tpshard.h declares.
EXPORTS = ("tp_last_error", "tp_version", "tp_layout_plan", "tp_check_broadcast_binary", "tp_infer_matmul_dims_mapping", "tp_shard_materialize", "tp_shard_materialize_batch", "tp_shard_gather",
           "tp_partial_reduce", "tp_partial_reduce_ex", "tp_colrow_mlp", "tp_colrow_mlp_noalloc", "tp_colrow_mlp_stack", "tp_colrow_mlp_backward", "tp_timing_enable", "tp_timing_read")

TP_KERNEL_NAMES = ("materialize", "gemm1", "gemm2", "reduce", "gemm_dgrad", "gemm_wgrad", "gather", "gemm2_reduce",
                   "gemm_dgrad_reduce", "reduce_tail")

TP_REDUCE_FUSION_AUTO = 0
TP_REDUCE_FUSION_OFF = 1

TP_WEIGHTS_MATH = 0
TP_WEIGHTS_LINEAR = 1


class TpError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"tpshard error {code} ({ERROR_NAMES.get(code, '?')}): {msg}")
        self.code = code
        self.kind = ERROR_NAMES.get(code, "?")


class tp_simple_sharding(C.Structure):
    _fields_ = [("dim_value", C.c_int64), ("num_shards", C.c_int64)]


class tp_sharded_dim(C.Structure):
    _fields_ = [("axis", C.c_int64), ("simple_sharding", C.POINTER(tp_simple_sharding)),
                ("num_simple_sharding", C.c_int64)]


class tp_device_group(C.Structure):
    _fields_ = [("key", C.c_int64), ("devices", C.POINTER(C.c_int64)), ("num_devices", C.c_int64)]


class tp_sharding_spec(C.Structure):
    _fields_ = [("device", C.POINTER(C.c_int64)), ("num_device", C.c_int64),
                ("device_map", C.POINTER(tp_device_group)), ("num_groups", C.c_int64),
                ("sharded_dim", C.POINTER(tp_sharded_dim)), ("num_sharded_dim", C.c_int64)]


class tp_process_mesh(C.Structure):
    _fields_ = [("shape", C.POINTER(C.c_int64)), ("ndim", C.c_int64), ("process_ids", C.POINTER(C.c_int64))]


class tp_layout(C.Structure):
    _fields_ = [("kind", C.c_int32), ("spec", tp_sharding_spec), ("mesh", tp_process_mesh),
                ("dims_mapping", C.POINTER(C.c_int64))]


class tp_mlp_args(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("act", C.c_int32),
                ("M", C.c_int64), ("H", C.c_int64), ("F", C.c_int64),
                ("X", C.c_void_p), ("A_i", C.c_void_p), ("B_i", C.c_void_p),
                ("Y_ws", C.c_void_p), ("Z_i", C.c_void_p),
                ("row_chunks", C.c_int64), ("col_chunks", C.c_int64), ("P", C.c_int64),
                ("peer_partials", C.POINTER(C.c_void_p)), ("Z_out", C.c_void_p),
                ("reduce_workgroups", C.c_int64), ("H_out", C.c_void_p), ("bias", C.c_void_p),
                ("seq_splits", C.c_int64), ("X_shards", C.POINTER(C.c_void_p)), ("Z_split", C.POINTER(C.c_void_p)),
                ("X_next", C.c_void_p), ("reduce_fusion", C.c_int32), ("A_ld", C.c_int64),
                ("weight_layout", C.c_int32), ("B_ld", C.c_int64)]


class tp_mlp_bwd_args(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("act", C.c_int32),
                ("M", C.c_int64), ("H", C.c_int64), ("F", C.c_int64),
                ("X", C.c_void_p), ("A_i", C.c_void_p), ("B_i", C.c_void_p),
                ("H_i", C.c_void_p), ("Y_i", C.c_void_p), ("dZ", C.c_void_p),
                ("dH_ws", C.c_void_p), ("dX_i", C.c_void_p), ("dA_i", C.c_void_p), ("dB_i", C.c_void_p),
                ("accumulate", C.c_int32), ("row_chunks", C.c_int64), ("P", C.c_int64),
                ("peer_dX", C.POINTER(C.c_void_p)), ("dX_out", C.c_void_p),
                ("reduce_workgroups", C.c_int64),
                ("seq_splits", C.c_int64), ("dZ_shards", C.POINTER(C.c_void_p)), ("dX_split", C.POINTER(C.c_void_p)),
                ("reduce_fusion", C.c_int32), ("weight_layout", C.c_int32)]


class tp_materialize_item(C.Structure):
    _fields_ = [("src", C.c_void_p), ("dtype", C.c_int32), ("shape", C.POINTER(C.c_int64)), ("ndim", C.c_int64),
                ("layout", C.POINTER(tp_layout)), ("dst", C.POINTER(C.c_void_p)), ("num_dst", C.c_int64),
                ("local_only", C.c_int32), ("local_device", C.c_int64)]


class tp_kernel_stat(C.Structure):
    _fields_ = [("launches", C.c_int64), ("total_ms", C.c_double), ("min_ms", C.c_double),
                ("max_ms", C.c_double), ("work", C.c_double)]


_lib = None


def load(path: str = LIB_PATH) -> C.CDLL:
    """Load the library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m sharded_gemm_amd.build` "
                           "(there is no fallback path)")
    lib = C.CDLL(path)
    i64p = C.POINTER(C.c_int64)
    lib.tp_last_error.restype = C.c_char_p
    lib.tp_last_error.argtypes = []
    lib.tp_version.restype = C.c_char_p
    lib.tp_version.argtypes = []
    lib.tp_layout_plan.restype = C.c_int
    lib.tp_layout_plan.argtypes = [i64p, C.c_int64, C.POINTER(tp_layout), i64p, i64p, C.c_int64, i64p, C.c_int64]
    lib.tp_shard_materialize.restype = C.c_int
    lib.tp_shard_materialize.argtypes = [C.c_void_p, C.c_int32, i64p, C.c_int64, C.POINTER(tp_layout),
                                         C.POINTER(C.c_void_p), C.c_int64, C.c_void_p]
    lib.tp_shard_materialize_batch.restype = C.c_int
    lib.tp_shard_materialize_batch.argtypes = [C.POINTER(tp_materialize_item), C.c_int64, C.c_void_p]
    lib.tp_shard_gather.restype = C.c_int
    lib.tp_shard_gather.argtypes = [C.POINTER(C.c_void_p), C.c_int64, C.c_int32, i64p, C.c_int64, C.POINTER(tp_layout),
                                    C.POINTER(C.c_void_p), C.c_int64, C.c_void_p]
    lib.tp_check_broadcast_binary.restype = C.c_int
    lib.tp_check_broadcast_binary.argtypes = [i64p, C.c_int64, C.POINTER(tp_layout), i64p, C.c_int64,
                                              C.POINTER(tp_layout), i64p, i64p, i64p, C.c_int64, i64p, i64p,
                                              C.c_int64]
    lib.tp_infer_matmul_dims_mapping.restype = C.c_int
    lib.tp_infer_matmul_dims_mapping.argtypes = [i64p, i64p, C.c_int64, C.c_int64, i64p, i64p]
    lib.tp_partial_reduce.restype = C.c_int
    lib.tp_partial_reduce.argtypes = [C.POINTER(C.c_void_p), C.c_int64, C.c_int64, C.c_int64, C.c_int64,
                                      C.c_int32, C.c_int64, C.POINTER(C.c_void_p), C.c_int64, C.c_void_p]
    lib.tp_partial_reduce_ex.argtypes = [C.POINTER(C.c_void_p), C.c_int64, C.c_int64, C.c_int64, C.c_int64,
                                         C.c_int32, C.c_int64, C.POINTER(C.c_void_p), C.c_int64, C.c_int32,
                                         C.c_void_p, C.c_void_p]
    lib.tp_partial_reduce_ex.restype = C.c_int
    lib.tp_colrow_mlp.restype = C.c_int
    lib.tp_colrow_mlp.argtypes = [C.POINTER(tp_mlp_args), C.c_void_p, C.c_void_p]
    lib.tp_colrow_mlp_noalloc.restype = C.c_int
    lib.tp_colrow_mlp_noalloc.argtypes = [C.POINTER(tp_mlp_args), C.c_void_p, C.c_void_p]
    lib.tp_colrow_mlp_stack.restype = C.c_int
    lib.tp_colrow_mlp_stack.argtypes = [C.POINTER(tp_mlp_args), C.c_int64, C.c_void_p, C.c_void_p]
    lib.tp_colrow_mlp_backward.argtypes = [C.POINTER(tp_mlp_bwd_args), C.c_void_p, C.c_void_p]
    lib.tp_colrow_mlp_backward.restype = C.c_int
    lib.tp_timing_enable.restype = C.c_int
    lib.tp_timing_enable.argtypes = [C.c_int32]
    lib.tp_timing_read.restype = C.c_int
    lib.tp_timing_read.argtypes = [C.POINTER(tp_kernel_stat)]
    _lib = lib
    return lib


def _check(rc: int):
    if rc != TP_OK:
        raise TpError(rc, load().tp_last_error().decode())


def _i64_array(vals):
    vals = [int(v) for v in vals]
    return (C.c_int64 * max(1, len(vals)))(*vals)


def make_layout(layout: dict):
    """Build a ``tp_layout`` from a dict.  Returns ``(struct, keepalive)``.

    ShardingSpec form::   {"device": [...], "device_map": {-1: [...]},
                           "sharded_dim": [{"axis": a, "num_shards": n, "dim_value": d}
                                           or {"axis": a, "simple_sharding": [{...}, ...]}]}
    Mesh form::           {"mesh_shape": [...], "process_ids": [...], "dims_mapping": [...]}
    """
    keep = []
    lay = tp_layout()
    if "dims_mapping" in layout:
        lay.kind = TP_LAYOUT_DIMS_MAPPING
        shp = _i64_array(layout["mesh_shape"])
        ids = _i64_array(layout["process_ids"])
        dm = _i64_array(layout["dims_mapping"])
        keep += [shp, ids, dm]
        lay.mesh = tp_process_mesh(C.cast(shp, C.POINTER(C.c_int64)), len(layout["mesh_shape"]),
                                   C.cast(ids, C.POINTER(C.c_int64)))
        lay.dims_mapping = C.cast(dm, C.POINTER(C.c_int64))
        return lay, keep
    lay.kind = TP_LAYOUT_SPEC
    dev = _i64_array(layout.get("device", []))
    keep.append(dev)
    groups = list(layout.get("device_map", {}).items())
    garr = (tp_device_group * max(1, len(groups)))()
    for g, (key, ids) in enumerate(groups):
        arr = _i64_array(ids)
        keep.append(arr)
        garr[g] = tp_device_group(int(key), C.cast(arr, C.POINTER(C.c_int64)), len(ids))
    keep.append(garr)
    sds = list(layout.get("sharded_dim", []))
    sarr = (tp_sharded_dim * max(1, len(sds)))()
    for m, sd in enumerate(sds):
        ss = sd["simple_sharding"] if "simple_sharding" in sd else [
            {"num_shards": sd["num_shards"], "dim_value": sd.get("dim_value", 0)}]
        ssarr = (tp_simple_sharding * max(1, len(ss)))()
        for q, e in enumerate(ss):
            ssarr[q] = tp_simple_sharding(int(e.get("dim_value", 0) or 0), int(e["num_shards"]))
        keep.append(ssarr)
        sarr[m] = tp_sharded_dim(int(sd["axis"]), C.cast(ssarr, C.POINTER(tp_simple_sharding)), len(ss))
    keep.append(sarr)
    lay.spec = tp_sharding_spec(C.cast(dev, C.POINTER(C.c_int64)), len(layout.get("device", [])),
                                C.cast(garr, C.POINTER(tp_device_group)), len(groups),
                                C.cast(sarr, C.POINTER(tp_sharded_dim)), len(sds))
    return lay, keep


def tp_layout_plan(shape, layout: dict, num_dst: int = 0, max_shards: int = 4096):
    """Host-only plan: ``(num_shards, boxes[k][axis] = (start, stop), shard_of_device)``."""
    lib = load()
    lay, keep = make_layout(layout)
    shp = _i64_array(shape)
    ndim = len(shape)
    n = C.c_int64(0)
    boxes = (C.c_int64 * max(1, max_shards * 2 * max(ndim, 1)))()
    sod = (C.c_int64 * max(1, num_dst))()
    _check(lib.tp_layout_plan(C.cast(shp, C.POINTER(C.c_int64)), ndim, C.byref(lay), C.byref(n),
                              C.cast(boxes, C.POINTER(C.c_int64)), max_shards,
                              C.cast(sod, C.POINTER(C.c_int64)), num_dst))
    k = min(n.value, max_shards)
    out_boxes = [[(boxes[(s * ndim + i) * 2], boxes[(s * ndim + i) * 2 + 1]) for i in range(ndim)]
                 for s in range(k)]
    return n.value, out_boxes, [sod[d] for d in range(num_dst)]


def _stream_ptr(stream):
    if stream is None:
        import torch
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if hasattr(stream, "cuda_stream"):
        return C.c_void_p(stream.cuda_stream)
    return C.c_void_p(int(stream))


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return TP_F32
    if t.dtype == torch.bfloat16:
        return TP_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def tp_shard_materialize(src, layout: dict, dst, stream=None):
    """Split/replicate ``src`` into ``dst`` (dict or list: device id -> tensor)."""
    lib = load()
    lay, keep = make_layout(layout)
    items = dst.items() if isinstance(dst, dict) else enumerate(dst)
    items = list(items)
    num_dst = (max(d for d, _ in items) + 1) if items else 0
    ptrs = (C.c_void_p * max(1, num_dst))()
    for d, t in items:
        ptrs[d] = _ptr(t) if t is not None else None
    shp = _i64_array(src.shape)
    _check(lib.tp_shard_materialize(C.c_void_p(_ptr(src)), _dtype_code(src), C.cast(shp, C.POINTER(C.c_int64)),
                                    src.dim(), C.byref(lay), C.cast(ptrs, C.POINTER(C.c_void_p)), num_dst,
                                    _stream_ptr(stream)))


def _tensors(*objs):
    """The tensors among objs, looking one level into lists, tuples and dict values."""
    out = []
    for o in objs:
        if hasattr(o, "data_ptr"):
            out.append(o)
        elif isinstance(o, dict):
            out += [v for v in o.values() if hasattr(v, "data_ptr")]
        elif isinstance(o, (list, tuple)):
            out += [v for v in o if hasattr(v, "data_ptr")]
    return out


class Prepared:
    """A library call whose arguments were marshalled once: calling it passes
    the same argument structures again, so a loop pays one C call per launch
    sequence.  It holds references to the tensors it points into, and a replay
    after any of them has moved (resized or re-pointed) raises instead of
    touching stale memory."""

    def __init__(self, fn, args, keep, streams, tensors=()):
        self._fn, self._args, self._keep, self._streams = fn, args, keep, streams
        self._tensors = [(t, t.data_ptr()) for t in tensors]

    def __call__(self, *streams):
        for t, p in self._tensors:
            if t.data_ptr() != p:
                raise TpError(-1, "a tensor of a prepared call has moved since it was prepared")
        ptrs = [_stream_ptr(s) for s in streams] if streams else self._streams
        if len(ptrs) < len(self._streams):
            ptrs = list(ptrs) + [ptrs[-1]] * (len(self._streams) - len(ptrs))
        _check(self._fn(*self._args, *ptrs))


def tp_shard_materialize_batch(jobs, stream=None, prepare=False):
    """Several tp_shard_materialize calls in one: ``jobs`` is a list of
    (src, layout, dst) with dst a dict or list (device id -> tensor), or of
    (src, layout, dst, local_device) to write only that device's share (the
    other entries of dst may be absent).  With ``prepare=True`` nothing runs; a
    ``Prepared`` call taking the stream is returned."""
    lib = load()
    keep, items = [], []
    for job in jobs:
        src, layout, dst = job[:3]
        local = job[3] if len(job) > 3 else None
        lay, k = make_layout(layout)
        pairs = list(dst.items() if isinstance(dst, dict) else enumerate(dst))
        num_dst = (max(d for d, _ in pairs) + 1) if pairs else 0
        ptrs = (C.c_void_p * max(1, num_dst))()
        for d, t in pairs:
            ptrs[d] = _ptr(t) if t is not None else None
        shp = _i64_array(src.shape)
        keep += [lay, k, ptrs, shp]
        items.append(tp_materialize_item(src=_ptr(src), dtype=_dtype_code(src), shape=C.cast(shp, C.POINTER(C.c_int64)),
                                         ndim=src.dim(), layout=C.pointer(lay),
                                         dst=C.cast(ptrs, C.POINTER(C.c_void_p)), num_dst=num_dst,
                                         local_only=0 if local is None else 1,
                                         local_device=0 if local is None else int(local)))
    arr = (tp_materialize_item * max(1, len(items)))(*items)
    if prepare:
        return Prepared(lib.tp_shard_materialize_batch, (arr, len(items)), keep, [_stream_ptr(stream)],
                        _tensors(*[j[0] for j in jobs], *[j[2] for j in jobs]))
    _check(lib.tp_shard_materialize_batch(arr, len(items), _stream_ptr(stream)))


def tp_check_broadcast_binary(shape1, layout1: dict, shape2, layout2: dict):
    """Output sharding of a broadcasting binary elementwise op: (out_shape,
    [(box, devices)]) with boxes as ((start, stop), ...) row-major over the
    output shards.  Host only."""
    lib = load()
    l1, k1 = make_layout(layout1)
    l2, k2 = make_layout(layout2)
    s1, s2 = _i64_array(shape1), _i64_array(shape2)
    r = max(len(shape1), len(shape2))
    out_shape = (C.c_int64 * max(1, r))()
    n = C.c_int64()
    args = [C.cast(s1, C.POINTER(C.c_int64)), len(shape1), C.byref(l1), C.cast(s2, C.POINTER(C.c_int64)),
            len(shape2), C.byref(l2), C.cast(out_shape, C.POINTER(C.c_int64)), C.byref(n)]
    _check(lib.tp_check_broadcast_binary(*args, None, 0, None, None, 0))
    S = n.value
    boxes = (C.c_int64 * max(1, 2 * r * S))()
    offs = (C.c_int64 * (S + 1))()
    _check(lib.tp_check_broadcast_binary(*args, C.cast(boxes, C.POINTER(C.c_int64)), S,
                                         C.cast(offs, C.POINTER(C.c_int64)), None, 0))
    devs = (C.c_int64 * max(1, offs[S]))()
    _check(lib.tp_check_broadcast_binary(*args, C.cast(boxes, C.POINTER(C.c_int64)), S,
                                         C.cast(offs, C.POINTER(C.c_int64)), C.cast(devs, C.POINTER(C.c_int64)),
                                         offs[S]))
    shards = []
    for k in range(S):
        box = tuple((boxes[(k * r + a) * 2], boxes[(k * r + a) * 2 + 1]) for a in range(r))
        shards.append((box, [devs[i] for i in range(offs[k], offs[k + 1])]))
    return [out_shape[a] for a in range(r)], shards


def tp_infer_matmul_dims_mapping(x_map, y_map, mesh_ndim):
    """(z_map, partial_mesh_dim) of matmul(X[..., M, K], Y[..., K, N]).  Host only."""
    lib = load()
    nd = len(x_map)
    if len(y_map) != nd:
        raise ValueError("x_map and y_map need the same length")
    xa, ya = _i64_array(x_map), _i64_array(y_map)
    z = (C.c_int64 * max(1, nd))()
    part = C.c_int64()
    _check(lib.tp_infer_matmul_dims_mapping(C.cast(xa, C.POINTER(C.c_int64)), C.cast(ya, C.POINTER(C.c_int64)), nd,
                                            mesh_ndim, C.cast(z, C.POINTER(C.c_int64)), C.byref(part)))
    return [z[i] for i in range(nd)], part.value


def tp_shard_gather(src, layout: dict, out, shape, stream=None):
    """All-gather: write the full tensor of ``shape`` assembled from the shards in
    ``src`` (dict or list: device id -> tensor, None where not read) into every
    tensor of the list ``out``."""
    lib = load()
    lay, keep = make_layout(layout)
    items = list(src.items() if isinstance(src, dict) else enumerate(src))
    num_src = (max(d for d, _ in items) + 1) if items else 0
    ptrs = (C.c_void_p * max(1, num_src))()
    dtype = None
    for d, t in items:
        ptrs[d] = _ptr(t) if t is not None else None
        if t is not None and dtype is None:
            dtype = _dtype_code(t)
    outs = list(out)
    if dtype is None:
        dtype = _dtype_code(outs[0])
    optr = (C.c_void_p * max(1, len(outs)))(*[_ptr(t) for t in outs])
    shp = _i64_array(shape)
    _check(lib.tp_shard_gather(C.cast(ptrs, C.POINTER(C.c_void_p)), num_src, dtype, C.cast(shp, C.POINTER(C.c_int64)),
                               len(shape), C.byref(lay), C.cast(optr, C.POINTER(C.c_void_p)), len(outs),
                               _stream_ptr(stream)))


def _check_bias(bias, cols):
    """A row-parallel bias is a contiguous fp32 vector of the output's width."""
    if bias is None:
        return
    import torch
    if not hasattr(bias, "data_ptr") or bias.dtype != torch.float32:
        raise TypeError("bias must be an fp32 tensor")
    if tuple(bias.shape) != (int(cols),) or not bias.is_contiguous():
        raise ValueError(f"bias must be a contiguous fp32 [{int(cols)}]")


def _seq_arrays(shards, split, M=None, H=None, in_dtype=None, shards_name="X_shards", split_name="Z_split"):
    """(S, ctypes array or None, ctypes array or None) for the sequence-parallel
    fields.  Each block is a contiguous [M/S, H] tensor: the shards in the
    input dtype, the split outputs fp32 (the library trusts these sizes)."""
    import torch
    shards = list(shards) if shards is not None else None
    split = list(split) if split is not None else None
    lens = {len(x) for x in (shards, split) if x is not None}
    if len(lens) > 1:
        raise ValueError("the input shards and the split outputs must have the same count")
    S = lens.pop() if lens else 0
    if S and M is not None:
        if M % S:
            raise ValueError(f"{S} sequence blocks do not divide M = {M}")
        want = (M // S, H)
        for name, xs, dt in ((shards_name, shards, in_dtype), (split_name, split, torch.float32)):
            for t in xs or ():
                if not hasattr(t, "data_ptr") or t.dtype != dt:
                    raise TypeError(f"every {name} block must be a {dt} tensor")
                if tuple(t.shape) != want or not t.is_contiguous():
                    raise ValueError(f"every {name} block must be a contiguous [{want[0]}, {want[1]}]")

    def arr(xs):
        return C.cast((C.c_void_p * len(xs))(*[_ptr(t) for t in xs]), C.POINTER(C.c_void_p)) if xs else None
    return S, arr(shards), arr(split)


def tp_partial_reduce(partials, out, mode=TP_REDUCE_FULL, rows=None, cols=None, ld_in=None, ld_out=None,
                      stream=None, op=TP_REDUCE_OP_SUM, bias=None):
    """Reduce fp32 ``partials`` (list of tensors or raw device pointers) into ``out`` (list)
    with ``op`` (sum, max or min), then add ``bias`` (fp32 [cols]) if given.

    With tensors, rows/cols/ld default to the 2-D shape of partials[0]."""
    lib = load()
    P = len(partials)
    t0 = partials[0]
    is_tensor = hasattr(t0, "data_ptr")
    if rows is None:
        rows, cols = int(t0.shape[0]), int(t0.shape[1])
    if ld_in is None:
        ld_in = int(t0.stride(0)) if is_tensor else cols
    if ld_out is None:
        ld_out = int(out[0].stride(0)) if hasattr(out[0], "data_ptr") else cols
    _check_bias(bias, cols)
    pin = (C.c_void_p * P)(*[(p.data_ptr() if hasattr(p, "data_ptr") else p) for p in partials])
    pout = (C.c_void_p * len(out))(*[(o.data_ptr() if hasattr(o, "data_ptr") else o) for o in out])
    if op == TP_REDUCE_OP_SUM and bias is None:
        _check(lib.tp_partial_reduce(C.cast(pin, C.POINTER(C.c_void_p)), P, rows, cols, ld_in, mode, len(out),
                                     C.cast(pout, C.POINTER(C.c_void_p)), ld_out, _stream_ptr(stream)))
    else:
        _check(lib.tp_partial_reduce_ex(C.cast(pin, C.POINTER(C.c_void_p)), P, rows, cols, ld_in, mode, len(out),
                                        C.cast(pout, C.POINTER(C.c_void_p)), ld_out, op, _ptr(bias),
                                        _stream_ptr(stream)))


def _mlp_args(X, A_i, B_i, Y_ws, Z_i, *, row_chunks=1, col_chunks=1, peer_partials=(), Z_out=None,
              act=TP_ACT_GELU_ERF, reduce_workgroups=0, H_out=None, bias=None, X_shards=None, Z_split=None,
              X_next=None, reduce_fusion=TP_REDUCE_FUSION_AUTO, weight_layout=TP_WEIGHTS_MATH):
    """(tp_mlp_args, keep-alive list) for one forward layer, shapes checked.
    X may be None with X_shards: GEMM1 then reads the blocks where they lie."""
    if X is None:
        if not X_shards:
            raise ValueError("X may be None only with X_shards")
        X_shards = list(X_shards)
        x0 = X_shards[0]
        if not hasattr(x0, "data_ptr") or x0.dim() != 2:
            raise TypeError("every X_shards block must be a 2-D tensor")
        M, H, xref = int(x0.shape[0]) * len(X_shards), int(x0.shape[1]), x0
    else:
        M, H, xref = int(X.shape[0]), int(X.shape[1]), X
    linear = weight_layout == TP_WEIGHTS_LINEAR
    F = int(A_i.shape[0] if linear else A_i.shape[1])
    peers = list(peer_partials)
    wa, wb = ((F, H), (H, F)) if linear else ((H, F), (F, H))
    if tuple(A_i.shape) != wa or tuple(B_i.shape) != wb or tuple(Z_i.shape) != (M, H) \
            or (Y_ws is not None and tuple(Y_ws.shape) != (M, F)):
        raise ValueError(f"shapes must be X[M,H], A_i{list(wa)}, B_i{list(wb)}, Y_ws[M,F], Z_i[M,H]")

    # A weight may be a column slice of the full weight (unit column stride, a
    # row stride of at least its row length): it is then read in place.
    def ld_of(t, name):
        if t.is_contiguous():
            return 0
        if t.dim() != 2 or t.stride(1) != 1 or t.stride(0) < t.shape[1]:
            raise ValueError(f"{name} must be contiguous or a column slice (unit column stride, row stride >= "
                             f"its row length)")
        return int(t.stride(0))
    A_ld, B_ld = ld_of(A_i, "A_i"), ld_of(B_i, "B_i")
    if not (xref.dtype == A_i.dtype == B_i.dtype) or (Y_ws is not None and Y_ws.dtype != xref.dtype):
        raise TypeError("X, A_i, B_i and Y_ws must share one dtype")
    for t in (H_out, X_next):
        if t is not None and t.dtype != xref.dtype:
            raise TypeError("H_out and X_next are in the input dtype")
    if H_out is not None and tuple(H_out.shape) != (M, F):
        raise ValueError("H_out must be [M, F]")
    if X_next is not None and tuple(X_next.shape) != (M, H):
        raise ValueError("X_next must be [M, H]")
    import torch
    for t in [Z_i, *peers] + ([Z_out] if Z_out is not None else []):
        if t.dtype != torch.float32 or tuple(t.shape) != (M, H):
            raise TypeError("Z_i, peer partials and Z_out must be fp32 [M, H]")
    _check_bias(bias, H)
    S, xs, zs = _seq_arrays(X_shards, Z_split, M, H, xref.dtype, "X_shards", "Z_split")
    parr = (C.c_void_p * max(1, len(peers)))(*[_ptr(p) for p in peers])
    args = tp_mlp_args(dtype=_dtype_code(xref), act=act, M=M, H=H, F=F,
                       X=_ptr(X), A_i=A_i.data_ptr(), B_i=B_i.data_ptr(), Y_ws=_ptr(Y_ws), Z_i=_ptr(Z_i),
                       row_chunks=row_chunks, col_chunks=col_chunks, P=1 + len(peers),
                       peer_partials=C.cast(parr, C.POINTER(C.c_void_p)) if peers else None,
                       Z_out=_ptr(Z_out), reduce_workgroups=reduce_workgroups, H_out=_ptr(H_out), bias=_ptr(bias),
                       X_next=_ptr(X_next), reduce_fusion=reduce_fusion, A_ld=A_ld,
                       weight_layout=weight_layout, B_ld=B_ld)
    args.seq_splits, args.X_shards, args.Z_split = S, xs, zs
    return args, [parr, xs, zs]


def tp_colrow_mlp(X, A_i, B_i, Y_ws, Z_i, *, s_compute=None, s_reduce=None, prepare=False, **kw):
    """One rank's MLP share: Y_ws = act(X A_i); Z_i = Y_ws B_i; Z_out = Z_i + sum(peers) (+ bias);
    optionally H_out = X A_i (the pre-activation kept for the backward) and X_next = the
    sum rounded to the input dtype (the next layer's input).

    Keywords: row_chunks, col_chunks, peer_partials, Z_out, act, reduce_workgroups, H_out,
    bias, X_shards, Z_split, X_next, weight_layout (TP_WEIGHTS_LINEAR: A_i is [F, H] and
    B_i [H, F], as a linear layer stores its weight; either may be a column slice of the
    full weight, read in place), reduce_fusion (TP_REDUCE_FUSION_AUTO lets GEMM2's
    epilogue take the reduction where nothing would run beside it; TP_REDUCE_FUSION_OFF
    keeps the separate reduction kernel; same bits either way).  Sequence parallelism: with ``X_shards`` (S tensors
    [M/S, H]) X is a workspace the call fills by all-gathering them, or None: GEMM1 then reads the blocks where
    they lie (the all-gather folded into its operand loads; X is not written); with ``Z_split``
    (S tensors [M/S, H] fp32) the sum is reduce-scattered into the blocks instead of
    written to Z_out.  With ``prepare=True`` nothing runs; a ``Prepared`` call taking
    (s_compute, s_reduce) is returned."""
    lib = load()
    args, keep = _mlp_args(X, A_i, B_i, Y_ws, Z_i, **kw)
    sc = _stream_ptr(s_compute)
    sr = _stream_ptr(s_reduce) if s_reduce is not None else sc
    if prepare:
        return Prepared(lib.tp_colrow_mlp, (C.byref(args),), keep + [args], [sc, sr],
                        _tensors(X, A_i, B_i, Y_ws, Z_i, *kw.values()))
    _check(lib.tp_colrow_mlp(C.byref(args), sc, sr))


def tp_colrow_mlp_noalloc(X, A_i, B_i, Z_i, *, s_compute=None, s_reduce=None, prepare=False, **kw):
    """tp_colrow_mlp without a Y workspace: the library keeps Y (one row chunk
    at a time, at most 32 MiB) in its own fixed device array and allocates
    nothing.  Same keywords and results as tp_colrow_mlp, except that Y is not
    returned.  Calls that overlap on one GPU race on that array."""
    lib = load()
    args, keep = _mlp_args(X, A_i, B_i, None, Z_i, **kw)
    sc = _stream_ptr(s_compute)
    sr = _stream_ptr(s_reduce) if s_reduce is not None else sc
    if prepare:
        return Prepared(lib.tp_colrow_mlp_noalloc, (C.byref(args),), keep + [args], [sc, sr],
                        _tensors(X, A_i, B_i, Z_i, *kw.values()))
    _check(lib.tp_colrow_mlp_noalloc(C.byref(args), sc, sr))


def tp_colrow_mlp_stack(layers, s_compute=None, s_reduce=None, prepare=False):
    """Forward layers in sequence with the inter-layer overlap (or one after another
    where each layer alone would keep to s_compute); ``layers`` is a list of dicts of
    tp_colrow_mlp's arguments (X, A_i, B_i, Y_ws, Z_i and keywords), each layer but
    the last writing the next one's X through X_next."""
    lib = load()
    built = [_mlp_args(**dict(layer)) for layer in layers]
    arr = (tp_mlp_args * max(1, len(built)))(*[b[0] for b in built])
    sc = _stream_ptr(s_compute)
    sr = _stream_ptr(s_reduce) if s_reduce is not None else sc
    if prepare:
        return Prepared(lib.tp_colrow_mlp_stack, (arr, len(built)), [built], [sc, sr],
                        _tensors(*[v for layer in layers for v in dict(layer).values()]))
    _check(lib.tp_colrow_mlp_stack(arr, len(built), sc, sr))


def tp_colrow_mlp_backward(X, A_i, B_i, H_i, Y_i, dZ, dH_ws, dX_i, dA_i, dB_i, *, row_chunks=1, peer_dX=(),
                           dX_out=None, act=TP_ACT_GELU_ERF, accumulate=False, s_compute=None, s_reduce=None,
                           reduce_workgroups=0, dZ_shards=None, dX_split=None,
                           reduce_fusion=TP_REDUCE_FUSION_AUTO, weight_layout=TP_WEIGHTS_MATH, prepare=False):
    """Backward of one rank's MLP share: dH_ws = (dZ B_i^T) * act'(H_i); dX_i = dH_ws A_i^T;
    dX_out = dX_i + sum(peers); dA_i (+)= X^T dH_ws; dB_i (+)= Y_i^T dZ.
    reduce_fusion as in tp_colrow_mlp (for the sum of dX).  weight_layout
    TP_WEIGHTS_LINEAR: A_i, dA_i are [F, H] and B_i, dB_i [H, F] (a linear layer's
    [out, in]).

    Sequence parallelism: with ``dZ_shards`` dZ is a workspace the call fills by
    all-gathering them; with ``dX_split`` the input gradient is reduce-scattered."""
    lib = load()
    linear = weight_layout == TP_WEIGHTS_LINEAR
    M, H = int(X.shape[0]), int(X.shape[1])
    F = int(A_i.shape[0] if linear else A_i.shape[1])
    peers = list(peer_dX)
    wa, wb = ((F, H), (H, F)) if linear else ((H, F), (F, H))
    if tuple(A_i.shape) != wa or tuple(B_i.shape) != wb or tuple(Y_i.shape) != (M, F) \
            or tuple(dZ.shape) != (M, H) or tuple(dH_ws.shape) != (M, F) or tuple(dX_i.shape) != (M, H) \
            or tuple(dA_i.shape) != wa or tuple(dB_i.shape) != wb \
            or (H_i is not None and tuple(H_i.shape) != (M, F)):
        raise ValueError(f"shapes must be X, dZ, dX_i [M,H]; A_i, dA_i {list(wa)}; B_i, dB_i {list(wb)}; "
                         "H_i, Y_i, dH_ws [M,F]")
    ins = [X, A_i, B_i, Y_i, dZ, dH_ws] + ([H_i] if H_i is not None else [])
    if any(t.dtype != X.dtype for t in ins):
        raise TypeError("X, A_i, B_i, H_i, Y_i, dZ and dH_ws must share one dtype")
    import torch
    for t in [dX_i, dA_i, dB_i, *peers] + ([dX_out] if dX_out is not None else []):
        if t.dtype != torch.float32:
            raise TypeError("dX_i, dA_i, dB_i, peer dX and dX_out must be fp32")
    for t in peers + ([dX_out] if dX_out is not None else []):
        if tuple(t.shape) != (M, H):
            raise ValueError("peer dX and dX_out must be [M, H]")
    parr = (C.c_void_p * max(1, len(peers)))(*[_ptr(p) for p in peers])
    args = tp_mlp_bwd_args(dtype=_dtype_code(X), act=act, M=M, H=H, F=F,
                           X=_ptr(X), A_i=_ptr(A_i), B_i=_ptr(B_i), H_i=_ptr(H_i), Y_i=_ptr(Y_i), dZ=_ptr(dZ),
                           dH_ws=_ptr(dH_ws), dX_i=_ptr(dX_i), dA_i=_ptr(dA_i), dB_i=_ptr(dB_i),
                           accumulate=1 if accumulate else 0, row_chunks=row_chunks, P=1 + len(peers),
                           peer_dX=C.cast(parr, C.POINTER(C.c_void_p)) if peers else None,
                           dX_out=_ptr(dX_out), reduce_workgroups=reduce_workgroups, reduce_fusion=reduce_fusion,
                           weight_layout=weight_layout)
    S, gs, xs = _seq_arrays(dZ_shards, dX_split, M, H, X.dtype, "dZ_shards", "dX_split")
    args.seq_splits, args.dZ_shards, args.dX_split = S, gs, xs
    sc = _stream_ptr(s_compute)
    sr = _stream_ptr(s_reduce) if s_reduce is not None else sc
    if prepare:
        return Prepared(lib.tp_colrow_mlp_backward, (C.byref(args),), [args, parr, gs, xs], [sc, sr],
                        _tensors(X, A_i, B_i, H_i, Y_i, dZ, dH_ws, dX_i, dA_i, dB_i, peers, dX_out, dZ_shards,
                                 dX_split))
    _check(lib.tp_colrow_mlp_backward(C.byref(args), sc, sr))


def tp_timing_enable(on: bool = True):
    _check(load().tp_timing_enable(1 if on else 0))


def tp_timing_read():
    """{kernel name: dict(launches, total_ms, min_ms, max_ms, work)} since the last read."""
    arr = (tp_kernel_stat * len(TP_KERNEL_NAMES))()
    _check(load().tp_timing_read(C.cast(arr, C.POINTER(tp_kernel_stat))))
    return {name: dict(launches=arr[k].launches, total_ms=arr[k].total_ms, min_ms=arr[k].min_ms,
                       max_ms=arr[k].max_ms, work=arr[k].work) for k, name in enumerate(TP_KERNEL_NAMES)}


def version() -> str:
    return load().tp_version().decode()
