"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every symbol the header declares, plans layouts exactly as the oracle does,
and rejects bad arguments with the oracle's error kinds before touching HIP."""
import ctypes as C
import os
import random
import re

import numpy as np
import pytest
import torch

import sharded_gemm_amd as tp
from sharded_gemm_amd import _abi
from oracle import layout as L

import test_oracle_layout as TL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _ensure_built():
    if not os.path.exists(_abi.LIB_PATH):
        from sharded_gemm_amd import build
        build.build()


def setup_module(_):
    _ensure_built()


def _header_functions():
    src = open(os.path.join(ROOT, "include", "tpshard.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tp_[a-z_]+)\s*\(", src)))


def test_header_symbols_exported():
    lib = _abi.load()
    names = _header_functions()
    assert set(names) == set(_abi.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert tp.version().startswith("tpshard")
    # Every entry point has its prototype declared on the binding side, so
    # 64-bit sizes and pointers are never passed as C ints.
    for n in names:
        assert getattr(lib, n).argtypes is not None, n
        assert getattr(lib, n).restype is not None, n


def test_kernel_kinds_match_header():
    """The binding's per-kernel timing names follow the header's TP_KERNEL_*
    enum, value for value, and the table is TP_KERNEL_KINDS long."""
    src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "tpshard.h")).read(), flags=re.S)
    kinds = {name.lower(): int(v) for name, v in re.findall(r"\bTP_KERNEL_([A-Z0-9_]+)\s*=\s*(\d+)", src)}
    n = kinds.pop("kinds")
    assert len(_abi.TP_KERNEL_NAMES) == n
    assert {name: k for k, name in enumerate(_abi.TP_KERNEL_NAMES)} == kinds


def test_reduce_fusion_constants_match_header():
    src = open(os.path.join(ROOT, "include", "tpshard.h")).read()
    vals = dict(re.findall(r"\b(TP_REDUCE_FUSION_[A-Z]+)\s*=\s*(\d+)", src))
    assert {k: int(v) for k, v in vals.items()} == {"TP_REDUCE_FUSION_AUTO": tp.TP_REDUCE_FUSION_AUTO,
                                                     "TP_REDUCE_FUSION_OFF": tp.TP_REDUCE_FUSION_OFF}
    vals = dict(re.findall(r"\b(TP_WEIGHTS_[A-Z]+)\s*=\s*(\d+)", src))
    assert {k: int(v) for k, v in vals.items()} == {"TP_WEIGHTS_MATH": tp.TP_WEIGHTS_MATH,
                                                     "TP_WEIGHTS_LINEAR": tp.TP_WEIGHTS_LINEAR}


def _oracle_plan(shape, spec):
    boxes, groups = L.shard_boxes(shape, spec)
    return boxes, groups


@pytest.mark.parametrize("with_map", [False, True])
def test_plan_matches_oracle_brute_force(with_map):
    rnd = random.Random(5 + with_map)
    for shape, axes, counts in TL._all_cases(max_cases=600, seed=13):
        nsh = int(np.prod(counts)) if counts else 1
        if with_map:
            devs = list(range(2 * nsh))
            rnd.shuffle(devs)
            spec = {"device": [-(k + 1) for k in range(nsh)],
                    "device_map": {-(k + 1): [devs[2 * k], devs[2 * k + 1]] for k in range(nsh)}}
        else:
            devs = list(range(nsh))
            rnd.shuffle(devs)
            spec = {"device": devs}
        spec["sharded_dim"] = [{"axis": a - len(shape) if k % 2 else a, "num_shards": n}
                               for k, (a, n) in enumerate(zip(axes, counts))]
        boxes, groups = _oracle_plan(shape, spec)
        ndst = max(max(g) for g in groups) + 2
        n, cboxes, sod = tp.tp_layout_plan(shape, spec, num_dst=ndst)
        assert n == len(boxes)
        assert [tuple(map(tuple, b)) for b in cboxes] == [tuple(b) for b in boxes]
        for k, grp in enumerate(groups):
            for d in grp:
                assert sod[d] == k
        assert sum(1 for s in sod if s >= 0) == sum(len(g) for g in groups)


def test_plan_mesh_matches_oracle():
    t = np.arange(4 * 6 * 8, dtype=np.float32).reshape(4, 6, 8)
    for mesh, dm in [([2, 4], [0, -1, 1]), ([2, 2], [1, -1, 0]), ([2, 3], [-1, 1, 0]), ([3, 2], [-1, 0, -1]),
                     ([2, 2, 2], [2, -1, 0]), ([4], [-1, -1, -1])]:
        ids = list(range(10, 10 + int(np.prod(mesh))))
        try:
            ref = L.split_dims_mapping(t, mesh, ids, dm)
        except L.OracleLayoutError as e:
            with pytest.raises(tp.TpError) as ce:
                tp.tp_layout_plan(t.shape, {"mesh_shape": mesh, "process_ids": ids, "dims_mapping": dm})
            assert ce.value.kind == e.kind
            continue
        n, boxes, sod = tp.tp_layout_plan(t.shape, {"mesh_shape": mesh, "process_ids": ids, "dims_mapping": dm},
                                          num_dst=max(ids) + 1)
        for d in ids:
            box = boxes[sod[d]]
            assert np.array_equal(t[tuple(slice(a, b) for a, b in box)], ref[d])


@pytest.mark.parametrize("spec,shape,kind", TL.test_rejections.pytestmark[0].args[1])
def test_plan_rejects_like_oracle(spec, shape, kind):
    with pytest.raises(tp.TpError) as e:
        tp.tp_layout_plan(shape, spec, num_dst=8)
    assert e.value.kind == kind


@pytest.mark.parametrize("mesh,ids,dm,shape,kind", TL.test_mesh_rejections.pytestmark[0].args[1])
def test_mesh_rejects_like_oracle(mesh, ids, dm, shape, kind):
    if len(ids) != int(np.prod(mesh)) or len(dm) != len(shape):
        pytest.skip("array length is implied by the C arguments")
    with pytest.raises(tp.TpError) as e:
        tp.tp_layout_plan(shape, {"mesh_shape": mesh, "process_ids": ids, "dims_mapping": dm})
    assert e.value.kind == kind


# --- argument validation of the launching entry points (returns before any HIP call) ---

FAKE = 1 << 40   # device-looking addresses; never dereferenced on these paths


@pytest.fixture(autouse=True)
def _no_visible_gpu():
    """These tests hand the library made-up device addresses and expect it to
    refuse them before any launch; where a GPU is visible a mistake in such a
    test could reach a kernel, so they run only where none is."""
    if torch.cuda.is_available():
        pytest.skip("validation tests with made-up device addresses run on hosts without a GPU")


def _mlp_args(**kw):
    a = _abi.tp_mlp_args(dtype=_abi.TP_BF16, act=_abi.TP_ACT_GELU_ERF, M=64, H=64, F=64,
                         X=FAKE, A_i=FAKE + (1 << 20), B_i=FAKE + (2 << 20), Y_ws=FAKE + (3 << 20),
                         Z_i=FAKE + (4 << 20), row_chunks=1, col_chunks=1, P=1, peer_partials=None, Z_out=None,
                         reduce_workgroups=0)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), _abi.TP_ERR_ARG),
    (dict(act=5), _abi.TP_ERR_ARG),
    (dict(M=0), _abi.TP_ERR_ARG),
    (dict(X=None), _abi.TP_ERR_ARG),
    (dict(row_chunks=3), _abi.TP_ERR_INDIVISIBLE),
    (dict(col_chunks=5), _abi.TP_ERR_INDIVISIBLE),
    (dict(row_chunks=0), _abi.TP_ERR_ARG),
    (dict(P=2), _abi.TP_ERR_ARG),
    (dict(P=65), _abi.TP_ERR_ARG),
    (dict(Y_ws=FAKE + 100), _abi.TP_ERR_ARG),          # overlaps X
    (dict(Z_i=FAKE + (3 << 20) + 64), _abi.TP_ERR_ARG),  # overlaps Y_ws
    (dict(reduce_workgroups=-1), _abi.TP_ERR_ARG),
    (dict(reduce_fusion=2), _abi.TP_ERR_ARG),
    (dict(reduce_fusion=-1), _abi.TP_ERR_ARG),
    (dict(weight_layout=2), _abi.TP_ERR_ARG),
    (dict(B_ld=63), _abi.TP_ERR_ARG),                   # B_i rows are H = 64 long
    (dict(A_ld=63), _abi.TP_ERR_ARG),                   # A_i rows are F = 64 long
    (dict(weight_layout=1, M=64, H=64, F=32, A_ld=32), _abi.TP_ERR_ARG),   # linear A_i rows are H = 64 long
    (dict(weight_layout=1, M=64, H=64, F=32, B_ld=31), _abi.TP_ERR_ARG),   # linear B_i rows are F = 32 long
])
def test_mlp_validation(kw, code):
    lib = _abi.load()
    a = _mlp_args(**kw)
    assert lib.tp_colrow_mlp(C.byref(a), None, None) == code
    assert lib.tp_last_error().decode() != ""


def test_mlp_peer_validation():
    lib = _abi.load()
    peers = (C.c_void_p * 1)(None)
    a = _mlp_args(P=2, peer_partials=C.cast(peers, C.POINTER(C.c_void_p)), Z_out=FAKE + (9 << 20))
    assert lib.tp_colrow_mlp(C.byref(a), None, None) == _abi.TP_ERR_ARG
    peers[0] = FAKE + (4 << 20) + 8   # overlaps Z_i
    assert lib.tp_colrow_mlp(C.byref(a), None, None) == _abi.TP_ERR_ARG


def _reduce(P=2, rows=8, cols=8, ld_in=8, mode=0, S=1, ld_out=8, parts=None, outs=None):
    lib = _abi.load()
    parts = parts if parts is not None else [FAKE + p * (1 << 20) for p in range(P)]
    outs = outs if outs is not None else [FAKE + (100 << 20) + j * (1 << 20) for j in range(S)]
    pin = (C.c_void_p * max(1, len(parts)))(*parts)
    pout = (C.c_void_p * max(1, len(outs)))(*outs)
    return lib.tp_partial_reduce(C.cast(pin, C.POINTER(C.c_void_p)), P, rows, cols, ld_in, mode, S,
                                 C.cast(pout, C.POINTER(C.c_void_p)), ld_out, None)


def test_reduce_validation():
    assert _reduce(P=0) == _abi.TP_ERR_ARG
    assert _reduce(P=65) == _abi.TP_ERR_UNSUPPORTED
    assert _reduce(ld_in=4) == _abi.TP_ERR_ARG
    assert _reduce(mode=3) == _abi.TP_ERR_ARG
    assert _reduce(mode=0, S=2) == _abi.TP_ERR_ARG
    assert _reduce(mode=1, S=3) == _abi.TP_ERR_INDIVISIBLE
    assert _reduce(mode=1, S=65, rows=65) == _abi.TP_ERR_UNSUPPORTED
    assert _reduce(parts=[FAKE, None]) == _abi.TP_ERR_ARG
    assert _reduce(outs=[FAKE + 16]) == _abi.TP_ERR_ARG        # overlaps partial 0, not in place
    assert _reduce(mode=1, S=2, outs=[FAKE + (100 << 20), FAKE + (100 << 20) + 32]) == _abi.TP_ERR_ARG


def test_materialize_validation():
    lib = _abi.load()
    spec = {"device": [0, 1], "sharded_dim": [{"axis": 0, "num_shards": 2}]}
    lay, keep = _abi.make_layout(spec)
    shape = (C.c_int64 * 2)(4, 4)
    good = (C.c_void_p * 2)(FAKE + (1 << 20), FAKE + (2 << 20))
    dptr = C.cast(good, C.POINTER(C.c_void_p))
    sp = C.cast(shape, C.POINTER(C.c_int64))
    assert lib.tp_shard_materialize(C.c_void_p(FAKE), 9, sp, 2, C.byref(lay), dptr, 2, None) == _abi.TP_ERR_ARG
    assert lib.tp_shard_materialize(None, 0, sp, 2, C.byref(lay), dptr, 2, None) == _abi.TP_ERR_ARG
    assert lib.tp_shard_materialize(C.c_void_p(FAKE), 0, sp, 2, C.byref(lay), dptr, 1, None) == _abi.TP_ERR_ARG
    bad = (C.c_void_p * 2)(FAKE + (1 << 20), None)
    assert lib.tp_shard_materialize(C.c_void_p(FAKE), 0, sp, 2, C.byref(lay),
                                    C.cast(bad, C.POINTER(C.c_void_p)), 2, None) == _abi.TP_ERR_ARG
    ovl = (C.c_void_p * 2)(FAKE + 8, FAKE + (2 << 20))
    assert lib.tp_shard_materialize(C.c_void_p(FAKE), 0, sp, 2, C.byref(lay),
                                    C.cast(ovl, C.POINTER(C.c_void_p)), 2, None) == _abi.TP_ERR_ARG
    ind = (C.c_int64 * 2)(3, 4)
    assert lib.tp_shard_materialize(C.c_void_p(FAKE), 0, C.cast(ind, C.POINTER(C.c_int64)), 2, C.byref(lay),
                                    dptr, 2, None) == _abi.TP_ERR_INDIVISIBLE


def test_materialize_local_device_validation():
    """local_only must be 0 or 1; local_device must lie in [0, num_dst) and be
    named by the layout; with it, the other dst entries may be NULL."""
    lib = _abi.load()
    spec = {"device": [0, 1], "sharded_dim": [{"axis": 0, "num_shards": 2}]}
    lay, keep = _abi.make_layout(spec)
    shape = (C.c_int64 * 2)(4, 4)
    sp = C.cast(shape, C.POINTER(C.c_int64))

    def item(ptrs, n, only, dev):
        arr = (C.c_void_p * max(1, n))(*ptrs)
        return arr, _abi.tp_materialize_item(src=FAKE, dtype=_abi.TP_F32, shape=sp, ndim=2, layout=C.pointer(lay),
                                             dst=C.cast(arr, C.POINTER(C.c_void_p)), num_dst=n, local_only=only,
                                             local_device=dev)
    for only, dev, n in ((2, 0, 2), (1, -1, 2), (1, 2, 2), (1, 3, 4)):
        arr, it = item([FAKE + (1 << 20)] * n, n, only, dev)
        assert lib.tp_shard_materialize_batch(C.byref(it), 1, None) == _abi.TP_ERR_ARG, (only, dev, n)
        assert lib.tp_last_error().decode() != ""
    # device 1's share alone with dst[0] NULL is accepted by validation; a NULL
    # dst[1] is not
    arr, it = item([None, None], 2, 1, 1)
    assert lib.tp_shard_materialize_batch(C.byref(it), 1, None) == _abi.TP_ERR_ARG


def test_missing_library_fails_loudly(tmp_path):
    saved = _abi._lib
    try:
        _abi._lib = None
        with pytest.raises(RuntimeError):
            _abi.load(str(tmp_path / "nope.so"))
    finally:
        _abi._lib = saved


def test_forward_saved_preactivation_validation():
    lib = _abi.load()
    assert lib.tp_colrow_mlp(C.byref(_mlp_args(act=_abi.TP_ACT_NONE, H_out=FAKE + (9 << 20))), None, None) == _abi.TP_ERR_ARG
    # H_out overlapping Y_ws
    assert lib.tp_colrow_mlp(C.byref(_mlp_args(H_out=FAKE + (3 << 20) + 64)), None, None) == _abi.TP_ERR_ARG


def _bwd_args(**kw):
    a = _abi.tp_mlp_bwd_args(dtype=_abi.TP_BF16, act=_abi.TP_ACT_GELU_ERF, M=64, H=64, F=64,
                             X=FAKE, A_i=FAKE + (1 << 20), B_i=FAKE + (2 << 20), H_i=FAKE + (3 << 20),
                             Y_i=FAKE + (4 << 20), dZ=FAKE + (5 << 20), dH_ws=FAKE + (6 << 20),
                             dX_i=FAKE + (7 << 20), dA_i=FAKE + (8 << 20), dB_i=FAKE + (9 << 20),
                             accumulate=0, row_chunks=1, P=1, peer_dX=None, dX_out=None, reduce_workgroups=0)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), _abi.TP_ERR_ARG),
    (dict(act=5), _abi.TP_ERR_ARG),
    (dict(M=0), _abi.TP_ERR_ARG),
    (dict(dZ=None), _abi.TP_ERR_ARG),
    (dict(dB_i=None), _abi.TP_ERR_ARG),
    (dict(H_i=None), _abi.TP_ERR_ARG),                    # the GeLU derivative needs the pre-activation
    (dict(accumulate=2), _abi.TP_ERR_ARG),
    (dict(row_chunks=3), _abi.TP_ERR_INDIVISIBLE),
    (dict(row_chunks=0), _abi.TP_ERR_ARG),
    (dict(P=2), _abi.TP_ERR_ARG),                         # P > 1 needs peers and dX_out
    (dict(P=65), _abi.TP_ERR_ARG),
    (dict(dH_ws=FAKE + 100), _abi.TP_ERR_ARG),            # overlaps X
    (dict(dA_i=FAKE + (9 << 20) + 64), _abi.TP_ERR_ARG),  # overlaps dB_i
    (dict(dX_i=FAKE + (5 << 20)), _abi.TP_ERR_ARG),       # overlaps dZ
    (dict(reduce_workgroups=-1), _abi.TP_ERR_ARG),
    (dict(weight_layout=3), _abi.TP_ERR_ARG),
])
def test_backward_validation(kw, code):
    lib = _abi.load()
    a = _bwd_args(**kw)
    assert lib.tp_colrow_mlp_backward(C.byref(a), None, None) == code
    assert lib.tp_last_error().decode() != ""


def test_backward_peer_validation():
    lib = _abi.load()
    peers = (C.c_void_p * 1)(None)
    a = _bwd_args(P=2, peer_dX=C.cast(peers, C.POINTER(C.c_void_p)), dX_out=FAKE + (20 << 20))
    assert lib.tp_colrow_mlp_backward(C.byref(a), None, None) == _abi.TP_ERR_ARG
    peers[0] = FAKE + (7 << 20) + 8   # overlaps dX_i
    assert lib.tp_colrow_mlp_backward(C.byref(a), None, None) == _abi.TP_ERR_ARG


def _reduce_ex(op=0, bias=None, **kw):
    lib = _abi.load()
    P, rows, cols = 2, 8, 8
    parts = [FAKE + p * (1 << 20) for p in range(P)]
    outs = kw.get("outs", [FAKE + (100 << 20)])
    pin = (C.c_void_p * P)(*parts)
    pout = (C.c_void_p * len(outs))(*outs)
    return lib.tp_partial_reduce_ex(C.cast(pin, C.POINTER(C.c_void_p)), P, rows, cols, cols, 0, 1,
                                    C.cast(pout, C.POINTER(C.c_void_p)), cols, op, bias, None)


def test_reduce_ex_validation():
    assert _reduce_ex(op=3) == _abi.TP_ERR_ARG
    assert _reduce_ex(op=-1) == _abi.TP_ERR_ARG
    assert _reduce_ex(op=1, bias=FAKE + (100 << 20) + 16) == _abi.TP_ERR_ARG   # bias inside the output


def test_mlp_bias_needs_z_out():
    lib = _abi.load()
    assert lib.tp_colrow_mlp(C.byref(_mlp_args(bias=FAKE + (30 << 20))), None, None) == _abi.TP_ERR_ARG
    # bias overlapping Z_out
    a = _mlp_args(bias=FAKE + (9 << 20) + 4, Z_out=FAKE + (9 << 20))
    assert lib.tp_colrow_mlp(C.byref(a), None, None) == _abi.TP_ERR_ARG


def _ptrs(xs):
    return C.cast((C.c_void_p * max(1, len(xs)))(*xs), C.POINTER(C.c_void_p))


def test_gather_validation():
    lib = _abi.load()
    spec = {"device": [-1, -2], "device_map": {-1: [0, 1], -2: [2, 3]}, "sharded_dim": [{"axis": 0, "num_shards": 2}]}
    lay, keep = _abi.make_layout(spec)
    sp = C.cast((C.c_int64 * 2)(4, 4), C.POINTER(C.c_int64))
    src_ok = [FAKE + (1 << 20), None, FAKE + (2 << 20), None]    # replicas 1 and 3 are not read
    out_ok = [FAKE + (10 << 20), FAKE + (11 << 20)]

    def g(src=src_ok, nsrc=4, dtype=0, out=out_ok, nout=None, shape=sp):
        return lib.tp_shard_gather(_ptrs(src), nsrc, dtype, shape, 2, C.byref(lay), _ptrs(out),
                                   len(out) if nout is None else nout, None)
    assert g(dtype=9) == _abi.TP_ERR_ARG
    assert g(nsrc=3) == _abi.TP_ERR_ARG                       # the layout names device 3
    assert g(src=[None, FAKE, FAKE + (2 << 20), None]) == _abi.TP_ERR_ARG   # device 0 is read
    assert g(nout=0) == _abi.TP_ERR_ARG
    assert g(out=[FAKE + (10 << 20), None]) == _abi.TP_ERR_ARG
    assert g(out=[FAKE + (10 << 20), FAKE + (10 << 20) + 32]) == _abi.TP_ERR_ARG   # outputs overlap
    assert g(out=[FAKE + (1 << 20) + 8]) == _abi.TP_ERR_ARG                        # output overlaps a shard
    assert g(shape=C.cast((C.c_int64 * 2)(3, 4), C.POINTER(C.c_int64))) == _abi.TP_ERR_INDIVISIBLE


def test_sequence_parallel_validation():
    lib = _abi.load()
    xs = [FAKE + (40 << 20) + j * (1 << 20) for j in range(4)]
    zs = [FAKE + (50 << 20) + j * (1 << 20) for j in range(4)]

    def fwd(**kw):
        return lib.tp_colrow_mlp(C.byref(_mlp_args(**kw)), None, None)
    assert fwd(X_shards=_ptrs(xs)) == _abi.TP_ERR_ARG                          # S not set
    assert fwd(seq_splits=65, X_shards=_ptrs(xs)) == _abi.TP_ERR_ARG
    assert fwd(seq_splits=-1) == _abi.TP_ERR_ARG
    assert fwd(seq_splits=3, X_shards=_ptrs(xs)) == _abi.TP_ERR_INDIVISIBLE     # 3 does not divide 64
    assert fwd(seq_splits=4, row_chunks=1, M=64, Z_split=_ptrs(zs), Z_out=FAKE + (60 << 20)) == _abi.TP_ERR_ARG
    assert fwd(seq_splits=4, X_shards=_ptrs([xs[0], None, xs[2], xs[3]])) == _abi.TP_ERR_ARG
    assert fwd(seq_splits=4, X_shards=_ptrs([xs[0], xs[1], FAKE + 8, xs[3]])) == _abi.TP_ERR_ARG   # shard inside X (written)
    assert fwd(seq_splits=4, Z_split=_ptrs([zs[0], zs[0] + 64, zs[2], zs[3]])) == _abi.TP_ERR_ARG   # blocks overlap
    # 24 rows: chunks of 8 (R = 3) and sequence blocks of 6 (S = 4) do not nest
    assert fwd(M=24, seq_splits=4, row_chunks=3, X_shards=_ptrs(xs)) == _abi.TP_ERR_UNSUPPORTED
    # X = NULL: GEMM1 would read the blocks in place, but a 64-row chunk over
    # blocks of 16 rows would put one tile across several blocks
    assert fwd(X=None, seq_splits=4, X_shards=_ptrs(xs)) == _abi.TP_ERR_UNSUPPORTED
    assert fwd(X=None, seq_splits=4, X_shards=_ptrs([xs[0], None, xs[2], xs[3]])) == _abi.TP_ERR_ARG

    def bwd(**kw):
        return lib.tp_colrow_mlp_backward(C.byref(_bwd_args(**kw)), None, None)
    assert bwd(dX_split=_ptrs(zs)) == _abi.TP_ERR_ARG
    assert bwd(seq_splits=3, dZ_shards=_ptrs(xs)) == _abi.TP_ERR_INDIVISIBLE
    assert bwd(seq_splits=4, dX_split=_ptrs(zs), dX_out=FAKE + (60 << 20)) == _abi.TP_ERR_ARG
    assert bwd(seq_splits=4, dZ_shards=_ptrs([xs[0], FAKE + (5 << 20) + 8, xs[2], xs[3]])) == _abi.TP_ERR_ARG  # in dZ
    assert bwd(M=24, seq_splits=4, row_chunks=3, dZ_shards=_ptrs(xs)) == _abi.TP_ERR_UNSUPPORTED


def test_32bit_index_limits_are_rejected():
    """Sizes past the kernels' 32-bit indexing are refused before any launch."""
    lib = _abi.load()
    # an MLP whose row chunk times column block reaches 2**31 elements
    assert lib.tp_colrow_mlp(C.byref(_mlp_args(M=1 << 16, H=1 << 15, F=64)), None, None) == _abi.TP_ERR_UNSUPPORTED
    # a reduce of 2**33 elements: 2**31 four-wide vectors
    parts = [FAKE, FAKE + (1 << 36)]
    outs = [FAKE + (2 << 36)]
    assert _reduce(P=2, rows=1 << 17, cols=1 << 16, ld_in=1 << 16, ld_out=1 << 16, parts=parts, outs=outs) == \
        _abi.TP_ERR_UNSUPPORTED
    # a shard of 2**36 bytes (bf16): 2**32 sixteen-byte vectors
    spec = {"device": [0], "sharded_dim": []}
    lay, keep = _abi.make_layout(spec)
    shape = (C.c_int64 * 1)(1 << 35)
    dst = (C.c_void_p * 1)(FAKE + (1 << 38))
    assert lib.tp_shard_materialize(C.c_void_p(FAKE), _abi.TP_BF16, C.cast(shape, C.POINTER(C.c_int64)), 1,
                                    C.byref(lay), C.cast(dst, C.POINTER(C.c_void_p)), 1, None) == _abi.TP_ERR_UNSUPPORTED


def test_group_beyond_launch_table_is_rejected():
    """One shard replicated to more than 64 devices cannot be written by one
    launch: rejected before any launch."""
    lib = _abi.load()
    spec = {"device": [-1], "device_map": {-1: list(range(65))}, "sharded_dim": []}
    lay, keep = _abi.make_layout(spec)
    shape = (C.c_int64 * 1)(64)
    dst = (C.c_void_p * 65)(*[FAKE + (d + 1) * (1 << 20) for d in range(65)])
    assert lib.tp_shard_materialize(C.c_void_p(FAKE), _abi.TP_F32, C.cast(shape, C.POINTER(C.c_int64)), 1,
                                    C.byref(lay), C.cast(dst, C.POINTER(C.c_void_p)), 65, None) == _abi.TP_ERR_UNSUPPORTED


def test_materialize_batch_validation():
    lib = _abi.load()
    spec = {"device": [0, 1], "sharded_dim": [{"axis": 0, "num_shards": 2}]}
    lay, keep = _abi.make_layout(spec)
    shape = (C.c_int64 * 2)(4, 4)
    d1 = (C.c_void_p * 2)(FAKE + (1 << 20), FAKE + (2 << 20))
    d2 = (C.c_void_p * 2)(FAKE + (3 << 20), FAKE + (4 << 20))

    def item(src, dst, dtype=_abi.TP_F32):
        return _abi.tp_materialize_item(src=src, dtype=dtype, shape=C.cast(shape, C.POINTER(C.c_int64)), ndim=2,
                                        layout=C.pointer(lay), dst=C.cast(dst, C.POINTER(C.c_void_p)), num_dst=2)
    arr = (_abi.tp_materialize_item * 2)(item(FAKE, d1), item(FAKE + (5 << 20), d2, dtype=9))
    assert lib.tp_shard_materialize_batch(arr, 2, None) == _abi.TP_ERR_ARG            # item 1: bad dtype
    assert "item 1" in lib.tp_last_error().decode()
    arr = (_abi.tp_materialize_item * 2)(item(FAKE, d1), item(FAKE + (1 << 20) + 8, d2))
    assert lib.tp_shard_materialize_batch(arr, 2, None) == _abi.TP_ERR_ARG            # item 1 reads item 0's output
    dsame = (C.c_void_p * 2)(FAKE + (1 << 20), FAKE + (6 << 20))
    arr = (_abi.tp_materialize_item * 2)(item(FAKE, d1), item(FAKE + (5 << 20), dsame))
    assert lib.tp_shard_materialize_batch(arr, 2, None) == _abi.TP_ERR_ARG            # two items write one buffer
    assert lib.tp_shard_materialize_batch(None, 1, None) == _abi.TP_ERR_ARG
    assert lib.tp_shard_materialize_batch(arr, -1, None) == _abi.TP_ERR_ARG


def test_binding_checks_sequence_blocks_and_bias():
    """The binding refuses sequence blocks and biases whose dtype, shape or
    layout differ from what the library assumes (it trusts their sizes), before
    any call into it.  Host tensors: nothing here reaches a kernel."""
    M, H, F, S = 64, 32, 16, 4
    X = torch.zeros((M, H), dtype=torch.bfloat16)
    A = torch.zeros((H, F), dtype=torch.bfloat16)
    B = torch.zeros((F, H), dtype=torch.bfloat16)
    Y = torch.zeros((M, F), dtype=torch.bfloat16)
    Z = torch.zeros((M, H))
    xs = [torch.zeros((M // S, H), dtype=torch.bfloat16) for _ in range(S)]
    zs = [torch.zeros((M // S, H)) for _ in range(S)]

    def fwd(**kw):
        tp.tp_colrow_mlp(X, A, B, Y, Z, **kw)
    with pytest.raises(TypeError):
        fwd(Z_split=[z.to(torch.bfloat16) for z in zs])                  # bf16 split output
    with pytest.raises(ValueError):
        fwd(Z_split=[torch.zeros((M // S - 1, H)) for _ in range(S)])    # short blocks
    with pytest.raises(ValueError):
        fwd(Z_split=[torch.zeros((H, M // S)).t() for _ in range(S)])    # not contiguous
    with pytest.raises(ValueError):
        fwd(X_shards=[torch.zeros((M // 3, H), dtype=torch.bfloat16) for _ in range(3)])   # 3 does not divide 64
    with pytest.raises(TypeError):
        fwd(X_shards=[x.float() for x in xs])                            # not X's dtype
    with pytest.raises(ValueError):
        fwd(X_shards=xs, Z_split=zs[:2])                                 # counts differ
    with pytest.raises(ValueError):
        tp.tp_colrow_mlp(None, A, B, Y, Z)                               # X = None needs X_shards
    with pytest.raises(ValueError):                                      # linear layout: A_i [F, H], B_i [H, F]
        fwd(weight_layout=tp.TP_WEIGHTS_LINEAR)
    with pytest.raises(ValueError):                                      # a weight with a column stride
        tp.tp_colrow_mlp(X, A, torch.zeros((H, F), dtype=torch.bfloat16).t(), Y, Z, s_compute=0, s_reduce=0)
    with pytest.raises(tp.TpError) as e:                                 # read in place: blocks of 16 rows
        tp.tp_colrow_mlp(None, A, B, Y, Z, X_shards=xs, s_compute=0, s_reduce=0)
    assert e.value.kind == "unsupported"
    with pytest.raises(TypeError):
        fwd(Z_out=torch.zeros((M, H)), bias=torch.zeros(H, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        fwd(Z_out=torch.zeros((M, H)), bias=torch.zeros(H - 1))
    with pytest.raises(ValueError):
        fwd(Z_out=torch.zeros((M, H)), bias=torch.zeros((H, 2))[:, 0])   # strided

    with pytest.raises(TypeError):
        tp.tp_partial_reduce([Z, Z.clone()], [torch.zeros((M, H))], bias=torch.zeros(H, dtype=torch.float64))
    with pytest.raises(ValueError):
        tp.tp_partial_reduce([Z, Z.clone()], [torch.zeros((M, H))], bias=torch.zeros(H + 1))

    dZ = torch.zeros((M, H), dtype=torch.bfloat16)
    dH = torch.zeros((M, F), dtype=torch.bfloat16)
    dX = torch.zeros((M, H))
    dA = torch.zeros((H, F))
    dB = torch.zeros((F, H))

    def bwd(**kw):
        tp.tp_colrow_mlp_backward(X, A, B, Y, Y, dZ, dH, dX, dA, dB, **kw)
    with pytest.raises(TypeError):
        bwd(dX_split=[z.to(torch.bfloat16) for z in zs])
    with pytest.raises(ValueError):
        bwd(dX_split=[torch.zeros((M // S, H + 1)) for _ in range(S)])
    with pytest.raises(TypeError):
        bwd(dZ_shards=[x.float() for x in xs])
    with pytest.raises(ValueError):
        bwd(dZ_shards=[torch.zeros((M // S + 1, H), dtype=torch.bfloat16) for _ in range(S)])


def test_noalloc_validation():
    """The allocation-free forward refuses a Y workspace and a row chunk of Y
    beyond its 32 MiB scratch before it touches the device."""
    lib = _abi.load()
    a = _mlp_args()
    a.Y_ws = FAKE + (3 << 20)
    assert lib.tp_colrow_mlp_noalloc(C.byref(a), None, None) == _abi.TP_ERR_ARG
    assert "Y_ws" in lib.tp_last_error().decode()
    a = _mlp_args(M=4096, F=8192, Y_ws=None)          # one chunk of 64 MiB of bf16
    assert lib.tp_colrow_mlp_noalloc(C.byref(a), None, None) == _abi.TP_ERR_UNSUPPORTED
    assert "scratch" in lib.tp_last_error().decode()
    a = _mlp_args(dtype=9, Y_ws=None)
    assert lib.tp_colrow_mlp_noalloc(C.byref(a), None, None) == _abi.TP_ERR_ARG
    assert lib.tp_colrow_mlp_noalloc(None, None, None) == _abi.TP_ERR_ARG


def test_column_slice_validation():
    """A_ld below F is refused; a column slice's strided extent counts in the overlap checks."""
    lib = _abi.load()
    a = _mlp_args(A_ld=32)                         # F = 64
    assert lib.tp_colrow_mlp(C.byref(a), None, None) == _abi.TP_ERR_ARG
    # A_i rows 256 elements apart: its last row reaches past Y_ws's start
    a = _mlp_args(A_ld=256 * 64, Y_ws=FAKE + (1 << 20) + 63 * 256 * 64 * 2 + 16)
    assert lib.tp_colrow_mlp(C.byref(a), None, None) == _abi.TP_ERR_ARG
    with pytest.raises(ValueError):
        tp.tp_colrow_mlp(torch.zeros((64, 64), dtype=torch.bfloat16), torch.zeros((64, 128), dtype=torch.bfloat16)[:, ::2],
                         torch.zeros((64, 64), dtype=torch.bfloat16), torch.zeros((64, 64), dtype=torch.bfloat16),
                         torch.zeros((64, 64)))
