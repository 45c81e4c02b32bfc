"""The host sharding checker in the C library against the checker oracle:
same output shards and device sets, same rejections (host only, no GPU)."""
import itertools
import random

import numpy as np
import pytest

import sharded_gemm_amd as tp
from sharded_gemm_amd import _abi
from oracle import checker as K
from oracle.layout import OracleLayoutError

import test_oracle_checker as TK

KIND = {"spec": _abi.TP_ERR_SPEC, "arg": _abi.TP_ERR_ARG, "indivisible": _abi.TP_ERR_INDIVISIBLE,
        "unsupported": _abi.TP_ERR_UNSUPPORTED}


def setup_module(_):
    import test_abi_cpu
    test_abi_cpu._ensure_built()


def _both(fn_c, fn_o):
    try:
        ref = fn_o()
    except OracleLayoutError as e:
        with pytest.raises(tp.TpError) as ce:
            fn_c()
        assert ce.value.code == KIND[e.kind], (e, ce.value)
        return None
    got = fn_c()
    return got, ref


def test_page_examples():
    c = TK._load()["composition"]
    got = tp.tp_check_broadcast_binary(c["shape1"], TK._spec(c["spec1"]), c["shape2"], TK._spec(c["spec2"]))
    assert [d for _, d in got[1]] == c["expected_devices"]
    bad = TK._load()["invalid_add"]
    with pytest.raises(tp.TpError) as e:
        tp.tp_check_broadcast_binary(bad["shape"], TK._spec(bad["spec1"]), bad["shape"], TK._spec(bad["spec2"]))
    assert e.value.kind == "spec"
    m = TK._load()["matmul"]
    assert tp.tp_infer_matmul_dims_mapping(m["x_map"], m["y_map"], m["mesh_ndim"]) == (m["expected_z_map"], -1)


def test_broadcast_matches_oracle_brute_force():
    rnd = random.Random(41)
    devices = list(range(8))
    n = 0
    for _ in range(1500):
        r = rnd.choice([1, 2, 3])
        base = [rnd.choice([2, 3, 4, 6]) for _ in range(r)]
        s1 = [d if rnd.random() < 0.7 else 1 for d in base]
        s2 = [d if rnd.random() < 0.7 else 1 for d in base]
        if rnd.random() < 0.2 and r > 1:
            s2 = s2[1:]
        if rnd.random() < 0.05:
            s2 = [d + 1 for d in s2]            # shapes that do not broadcast (mostly)
        sp1, sp2 = TK._random_spec(rnd, s1, devices), TK._random_spec(rnd, s2, devices)
        res = _both(lambda: tp.tp_check_broadcast_binary(s1, sp1, s2, sp2), lambda: K.broadcast_binary(s1, sp1, s2, sp2))
        if res is None:
            continue
        (gshape, gshards), (oshape, oshards) = res
        assert list(gshape) == list(oshape)
        assert [(tuple(b), list(d)) for b, d in gshards] == [(tuple(b), list(d)) for b, d in oshards]
        n += 1
    assert n > 150


@pytest.mark.parametrize("q", [1, 2, 3])
@pytest.mark.parametrize("ndim", [2, 3])
def test_matmul_matches_oracle_every_mapping(q, ndim):
    opts = list(range(-2, q + 1))     # includes out-of-range values
    for xm in itertools.product(opts, repeat=ndim):
        for ym in itertools.product(opts, repeat=ndim):
            res = _both(lambda: tp.tp_infer_matmul_dims_mapping(list(xm), list(ym), q),
                        lambda: K.matmul_dims_mapping(list(xm), list(ym), q))
            if res is None:
                continue
            (z, part), (oz, opart) = res
            assert z == oz and part == (opart[0] if opart else -1), (xm, ym)


def test_null_and_range_errors():
    import ctypes as C
    lib = _abi.load()
    a = (C.c_int64 * 2)(0, -1)
    z = (C.c_int64 * 2)()
    p = C.c_int64()
    ptr = lambda x: C.cast(x, C.POINTER(C.c_int64))
    assert lib.tp_infer_matmul_dims_mapping(None, ptr(a), 2, 2, ptr(z), C.byref(p)) == _abi.TP_ERR_ARG
    assert lib.tp_infer_matmul_dims_mapping(ptr(a), ptr(a), 1, 2, ptr(z), C.byref(p)) == _abi.TP_ERR_ARG
    assert lib.tp_infer_matmul_dims_mapping(ptr(a), ptr(a), 2, 0, ptr(z), C.byref(p)) == _abi.TP_ERR_ARG
