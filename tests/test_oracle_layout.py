"""Pins for the layout oracle: the pages' worked examples, invariants, a
library special case and brute force against an independent inverse formula."""
import itertools
import json
import os
import random

import numpy as np
import pytest

from oracle import layout as L

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "onnx_sharding_examples.json")


def _load():
    with open(GOLDEN) as f:
        return json.load(f)


def _spec_from_json(js):
    spec = dict(js)
    if "device_map" in spec:
        spec["device_map"] = {int(k): v for k, v in spec["device_map"].items()}
    return spec


@pytest.mark.parametrize("case", _load()["cases"], ids=lambda c: c["name"])
def test_page_examples(case):
    t = np.array(_load()["tensor"], dtype=np.float32)
    got = L.split(t, _spec_from_json(case["spec"]))
    exp = {int(k): np.array(v, dtype=np.float32) for k, v in case["expected"].items()}
    assert sorted(got) == sorted(exp)
    for d in exp:
        assert got[d].shape == exp[d].shape, d
        assert np.array_equal(got[d], exp[d]), (d, got[d], exp[d])


@pytest.mark.parametrize("case", _load()["mesh_cases"], ids=lambda c: c["name"])
def test_page_2d_sbp_example(case):
    t = np.array(_load()["tensor"], dtype=np.float32)
    got = L.split_dims_mapping(t, case["mesh_shape"], case["process_ids"], case["dims_mapping"])
    exp = {int(k): np.array(v, dtype=np.float32) for k, v in case["expected"].items()}
    assert sorted(got) == sorted(exp)
    for d in exp:
        assert np.array_equal(got[d], exp[d])


@pytest.mark.parametrize("case", _load()["hierarchy_cases"], ids=lambda c: str(c["hierarchy"]))
def test_page_hierarchy(case):
    assert L.mesh_shape(case["ranks"]) == case["hierarchy"]


def test_dims_mapping_meaning_bsh():
    # Paddle SPMD page, "dims_mapping": [B,S,H] with [0,-1,1] cuts B along mesh
    # dim x, H along mesh dim y and keeps S whole.
    B, S, H = 4, 3, 6
    t = np.arange(B * S * H, dtype=np.float32).reshape(B, S, H)
    mesh = [2, 3]
    ids = [10, 11, 12, 13, 14, 15]
    got = L.split_dims_mapping(t, mesh, ids, [0, -1, 1])
    for x in range(2):
        for y in range(3):
            piece = got[ids[x * 3 + y]]
            assert piece.shape == (B // 2, S, H // 3)
            assert np.array_equal(piece, t[x * 2:(x + 1) * 2, :, y * 2:(y + 1) * 2])


def test_broadcast_replicas_equal_source():
    rng = np.random.default_rng(0)
    t = rng.standard_normal((3, 5, 2)).astype(np.float32)
    spec = {"device": [-7], "device_map": {-7: [4, 1, 9]}, "sharded_dim": []}
    got = L.split(t, spec)
    assert sorted(got) == [1, 4, 9]
    for d in got:
        assert np.array_equal(got[d], t)


def _shards_by_inverse_formula(t, axes, counts, groups):
    """Independent of the oracle: walk every *global* element, find the shard
    it falls in and its local index, and scatter it there."""
    shape = t.shape
    widths = {a: shape[a] // n for a, n in zip(axes, counts)}
    out_shape = [shape[i] // dict(zip(axes, counts)).get(i, 1) for i in range(len(shape))]
    nsh = int(np.prod(counts)) if counts else 1
    shards = [np.zeros(out_shape, dtype=t.dtype) for _ in range(nsh)]
    for g in itertools.product(*[range(s) for s in shape]):
        k = 0
        for a, n in zip(axes, counts):
            k = k * n + g[a] // widths[a]
        local = tuple(g[i] % widths[i] if i in widths else g[i] for i in range(len(shape)))
        shards[k][local] = t[g]
    res = {}
    for k, grp in enumerate(groups):
        for d in grp:
            res[d] = shards[k]
    return res


def _all_cases(max_cases=1500, seed=7):
    dims = [1, 2, 3, 4, 6]
    cases = []
    for r in (1, 2, 3):
        for shape in itertools.product(dims, repeat=r):
            for m in range(0, r + 1):
                for axes in itertools.permutations(range(r), m):
                    divs = [[n for n in range(1, shape[a] + 1) if shape[a] % n == 0] for a in axes]
                    for counts in itertools.product(*divs):
                        cases.append((shape, axes, counts))
    random.Random(seed).shuffle(cases)
    return cases[:max_cases]


@pytest.mark.parametrize("with_map", [False, True])
def test_brute_force_against_inverse_formula(with_map):
    rnd = random.Random(11 + with_map)
    for shape, axes, counts in _all_cases():
        t = np.arange(1, int(np.prod(shape)) + 1, dtype=np.float64).reshape(shape)
        nsh = int(np.prod(counts)) if counts else 1
        if with_map:
            devs = list(range(2 * nsh))
            rnd.shuffle(devs)
            groups = [[devs[2 * k], devs[2 * k + 1]] for k in range(nsh)]
            spec = {"device": [-(k + 1) for k in range(nsh)],
                    "device_map": {-(k + 1): groups[k] for k in range(nsh)}}
        else:
            devs = list(range(nsh))
            rnd.shuffle(devs)
            groups = [[d] for d in devs]
            spec = {"device": devs}
        # Mix negative axis spellings in (normalised by +rank).
        spec["sharded_dim"] = [{"axis": a - len(shape) if (a + k) % 2 else a, "num_shards": n}
                               for k, (a, n) in enumerate(zip(axes, counts))]
        got = L.split(t, spec)
        exp = _shards_by_inverse_formula(t, list(axes), list(counts), groups)
        assert sorted(got) == sorted(exp)
        for d in exp:
            assert np.array_equal(got[d], exp[d]), (shape, axes, counts, d)


def test_concat_restores_tensor():
    # OneFlow SBP "split": concatenating the physical pieces restores the tensor.
    rng = np.random.default_rng(3)
    t = rng.standard_normal((4, 6, 10)).astype(np.float32)
    spec = {"device": list(range(6)),
            "sharded_dim": [{"axis": 2, "num_shards": 2}, {"axis": 1, "num_shards": 3}]}
    got = L.split(t, spec)
    # first listed axis (2) outermost: shard k = s2 * 3 + s1
    cols = [np.concatenate([got[s2 * 3 + s1] for s1 in range(3)], axis=1) for s2 in range(2)]
    assert np.array_equal(np.concatenate(cols, axis=2), t)


def test_nested_numpy_split_special_case():
    # Library special case: np.split along the first listed axis, then each
    # piece along the second, yields the shards in a-outer / b-inner order.
    rng = np.random.default_rng(5)
    t = rng.standard_normal((6, 8)).astype(np.float32)
    spec = {"device": list(range(6)),
            "sharded_dim": [{"axis": 0, "num_shards": 3}, {"axis": -1, "num_shards": 2}]}
    got = L.split(t, spec)
    ref = [q for p in np.split(t, 3, axis=0) for q in np.split(p, 2, axis=1)]
    for k, q in enumerate(ref):
        assert np.array_equal(got[k], q)


def test_dims_mapping_matches_equivalent_spec():
    # Route agreement: mesh + dims_mapping, then broadcast each process's block
    # to 2 devices, equals one fused ShardingSpec with a device map.
    rng = np.random.default_rng(9)
    t = rng.standard_normal((4, 3, 8)).astype(np.float32)
    mesh = [2, 4]
    ids = list(range(8))
    by_mesh = L.split_dims_mapping(t, mesh, ids, [0, -1, 1])
    fused = {"device": [-(k + 1) for k in range(8)],
             "device_map": {-(k + 1): [2 * k, 2 * k + 1] for k in range(8)},
             "sharded_dim": [{"axis": 0, "num_shards": 2}, {"axis": 2, "num_shards": 4}]}
    got = L.split(t, fused)
    for k in range(8):
        for d in (2 * k, 2 * k + 1):
            assert np.array_equal(got[d], by_mesh[k])


@pytest.mark.parametrize("spec,shape,kind", [
    ({"device": [0, 1], "sharded_dim": [{"axis": 2, "num_shards": 2}]}, (2, 2), "spec"),
    ({"device": [0, 1], "sharded_dim": [{"axis": -3, "num_shards": 2}]}, (2, 2), "spec"),
    ({"device": [0, 1, 2, 3], "sharded_dim": [{"axis": 0, "num_shards": 2}, {"axis": -2, "num_shards": 2}]}, (2, 2), "spec"),
    ({"device": [0, 1, 2], "sharded_dim": [{"axis": 0, "num_shards": 2}]}, (2, 2), "spec"),
    ({"device": [0, 1, 2], "sharded_dim": [{"axis": 0, "num_shards": 3}]}, (4, 2), "indivisible"),
    ({"device": [0, 0], "sharded_dim": [{"axis": 0, "num_shards": 2}]}, (2, 2), "spec"),
    ({"device": [-1, 1], "device_map": {-1: [0, 1]}, "sharded_dim": [{"axis": 0, "num_shards": 2}]}, (2, 2), "spec"),
    ({"device": [-2], "device_map": {-1: [0, 1]}, "sharded_dim": []}, (2, 2), "spec"),
    ({"device": [1], "device_map": {1: [0, 1]}, "sharded_dim": []}, (2, 2), "spec"),
    ({"device": [0, 1], "sharded_dim": [{"axis": 0, "num_shards": 2, "dim_value": 3}]}, (2, 2), "spec"),
    ({"device": [0, 1], "sharded_dim": [{"axis": 0, "simple_sharding": [{"num_shards": 2}, {"num_shards": 1}]}]}, (2, 2), "unsupported"),
    ({"device": [], "sharded_dim": [{"axis": 0, "num_shards": 0}]}, (2, 2), "spec"),
])
def test_rejections(spec, shape, kind):
    with pytest.raises(L.OracleLayoutError) as e:
        L.split(np.zeros(shape, np.float32), spec)
    assert e.value.kind == kind


@pytest.mark.parametrize("mesh,ids,dm,shape,kind", [
    ([2, 2], [0, 1, 2, 3], [0, 0], (2, 2), "spec"),
    ([2, 2], [0, 1, 2, 3], [2, -1], (2, 2), "spec"),
    ([2, 2], [0, 1, 2], [0, -1], (2, 2), "spec"),
    ([2, 2], [0, 1, 2, 2], [0, -1], (2, 2), "spec"),
    ([3], [0, 1, 2], [0, -1], (2, 2), "indivisible"),
    ([2], [0, 1], [0], (2, 2), "spec"),
])
def test_mesh_rejections(mesh, ids, dm, shape, kind):
    with pytest.raises(L.OracleLayoutError) as e:
        L.split_dims_mapping(np.zeros(shape, np.float32), mesh, ids, dm)
    assert e.value.kind == kind


def test_zero_size_axis():
    t = np.zeros((0, 4), np.float32)
    got = L.split(t, {"device": [0, 1], "sharded_dim": [{"axis": 1, "num_shards": 2}]})
    assert got[0].shape == (0, 2) and got[1].shape == (0, 2)
