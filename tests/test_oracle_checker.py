"""Pins for the checker oracle: the pages' worked examples, and brute force
against what the layouts mean (which device holds which elements, and what
each process's local product is)."""
import itertools
import json
import os
import random

import numpy as np
import pytest

from oracle import checker as K
from oracle import layout as L
from oracle.layout import OracleLayoutError

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "checker_examples.json")


def _load():
    with open(GOLDEN) as f:
        return json.load(f)


def _spec(js):
    spec = dict(js)
    if "device_map" in spec:
        spec["device_map"] = {int(k): v for k, v in spec["device_map"].items()}
    return spec


def test_page_composition_example():
    c = _load()["composition"]
    out_shape, shards = K.broadcast_binary(c["shape1"], _spec(c["spec1"]), c["shape2"], _spec(c["spec2"]))
    assert out_shape == [4, 6]
    assert [d for _, d in shards] == c["expected_devices"]
    assert [b for b, _ in shards] == [((0, 2), (0, 3)), ((0, 2), (3, 6)), ((2, 4), (0, 3)), ((2, 4), (3, 6))]


def test_page_invalid_add_is_rejected():
    c = _load()["invalid_add"]
    with pytest.raises(OracleLayoutError) as e:
        K.broadcast_binary(c["shape"], _spec(c["spec1"]), c["shape"], _spec(c["spec2"]))
    assert e.value.kind == "spec"


def test_page_matmul_example():
    c = _load()["matmul"]
    z, partial = K.matmul_dims_mapping(c["x_map"], c["y_map"], c["mesh_ndim"])
    assert z == c["expected_z_map"] and partial == []


def test_empty_intersection_is_incompatible():
    s1 = {"device": [-1, -2], "device_map": {-1: [0, 1], -2: [2, 3]}, "sharded_dim": [{"axis": 0, "num_shards": 2}]}
    s2 = {"device": [-1, -2], "device_map": {-1: [4, 5], -2: [6, 7]}, "sharded_dim": [{"axis": 1, "num_shards": 2}]}
    with pytest.raises(OracleLayoutError) as e:
        K.broadcast_binary([4, 1], s1, [1, 6], s2)
    assert e.value.kind == "spec"


def test_shapes_that_do_not_broadcast():
    s = {"device": [0], "sharded_dim": []}
    with pytest.raises(OracleLayoutError) as e:
        K.broadcast_binary([4, 3], s, [4, 2], s)
    assert e.value.kind == "arg"


def _holds(pieces_boxes, d, need):
    """Device d's box covers the region `need` (tuples of (start, stop))."""
    return any(all(b0 <= n0 and n1 <= b1 for (b0, b1), (n0, n1) in zip(box, need))
               for dev, box in pieces_boxes if dev == d)


def _device_boxes(shape, spec, r):
    boxes, groups = L.shard_boxes(shape, spec)
    pad = r - len(shape)
    return [(d, tuple([(0, 1)] * pad + list(b))) for b, g in zip(boxes, groups) for d in g]


def _random_spec(rnd, shape, devices):
    axes = [a for a in range(len(shape)) if shape[a] > 1 and rnd.random() < 0.6]
    counts = [rnd.choice([n for n in (1, 2, 3) if shape[a] % n == 0]) for a in axes]
    while int(np.prod(counts)) > len(devices):
        axes, counts = axes[:-1], counts[:-1]
    nsh = int(np.prod(counts)) if counts else 1
    grp = rnd.choice([1, 2])
    pool = list(devices)
    rnd.shuffle(pool)
    if grp == 1 or len(pool) < 2 * nsh:
        spec = {"device": pool[:nsh]}
    else:
        spec = {"device": [-(k + 1) for k in range(nsh)],
                "device_map": {-(k + 1): pool[2 * k:2 * k + 2] for k in range(nsh)}}
    spec["sharded_dim"] = [{"axis": a, "num_shards": n} for a, n in zip(axes, counts)]
    return spec


def test_brute_force_device_sets_are_exactly_the_capable_devices():
    """For random shapes with size-1 axes and random specs: every inferred
    device holds all input elements its output shard reads and computes the
    right values from its own pieces; every other device lacks some element.
    A rejection happens exactly when a non-broadcast axis is cut differently or
    some output shard has no capable device."""
    rnd = random.Random(3)
    devices = list(range(8))
    accepted = rejected = 0
    for _ in range(1000):
        r = rnd.choice([1, 2, 3])
        base = [rnd.choice([2, 3, 4, 6]) for _ in range(r)]
        s1 = [d if rnd.random() < 0.7 else 1 for d in base]
        s2 = [d if rnd.random() < 0.7 else 1 for d in base]
        if rnd.random() < 0.2 and r > 1:
            s2 = s2[1:]                         # lower rank, aligned on trailing axes
        sp1, sp2 = _random_spec(rnd, s1, devices), _random_spec(rnd, s2, devices)
        x1 = np.arange(1, int(np.prod(s1)) + 1, dtype=np.float64).reshape(s1)
        x2 = 1000.0 * np.arange(1, int(np.prod(s2)) + 1, dtype=np.float64).reshape(s2)
        full = x1 + x2
        rr = full.ndim
        b1, b2 = _device_boxes(s1, sp1, rr), _device_boxes(s2, sp2, rr)
        p1 = [1] * (rr - len(s1)) + s1
        p2 = [1] * (rr - len(s2)) + s2
        n1 = [1] * (rr - len(s1)) + K._counts(s1, sp1)
        n2 = [1] * (rr - len(s2)) + K._counts(s2, sp2)
        cut_differently = any(p1[a] != 1 and p2[a] != 1 and n1[a] != n2[a] for a in range(rr))
        try:
            out_shape, shards = K.broadcast_binary(s1, sp1, s2, sp2)
        except OracleLayoutError as e:
            rejected += 1
            if cut_differently:
                assert e.kind == "spec"
                continue
            # otherwise some output shard must have no capable device
            nout = [max(n1[a] if p1[a] != 1 else 1, n2[a] if p2[a] != 1 else 1) for a in range(rr)]
            found_empty = False
            for idx in itertools.product(*[range(n) for n in nout]):
                w = [full.shape[a] // nout[a] for a in range(rr)]
                box = [(i * w[a], (i + 1) * w[a]) for a, i in enumerate(idx)]
                need1 = [box[a] if p1[a] != 1 else (0, 1) for a in range(rr)]
                need2 = [box[a] if p2[a] != 1 else (0, 1) for a in range(rr)]
                if not any(_holds(b1, d, need1) and _holds(b2, d, need2) for d in devices):
                    found_empty = True
            assert found_empty
            continue
        accepted += 1
        assert not cut_differently
        assert list(out_shape) == list(full.shape)
        pieces1, pieces2 = L.split(x1, sp1), L.split(x2, sp2)
        covered = np.zeros(full.shape, dtype=int)
        for box, devs in shards:
            sl = tuple(slice(a, b) for a, b in box)
            covered[sl] += 1
            need1 = [box[a] if p1[a] != 1 else (0, 1) for a in range(rr)]
            need2 = [box[a] if p2[a] != 1 else (0, 1) for a in range(rr)]
            for d in devices:
                capable = _holds(b1, d, need1) and _holds(b2, d, need2)
                assert capable == (d in devs), (s1, sp1, s2, sp2, box, d)
            for d in devs:
                # compute the output shard from device d's own pieces
                def local(piece, dbox, need, shp):
                    pad = rr - len(shp)
                    pc = piece.reshape([1] * pad + list(piece.shape))
                    return pc[tuple(slice(n0 - b0, n1 - b0) for (b0, _), (n0, n1) in zip(dbox, need))]
                d1 = [b for dv, b in b1 if dv == d][0]
                d2 = [b for dv, b in b2 if dv == d][0]
                got = local(pieces1[d], d1, need1, s1) + local(pieces2[d], d2, need2, s2)
                assert np.array_equal(np.broadcast_to(got, full[sl].shape), full[sl])
        assert (covered == 1).all()
    assert accepted > 100 and rejected > 100


def _blocks(shape, m, mesh):
    return [shape[i] // mesh[j] if j >= 0 else shape[i] for i, j in enumerate(m)]


@pytest.mark.parametrize("mesh", [[2, 2], [2, 3], [3, 2, 2]])
def test_brute_force_matmul_local_products(mesh):
    """Every dims_mapping pair on the mesh: when the merge accepts it, each
    process's local product X_p Y_p is the block of X Y that the inferred
    output mapping assigns it, summed over the partial mesh dims; when it
    rejects, the inputs cut one einsum axis by two mesh dims or one mesh dim
    cuts two axes."""
    q = len(mesh)
    M, Kd, N = 6, 12, 6
    rng = np.random.default_rng(q)
    X = rng.integers(-5, 5, size=(M, Kd)).astype(np.float64)
    Y = rng.integers(-5, 5, size=(Kd, N)).astype(np.float64)
    ids = list(range(int(np.prod(mesh))))
    opts = list(range(-1, q))
    acc = rej = 0
    for xm in itertools.product(opts, repeat=2):
        for ym in itertools.product(opts, repeat=2):
            valid_inputs = all(len([j for j in m if j >= 0]) == len({j for j in m if j >= 0}) for m in (xm, ym))
            try:
                z, partial = K.matmul_dims_mapping(list(xm), list(ym), q)
            except OracleLayoutError:
                rej += 1
                k_conflict = xm[1] >= 0 and ym[0] >= 0 and xm[1] != ym[0]
                kk = xm[1] if xm[1] >= 0 else ym[0]
                cut = [j for j in (xm[0], kk, ym[1]) if j >= 0]
                assert (not valid_inputs) or k_conflict or len(cut) != len(set(cut))
                continue
            acc += 1
            assert valid_inputs
            # After the merge both inputs carry the merged k mapping: an input
            # that kept k whole slices its replica locally (no communication).
            kk = xm[1] if xm[1] >= 0 else ym[0]
            xs = L.split_dims_mapping(X, mesh, ids, [xm[0], kk])
            ys = L.split_dims_mapping(Y, mesh, ids, [kk, ym[1]])
            Z = X @ Y
            sums = {}
            for lin, coord in enumerate(itertools.product(*[range(m) for m in mesh])):
                local = xs[lin] @ ys[lin]
                key = tuple(c if j not in partial else None for j, c in enumerate(coord))
                sums[key] = sums.get(key, 0) + local
            for key, val in sums.items():
                rows, cols = _blocks([M, N], z, mesh)
                r0 = key[z[0]] * rows if z[0] >= 0 else 0
                c0 = key[z[1]] * cols if z[1] >= 0 else 0
                assert np.array_equal(val, Z[r0:r0 + rows, c0:c0 + cols]), (xm, ym, z, partial, key)
    assert acc > 10 and rej > 10


def test_batched_matmul_and_partial():
    z, partial = K.matmul_dims_mapping([0, -1, 1], [-1, 1, -1], 2)
    assert z == [0, -1, -1] and partial == [1]
    z, partial = K.matmul_dims_mapping([-1, 0, -1], [1, -1, -1], 2)
    assert z == [1, 0, -1] and partial == []


@pytest.mark.parametrize("x,y,kind", [
    ([0, 1], [0, -1], "spec"),        # k cut by mesh dims 1 and 0: needs a reshard
    ([0, -1], [0, 1], "spec"),        # mesh dim 0 cuts both m and k
    ([0, 0], [-1, 1], "spec"),        # a mesh dim used twice within X
    ([2, -1], [-1, 1], "spec"),       # mesh dim out of range
    ([0], [-1, 1], "arg"),
])
def test_matmul_rejections(x, y, kind):
    with pytest.raises(OracleLayoutError) as e:
        K.matmul_dims_mapping(x, y, 2)
    assert e.value.kind == kind
