"""Pins for the oracle's gather (the inverse of a split: ColossalAI's
gather_output and the all-gather of sequence parallelism, sections 5.1 and
5.3; OneFlow's SBP section: split pieces concatenate back to the logical
tensor, broadcast pieces equal it).

The pieces fed to gather come from the pages' printed examples, from an
inverse formula written independently of the oracle, or from numpy's own
split, never from the oracle's split alone."""
import numpy as np
import pytest

import test_oracle_layout as TL
from oracle import layout as L
from oracle import mlp as O
from oracle import reduce as R
from oracle.layout import OracleLayoutError


@pytest.mark.parametrize("case", TL._load()["cases"], ids=lambda c: c["name"])
def test_page_examples_gather_back(case):
    """The pages' printed device contents assemble back to their tensor."""
    t = np.array(TL._load()["tensor"], dtype=np.float32)
    pieces = {int(k): np.array(v, dtype=np.float32) for k, v in case["expected"].items()}
    assert np.array_equal(L.gather(pieces, t.shape, TL._spec_from_json(case["spec"])), t)


@pytest.mark.parametrize("case", TL._load()["mesh_cases"], ids=lambda c: c["name"])
def test_page_2d_sbp_example_gathers_back(case):
    t = np.array(TL._load()["tensor"], dtype=np.float32)
    pieces = {int(k): np.array(v, dtype=np.float32) for k, v in case["expected"].items()}
    got = L.gather_dims_mapping(pieces, t.shape, case["mesh_shape"], case["process_ids"], case["dims_mapping"])
    assert np.array_equal(got, t)


def test_brute_force_pieces_from_inverse_formula():
    """Pieces built by the independent inverse formula (global index -> shard,
    local index) gather back to the tensor, over about 1500 layouts."""
    for shape, axes, counts in TL._all_cases(max_cases=800, seed=13):
        t = np.arange(1, int(np.prod(shape)) + 1, dtype=np.float64).reshape(shape)
        nsh = int(np.prod(counts)) if counts else 1
        groups = [[2 * k + 1, 2 * k] for k in range(nsh)]
        spec = {"device": [-(k + 1) for k in range(nsh)],
                "device_map": {-(k + 1): groups[k] for k in range(nsh)},
                "sharded_dim": [{"axis": a, "num_shards": n} for a, n in zip(axes, counts)]}
        pieces = TL._shards_by_inverse_formula(t, list(axes), list(counts), groups)
        assert np.array_equal(L.gather(pieces, shape, spec), t), (shape, axes, counts)


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_single_axis_gather_is_concatenation(axis):
    rng = np.random.default_rng(21 + axis)
    S, B, H, P = 8, 4, 12, 4
    t_shape = [S, B, H]
    pieces_list = []
    for _ in range(P):
        sh = list(t_shape)
        sh[axis] //= P
        pieces_list.append(rng.standard_normal(sh))
    spec = {"device": list(range(P)), "sharded_dim": [{"axis": axis, "num_shards": P}]}
    got = L.gather(dict(enumerate(pieces_list)), t_shape, spec)
    assert np.array_equal(got, np.concatenate(pieces_list, axis=axis))


def test_sequence_axis_dims_mapping_is_concatenation():
    """[S, B, H] with the sequence axis on mesh dim 0 ([SPMD] dims_mapping
    [0, -1, -1]); the second mesh dim replicates."""
    rng = np.random.default_rng(5)
    S, B, H = 8, 2, 6
    mesh, ids = [4, 2], [7, 6, 5, 4, 3, 2, 1, 0]
    blocks = [rng.standard_normal((S // 4, B, H)) for _ in range(4)]
    pieces = {ids[2 * c + r]: blocks[c] for c in range(4) for r in range(2)}
    got = L.gather_dims_mapping(pieces, (S, B, H), mesh, ids, [0, -1, -1])
    assert np.array_equal(got, np.concatenate(blocks, axis=0))


def test_replica_taken_from_first_listed_device():
    t = np.zeros((2, 2))
    spec = {"device": [-1, -2], "device_map": {-1: [3, 0], -2: [1, 2]},
            "sharded_dim": [{"axis": 0, "num_shards": 2}]}
    pieces = {3: np.full((1, 2), 1.0), 0: np.full((1, 2), 9.0), 1: np.full((1, 2), 2.0), 2: np.full((1, 2), 9.0)}
    assert np.array_equal(L.gather(pieces, t.shape, spec), np.array([[1.0, 1.0], [2.0, 2.0]]))
    mesh_pieces = {0: np.full((1, 2), 1.0), 1: np.full((1, 2), 9.0), 2: np.full((1, 2), 2.0), 3: np.full((1, 2), 9.0)}
    got = L.gather_dims_mapping(mesh_pieces, (2, 2), [2, 2], [0, 1, 2, 3], [0, -1])
    assert np.array_equal(got, np.array([[1.0, 1.0], [2.0, 2.0]]))


def test_reduce_scatter_then_all_gather_is_all_reduce():
    """ColossalAI sections 3 and 5.3: a ring all-reduce is a reduce-scatter
    followed by an all-gather.  On [S, B, H] with the sequence axis split,
    gathering the reduce-scatter blocks gives the all-reduced tensor."""
    rng = np.random.default_rng(17)
    S, B, H, P = 16, 2, 5, 4
    parts = [rng.integers(-50, 50, size=(S * B, H)).astype(np.float64) for _ in range(P)]
    blocks = R.reduce_split(parts, P)
    spec = {"device": list(range(P)), "sharded_dim": [{"axis": 0, "num_shards": P}]}
    pieces = {j: blocks[j].reshape(S // P, B, H) for j in range(P)}
    got = L.gather(pieces, (S, B, H), spec)
    exp = sum(p.reshape(S, B, H) for p in parts)
    assert np.array_equal(got, exp)


def test_gather_output_of_column_layer():
    """ColossalAI section 2: [Y_1 Y_2] = [X A_1  X A_2]; gathering the
    column-parallel outputs along the last axis gives the unsharded layer's
    output (GeLU acts elementwise, so it commutes with the gather)."""
    rng = np.random.default_rng(4)
    M, H, F, P = 5, 6, 8, 4
    X, A = rng.standard_normal((M, H)), rng.standard_normal((H, F))
    Ys = {i: O.hidden(X, A[:, i * F // P:(i + 1) * F // P]) for i in range(P)}
    spec = {"device": list(range(P)), "sharded_dim": [{"axis": 1, "num_shards": P}]}
    ref = X @ A
    assert np.allclose(L.gather(Ys, (M, F), spec), O.gelu(ref), atol=1e-12, rtol=0)


def test_rejections():
    spec = {"device": [0, 1], "sharded_dim": [{"axis": 0, "num_shards": 2}]}
    with pytest.raises(OracleLayoutError) as e:
        L.gather({0: np.zeros((1, 3))}, (2, 3), spec)
    assert e.value.kind == "arg"
    with pytest.raises(OracleLayoutError) as e:
        L.gather({0: np.zeros((1, 3)), 1: np.zeros((2, 3))}, (2, 3), spec)
    assert e.value.kind == "arg"
    with pytest.raises(OracleLayoutError) as e:
        L.gather({0: np.zeros((1, 3)), 1: np.zeros((1, 3))}, (3, 3), spec)
    assert e.value.kind == "indivisible"
