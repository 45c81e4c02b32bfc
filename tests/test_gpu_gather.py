"""GPU parity of tp_shard_gather (the all-gather of a layout) against the
oracle's gather, and of the reduce-scatter + all-gather decomposition of the
all-reduce: bit-exact throughout (bits are copied, sums are taken in the same
order)."""
import random

import numpy as np
import pytest
import torch

import sharded_gemm_amd as tp
from sharded_gemm_amd import inputs
from oracle import layout as L
from oracle import reduce as R

import test_oracle_layout as TL
from gpu_helpers import Guarded, announce, bits, require_gpu

pytestmark = pytest.mark.gpu


def setup_module(_):
    require_gpu()


def _pieces(shape, layout, dtype, seed, mesh=False):
    """Independent seeded pieces (every device its own values, replicas
    included) with the layout's shard extents: {device: cpu tensor}."""
    n, boxes, sod = tp.tp_layout_plan(shape, layout, num_dst=4096)
    ext = [b - a for a, b in boxes[0]] if boxes else list(shape)
    devs = [d for d, s in enumerate(sod) if s >= 0]
    dt = "bf16" if dtype == torch.bfloat16 else "f32"
    return {d: inputs.normal(ext, seed=seed + d, dtype=dt) for d in devs}


def _run(pieces_cpu, layout, shape, dtype, nout=1):
    src = {d: p.cuda() for d, p in pieces_cpu.items()}
    outs = [Guarded(shape, dtype) for _ in range(nout)]
    tp.tp_shard_gather(src, layout, [g.t for g in outs], shape)
    torch.cuda.synchronize()
    for j, g in enumerate(outs):
        assert g.guards_intact(), f"write outside out[{j}]"
    return [g.t.cpu() for g in outs]


def _oracle(pieces_cpu, layout, shape):
    if "mesh_shape" in layout:
        return L.gather_dims_mapping(pieces_cpu, shape, layout["mesh_shape"], layout["process_ids"],
                                     layout["dims_mapping"])
    return L.gather(pieces_cpu, shape, layout)


def _same_bits(got, ref64, dtype):
    r = torch.from_numpy(np.ascontiguousarray(ref64)).to(dtype)   # exact: the oracle widened the stored values
    assert tuple(got.shape) == tuple(r.shape)
    assert np.array_equal(bits(got), bits(r))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("case", TL._load()["cases"], ids=lambda c: c["name"])
def test_page_examples_gather_back(case, dtype):
    """The pages' printed device contents gather back to their tensor."""
    announce(f"gather page example {case['name']} {dtype}")
    t = torch.tensor(TL._load()["tensor"], dtype=dtype)
    pieces = {int(k): torch.tensor(v, dtype=dtype) for k, v in case["expected"].items()}
    got = _run(pieces, TL._spec_from_json(case["spec"]), tuple(t.shape), dtype, nout=2)
    for g in got:
        assert torch.equal(g, t)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_brute_force(dtype):
    rnd = random.Random(29)
    cases = TL._all_cases(max_cases=150, seed=31)
    announce(f"gather brute force {dtype} ({len(cases)} cases)")
    for i, (shape, axes, counts) in enumerate(cases):
        nsh = int(np.prod(counts)) if counts else 1
        if i % 2:
            spec = {"device": [-(k + 1) for k in range(nsh)],
                    "device_map": {-(k + 1): [2 * k + 1, 2 * k] for k in range(nsh)}}
        else:
            devs = list(range(nsh))
            rnd.shuffle(devs)
            spec = {"device": devs}
        spec["sharded_dim"] = [{"axis": a, "num_shards": n} for a, n in zip(axes, counts)]
        pieces = _pieces(shape, spec, dtype, seed=95000 + 100 * i)
        got = _run(pieces, spec, tuple(shape), dtype)
        _same_bits(got[0], _oracle(pieces, spec, shape), dtype)


@pytest.mark.parametrize("shape,sharded", [
    ((6, 4, 10), [(2, 10)]), ((6, 4, 10), [(2, 5)]), ((6, 4, 12), [(-1, 4)]), ((6, 4, 10), [(2, 2)]),
    ((6, 4, 16), [(2, 2)]), ((33, 7, 64), [(0, 3)]), ((5, 6, 7, 8), [(3, 2), (1, 3)]),
    ((4, 6, 8, 2), [(0, 2), (2, 4), (1, 3)]),
])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_vector_widths(shape, sharded, dtype):
    """Runs of 1 .. 8 elements and multi-axis boxes: every vector width."""
    nsh = 1
    for _, n in sharded:
        nsh *= n
    spec = {"device": list(range(nsh)), "sharded_dim": [{"axis": a, "num_shards": n} for a, n in sharded]}
    announce(f"gather vector widths {shape} {sharded} {dtype}")
    pieces = _pieces(shape, spec, dtype, seed=7700)
    got = _run(pieces, spec, shape, dtype, nout=3)
    ref = _oracle(pieces, spec, shape)
    for g in got:
        _same_bits(g, ref, dtype)


def test_replica_read_from_first_listed_device():
    announce("gather replicas: first listed device")
    spec = {"device": [-1, -2], "device_map": {-1: [3, 0], -2: [1, 2]}, "sharded_dim": [{"axis": 0, "num_shards": 2}]}
    pieces = {d: torch.full((1, 8), float(10 + d)) for d in range(4)}
    got = _run(pieces, spec, (2, 8), torch.float32)[0]
    assert torch.equal(got, torch.tensor([[13.0] * 8, [11.0] * 8]))
    _same_bits(got, L.gather(pieces, (2, 8), spec), torch.float32)


def test_mesh_dims_mapping_sequence_axis():
    """[S, B, H] with the sequence axis on mesh dim 0 of a 4 x 2 mesh ([SPMD]
    dims_mapping [0, -1, -1]): the replicas along mesh dim 1 are not read."""
    announce("gather dims_mapping sequence axis")
    shape = (512, 4, 1024)
    lay = {"mesh_shape": [4, 2], "process_ids": [7, 6, 5, 4, 3, 2, 1, 0], "dims_mapping": [0, -1, -1]}
    pieces = _pieces(shape, lay, torch.bfloat16, seed=9100)
    got = _run(pieces, lay, shape, torch.bfloat16, nout=2)
    ref = _oracle(pieces, lay, shape)
    for g in got:
        _same_bits(g, ref, torch.bfloat16)


def test_gather_inverts_materialize_full_size():
    """The 2x4-mesh layout at full size ([8, 2048, 8192] fp32, dims_mapping
    [0, -1, 1]): split, then gather back into two outputs, bit for bit."""
    announce("gather full size: materialize then gather")
    shape = (8, 2048, 8192)
    src_cpu = inputs.normal(shape, seed=9200)
    lay = {"mesh_shape": [2, 4], "process_ids": list(range(8)), "dims_mapping": [0, -1, 1]}
    src = src_cpu.cuda()
    shards = {d: torch.empty((4, 2048, 2048), device="cuda") for d in range(8)}
    tp.tp_shard_materialize(src, lay, shards)
    outs = [torch.empty(shape, device="cuda") for _ in range(2)]
    tp.tp_shard_gather(shards, lay, outs, shape)
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o.view(torch.int32), src.view(torch.int32))


@pytest.mark.parametrize("S,Bt,H,P", [(16, 2, 40, 4), (2048, 4, 1024, 8), (1024, 1, 4096, 8)])
def test_reduce_scatter_then_all_gather_is_all_reduce(S, Bt, H, P):
    """ColossalAI sections 3 and 5.3: reduce-scatter along the sequence axis
    (the SPLIT reduce), then all-gather the blocks: the all-reduced tensor, bit
    for bit against the FULL reduce on the GPU and against the oracle."""
    announce(f"RS + AG == AR S={S} B={Bt} H={H} P={P}")
    rows = S * Bt
    parts_cpu = [inputs.normal((rows, H), seed=9300 + p) for p in range(P)]
    parts = [p.cuda() for p in parts_cpu]
    blocks = [torch.empty((rows // P, H), device="cuda") for _ in range(P)]
    tp.tp_partial_reduce(parts, blocks, tp.TP_REDUCE_SPLIT)
    spec = {"device": list(range(P)), "sharded_dim": [{"axis": 0, "num_shards": P}]}
    full = [Guarded((S, Bt, H), torch.float32) for _ in range(2)]
    tp.tp_shard_gather({j: blocks[j].view(S // P, Bt, H) for j in range(P)}, spec, [g.t for g in full], (S, Bt, H))
    ar = torch.empty((rows, H), device="cuda")
    tp.tp_partial_reduce(parts, [ar])
    torch.cuda.synchronize()
    for g in full:
        assert g.guards_intact()
        assert torch.equal(g.t.view(rows, H).view(torch.int32), ar.view(torch.int32))
    ref = R.reduce_full(parts_cpu)
    assert np.abs(ar.cpu().double().numpy() - ref).max() <= 1e-6 * np.abs(np.stack([p.numpy() for p in parts_cpu])).sum(0).max()


def test_error_leaves_outputs_untouched():
    announce("gather error path")
    spec = {"device": [0, 1], "sharded_dim": [{"axis": 0, "num_shards": 2}]}
    pieces = {0: torch.ones((1, 4), device="cuda"), 1: torch.ones((1, 4), device="cuda")}
    out = Guarded((3, 4), torch.float32)
    with pytest.raises(tp.TpError) as e:
        tp.tp_shard_gather(pieces, spec, [out.t], (3, 4))   # 3 rows: indivisible
    assert e.value.kind == "indivisible"
    torch.cuda.synchronize()
    assert out.body_untouched() and out.guards_intact()


def test_empty_tensor_is_a_no_op():
    announce("gather empty tensor")
    spec = {"device": [0, 1], "sharded_dim": [{"axis": 1, "num_shards": 2}]}
    tp.tp_shard_gather({0: torch.empty((0, 2), device="cuda"), 1: torch.empty((0, 2), device="cuda")}, spec,
                       [torch.empty((0, 4), device="cuda")], (0, 4))
    torch.cuda.synchronize()


def test_rank8_many_shards_and_outputs():
    """Rank 8, 256 shards with replicas, gathered into 65 outputs (two groups of
    at most 64 per launch) and several launches of at most 32 shards."""
    shape = (2, 2, 2, 2, 2, 2, 2, 64)
    nsh = 256
    spec = {"device": [-(k + 1) for k in range(nsh)],
            "device_map": {-(k + 1): [2 * k + 1, 2 * k] for k in range(nsh)},
            "sharded_dim": [{"axis": a, "num_shards": 2} for a in range(8)]}
    announce("gather rank 8, 256 shards, 65 outputs")
    pieces = _pieces(shape, spec, torch.float32, seed=9600)
    got = _run(pieces, spec, shape, torch.float32, nout=65)
    ref = _oracle(pieces, spec, shape)
    for g in got:
        _same_bits(g, ref, torch.float32)
