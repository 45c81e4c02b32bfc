"""GPU parity of the short-run layout kernels: layouts whose innermost cut
leaves runs of under 16 bytes ([ONNX] "Sharding as a Split", the axis-1
example: one-element runs), split and gathered through whole-row blocks.
Bit-exact against the oracle, with replicas, dims_mapping layouts, both
enumeration orders, one device's share and the gather's replica choice."""
import numpy as np
import pytest
import torch

import sharded_gemm_amd as tp
from sharded_gemm_amd import inputs
from oracle import layout as L

from gpu_helpers import Guarded, announce, bits, require_gpu

pytestmark = pytest.mark.gpu


def setup_module(_):
    require_gpu()


CASES = [
    # (shape, layout, dtype); runs of L elements along the innermost cut axis
    ((4096, 8), {"device": list(range(8)), "sharded_dim": [{"axis": 1, "num_shards": 8}]}, "f32"),        # L = 1
    ((4096, 8), {"device": list(range(8)),
                 "sharded_dim": [{"axis": 0, "num_shards": 2}, {"axis": 1, "num_shards": 4}]}, "f32"),     # L = 2
    ((4096, 8), {"device": list(range(8)),
                 "sharded_dim": [{"axis": 1, "num_shards": 4}, {"axis": 0, "num_shards": 2}]}, "f32"),     # other order
    ((1024, 6), {"device": [-1, -2, -3], "device_map": {-1: [0, 3], -2: [1, 4], -3: [2, 5]},
                 "sharded_dim": [{"axis": 1, "num_shards": 3}]}, "bf16"),                                   # replicas
    ((64, 32, 4), {"mesh_shape": [2, 4], "process_ids": list(range(8)), "dims_mapping": [-1, 0, 1]}, "f32"),
    ((256, 3, 4), {"device": [0, 1], "sharded_dim": [{"axis": 2, "num_shards": 2}]}, "bf16"),
    ((2048, 12), {"device": [3, 1, 0, 2], "sharded_dim": [{"axis": 1, "num_shards": 4}]}, "bf16"),          # 6-byte runs
    ((16, 64, 8), {"device": list(range(16)),
                   "sharded_dim": [{"axis": 2, "num_shards": 8}, {"axis": 0, "num_shards": 2}]}, "bf16"),
    # 8-byte runs: odd n with replicas, n = 8 and 16, an outer cut with an axis inside it
    ((2048, 12), {"device": [-1, -2, -3], "device_map": {-1: [0, 3], -2: [1, 4], -3: [2, 5]},
                  "sharded_dim": [{"axis": 1, "num_shards": 3}]}, "bf16"),
    ((1024, 16), {"device": list(range(8)), "sharded_dim": [{"axis": 1, "num_shards": 8}]}, "f32"),
    ((512, 2, 32), {"device": list(range(16)),
                    "sharded_dim": [{"axis": 0, "num_shards": 2}, {"axis": 2, "num_shards": 8}]}, "bf16"),
    ((1024, 32), {"device": list(range(16)), "sharded_dim": [{"axis": 1, "num_shards": 16}]}, "f32"),
    # nine 512-row blocks: the gather's workgroups take two blocks each, one of them three
    ((4608, 8), {"device": [0, 1, 2, 3], "sharded_dim": [{"axis": 1, "num_shards": 4}]}, "f32"),
    ((4608, 12), {"device": [0, 1, 2, 3], "sharded_dim": [{"axis": 1, "num_shards": 4}]}, "bf16"),
    # not taken by the row-block kernels: blocks of fewer than 8 rows, 16-byte runs
    ((100, 8), {"device": list(range(8)), "sharded_dim": [{"axis": 1, "num_shards": 8}]}, "bf16"),
    ((8, 256, 12), {"device": list(range(6)),
                    "sharded_dim": [{"axis": 0, "num_shards": 2}, {"axis": 2, "num_shards": 3}]}, "f32"),
]


def _ids(c):
    shape, lay, dt = c
    return f"{'x'.join(map(str, shape))}-{dt}-{'mesh' if 'mesh_shape' in lay else len(lay['sharded_dim'])}"


def _oracle_split(src, lay):
    if "mesh_shape" in lay:
        return L.split_dims_mapping(src, lay["mesh_shape"], lay["process_ids"], lay["dims_mapping"])
    return L.split(src, lay)


def _as(ref, dtype):
    r = torch.from_numpy(np.ascontiguousarray(ref))
    return r.to(dtype)   # exact: the oracle widened the stored values


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_split_bit_exact(case):
    shape, lay, dt = case
    announce(f"short runs split {shape} {lay} {dt}")
    src = inputs.normal(shape, seed=7100 + len(shape), dtype=dt)
    ref = _oracle_split(src, lay)
    bufs = {d: Guarded(ref[d].shape, src.dtype) for d in ref}
    tp.tp_shard_materialize(src.cuda(), lay, {d: b.t for d, b in bufs.items()})
    torch.cuda.synchronize()
    for d, b in bufs.items():
        assert b.guards_intact(), d
        assert np.array_equal(bits(b.t.cpu()), bits(_as(ref[d], src.dtype))), d


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_gather_bit_exact(case):
    """Independent values on every device (replicas differ): the gather reads
    each shard from the first device its group lists, as the oracle does."""
    shape, lay, dt = case
    announce(f"short runs gather {shape} {lay} {dt}")
    n, boxes, sod = tp.tp_layout_plan(shape, lay, num_dst=64)
    ext = [b - a for a, b in boxes[0]]
    pieces = {d: inputs.normal(ext, seed=7200 + d, dtype=dt) for d, k in enumerate(sod) if k >= 0}
    if "mesh_shape" in lay:
        ref = L.gather_dims_mapping(pieces, shape, lay["mesh_shape"], lay["process_ids"], lay["dims_mapping"])
    else:
        ref = L.gather(pieces, shape, lay)
    dtype = pieces[next(iter(pieces))].dtype
    outs = [Guarded(shape, dtype) for _ in range(2)]
    tp.tp_shard_gather({d: p.cuda() for d, p in pieces.items()}, lay, [g.t for g in outs], shape)
    torch.cuda.synchronize()
    for g in outs:
        assert g.guards_intact()
        assert np.array_equal(bits(g.t.cpu()), bits(_as(ref, dtype)))


def test_local_share_and_batch():
    """One device's share of a short-run layout (the other shard positions are
    not written), and short-run and long-run tensors cut in one batched call."""
    announce("short runs local share and batch")
    shape, lay = (4096, 8), {"device": list(range(8)),
                             "sharded_dim": [{"axis": 0, "num_shards": 2}, {"axis": 1, "num_shards": 4}]}
    src = inputs.normal(shape, seed=7301)
    ref = L.split(src, lay)
    srcg = src.cuda()
    for d in (0, 5, 7):
        mine = Guarded(ref[d].shape, torch.float32)
        tp.tp_shard_materialize_batch([(srcg, lay, {d: mine.t}, d)])
        torch.cuda.synchronize()
        assert mine.guards_intact()
        assert np.array_equal(bits(mine.t.cpu()), bits(_as(ref[d], torch.float32))), d
    long_lay = {"device": [0, 1, 2, 3], "sharded_dim": [{"axis": 1, "num_shards": 4}]}
    w = inputs.normal((256, 1024), seed=7302, dtype="bf16")
    wref = L.split(w, long_lay)
    a = {d: Guarded(ref[d].shape, torch.float32) for d in ref}
    b = {d: Guarded(wref[d].shape, torch.bfloat16) for d in wref}
    tp.tp_shard_materialize_batch([(srcg, lay, {d: g.t for d, g in a.items()}), (w.cuda(), long_lay, {d: g.t for d, g in b.items()})])
    torch.cuda.synchronize()
    for d in ref:
        assert a[d].guards_intact() and np.array_equal(bits(a[d].t.cpu()), bits(_as(ref[d], torch.float32)))
    for d in wref:
        assert b[d].guards_intact() and np.array_equal(bits(b[d].t.cpu()), bits(_as(wref[d], torch.bfloat16)))


def test_misaligned_pointer_falls_back():
    """A destination that is not 16-byte aligned takes the per-shard kernel: same bits."""
    announce("short runs misaligned destination")
    shape, lay = (1024, 8), {"device": [0, 1, 2, 3], "sharded_dim": [{"axis": 1, "num_shards": 4}]}
    src = inputs.normal(shape, seed=7401)
    ref = L.split(src, lay)
    raw = torch.empty(4 * 2048 + 1, device="cuda")
    dst = {d: raw[1 + d * 2048:1 + (d + 1) * 2048].view(1024, 2) for d in range(4)}   # 4-byte aligned only
    tp.tp_shard_materialize(src.cuda(), lay, dst)
    torch.cuda.synchronize()
    for d in range(4):
        assert np.array_equal(bits(dst[d].cpu()), bits(_as(ref[d], torch.float32))), d


def test_full_size_split_and_gather():
    """The bench's short-run workload at its full size: fp32 [16777216, 8]
    (512 MiB) cut on axis 0 in 2 and axis 1 in 4 (8-byte runs), every shard
    against the oracle's split and the gather back equal to the source, bit
    for bit, in the launch configuration the bench times."""
    announce("short runs full size 16777216 x 8")
    shape = (16777216, 8)
    lay = {"device": list(range(8)), "sharded_dim": [{"axis": 0, "num_shards": 2}, {"axis": 1, "num_shards": 4}]}
    src = inputs.normal(shape, seed=7501)
    ref = L.split(src, lay)
    srcg = src.cuda()
    dst = {d: torch.empty(ref[d].shape, device="cuda") for d in ref}
    tp.tp_shard_materialize(srcg, lay, dst)
    full = torch.empty(shape, device="cuda")
    tp.tp_shard_gather(dst, lay, [full], shape)
    torch.cuda.synchronize()
    for d in ref:
        assert np.array_equal(bits(dst[d].cpu()), bits(_as(ref[d], torch.float32))), d
    assert torch.equal(full.cpu().view(torch.int32), src.view(torch.int32))
