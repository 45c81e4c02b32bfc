"""GPU parity of tp_shard_materialize against the layout oracle: bit-exact."""
import random

import numpy as np
import pytest
import torch

import sharded_gemm_amd as tp
from sharded_gemm_amd import inputs
from sharded_gemm_amd.workloads import RESHARD, TINY_LAYOUT_SPECS
from oracle import layout as L

import test_oracle_layout as TL
from gpu_helpers import Guarded, announce, bits, require_gpu

pytestmark = pytest.mark.gpu


def setup_module(_):
    require_gpu()


def _run(src_cpu, layout, dtype):
    """Materialise on the GPU into guarded buffers; return {device: cpu tensor}."""
    n, boxes, sod = tp.tp_layout_plan(src_cpu.shape, layout, num_dst=4096)
    ext = [b - a for a, b in boxes[0]] if boxes else list(src_cpu.shape)
    devs = [d for d, s in enumerate(sod) if s >= 0]
    bufs = {d: Guarded(ext, dtype) for d in devs}
    src = src_cpu.cuda()
    tp.tp_shard_materialize(src, layout, {d: b.t for d, b in bufs.items()})
    torch.cuda.synchronize()
    for d, b in bufs.items():
        assert b.guards_intact(), f"write outside dst[{d}]"
    return {d: b.t.cpu() for d, b in bufs.items()}


def _compare_with_oracle(src_cpu, got, ref):
    assert sorted(got) == sorted(ref)
    for d in ref:
        r = torch.from_numpy(np.ascontiguousarray(ref[d]))
        if src_cpu.dtype == torch.bfloat16:
            r = r.to(torch.bfloat16)   # exact: the oracle widened bf16 values to fp32
        assert tuple(got[d].shape) == tuple(r.shape), d
        assert np.array_equal(bits(got[d]), bits(r)), f"device {d} differs"


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("case", TL._load()["cases"], ids=lambda c: c["name"])
def test_page_examples(case, dtype):
    announce(f"layout page example {case['name']} {dtype}")
    src = torch.tensor(TL._load()["tensor"], dtype=dtype)
    spec = TL._spec_from_json(case["spec"])
    got = _run(src, spec, dtype)
    exp = {int(k): torch.tensor(v, dtype=dtype) for k, v in case["expected"].items()}
    for d in exp:
        assert torch.equal(got[d], exp[d]), (d, got[d], exp[d])
    _compare_with_oracle(src, got, L.split(src, spec))


def test_page_2d_sbp():
    case = TL._load()["mesh_cases"][0]
    announce("layout 2D SBP example")
    src = torch.tensor(TL._load()["tensor"], dtype=torch.float32)
    lay = {"mesh_shape": case["mesh_shape"], "process_ids": case["process_ids"], "dims_mapping": case["dims_mapping"]}
    got = _run(src, lay, torch.float32)
    for k, v in case["expected"].items():
        assert torch.equal(got[int(k)], torch.tensor(v, dtype=torch.float32))


def test_tiny_workload_specs():
    src = inputs.arange_tensor((2, 2))
    for name, spec in TINY_LAYOUT_SPECS.items():
        announce(f"tiny layout {name}")
        _compare_with_oracle(src, _run(src, spec, torch.float32), L.split(src, spec))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_brute_force(dtype):
    rnd = random.Random(17)
    cases = TL._all_cases(max_cases=150, seed=23)
    announce(f"layout brute force {dtype} ({len(cases)} cases)")
    for i, (shape, axes, counts) in enumerate(cases):
        nsh = int(np.prod(counts)) if counts else 1
        src = inputs.normal(shape, seed=90000 + i, dtype="bf16" if dtype == torch.bfloat16 else "f32")
        if i % 2:
            spec = {"device": [-(k + 1) for k in range(nsh)],
                    "device_map": {-(k + 1): [2 * k + 1, 2 * k] for k in range(nsh)}}
        else:
            devs = list(range(nsh))
            rnd.shuffle(devs)
            spec = {"device": devs}
        spec["sharded_dim"] = [{"axis": a, "num_shards": n} for a, n in zip(axes, counts)]
        _compare_with_oracle(src, _run(src, spec, dtype), L.split(src, spec))


@pytest.mark.parametrize("shape,sharded", [
    # contiguous runs of 1, 2, 3, 5 and 8 elements, plus multi-axis boxes:
    # every vector width of the copy (2, 4, 8, 16 bytes) gets exercised
    ((6, 4, 10), [(2, 10)]),
    ((6, 4, 10), [(2, 5)]),
    ((6, 4, 12), [(-1, 4)]),
    ((6, 4, 10), [(2, 2)]),
    ((6, 4, 16), [(2, 2)]),
    ((33, 7, 64), [(0, 3)]),
    ((5, 6, 7, 8), [(3, 2), (1, 3)]),
    ((4, 6, 8, 2), [(0, 2), (2, 4), (1, 3)]),
])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_vector_widths(shape, sharded, dtype):
    nsh = 1
    for _, n in sharded:
        nsh *= n
    spec = {"device": list(range(nsh)), "sharded_dim": [{"axis": a, "num_shards": n} for a, n in sharded]}
    announce(f"layout vector widths {shape} {sharded} {dtype}")
    src = inputs.normal(shape, seed=777, dtype="bf16" if dtype == torch.bfloat16 else "f32")
    _compare_with_oracle(src, _run(src, spec, dtype), L.split(src, spec))


def test_gpt2_weight_split():
    # Column slices of A [768, 3072] and row slices of B [3072, 768] for 4 ranks.
    announce("gpt2 weight split")
    A = inputs.normal((768, 3072), inputs.seed_for(2, inputs.SLOT_A), 0.02, "bf16")
    B = inputs.normal((3072, 768), inputs.seed_for(2, inputs.SLOT_B), 0.02, "bf16")
    sa = {"device": [0, 1, 2, 3], "sharded_dim": [{"axis": 1, "num_shards": 4}]}
    sb = {"device": [0, 1, 2, 3], "sharded_dim": [{"axis": 0, "num_shards": 4}]}
    _compare_with_oracle(A, _run(A, sa, torch.bfloat16), L.split(A, sa))
    _compare_with_oracle(B, _run(B, sb, torch.bfloat16), L.split(B, sb))


def test_reshard_full_size():
    """The 2x4-mesh workload at full size: dims_mapping [0,-1,1] on [8,2048,8192]
    fp32, then every shard to a device pair; the fused one-pass spec must give
    the same bits as materialise-then-broadcast, and both equal the oracle."""
    w = RESHARD
    announce("reshard full size: dims_mapping")
    src_cpu = inputs.normal(w.src_shape, inputs.seed_for(4, inputs.SLOT_LAYOUT))
    mesh = {"mesh_shape": list(w.mesh_shape), "process_ids": list(w.process_ids), "dims_mapping": list(w.dims_mapping)}
    src = src_cpu.cuda()
    shard_shape = (4, 2048, 2048)
    shards = {d: torch.empty(shard_shape, device="cuda") for d in range(8)}
    tp.tp_shard_materialize(src, mesh, shards)
    ref = L.split_dims_mapping(src_cpu, w.mesh_shape, w.process_ids, w.dims_mapping)
    torch.cuda.synchronize()
    for d in range(8):
        assert np.array_equal(bits(shards[d]), ref[d].view(np.int32)), d

    announce("reshard full size: broadcast of each shard to a device pair")
    pairs = {d: torch.empty(shard_shape, device="cuda") for d in range(16)}
    for k in range(8):
        bspec = {"device": [-1], "device_map": {-1: [2 * k, 2 * k + 1]}, "sharded_dim": []}
        tp.tp_shard_materialize(shards[k], bspec, {2 * k: pairs[2 * k], 2 * k + 1: pairs[2 * k + 1]})

    announce("reshard full size: fused split + replicate")
    fused_spec = {"device": [-(k + 1) for k in range(8)],
                  "device_map": {-(k + 1): [2 * k, 2 * k + 1] for k in range(8)},
                  "sharded_dim": [{"axis": 0, "num_shards": 2}, {"axis": 2, "num_shards": 4}]}
    fused = {d: Guarded(shard_shape, torch.float32) for d in range(16)}
    tp.tp_shard_materialize(src, fused_spec, {d: g.t for d, g in fused.items()})
    torch.cuda.synchronize()
    for d in range(16):
        assert fused[d].guards_intact()
        assert torch.equal(bits_t(fused[d].t), bits_t(pairs[d])), d
        assert np.array_equal(bits(fused[d].t), ref[d // 2].view(np.int32)), d


def bits_t(t):
    return t.view(torch.int32)


def test_rejected_spec_leaves_outputs_untouched():
    announce("layout error path")
    src = torch.arange(12, dtype=torch.float32, device="cuda").view(3, 4)
    outs = {d: Guarded((3, 2), torch.float32) for d in range(2)}
    bad = {"device": [0, 1], "sharded_dim": [{"axis": 0, "num_shards": 2}]}   # 3 rows: indivisible
    with pytest.raises(tp.TpError) as e:
        tp.tp_shard_materialize(src, bad, {d: g.t for d, g in outs.items()})
    assert e.value.kind == "indivisible"
    torch.cuda.synchronize()
    for g in outs.values():
        assert g.body_untouched() and g.guards_intact()


def test_empty_tensor_is_a_no_op():
    announce("layout empty tensor")
    src = torch.empty((0, 4), device="cuda")
    outs = {d: torch.empty((0, 2), device="cuda") for d in range(2)}
    tp.tp_shard_materialize(src, {"device": [0, 1], "sharded_dim": [{"axis": 1, "num_shards": 2}]}, outs)
    torch.cuda.synchronize()


def test_rank8_many_shards_and_replicas():
    """Rank 8 (the largest), every axis cut in two: 256 shards, each to a pair
    of devices (512 destinations), so the copy spans several launches of at
    most 32 shards and 64 destinations."""
    shape = (2, 2, 2, 2, 2, 2, 2, 64)
    nsh = 256
    spec = {"device": [-(k + 1) for k in range(nsh)],
            "device_map": {-(k + 1): [2 * k + 1, 2 * k] for k in range(nsh)},
            "sharded_dim": [{"axis": a, "num_shards": 2} for a in range(8)]}
    announce("layout rank 8, 256 shards x 2 replicas")
    src = inputs.normal(shape, seed=7900)
    _compare_with_oracle(src, _run(src, spec, torch.float32), L.split(src, spec))


def test_batch_equals_single_calls_and_oracle():
    """Several tensors in one tp_shard_materialize_batch call (mixed dtypes and
    layouts, six tensors so that the packing spills over launches): every
    destination equals the oracle's split."""
    announce("layout batch of 6 tensors")
    jobs, refs = [], []
    specs = [
        ((768, 3072), {"device": [0, 1, 2, 3], "sharded_dim": [{"axis": 1, "num_shards": 4}]}, "bf16"),
        ((3072, 768), {"device": [0, 1, 2, 3], "sharded_dim": [{"axis": 0, "num_shards": 4}]}, "bf16"),
        ((6, 4, 10), {"device": list(range(10)), "sharded_dim": [{"axis": 2, "num_shards": 5}, {"axis": 0, "num_shards": 2}]}, "f32"),
        ((2, 2, 2, 2, 2, 2, 2, 64), {"device": list(range(128)), "sharded_dim": [{"axis": a, "num_shards": 2} for a in range(7)]}, "f32"),
        ((33, 7, 64), {"device": [-1, -2, -3], "device_map": {-1: [0, 5], -2: [1, 4], -3: [2, 3]},
                       "sharded_dim": [{"axis": 0, "num_shards": 3}]}, "bf16"),
        ((4, 4), {"device": [-1], "device_map": {-1: [0, 1, 2]}, "sharded_dim": []}, "f32"),
    ]
    for i, (shape, spec, dt) in enumerate(specs):
        src = inputs.normal(shape, seed=9800 + i, dtype=dt)
        ref = L.split(src, spec)
        dst = {d: Guarded(v.shape, src.dtype) for d, v in ref.items()}
        jobs.append((src.cuda(), spec, {d: g.t for d, g in dst.items()}))
        refs.append((src, ref, dst))
    tp.tp_shard_materialize_batch(jobs)
    torch.cuda.synchronize()
    for src, ref, dst in refs:
        for d, g in dst.items():
            assert g.guards_intact()
        _compare_with_oracle(src, {d: g.t.cpu() for d, g in dst.items()}, ref)


def test_local_device_share_equals_its_shard():
    """An item with local_device writes that device's shard alone (the share
    one process materialises for itself), equal to the oracle's, for split,
    2-D split and replicated layouts; a device of a replicated group gets the
    group's shard."""
    announce("layout local-device shares")
    specs = [
        ((768, 3072), {"device": [0, 1, 2, 3], "sharded_dim": [{"axis": 1, "num_shards": 4}]}, "bf16"),
        ((3072, 768), {"device": [0, 1, 2, 3], "sharded_dim": [{"axis": 0, "num_shards": 4}]}, "bf16"),
        ((6, 4, 10), {"device": list(range(10)), "sharded_dim": [{"axis": 2, "num_shards": 5}, {"axis": 0, "num_shards": 2}]}, "f32"),
        ((33, 7, 64), {"device": [-1, -2, -3], "device_map": {-1: [0, 5], -2: [1, 4], -3: [2, 3]},
                       "sharded_dim": [{"axis": 0, "num_shards": 3}]}, "bf16"),
        ((4, 4), {"device": [-1], "device_map": {-1: [0, 1, 2]}, "sharded_dim": []}, "f32"),
    ]
    for i, (shape, spec, dt) in enumerate(specs):
        src = inputs.normal(shape, seed=9900 + i, dtype=dt)
        ref = L.split(src, spec)
        srcg = src.cuda()
        for d in sorted(ref)[:: max(1, len(ref) // 3)]:
            mine = Guarded(ref[d].shape, src.dtype)
            tp.tp_shard_materialize_batch([(srcg, spec, {d: mine.t}, d)])
            torch.cuda.synchronize()
            assert mine.guards_intact()
            _compare_with_oracle(src, {d: mine.t.cpu()}, {d: ref[d]})


def test_local_device_not_named_is_rejected():
    spec = {"device": [0, 1], "sharded_dim": [{"axis": 0, "num_shards": 2}]}
    out = Guarded((2, 4), torch.float32)
    src = torch.arange(16, dtype=torch.float32, device="cuda").view(4, 4)
    with pytest.raises(tp.TpError) as e:
        tp.tp_shard_materialize_batch([(src, spec, {2: out.t}, 2)])
    assert e.value.kind == "arg"
    torch.cuda.synchronize()
    assert out.body_untouched() and out.guards_intact()


def test_batch_error_leaves_every_item_untouched():
    announce("layout batch error path")
    ok_src = torch.arange(16, dtype=torch.float32, device="cuda").view(4, 4)
    ok_out = {d: Guarded((2, 4), torch.float32) for d in range(2)}
    bad_src = torch.arange(12, dtype=torch.float32, device="cuda").view(3, 4)
    bad_out = {d: Guarded((1, 4), torch.float32) for d in range(2)}
    spec = {"device": [0, 1], "sharded_dim": [{"axis": 0, "num_shards": 2}]}
    with pytest.raises(tp.TpError) as e:
        tp.tp_shard_materialize_batch([(ok_src, spec, {d: g.t for d, g in ok_out.items()}),
                                       (bad_src, spec, {d: g.t for d, g in bad_out.items()})])
    assert e.value.kind == "indivisible"
    torch.cuda.synchronize()
    for g in list(ok_out.values()) + list(bad_out.values()):
        assert g.body_untouched() and g.guards_intact()


def test_prepared_batch_replays():
    announce("layout prepared batch")
    A = inputs.normal((768, 3072), seed=9900, dtype="bf16").cuda()
    sa = {"device": [0, 1, 2, 3], "sharded_dim": [{"axis": 1, "num_shards": 4}]}
    outs = {d: torch.empty((768, 768), dtype=torch.bfloat16, device="cuda") for d in range(4)}
    call = tp.tp_shard_materialize_batch([(A, sa, outs)], prepare=True)
    ref = L.split(A.cpu(), sa)
    for _ in range(2):
        for o in outs.values():
            o.zero_()
        call(torch.cuda.current_stream())
        torch.cuda.synchronize()
        _compare_with_oracle(A.cpu(), {d: o.cpu() for d, o in outs.items()}, ref)
