"""GPU parity of tp_partial_reduce against the reduction oracle."""
import numpy as np
import pytest
import torch

import sharded_gemm_amd as tp
from sharded_gemm_amd import inputs
from sharded_gemm_amd.workloads import RESHARD
from oracle import reduce as R

from gpu_helpers import Guarded, announce, bits, rel_err, require_gpu

pytestmark = pytest.mark.gpu

TOL = 1e-6   # max|err| / max|ref| for fp32 sums vs the fp64 oracle


def setup_module(_):
    require_gpu()


@pytest.mark.parametrize("P", [1, 2, 3, 8, 13])
@pytest.mark.parametrize("rows,cols,ld", [(1, 1, 1), (7, 3, 5), (64, 1027, 1027), (300, 256, 384),
                                          (129, 768, 768), (4, 4100, 4104)])
def test_full(P, rows, cols, ld):
    announce(f"reduce FULL P={P} rows={rows} cols={cols} ld={ld}")
    parts_cpu = [inputs.normal((rows, ld), seed=5000 + p) for p in range(P)]
    parts = [p.cuda() for p in parts_cpu]
    out = Guarded((rows, ld), torch.float32)
    tp.tp_partial_reduce(parts, [out.t], tp.TP_REDUCE_FULL, rows=rows, cols=cols, ld_in=ld, ld_out=ld)
    torch.cuda.synchronize()
    assert out.guards_intact()
    got = out.t.cpu()
    ref = R.reduce_full([p[:, :cols] for p in parts_cpu])
    assert rel_err(got[:, :cols], ref) <= TOL
    if ld > cols:   # padding columns are not written
        pad = bits(got[:, cols:])
        assert (pad == np.int32(0x7FC0DEAD)).all()


def test_integer_partials_bit_exact():
    announce("reduce FULL integer partials, bit-exact")
    P, rows, cols = 8, 333, 517
    parts_cpu = [inputs.small_ints((rows, cols), seed=6000 + p, lo=-1024, hi=1024) for p in range(P)]
    out = torch.empty((rows, cols), device="cuda")
    tp.tp_partial_reduce([p.cuda() for p in parts_cpu], [out])
    ref = R.reduce_full(parts_cpu)
    assert np.array_equal(out.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("rows,cols", [(0, 16), (16, 0)])
def test_empty_block_is_a_no_op(rows, cols):
    """A block with no rows or no columns launches nothing and leaves the
    output untouched, in both modes."""
    announce(f"reduce empty block rows={rows} cols={cols}")
    parts = [torch.zeros((16, 16), device="cuda") for _ in range(3)]
    full = Guarded((16, 16), torch.float32)
    tp.tp_partial_reduce(parts, [full.t], tp.TP_REDUCE_FULL, rows=rows, cols=cols, ld_in=16, ld_out=16)
    outs = [Guarded((8, 16), torch.float32) for _ in range(2)]
    tp.tp_partial_reduce(parts, [o.t for o in outs], tp.TP_REDUCE_SPLIT, rows=rows, cols=cols, ld_in=16, ld_out=16)
    torch.cuda.synchronize()
    for g in [full] + outs:
        assert g.guards_intact()
        assert (bits(g.t.cpu()) == np.int32(0x7FC0DEAD)).all()


def test_in_place():
    announce("reduce FULL in place")
    parts_cpu = [inputs.normal((96, 200), seed=7000 + p) for p in range(4)]
    parts = [p.cuda() for p in parts_cpu]
    tp.tp_partial_reduce(parts, [parts[0]])
    assert rel_err(parts[0].cpu(), R.reduce_full(parts_cpu)) <= TOL


@pytest.mark.parametrize("P,S,rows,cols", [(2, 2, 8, 5), (4, 4, 64, 1000), (3, 6, 96, 64)])
def test_split_small(P, S, rows, cols):
    announce(f"reduce SPLIT P={P} S={S} {rows}x{cols}")
    parts_cpu = [inputs.normal((rows, cols), seed=8000 + p) for p in range(P)]
    outs = [Guarded((rows // S, cols), torch.float32) for _ in range(S)]
    tp.tp_partial_reduce([p.cuda() for p in parts_cpu], [o.t for o in outs], tp.TP_REDUCE_SPLIT)
    torch.cuda.synchronize()
    ref = R.reduce_split(parts_cpu, S)
    for j in range(S):
        assert outs[j].guards_intact()
        assert rel_err(outs[j].t.cpu(), ref[j]) <= TOL


def test_split_full_size():
    """8 fp32 partials [8192, 8192] -> 8 row shards [1024, 8192]."""
    w = RESHARD
    announce("reduce SPLIT full size 8 x [8192,8192] -> 8 x [1024,8192]")
    parts = [inputs.normal(w.partial_shape, inputs.seed_for(4, inputs.SLOT_PARTIAL + p), device="cuda")
             for p in range(w.num_partials)]
    rows = w.partial_shape[0] // w.num_splits
    outs = [torch.empty((rows, w.partial_shape[1]), device="cuda") for _ in range(w.num_splits)]
    tp.tp_partial_reduce(parts, outs, tp.TP_REDUCE_SPLIT)
    torch.cuda.synchronize()
    parts_cpu = [p.cpu() for p in parts]
    ref = R.reduce_split(parts_cpu, w.num_splits)
    for j in range(w.num_splits):
        assert rel_err(outs[j].cpu(), ref[j]) <= TOL, j


def test_error_leaves_output_untouched():
    announce("reduce error path")
    parts = [torch.zeros((6, 4), device="cuda") for _ in range(2)]
    outs = [Guarded((2, 4), torch.float32) for _ in range(4)]
    with pytest.raises(tp.TpError) as e:
        tp.tp_partial_reduce(parts, [o.t for o in outs], tp.TP_REDUCE_SPLIT)   # 6 rows, 4 splits
    assert e.value.kind == "indivisible"
    torch.cuda.synchronize()
    assert all(o.body_untouched() for o in outs)


# ---- partial max / min and the bias ------------------------------------------

OPS = {tp.TP_REDUCE_OP_SUM: "sum", tp.TP_REDUCE_OP_MAX: "max", tp.TP_REDUCE_OP_MIN: "min"}


@pytest.mark.parametrize("op", [tp.TP_REDUCE_OP_MAX, tp.TP_REDUCE_OP_MIN])
@pytest.mark.parametrize("P,rows,cols,ld", [(1, 5, 3, 3), (3, 64, 1027, 1027), (8, 300, 256, 384), (13, 129, 768, 768)])
def test_max_min_bit_exact(op, P, rows, cols, ld):
    """max / min pick one of the inputs, so the result is bit-exact."""
    announce(f"reduce FULL op={OPS[op]} P={P} rows={rows} cols={cols} ld={ld}")
    parts_cpu = [inputs.normal((rows, ld), seed=8000 + p) for p in range(P)]
    out = Guarded((rows, ld), torch.float32)
    tp.tp_partial_reduce([p.cuda() for p in parts_cpu], [out.t], rows=rows, cols=cols, ld_in=ld, ld_out=ld, op=op)
    torch.cuda.synchronize()
    assert out.guards_intact()
    ref = R.reduce_full([p[:, :cols] for p in parts_cpu], OPS[op])
    assert np.array_equal(out.t.cpu()[:, :cols].numpy().astype(np.float64), ref)


def test_max_min_nan_loses_to_a_number():
    announce("reduce max/min with NaN")
    a = torch.tensor([[float("nan"), 1.0, float("nan"), -3.0]], device="cuda")
    b = torch.tensor([[2.0, float("nan"), float("nan"), 5.0]], device="cuda")
    for op in (tp.TP_REDUCE_OP_MAX, tp.TP_REDUCE_OP_MIN):
        out = torch.empty_like(a)
        tp.tp_partial_reduce([a, b], [out], op=op)
        ref = R.reduce_full([a.cpu(), b.cpu()], OPS[op])
        got = out.cpu().numpy().astype(np.float64)
        assert np.array_equal(np.isnan(got), np.isnan(ref))
        assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])


@pytest.mark.parametrize("op", [tp.TP_REDUCE_OP_SUM, tp.TP_REDUCE_OP_MAX, tp.TP_REDUCE_OP_MIN])
@pytest.mark.parametrize("mode,S,rows,cols,boff", [("full", 1, 96, 1000, 0), ("full", 1, 33, 517, 0),
                                                   ("full", 1, 96, 1000, 1), ("split", 4, 64, 1000, 0),
                                                   ("split", 8, 8192, 1024, 0)])
def test_bias_integer_exact(op, mode, S, rows, cols, boff):
    """out = op over partials + bias, on integers: exact.  boff = 1 misaligns the
    bias by one element (scalar path)."""
    announce(f"reduce {mode} op={OPS[op]} + bias rows={rows} cols={cols} S={S} bias offset {boff}")
    P = 5
    parts_cpu = [inputs.small_ints((rows, cols), seed=8100 + p, lo=-1000, hi=1000) for p in range(P)]
    bias_cpu = inputs.small_ints((cols + boff,), seed=8199, lo=-100, hi=100)
    bias = bias_cpu.cuda()
    outs = [torch.empty((rows // S, cols), device="cuda") for _ in range(S)]
    tp.tp_partial_reduce([p.cuda() for p in parts_cpu], outs, tp.TP_REDUCE_FULL if mode == "full" else tp.TP_REDUCE_SPLIT,
                         op=op, bias=bias[boff:])
    ref = R.reduce_split(parts_cpu, S, OPS[op], bias_cpu[boff:])
    for o, r in zip(outs, ref):
        assert np.array_equal(o.cpu().numpy().astype(np.float64), r)


def test_bias_with_random_sum():
    announce("reduce FULL sum + bias, random")
    parts_cpu = [inputs.normal((512, 768), seed=8300 + p) for p in range(4)]
    bias_cpu = inputs.normal((768,), seed=8399)
    out = torch.empty((512, 768), device="cuda")
    tp.tp_partial_reduce([p.cuda() for p in parts_cpu], [out], bias=bias_cpu.cuda())
    assert rel_err(out.cpu(), R.reduce_full(parts_cpu, "sum", bias_cpu)) <= TOL


# ---- maximum sizes ------------------------------------------------------------

def test_max_partials_and_splits_integer_exact():
    """P = 64 partials (eight load groups) and S = 64 output blocks, the
    largest the library takes: integer sums, exact."""
    announce("reduce P=64 FULL and P=64 S=64 SPLIT")
    P, rows, cols = 64, 256, 520
    parts_cpu = [inputs.small_ints((rows, cols), seed=8500 + p, lo=-1000, hi=1000) for p in range(P)]
    parts = [p.cuda() for p in parts_cpu]
    out = Guarded((rows, cols), torch.float32)
    tp.tp_partial_reduce(parts, [out.t])
    blocks = [Guarded((rows // 64, cols), torch.float32) for _ in range(64)]
    tp.tp_partial_reduce(parts, [b.t for b in blocks], tp.TP_REDUCE_SPLIT)
    torch.cuda.synchronize()
    full = R.reduce_full(parts_cpu)
    assert out.guards_intact() and np.array_equal(out.t.cpu().numpy().astype(np.float64), full)
    ref = R.reduce_split(parts_cpu, 64)
    for b, r in zip(blocks, ref):
        assert b.guards_intact() and np.array_equal(b.t.cpu().numpy().astype(np.float64), r)
