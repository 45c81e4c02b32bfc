"""GPU parity of the sequence-parallel MLP (ColossalAI section 5.3: the column
layer all-gathers its input along the sequence axis and the row layer
reduce-scatters its output; in the backward the output gradient is
all-gathered and the input gradient reduce-scattered) against the oracle."""
import numpy as np
import pytest
import torch

import sharded_gemm_amd as tp
from sharded_gemm_amd import inputs
from sharded_gemm_amd.workloads import GPT3_175B, GPT3_6P7B
from oracle import mlp as O
from oracle import reduce as R

from gpu_helpers import Guarded, announce, bits, rel_err, require_gpu

pytestmark = pytest.mark.gpu

TOL_BF16 = 1e-2


def setup_module(_):
    require_gpu()


def _one_hot(H, F, seed):
    g = torch.Generator().manual_seed(seed)
    rows = torch.randint(0, H, (F,), generator=g)
    vals = torch.randint(1, 5, (F,), generator=g) * (torch.randint(0, 2, (F,), generator=g) * 2 - 1)
    A = torch.zeros((H, F))
    A[rows, torch.arange(F)] = vals.float()
    return A.to(torch.bfloat16)


def _f64(t):
    return t.double().numpy()


def sp_forward(X_blocks, A, B, peers, *, Rc=1, Cc=1, act=tp.TP_ACT_GELU_ERF, bias=None, two_streams=True,
               fusion=tp.TP_REDUCE_FUSION_AUTO, in_place=False, noalloc=False):
    """tp_colrow_mlp with X_shards and Z_split into guarded buffers; returns CPU
    copies (X gathered, Y, Z_i, [Z blocks]).  in_place: X = None, GEMM1 reads
    the blocks where they lie (the returned X is then the untouched workspace).
    noalloc: through the allocation-free entry point, which keeps the row
    chunks (the returned Y is then the untouched workspace)."""
    S = len(X_blocks)
    Ms, H = X_blocks[0].shape
    M, F = Ms * S, A.shape[1]
    Xw = Guarded((M, H), X_blocks[0].dtype)
    Y = Guarded((M, F), X_blocks[0].dtype)
    Z = Guarded((M, H), torch.float32)
    Zs = [Guarded((Ms, H), torch.float32) for _ in range(S)]
    s0 = torch.cuda.current_stream()
    s1 = torch.cuda.Stream() if two_streams else s0
    kw = dict(row_chunks=Rc, col_chunks=Cc, peer_partials=list(peers), act=act, s_compute=s0, s_reduce=s1, bias=bias,
              X_shards=list(X_blocks), Z_split=[g.t for g in Zs], reduce_fusion=fusion)
    if noalloc:
        tp.tp_colrow_mlp_noalloc(None if in_place else Xw.t, A, B, Z.t, **kw)
    else:
        tp.tp_colrow_mlp(None if in_place else Xw.t, A, B, Y.t, Z.t, **kw)
    torch.cuda.synchronize()
    for g in [Xw, Y, Z] + Zs:
        assert g.guards_intact(), "write outside an output buffer"
    if in_place:
        assert Xw.body_untouched(), "X = None: nothing is gathered"
    return Xw.t.cpu(), Y.t.cpu(), Z.t.cpu(), [g.t.cpu() for g in Zs]


@pytest.mark.parametrize("M,H,F,Rc,Cc,P,S", [
    (512, 384, 256, 2, 3, 4, 4),      # a row chunk spans two sequence blocks
    (1024, 256, 128, 4, 1, 2, 2),     # a sequence block holds two row chunks
    (96, 72, 40, 3, 2, 3, 3),         # chunks and blocks coincide
    (1030, 640, 320, 2, 5, 5, 2),     # ragged tiles
    (256, 128, 64, 1, 1, 2, 4),       # one block: serial schedule
    (4096, 768, 768, 2, 1, 4, 4),     # GPT-2-small shape
])
def test_forward_integer_exact(M, H, F, Rc, Cc, P, S):
    """Integer chain: the gathered X equals the concatenated blocks, Z_i the
    oracle's partial and block j the oracle's rows j of the full sum."""
    announce(f"seqpar forward integer exact M={M} H={H} F={F} R={Rc} C={Cc} P={P} S={S}")
    Ms = M // S
    Xb = [inputs.small_ints((Ms, H), seed=600 + j, lo=-4, hi=4, dtype="bf16") for j in range(S)]
    A = _one_hot(H, F, 650)
    B = inputs.small_ints((F, H), seed=651, lo=-4, hi=4, dtype="bf16")
    peers = [inputs.small_ints((M, H), seed=660 + p, lo=-512, hi=512) for p in range(P - 1)]
    bias = inputs.small_ints((H,), seed=659, lo=-64, hi=64)
    Xg, Y, Z, Zs = sp_forward([x.cuda() for x in Xb], A.cuda(), B.cuda(), [p.cuda() for p in peers], Rc=Rc, Cc=Cc,
                              act=tp.TP_ACT_NONE, bias=bias.cuda())
    X = torch.cat(Xb)
    assert np.array_equal(bits(Xg), bits(X))
    z_ref = O.mlp_rank(X, A, B, O.GELU_NONE)
    assert np.array_equal(_f64(Z), z_ref)
    ref = R.reduce_split([z_ref] + [_f64(p) for p in peers], S, "sum", _f64(bias))
    for j in range(S):
        assert np.array_equal(_f64(Zs[j]), ref[j]), j


@pytest.mark.parametrize("M,H,F,Rc,Cc,P,S", [
    (4096, 768, 768, 1, 1, 4, 4),     # GPT-2-small: each row of the chunk to one of 4 blocks
    (1024, 384, 256, 2, 2, 4, 4),     # a chunk covers 2 blocks, 2 column blocks
    (1024, 384, 256, 4, 1, 3, 2),     # a chunk lies inside one block
    (1200, 264, 160, 1, 1, 2, 8),     # 8 blocks in the chunk: separate reduce-scatter
    # the 256-row tiles, the tile staged through LDS: a chunk over 4 blocks (8 ranks), a chunk inside a block,
    # ragged rows over 2 blocks
    (4096, 4096, 512, 1, 1, 8, 4),
    (4096, 2048, 512, 2, 1, 8, 2),
    (3000, 4096, 256, 1, 1, 4, 2),
])
def test_forward_reduce_fusion_same_bits(M, H, F, Rc, Cc, P, S):
    """The reduce-scatter folded into GEMM2's epilogue (one stream: one GEMM1
    over all rows, every block folds) gives the separate kernel's bits in
    every sequence block."""
    announce(f"seqpar reduce fusion M={M} H={H} F={F} R={Rc} C={Cc} P={P} S={S}")
    Ms = M // S
    Xb = [inputs.normal((Ms, H), seed=780 + j, dtype="bf16").cuda() for j in range(S)]
    A = inputs.normal((H, F), seed=790, std=0.05, dtype="bf16").cuda()
    B = inputs.normal((F, H), seed=791, std=0.05, dtype="bf16").cuda()
    peers = [inputs.normal((M, H), seed=795 + p).cuda() for p in range(P - 1)]
    bias = inputs.normal((H,), seed=799).cuda()
    kw = dict(Rc=Rc, Cc=Cc, bias=bias, two_streams=False)
    got = sp_forward(Xb, A, B, peers, **kw)
    ref = sp_forward(Xb, A, B, peers, fusion=tp.TP_REDUCE_FUSION_OFF, **kw)
    for a, b in zip(got[:3], ref[:3]):
        assert np.array_equal(bits(a), bits(b))
    for j in range(S):
        assert np.array_equal(bits(got[3][j]), bits(ref[3][j])), j



@pytest.mark.parametrize("M,H,F,Rc,Cc,P,S,dt", [
    (1024, 384, 256, 2, 1, 4, 2, "bf16"),     # each row chunk inside one block: read at an offset
    (2048, 512, 256, 1, 1, 4, 4, "bf16"),     # a chunk over 4 blocks of 512 rows, small tiles
    (4096, 768, 768, 1, 1, 4, 4, "bf16"),     # GPT-2-small shape
    (4096, 1024, 2048, 2, 1, 8, 8, "bf16"),   # chunks over 4 blocks each, the 256-row tiles
    (3072, 512, 1536, 1, 2, 2, 4, "bf16"),    # 768-row blocks, the 256-row tiles, two column blocks
    (1030, 640, 320, 2, 1, 3, 2, "bf16"),     # ragged rows inside one block each
    (256, 96, 64, 4, 1, 2, 2, "f32"),         # fp32, chunks inside blocks
])
def test_forward_blocks_read_in_place_same_bits(M, H, F, Rc, Cc, P, S, dt):
    """With X = None GEMM1 reads the sequence blocks where they lie instead of
    gathering them first: the same Y, Z_i and reduce-scattered sum, bit for bit."""
    announce(f"seqpar blocks in place M={M} H={H} F={F} R={Rc} C={Cc} P={P} S={S} {dt}")
    Ms = M // S
    Xb = [inputs.normal((Ms, H), seed=880 + j, dtype=dt).cuda() for j in range(S)]
    A = inputs.normal((H, F), seed=890, std=0.05, dtype=dt).cuda()
    B = inputs.normal((F, H), seed=891, std=0.05, dtype=dt).cuda()
    peers = [inputs.normal((M, H), seed=895 + p).cuda() for p in range(P - 1)]
    kw = dict(Rc=Rc, Cc=Cc)
    got = sp_forward(Xb, A, B, peers, in_place=True, **kw)
    ref = sp_forward(Xb, A, B, peers, **kw)
    for a, b in zip(got[1:3], ref[1:3]):
        assert np.array_equal(bits(a), bits(b))
    for j in range(S):
        assert np.array_equal(bits(got[3][j]), bits(ref[3][j])), j
    if Rc > 1:
        # The chunks kept (a one-stream schedule may read every block in one GEMM1): each chunk's rows
        # at an offset into its block, or its blocks in turn.
        kept = sp_forward(Xb, A, B, peers, in_place=True, noalloc=True, **kw)
        assert np.array_equal(bits(kept[2]), bits(ref[2]))
        for j in range(S):
            assert np.array_equal(bits(kept[3][j]), bits(ref[3][j])), j


@pytest.mark.parametrize("in_place", [True, False])
def test_one_stream_gemm1_over_all_rows(in_place):
    """One stream, 8 sequence blocks, R = 2: each chunk's sum folds into its
    GEMM2 (4 blocks apiece), so GEMM1 runs once over all rows, read in place
    from the 8 blocks or from X gathered whole first, and each chunk keeps its
    GEMM2.  The same bits as the chunked two-stream schedule with the separate
    reduce-scatter."""
    announce(f"seqpar one stream, GEMM1 over all rows, in_place={in_place}")
    M, H, F, P, S, Rc = 4096, 2048, 512, 8, 8, 2
    Ms = M // S
    Xb = [inputs.normal((Ms, H), seed=980 + j, dtype="bf16").cuda() for j in range(S)]
    A = inputs.normal((H, F), seed=990, std=0.05, dtype="bf16").cuda()
    B = inputs.normal((F, H), seed=991, std=0.05, dtype="bf16").cuda()
    peers = [inputs.normal((M, H), seed=995 + p).cuda() for p in range(P - 1)]
    tp.tp_timing_enable(True)
    try:
        tp.tp_timing_read()
        got = sp_forward(Xb, A, B, peers, Rc=Rc, two_streams=False, in_place=in_place)
        st = tp.tp_timing_read()
    finally:
        tp.tp_timing_enable(False)
    assert st["gemm1"]["launches"] == 1
    assert st["gemm1"]["work"] == 2.0 * M * F * H
    assert st["gemm2_reduce"]["launches"] == Rc and st["gemm2"]["launches"] == 0
    ref = sp_forward(Xb, A, B, peers, Rc=Rc, fusion=tp.TP_REDUCE_FUSION_OFF, in_place=in_place)
    for a, b in zip(got[1:3], ref[1:3]):
        assert np.array_equal(bits(a), bits(b))
    for j in range(S):
        assert np.array_equal(bits(got[3][j]), bits(ref[3][j])), j


def test_forward_blocks_in_place_rejects_blocks_off_the_tile():
    """A row chunk over blocks of 128 rows cannot be read in place (a 256-row
    tile would straddle two blocks): rejected before any launch."""
    announce("seqpar blocks in place, rejected")
    M, H, F, S = 1024, 256, 128, 8
    Xb = [torch.zeros((M // S, H), dtype=torch.bfloat16, device="cuda") for _ in range(S)]
    A = torch.zeros((H, F), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((F, H), dtype=torch.bfloat16, device="cuda")
    Y = Guarded((M, F), torch.bfloat16)
    Z = Guarded((M, H), torch.float32)
    Zs = [Guarded((M // S, H), torch.float32) for _ in range(S)]
    with pytest.raises(tp.TpError) as e:
        tp.tp_colrow_mlp(None, A, B, Y.t, Z.t, X_shards=Xb, Z_split=[g.t for g in Zs])
    assert e.value.kind == "unsupported"
    torch.cuda.synchronize()
    for g in [Y, Z] + Zs:
        assert g.body_untouched() and g.guards_intact()

def test_forward_gelu_matches_unsplit_path_bitwise():
    """GeLU on random bf16 inputs: the sequence-parallel call gives the same bits
    as gathering X by hand and running the all-reduce form, and the blocks are
    within tolerance of the oracle."""
    announce("seqpar forward gelu vs unsplit path")
    M, H, F, P, S, Rc = 2048, 768, 768, 4, 4, 2
    Xb = [inputs.normal((M // S, H), seed=700 + j, dtype="bf16") for j in range(S)]
    A = inputs.normal((H, F), seed=710, std=0.02, dtype="bf16")
    B = inputs.normal((F, H), seed=711, std=0.02, dtype="bf16")
    peers = [inputs.normal((M, H), seed=720 + p) for p in range(P - 1)]
    Xg, Y, Z, Zs = sp_forward([x.cuda() for x in Xb], A.cuda(), B.cuda(), [p.cuda() for p in peers], Rc=Rc)
    X = torch.cat(Xb).cuda()
    Y2 = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    Z2 = torch.empty((M, H), device="cuda")
    Zo = torch.empty((M, H), device="cuda")
    tp.tp_colrow_mlp(X, A.cuda(), B.cuda(), Y2, Z2, row_chunks=Rc, peer_partials=[p.cuda() for p in peers], Z_out=Zo,
                     s_reduce=torch.cuda.Stream())
    torch.cuda.synchronize()
    assert np.array_equal(bits(Y), bits(Y2.cpu()))
    assert np.array_equal(bits(Z), bits(Z2.cpu()))
    full = torch.cat(Zs)
    assert np.array_equal(bits(full), bits(Zo.cpu()))
    rows = np.arange(0, M, 37)
    ref = O.mlp_rank_rows(torch.cat(Xb), A, B, rows) + sum(_f64(p)[rows] for p in peers)
    assert rel_err(full[torch.from_numpy(rows)], ref) <= TOL_BF16


@pytest.mark.parametrize("M,H,F,Rc,Cc,P,S,with_bias", [
    (256, 96, 64, 1, 1, 3, 4, True),     # one chunk covers 4 blocks: every row to its block (nout 4)
    (256, 96, 64, 2, 1, 2, 4, False),    # a chunk covers 2 blocks (nout 2)
    (192, 80, 48, 1, 2, 2, 3, True),     # 3 blocks, 2 column blocks
    (256, 64, 32, 4, 1, 3, 2, True),     # a chunk lies inside one block
    (200, 72, 40, 1, 1, 2, 8, False),    # 8 blocks in the chunk: beyond the epilogue's outputs
    (64, 256, 512, 1, 1, 2, 2, True),    # the tiny workload's shape
])
def test_forward_fp32_integer_exact(M, H, F, Rc, Cc, P, S, with_bias):
    """fp32 path (the tiny workload's kernels) with the reduce-scatter: the
    epilogue's form on the serial schedule and the separate kernel on two
    streams give the same bits, each block equal to the oracle's rows."""
    announce(f"seqpar fp32 integer exact M={M} H={H} F={F} R={Rc} C={Cc} P={P} S={S} bias={with_bias}")
    Ms = M // S
    Xb = [inputs.small_ints((Ms, H), seed=900 + j, lo=-4, hi=4) for j in range(S)]
    A = _one_hot(H, F, 950).float()
    B = inputs.small_ints((F, H), seed=951, lo=-4, hi=4)
    peers = [inputs.small_ints((M, H), seed=960 + p, lo=-512, hi=512) for p in range(P - 1)]
    bias = inputs.small_ints((H,), seed=959, lo=-64, hi=64) if with_bias else None
    dev = dict(X_blocks=[x.cuda() for x in Xb], A=A.cuda(), B=B.cuda(), peers=[p.cuda() for p in peers])
    kw = dict(Rc=Rc, Cc=Cc, act=tp.TP_ACT_NONE, bias=bias.cuda() if with_bias else None)
    fused = sp_forward(**dev, two_streams=False, **kw)
    apart = sp_forward(**dev, two_streams=False, fusion=tp.TP_REDUCE_FUSION_OFF, **kw)
    beside = sp_forward(**dev, two_streams=True, **kw)
    for got in (apart, beside):
        for a, b in zip(got[:3], fused[:3]):
            assert np.array_equal(bits(a), bits(b))
        for j in range(S):
            assert np.array_equal(bits(got[3][j]), bits(fused[3][j])), j
    X = torch.cat(Xb)
    assert np.array_equal(bits(fused[0]), bits(X))
    z_ref = O.mlp_rank(X, A, B, O.GELU_NONE)
    assert np.array_equal(_f64(fused[2]), z_ref)
    ref = R.reduce_split([z_ref] + [_f64(p) for p in peers], S, "sum", _f64(bias) if with_bias else None)
    for j in range(S):
        assert np.array_equal(_f64(fused[3][j]), ref[j]), j


def _chunk_rows(M, Rc, per_chunk):
    Mr = M // Rc
    rows = []
    for r in range(Rc):
        rows += list(np.unique(np.linspace(r * Mr, (r + 1) * Mr - 1, per_chunk).astype(np.int64)))
    return np.array(rows)


@pytest.mark.parametrize("w", [GPT3_175B, GPT3_6P7B], ids=lambda w: w.name)
@pytest.mark.parametrize("in_place", [True, False])
def test_forward_gpt3_sampled(w, in_place):
    """A GPT-3 per-rank shape as the bench's sequence-parallel step runs it
    (TP = 8: 8 sequence blocks, R row chunks, C column blocks, two streams
    offered; GEMM1 reading the blocks where they lie, or after gathering them,
    when the gathered input must equal the blocks; for 6.7B with the blocks in
    place the call keeps to one stream and one GEMM1 reads all 8 blocks), and
    128 rows of the reduce-scattered output (64 per row chunk, each chunk's
    first and last among them) match the oracle's rank-0 rows plus the drawn
    peers' rows."""
    announce(f"seqpar forward {w.name} sampled in_place={in_place}")
    M, H, F, P, S = w.M, w.H, w.F, w.P, w.P
    Ms = M // S
    Xb = [inputs.normal((Ms, H), inputs.seed_for(w.cfg, inputs.SLOT_X) + 100 * j, 1.0, "bf16", "cuda")
          for j in range(S)]
    A = inputs.normal((H, F), inputs.seed_for(w.cfg, inputs.SLOT_A), 0.02, "bf16", "cuda")
    B = inputs.normal((F, H), inputs.seed_for(w.cfg, inputs.SLOT_B), 0.02, "bf16", "cuda")
    peers = [inputs.normal((M, H), inputs.seed_for(w.cfg, inputs.SLOT_PARTIAL + p), 1.0, "f32", "cuda")
             for p in range(P - 1)]
    Xg, Y, Z, Zs = sp_forward(Xb, A, B, peers, Rc=w.R, Cc=w.C, in_place=in_place)
    X = torch.cat([x.cpu() for x in Xb])
    if not in_place:
        assert np.array_equal(bits(Xg), bits(X))
    rows = _chunk_rows(M, w.R, 64)
    announce(f"seqpar forward {w.name}: oracle on {len(rows)} rows")
    z0 = O.mlp_rank_rows(X, A.cpu(), B.cpu(), rows)
    assert rel_err(Z[torch.from_numpy(rows)], z0) <= TOL_BF16
    ref = z0 + sum(p[torch.from_numpy(rows).cuda()].cpu().double().numpy() for p in peers)
    full = torch.cat(Zs)
    assert rel_err(full[torch.from_numpy(rows)], ref) <= TOL_BF16


def sp_backward(X, A, B, Y, dZ_blocks, peers, *, Rc=1, act=tp.TP_ACT_NONE, H_i=None, two_streams=True):
    S = len(dZ_blocks)
    Ms, H = dZ_blocks[0].shape
    M, F = Ms * S, A.shape[1]
    dZw = Guarded((M, H), X.dtype)
    dH = Guarded((M, F), X.dtype)
    dX = Guarded((M, H), torch.float32)
    dA = Guarded((H, F), torch.float32)
    dB = Guarded((F, H), torch.float32)
    dXs = [Guarded((Ms, H), torch.float32) for _ in range(S)]
    s0 = torch.cuda.current_stream()
    s1 = torch.cuda.Stream() if two_streams else s0
    tp.tp_colrow_mlp_backward(X, A, B, H_i, Y, dZw.t, dH.t, dX.t, dA.t, dB.t, row_chunks=Rc, peer_dX=list(peers),
                              act=act, s_compute=s0, s_reduce=s1, dZ_shards=list(dZ_blocks),
                              dX_split=[g.t for g in dXs])
    torch.cuda.synchronize()
    for g in [dZw, dH, dX, dA, dB] + dXs:
        assert g.guards_intact(), "write outside an output buffer"
    return dZw.t.cpu(), dX.t.cpu(), dA.t.cpu(), dB.t.cpu(), [g.t.cpu() for g in dXs]


@pytest.mark.parametrize("M,H,F,Rc,P,S", [
    (512, 384, 256, 2, 4, 4), (1024, 256, 128, 4, 2, 2), (300, 264, 136, 3, 3, 3), (256, 128, 64, 1, 1, 4),
    (4096, 768, 768, 2, 4, 8),
])
def test_backward_integer_exact(M, H, F, Rc, P, S):
    """Integer chain through the backward: dZ gathered from its blocks, the
    weight gradients and the reduce-scattered input gradient exact."""
    announce(f"seqpar backward integer exact M={M} H={H} F={F} R={Rc} P={P} S={S}")
    Ms = M // S
    X = inputs.small_ints((M, H), seed=801, lo=-4, hi=4, dtype="bf16")
    A = _one_hot(H, F, 802)
    B = _one_hot(H, F, 803).t().contiguous()
    dZb = [inputs.small_ints((Ms, H), seed=810 + j, lo=-4, hi=4, dtype="bf16") for j in range(S)]
    peers = [inputs.small_ints((M, H), seed=830 + p, lo=-512, hi=512) for p in range(P - 1)]
    Xd, Ad, Bd = X.cuda(), A.cuda(), B.cuda()
    Y = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    Z = torch.empty((M, H), device="cuda")
    tp.tp_colrow_mlp(Xd, Ad, Bd, Y, Z, act=tp.TP_ACT_NONE)
    dZg, dX, dA, dB, dXs = sp_backward(Xd, Ad, Bd, Y, [d.cuda() for d in dZb], [p.cuda() for p in peers], Rc=Rc)
    dZ = torch.cat(dZb)
    assert np.array_equal(bits(dZg), bits(dZ))
    g = O.backward_rank(X, A, B, dZ, O.GELU_NONE)
    assert np.array_equal(_f64(dX), g["dX_i"])
    assert np.array_equal(_f64(dA), g["dA_i"])
    assert np.array_equal(_f64(dB), g["dB_i"])
    ref = R.reduce_split([g["dX_i"]] + [_f64(p) for p in peers], S)
    for j in range(S):
        assert np.array_equal(_f64(dXs[j]), ref[j]), j


def test_backward_gelu_tolerance():
    announce("seqpar backward gelu tolerance")
    M, H, F, P, S, Rc = 1024, 512, 384, 2, 4, 2
    X = inputs.normal((M, H), seed=851, dtype="bf16")
    A = inputs.normal((H, F), seed=852, std=0.05, dtype="bf16")
    B = inputs.normal((F, H), seed=853, std=0.05, dtype="bf16")
    dZb = [inputs.normal((M // S, H), seed=860 + j, dtype="bf16") for j in range(S)]
    peers = [inputs.normal((M, H), seed=870)]
    Xd, Ad, Bd = X.cuda(), A.cuda(), B.cuda()
    Y = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    Z = torch.empty((M, H), device="cuda")
    Hs = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    tp.tp_colrow_mlp(Xd, Ad, Bd, Y, Z, H_out=Hs)
    dZg, dX, dA, dB, dXs = sp_backward(Xd, Ad, Bd, Y, [d.cuda() for d in dZb], [p.cuda() for p in peers], Rc=Rc,
                                       act=tp.TP_ACT_GELU_ERF, H_i=Hs)
    g = O.backward_rank(X, A, B, torch.cat(dZb), O.GELU_ERF)
    assert rel_err(dA, g["dA_i"]) <= TOL_BF16
    assert rel_err(dB, g["dB_i"]) <= TOL_BF16
    assert rel_err(torch.cat(dXs), g["dX_i"] + _f64(peers[0])) <= TOL_BF16


def test_backward_gpt3_175b_sampled():
    """The bench's sequence-parallel backward at the GPT-3 175B per-rank shape
    (TP = 8 blocks, R = 2): dZ gathered from its blocks, 128 rows of the
    reduce-scattered input gradient and 32 columns of dA / rows of dB against
    the oracle."""
    w = GPT3_175B
    announce(f"seqpar backward {w.name} sampled")
    M, H, F, P, S = w.M, w.H, w.F, w.P, w.P
    X = inputs.normal((M, H), inputs.seed_for(w.cfg, inputs.SLOT_X), 1.0, "bf16", "cuda")
    A = inputs.normal((H, F), inputs.seed_for(w.cfg, inputs.SLOT_A), 0.02, "bf16", "cuda")
    B = inputs.normal((F, H), inputs.seed_for(w.cfg, inputs.SLOT_B), 0.02, "bf16", "cuda")
    dZb = [inputs.normal((M // S, H), inputs.seed_for(w.cfg, inputs.SLOT_DZ) + 100 * j, 1.0, "bf16", "cuda")
           for j in range(S)]
    peers = [inputs.normal((M, H), inputs.seed_for(w.cfg, inputs.SLOT_PARTIAL + p), 1.0, "f32", "cuda")
             for p in range(P - 1)]
    Y = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    Z = torch.empty((M, H), device="cuda")
    Hs = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    tp.tp_colrow_mlp(X, A, B, Y, Z, H_out=Hs)
    del Z
    dZg, dX, dA, dB, dXs = sp_backward(X, A, B, Y, dZb, peers, Rc=w.R, act=tp.TP_ACT_GELU_ERF, H_i=Hs)
    dZ = torch.cat([d.cpu() for d in dZb])
    assert np.array_equal(bits(dZg), bits(dZ))
    Xc, Ac, Bc = X.cpu(), A.cpu(), B.cpu()
    rows = _chunk_rows(M, w.R, 64)
    cols = np.sort(np.random.default_rng(1).choice(F, 32, replace=False))
    announce(f"seqpar backward {w.name}: oracle on {len(rows)} rows and {len(cols)} columns")
    gr = O.backward_rank(Xc[rows], Ac, Bc, dZ[rows])
    assert rel_err(dX[torch.from_numpy(rows)], gr["dX_i"]) <= TOL_BF16
    ridx = torch.from_numpy(rows)
    ref = gr["dX_i"] + sum(p[ridx.cuda()].cpu().double().numpy() for p in peers)
    assert rel_err(torch.cat(dXs)[ridx], ref) <= TOL_BF16
    gc = O.backward_rank(Xc, Ac[:, cols], Bc[cols, :], dZ)
    assert rel_err(dA[:, cols], gc["dA_i"]) <= TOL_BF16
    assert rel_err(dB[cols, :], gc["dB_i"]) <= TOL_BF16


def test_error_leaves_outputs_untouched():
    """Chunks of 8 rows and blocks of 6 do not nest: rejected before any launch."""
    announce("seqpar error path")
    M, H, F, S = 24, 16, 16, 4
    Xb = [torch.zeros((M // S, H), dtype=torch.bfloat16, device="cuda") for _ in range(S)]
    A = torch.zeros((H, F), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((F, H), dtype=torch.bfloat16, device="cuda")
    Xw = Guarded((M, H), torch.bfloat16)
    Y = Guarded((M, F), torch.bfloat16)
    Z = Guarded((M, H), torch.float32)
    Zs = [Guarded((M // S, H), torch.float32) for _ in range(S)]
    with pytest.raises(tp.TpError) as e:
        tp.tp_colrow_mlp(Xw.t, A, B, Y.t, Z.t, row_chunks=3, X_shards=Xb, Z_split=[g.t for g in Zs])
    assert e.value.kind == "unsupported"
    torch.cuda.synchronize()
    for g in [Xw, Y, Z] + Zs:
        assert g.body_untouched() and g.guards_intact()
