"""GPU parity of tp_colrow_mlp_backward (dH with the fused GeLU derivative, the
partial input gradient and its reduce over ranks, the weight gradients) and of
the forward's saved pre-activation, against the oracle's backward."""
import numpy as np
import pytest
import torch

import sharded_gemm_amd as tp
from sharded_gemm_amd import inputs
from sharded_gemm_amd.workloads import GPT3_175B, GPT3_6P7B, TINY
from oracle import layout as L
from oracle import mlp as O
from oracle import reduce as R

from gpu_helpers import Guarded, announce, bits, rel_err, require_gpu

pytestmark = pytest.mark.gpu

TOL_BF16 = 1e-2   # max|err|/max|ref|: bf16 operands, fp32 accumulation, H, Y and dH rounded to bf16
TOL_F32 = 1e-5    # same measure, fp32 throughout


def setup_module(_):
    require_gpu()


def forward(X, A_i, B_i, *, act=tp.TP_ACT_GELU_ERF, save_h=True):
    """The forward on the GPU; returns device Y and (for GeLU) H."""
    M, H = X.shape
    F = A_i.shape[1]
    Y = torch.empty((M, F), dtype=X.dtype, device="cuda")
    Z = torch.empty((M, H), dtype=torch.float32, device="cuda")
    Hs = torch.empty((M, F), dtype=X.dtype, device="cuda") if (save_h and act == tp.TP_ACT_GELU_ERF) else None
    tp.tp_colrow_mlp(X, A_i, B_i, Y, Z, act=act, H_out=Hs)
    return Y, Hs


def backward(X, A_i, B_i, H_i, Y_i, dZ, *, R=1, peers=(), act=tp.TP_ACT_GELU_ERF, two_streams=True,
             dA0=None, dB0=None):
    """One backward call into canary-guarded outputs; returns CPU copies
    (dH, dX_i, dX_out, dA_i, dB_i).  dA0 / dB0: starting weight gradients
    (then accumulate = 1)."""
    M, H = X.shape
    F = A_i.shape[1]
    dH = Guarded((M, F), X.dtype)
    dX = Guarded((M, H), torch.float32)
    dXo = Guarded((M, H), torch.float32) if peers else None
    dA = Guarded((H, F), torch.float32)
    dB = Guarded((F, H), torch.float32)
    acc = dA0 is not None
    if acc:
        dA.t.copy_(dA0)
        dB.t.copy_(dB0)
    s0 = torch.cuda.current_stream()
    s1 = torch.cuda.Stream() if two_streams else s0
    tp.tp_colrow_mlp_backward(X, A_i, B_i, H_i, Y_i, dZ, dH.t, dX.t, dA.t, dB.t, row_chunks=R, peer_dX=list(peers),
                              dX_out=dXo.t if dXo is not None else None, act=act, accumulate=acc,
                              s_compute=s0, s_reduce=s1)
    torch.cuda.synchronize()
    for g in (dH, dX, dA, dB) + ((dXo,) if dXo is not None else ()):
        assert g.guards_intact(), "write outside an output buffer"
    return dH.t.cpu(), dX.t.cpu(), (dXo.t.cpu() if dXo is not None else None), dA.t.cpu(), dB.t.cpu()


def _one_hot(H, F, seed):
    """[H, F] with one small nonzero integer per column."""
    g = torch.Generator().manual_seed(seed)
    rows = torch.randint(0, H, (F,), generator=g)
    vals = torch.randint(1, 5, (F,), generator=g) * (torch.randint(0, 2, (F,), generator=g) * 2 - 1)
    A = torch.zeros((H, F))
    A[rows, torch.arange(F)] = vals.float()
    return A.to(torch.bfloat16)


def _f64(t):
    return t.double().numpy()


# ---------------------------------------------------------------- exact cases

@pytest.mark.parametrize("M,H,F,Rc,P", [
    (77, 45, 51, 1, 1), (300, 264, 136, 3, 2), (1024, 1024, 512, 4, 3), (4096, 768, 768, 2, 4),
    # weight gradient on the ping-pong kernel with A given transposed (256 x 192)
    (256, 2048, 6144, 1, 2),
    # dH GEMM on the ping-pong kernel with W given transposed (256 x 192)
    (4096, 256, 6144, 2, 2),
    # every GEMM on the ping-pong kernel's 256 x 128 tiles (dA, dB with A transposed)
    (4000, 2000, 2000, 1, 2), (4000, 2000, 2000, 2, 2),
    # dA on 256 x 192 tiles with A transposed
    (512, 2048, 6144, 2, 2),
    # dA and dB in one grouped launch, 45 tiles each (the second problem's tiles start off the XCD stride)
    (256, 576, 320, 1, 2),
    # the same, 32-deep stages (160 tokens)
    (160, 576, 320, 2, 2),
])
def test_backward_integer_exact(M, H, F, Rc, P):
    """One-hot A_i (columns) and B_i (rows) keep every value a small integer:
    dH = dZ B_i^T is exact in bf16 and dX, dA, dB, dX_out are exact in fp32,
    so all must equal the oracle bit for bit."""
    announce(f"backward integer exact M={M} H={H} F={F} R={Rc} P={P}")
    X = inputs.small_ints((M, H), seed=401, lo=-4, hi=4, dtype="bf16")
    A = _one_hot(H, F, 402)
    B = _one_hot(H, F, 403).t().contiguous()
    dZ = inputs.small_ints((M, H), seed=404, lo=-4, hi=4, dtype="bf16")
    peers = [inputs.small_ints((M, H), seed=410 + p, lo=-512, hi=512) for p in range(P - 1)]
    Xd, Ad, Bd, dZd = X.cuda(), A.cuda(), B.cuda(), dZ.cuda()
    Y, _ = forward(Xd, Ad, Bd, act=tp.TP_ACT_NONE)
    dH, dX, dXo, dA, dB = backward(Xd, Ad, Bd, None, Y, dZd, R=Rc, peers=[p.cuda() for p in peers],
                                   act=tp.TP_ACT_NONE)
    g = O.backward_rank(X, A, B, dZ, O.GELU_NONE)
    assert np.array_equal(_f64(dH), g["dH"])
    assert np.array_equal(_f64(dX), g["dX_i"])
    assert np.array_equal(_f64(dA), g["dA_i"])
    assert np.array_equal(_f64(dB), g["dB_i"])
    if P > 1:
        assert np.array_equal(_f64(dXo), R.reduce_full([g["dX_i"]] + [p.double().numpy() for p in peers]))


@pytest.mark.parametrize("M,H,F,dt", [
    (512, 384, 256, "bf16"),
    # the accumulating weight-gradient GEMMs (A transposed) on larger tiles, and
    # in the grouped launch with 64- and 32-deep stages
    (4000, 2000, 2000, "bf16"), (512, 2048, 6144, "bf16"), (256, 576, 320, "bf16"), (160, 576, 320, "bf16"),
    # the fp32 GEMM continuing from C, off its tile sizes
    (130, 129, 65, "f32"),
])
def test_backward_accumulates_weight_gradients(M, H, F, dt):
    """accumulate = 1 continues from the given dA_i, dB_i: exact integers twice over."""
    announce(f"backward accumulate M={M} H={H} F={F} {dt}")
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    X = inputs.small_ints((M, H), seed=421, lo=-4, hi=4, dtype=dt).cuda()
    A = _one_hot(H, F, 422).to(tdt).cuda()
    B = _one_hot(H, F, 423).t().contiguous().to(tdt).cuda()
    dZ = inputs.small_ints((M, H), seed=424, lo=-4, hi=4, dtype=dt).cuda()
    Y, _ = forward(X, A, B, act=tp.TP_ACT_NONE)
    _, _, _, dA1, dB1 = backward(X, A, B, None, Y, dZ, R=2, act=tp.TP_ACT_NONE)
    _, _, _, dA2, dB2 = backward(X, A, B, None, Y, dZ, R=2, act=tp.TP_ACT_NONE, dA0=dA1.cuda(), dB0=dB1.cuda())
    assert torch.equal(dA2, 2 * dA1) and torch.equal(dB2, 2 * dB1)


# ---------------------------------------------------------------- GeLU, tolerance

@pytest.mark.parametrize("M,H,F,Rc,P", [(333, 320, 200, 1, 2), (1500, 2048, 1024, 3, 3), (4096, 768, 768, 1, 4)])
def test_backward_gelu(M, H, F, Rc, P):
    announce(f"backward gelu M={M} H={H} F={F} R={Rc} P={P}")
    X = inputs.normal((M, H), 501, 1.0, "bf16")
    A = inputs.normal((H, F), 502, 1.0 / np.sqrt(H), "bf16")
    B = inputs.normal((F, H), 503, 1.0 / np.sqrt(F), "bf16")
    dZ = inputs.normal((M, H), 504, 1.0, "bf16")
    peers = [inputs.normal((M, H), 510 + p) for p in range(P - 1)]
    Xd, Ad, Bd, dZd = X.cuda(), A.cuda(), B.cuda(), dZ.cuda()
    Y, Hs = forward(Xd, Ad, Bd)
    # The saved pre-activation is X A_i rounded to bf16.
    assert rel_err(Hs, O.hidden(X, A, O.GELU_NONE)) <= TOL_BF16
    dH, dX, dXo, dA, dB = backward(Xd, Ad, Bd, Hs, Y, dZd, R=Rc, peers=[p.cuda() for p in peers])
    g = O.backward_rank(X, A, B, dZ)
    assert rel_err(dH, g["dH"]) <= TOL_BF16
    assert rel_err(dX, g["dX_i"]) <= TOL_BF16
    assert rel_err(dA, g["dA_i"]) <= TOL_BF16
    assert rel_err(dB, g["dB_i"]) <= TOL_BF16
    assert rel_err(dXo, R.reduce_full([g["dX_i"]] + [p.double().numpy() for p in peers])) <= TOL_BF16


@pytest.mark.parametrize("M,H,F,Rc,P", [(77, 45, 51, 1, 2), (300, 264, 136, 3, 2), (130, 129, 65, 2, 3),
                                        (1, 1, 1, 1, 2)])
def test_backward_gelu_fp32_ragged(M, H, F, Rc, P):
    """fp32 throughout, sizes off the 32 x 32 tile and the 64-deep k slab: the
    fused GeLU derivative, and the transposed operands of the weight
    gradients, taken over all rows at once."""
    announce(f"backward gelu fp32 M={M} H={H} F={F} R={Rc} P={P}")
    X = inputs.normal((M, H), 521, 1.0)
    A = inputs.normal((H, F), 522, 1.0 / np.sqrt(H))
    B = inputs.normal((F, H), 523, 1.0 / np.sqrt(F))
    dZ = inputs.normal((M, H), 524, 1.0)
    peers = [inputs.normal((M, H), 530 + p) for p in range(P - 1)]
    Xd, Ad, Bd, dZd = X.cuda(), A.cuda(), B.cuda(), dZ.cuda()
    Y, Hs = forward(Xd, Ad, Bd)
    assert rel_err(Hs, O.hidden(X, A, O.GELU_NONE)) <= TOL_F32
    dH, dX, dXo, dA, dB = backward(Xd, Ad, Bd, Hs, Y, dZd, R=Rc, peers=[p.cuda() for p in peers])
    g = O.backward_rank(X, A, B, dZ)
    assert rel_err(dH, g["dH"]) <= TOL_F32
    assert rel_err(dX, g["dX_i"]) <= TOL_F32
    assert rel_err(dA, g["dA_i"]) <= TOL_F32
    assert rel_err(dB, g["dB_i"]) <= TOL_F32
    assert rel_err(dXo, R.reduce_full([g["dX_i"]] + [p.double().numpy() for p in peers])) <= TOL_F32


def _bwd_fusion(Xd, Ad, Bd, Hs, Y, dZd, peers, *, fusion, R=1, in_place=False):
    M, H = Xd.shape
    F = Ad.shape[1]
    dH = Guarded((M, F), Xd.dtype)
    dX = Guarded((M, H), torch.float32)
    dXo = None if in_place else Guarded((M, H), torch.float32)
    dA, dB = Guarded((H, F), torch.float32), Guarded((F, H), torch.float32)
    tp.tp_colrow_mlp_backward(Xd, Ad, Bd, Hs, Y, dZd, dH.t, dX.t, dA.t, dB.t, row_chunks=R, peer_dX=peers,
                              dX_out=dX.t if in_place else dXo.t, reduce_fusion=fusion,
                              s_compute=torch.cuda.current_stream(), s_reduce=torch.cuda.Stream())
    torch.cuda.synchronize()
    outs = [g for g in (dH, dX, dXo, dA, dB) if g is not None]
    assert all(g.guards_intact() for g in outs), "write outside an output buffer"
    return [g.t.cpu() for g in outs]


@pytest.mark.parametrize("M,H,F,P,Rc,in_place", [
    (4096, 768, 768, 4, 1, False),    # the GPT-2-small rank at TP = 4
    (4096, 768, 768, 4, 1, True),     # dX_out = dX_i (the all-reduce's form)
    (512, 384, 256, 3, 2, False),     # every chunk folds
    (300, 264, 160, 2, 3, False),     # ragged rows
    (512, 384, 256, 5, 1, False),     # 4 peers: reduction on s_reduce
    (520, 392, 200, 3, 1, False),     # K % 32 != 0: reduction on s_reduce
])
def test_backward_reduce_fusion_same_bits(M, H, F, P, Rc, in_place):
    """The dX GEMM with the ranks' sum in its epilogue gives the bits of the dX
    GEMM followed by the separate reduction: dH, dX_i, dX_out, dA_i, dB_i."""
    announce(f"backward reduce fusion M={M} H={H} F={F} P={P} R={Rc} in_place={in_place}")
    X = inputs.normal((M, H), 541, 1.0, "bf16")
    A = inputs.normal((H, F), 542, 1.0 / np.sqrt(H), "bf16")
    B = inputs.normal((F, H), 543, 1.0 / np.sqrt(F), "bf16")
    dZ = inputs.normal((M, H), 544, 1.0, "bf16")
    peers_cpu = [inputs.normal((M, H), 550 + p) for p in range(P - 1)]
    Xd, Ad, Bd, dZd = X.cuda(), A.cuda(), B.cuda(), dZ.cuda()
    peers = [p.cuda() for p in peers_cpu]
    Y, Hs = forward(Xd, Ad, Bd)
    fused = _bwd_fusion(Xd, Ad, Bd, Hs, Y, dZd, peers, fusion=tp.TP_REDUCE_FUSION_AUTO, R=Rc, in_place=in_place)
    apart = _bwd_fusion(Xd, Ad, Bd, Hs, Y, dZd, peers, fusion=tp.TP_REDUCE_FUSION_OFF, R=Rc, in_place=in_place)
    for a, b in zip(fused, apart):
        assert np.array_equal(bits(a), bits(b))
    g = O.backward_rank(X, A, B, dZ)
    total = R.reduce_full([g["dX_i"]] + [p.double().numpy() for p in peers_cpu])
    dX_sum = fused[1] if in_place else fused[2]
    assert rel_err(dX_sum, total) <= TOL_BF16
    assert rel_err(fused[-2], g["dA_i"]) <= TOL_BF16 and rel_err(fused[-1], g["dB_i"]) <= TOL_BF16


def test_backward_timing_reports_the_fused_kernel():
    """Per-kernel timing sees one gemm_dgrad_reduce launch per chunk, whose work
    is its algorithmic bytes, and no separate reduction."""
    announce("backward timing of the fused kernel")
    M, H, F, P, Rc = 512, 384, 256, 3, 2
    X = inputs.normal((M, H), 561, 1.0, "bf16").cuda()
    A = inputs.normal((H, F), 562, 1.0 / np.sqrt(H), "bf16").cuda()
    B = inputs.normal((F, H), 563, 1.0 / np.sqrt(F), "bf16").cuda()
    dZ = inputs.normal((M, H), 564, 1.0, "bf16").cuda()
    peers = [inputs.normal((M, H), 570 + p).cuda() for p in range(P - 1)]
    Y, Hs = forward(X, A, B)
    dH = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    dX, dXo = torch.empty((M, H), device="cuda"), torch.empty((M, H), device="cuda")
    dA, dB = torch.empty((H, F), device="cuda"), torch.empty((F, H), device="cuda")
    torch.cuda.synchronize()
    tp.tp_timing_enable(True)
    try:
        tp.tp_timing_read()
        tp.tp_colrow_mlp_backward(X, A, B, Hs, Y, dZ, dH, dX, dA, dB, row_chunks=Rc, peer_dX=peers, dX_out=dXo)
        st = tp.tp_timing_read()
    finally:
        tp.tp_timing_enable(False)
    Mr = M // Rc
    assert st["gemm_dgrad_reduce"]["launches"] == Rc and st["reduce"]["launches"] == 0
    assert st["gemm_dgrad"]["launches"] == Rc          # the dH GEMMs
    assert st["gemm_dgrad_reduce"]["work"] == Rc * (2 * (Mr * F + F * H) + 4 * (P - 1) * Mr * H + 2 * 4 * Mr * H)


@pytest.mark.parametrize("P,fused", [(4, True), (5, False)])
def test_backward_fusion_taken_where_the_rule_says(P, fused):
    """The dX sum folds into the dX GEMM for P <= 4, and runs as its own kernel
    on s_reduce for P = 5."""
    announce(f"backward fusion rule P={P}")
    M, H, F = 512, 384, 256
    z = lambda *shape, dt=torch.bfloat16: torch.zeros(shape, dtype=dt, device="cuda")
    X, A, B, dZ = z(M, H), z(H, F), z(F, H), z(M, H)
    Y, Hs, dH = z(M, F), z(M, F), z(M, F)
    dX, dA, dB = z(M, H, dt=torch.float32), z(H, F, dt=torch.float32), z(F, H, dt=torch.float32)
    peers = [z(M, H, dt=torch.float32) for _ in range(P - 1)]
    tp.tp_timing_enable(True)
    try:
        tp.tp_timing_read()
        tp.tp_colrow_mlp_backward(X, A, B, Hs, Y, dZ, dH, dX, dA, dB, peer_dX=peers, dX_out=dX,
                                  s_reduce=torch.cuda.Stream())
        torch.cuda.synchronize()
        st = tp.tp_timing_read()
    finally:
        tp.tp_timing_enable(False)
    assert st["gemm_dgrad_reduce"]["launches"] == (1 if fused else 0)
    assert st["reduce"]["launches"] == (0 if fused else 1)


def test_backward_chunks_do_not_change_a_bit():
    """Row chunks split dH and dX by rows and continue one accumulation of the
    weight gradients, so R = 1, 2, 4 give identical bits (serial or two streams)."""
    announce("backward chunked == serial")
    M, H, F = 2048, 1024, 512
    X = inputs.normal((M, H), 521, 1.0, "bf16").cuda()
    A = inputs.normal((H, F), 522, 1.0 / np.sqrt(H), "bf16").cuda()
    B = inputs.normal((F, H), 523, 1.0 / np.sqrt(F), "bf16").cuda()
    dZ = inputs.normal((M, H), 524, 1.0, "bf16").cuda()
    peers = [inputs.normal((M, H), 530 + p).cuda() for p in range(3)]
    Y, Hs = forward(X, A, B)
    ref = backward(X, A, B, Hs, Y, dZ, R=1, peers=peers, two_streams=False)
    for Rc, two in [(2, True), (4, True), (4, False)]:
        got = backward(X, A, B, Hs, Y, dZ, R=Rc, peers=peers, two_streams=two)
        for a, b in zip(got, ref):
            assert np.array_equal(bits(a), bits(b))


def _chunk_rows(M, Rc, per_chunk):
    """Rows of each row chunk: its first and last row plus evenly spread ones."""
    Mr = M // Rc
    rows = []
    for r in range(Rc):
        rows += list(np.unique(np.linspace(r * Mr, (r + 1) * Mr - 1, per_chunk).astype(np.int64)))
    return np.array(rows)


@pytest.mark.parametrize("w", [GPT3_6P7B, GPT3_175B], ids=lambda w: w.name)
def test_backward_tp8_sampled(w):
    """Full GPT-3 per-rank shapes at TP = 8 (R = 2), as the bench times them:
    128 rows of dH / dX / dX_out (64 per row chunk, each chunk's first and last
    among them) and 32 columns of dA / rows of dB against the oracle.  Each row
    of dH depends on its own rows of X and dZ; each column f of dA (row f of dB)
    on column f of A_i and row f of B_i alone, so the samples are exact
    restrictions.  The peers' input gradients are drawn, not computed."""
    announce(f"backward {w.name} sampled")
    M, H, F, P = w.M, w.H, w.F, w.P
    X = inputs.normal((M, H), inputs.seed_for(w.cfg, inputs.SLOT_X), 1.0, "bf16", "cuda")
    A = inputs.normal((H, F), inputs.seed_for(w.cfg, inputs.SLOT_A), 0.02, "bf16", "cuda")
    B = inputs.normal((F, H), inputs.seed_for(w.cfg, inputs.SLOT_B), 0.02, "bf16", "cuda")
    dZ = inputs.normal((M, H), inputs.seed_for(w.cfg, inputs.SLOT_DZ), 1.0, "bf16", "cuda")
    peers = [inputs.normal((M, H), inputs.seed_for(w.cfg, inputs.SLOT_PARTIAL + p), 1.0, "f32", "cuda")
             for p in range(P - 1)]
    Y, Hs = forward(X, A, B)
    dH, dX, dXo, dA, dB = backward(X, A, B, Hs, Y, dZ, R=w.R, peers=peers)
    del Y, Hs
    Xc, Ac, Bc, dZc = X.cpu(), A.cpu(), B.cpu(), dZ.cpu()
    rows = _chunk_rows(M, w.R, 64)
    cols = np.sort(np.random.default_rng(0).choice(F, 32, replace=False))
    announce(f"backward {w.name}: oracle on {len(rows)} rows and {len(cols)} columns")
    gr = O.backward_rank(Xc[rows], Ac, Bc, dZc[rows])
    assert rel_err(dH[rows], gr["dH"]) <= TOL_BF16
    assert rel_err(dX[rows], gr["dX_i"]) <= TOL_BF16
    peer_rows = [p[rows].cpu().double().numpy() for p in peers]
    assert rel_err(dXo[rows], R.reduce_full([gr["dX_i"]] + peer_rows)) <= TOL_BF16
    gc = O.backward_rank(Xc, Ac[:, cols], Bc[cols, :], dZc)
    assert rel_err(dA[:, cols], gc["dA_i"]) <= TOL_BF16
    assert rel_err(dB[cols, :], gc["dB_i"]) <= TOL_BF16


def test_backward_tiny_fp32_two_ranks():
    """The tiny fp32 configuration: both ranks' backward on the GPU, rank 0
    reducing rank 1's input gradient; the sum and the weight gradients against
    the oracle's full two-rank backward."""
    w = TINY
    announce(f"backward {w.name} fp32 two ranks")
    M, H, P, F = w.M, w.H, w.P, w.F
    X = inputs.normal((M, H), inputs.seed_for(1, inputs.SLOT_X), 1.0, "f32")
    A = inputs.normal((H, P * F), inputs.seed_for(1, inputs.SLOT_A), 1.0 / np.sqrt(H), "f32")
    B = inputs.normal((P * F, H), inputs.seed_for(1, inputs.SLOT_B), 1.0 / np.sqrt(P * F), "f32")
    dZ = inputs.normal((M, H), 1004, 1.0, "f32")
    A_sh = L.split(A, {"device": list(range(P)), "sharded_dim": [{"axis": 1, "num_shards": P}]})
    B_sh = L.split(B, {"device": list(range(P)), "sharded_dim": [{"axis": 0, "num_shards": P}]})
    outs = []
    for i in (1, 0):
        Ai = torch.from_numpy(np.ascontiguousarray(A_sh[i])).float().cuda()
        Bi = torch.from_numpy(np.ascontiguousarray(B_sh[i])).float().cuda()
        Y, Hs = forward(X.cuda(), Ai, Bi)
        peers = [outs[0][1].cuda()] if i == 0 else []
        outs.append(backward(X.cuda(), Ai, Bi, Hs, Y, dZ.cuda(), peers=peers))
    dX_ref, dA_ref, dB_ref = O.backward_all_ranks(X, [A_sh[0], A_sh[1]], [B_sh[0], B_sh[1]], dZ)
    rank0 = outs[1]
    assert rel_err(rank0[2], dX_ref) <= TOL_F32
    assert rel_err(rank0[3], dA_ref[0]) <= TOL_F32 and rel_err(rank0[4], dB_ref[0]) <= TOL_F32
    assert rel_err(outs[0][3], dA_ref[1]) <= TOL_F32 and rel_err(outs[0][4], dB_ref[1]) <= TOL_F32


def test_backward_error_path():
    """A rejected call raises and leaves its outputs untouched."""
    announce("backward error path")
    M, H, F = 64, 64, 64
    X = torch.zeros((M, H), dtype=torch.bfloat16, device="cuda")
    A = torch.zeros((H, F), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((F, H), dtype=torch.bfloat16, device="cuda")
    Y = torch.zeros((M, F), dtype=torch.bfloat16, device="cuda")
    dZ = torch.zeros((M, H), dtype=torch.bfloat16, device="cuda")
    dH = Guarded((M, F), torch.bfloat16)
    dX = Guarded((M, H), torch.float32)
    dA = Guarded((H, F), torch.float32)
    dB = Guarded((F, H), torch.float32)
    with pytest.raises(tp.TpError):   # GeLU needs the saved pre-activation
        tp.tp_colrow_mlp_backward(X, A, B, None, Y, dZ, dH.t, dX.t, dA.t, dB.t)
    with pytest.raises(tp.TpError):   # 3 row chunks do not divide 64 rows
        tp.tp_colrow_mlp_backward(X, A, B, Y, Y, dZ, dH.t, dX.t, dA.t, dB.t, row_chunks=3)
    torch.cuda.synchronize()
    for g in (dH, dX, dA, dB):
        assert g.body_untouched() and g.guards_intact()


def test_prepared_backward_replays():
    """A backward call marshalled once (prepare=True) and replayed twice, its
    outputs overwritten between the replays, gives the direct call's bits."""
    announce("backward prepared call")
    M, H, F, P = 1024, 512, 384, 3
    X = inputs.normal((M, H), 601, 1.0, "bf16").cuda()
    A = inputs.normal((H, F), 602, 1.0 / np.sqrt(H), "bf16").cuda()
    B = inputs.normal((F, H), 603, 1.0 / np.sqrt(F), "bf16").cuda()
    dZ = inputs.normal((M, H), 604, 1.0, "bf16").cuda()
    peers = [inputs.normal((M, H), 610 + p).cuda() for p in range(P - 1)]
    Y, Hs = forward(X, A, B)
    ref = backward(X, A, B, Hs, Y, dZ, R=2, peers=peers)
    outs = [torch.empty((M, F), dtype=torch.bfloat16, device="cuda"), torch.empty((M, H), device="cuda"),
            torch.empty((M, H), device="cuda"), torch.empty((H, F), device="cuda"), torch.empty((F, H), device="cuda")]
    dH, dX, dXo, dA, dB = outs
    call = tp.tp_colrow_mlp_backward(X, A, B, Hs, Y, dZ, dH, dX, dA, dB, row_chunks=2, peer_dX=peers, dX_out=dXo,
                                     s_compute=torch.cuda.current_stream(), s_reduce=torch.cuda.Stream(),
                                     prepare=True)
    for _ in range(2):
        for o in outs:
            o.fill_(float("nan"))
        call()
        torch.cuda.synchronize()
        for a, b in zip([o.cpu() for o in outs], ref):
            assert np.array_equal(bits(a), bits(b))
