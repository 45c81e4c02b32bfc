"""GPU parity of tp_colrow_mlp (GEMM1 + GeLU, GEMM2, two-stream chunked
reduce) against the MLP oracle."""
import numpy as np
import pytest
import torch

import sharded_gemm_amd as tp
from sharded_gemm_amd import inputs
from sharded_gemm_amd.workloads import GPT2_SMALL, GPT3_175B, GPT3_6P7B, TINY
from oracle import layout as L
from oracle import mlp as O
from oracle import reduce as R

from gpu_helpers import Guarded, announce, bits, rel_err, require_gpu

pytestmark = pytest.mark.gpu

TOL_BF16 = 1e-2   # max|err|/max|ref|, bf16 inputs, fp32 accumulation, Y rounded to bf16
TOL_F32 = 1e-5    # same measure, fp32 throughout


def setup_module(_):
    require_gpu()


def _call_rank(X, A_i, B_i, *, R, C, peers, act, two_streams, fusion=tp.TP_REDUCE_FUSION_AUTO, noalloc=False):
    M, H = X.shape
    F = A_i.shape[1]
    Y = None if noalloc else Guarded((M, F), X.dtype)
    Z = Guarded((M, H), torch.float32)
    Zo = Guarded((M, H), torch.float32) if peers else None
    s0 = torch.cuda.current_stream()
    kw = dict(row_chunks=R, col_chunks=C, peer_partials=list(peers), Z_out=Zo.t if Zo is not None else None,
              act=act, reduce_fusion=fusion, s_compute=s0, s_reduce=torch.cuda.Stream() if two_streams else s0)
    if noalloc:
        tp.tp_colrow_mlp_noalloc(X, A_i, B_i, Z.t, **kw)
    else:
        tp.tp_colrow_mlp(X, A_i, B_i, Y.t, Z.t, **kw)
    torch.cuda.synchronize()
    for g in (Y, Z, Zo):
        assert g is None or g.guards_intact(), "write outside an output buffer"
    return [g.t.cpu() if g is not None else None for g in (Y, Z, Zo)]


def run_rank(X, A_i, B_i, *, R=1, C=1, peers=(), act=tp.TP_ACT_GELU_ERF, two_streams=False):
    """One tp_colrow_mlp call into canary-guarded outputs; returns CPU copies
    of Y, Z_i and Z_out.  Where the schedule may merge the row chunks (one
    GEMM1 over all rows, or on one stream the layer as one block), two
    schedules that keep them apart run too and must give the same bits: the
    allocation-free entry point (every chunk's GEMM1 apart, Y kept one chunk at
    a time) and two streams with each block's separate reduction beside the
    next block's GEMM2."""
    kw = dict(R=R, C=C, peers=peers, act=act)
    out = _call_rank(X, A_i, B_i, two_streams=two_streams, **kw)
    if R * C > 1:
        kept = _call_rank(X, A_i, B_i, two_streams=two_streams, noalloc=True, **kw)
        for a, b in zip(out[1:], kept[1:]):
            assert (a is None and b is None) or np.array_equal(bits(a), bits(b))
        if peers:
            kept = _call_rank(X, A_i, B_i, two_streams=True, fusion=tp.TP_REDUCE_FUSION_OFF, **kw)
            for a, b in zip(out, kept):
                assert np.array_equal(bits(a), bits(b))
    return tuple(out)


def _bf16_exact(x64):
    """RNE rounding of exact fp64 values to bf16 (the same decision the kernel takes)."""
    return torch.from_numpy(np.asarray(x64)).to(torch.bfloat16)


# ---------------------------------------------------------------- exact cases

@pytest.mark.parametrize("M,H,F", [(300, 264, 136), (256, 512, 512), (77, 45, 51), (1, 8, 8), (513, 1040, 264),
                                   (333, 320, 200), (515, 256, 96), (1000, 512, 264), (4100, 1024, 776),
                                   # ping-pong kernel, 256 x 256 tiles (ragged M and N; 1, 2 and 7 stages)
                                   (4100, 64, 6152), (4100, 128, 6152), (4100, 448, 6152),
                                   # ping-pong kernel, 256 x 192 tiles (1, 2, 3 and 5 stages: the
                                   # split rings' repeated fetches of the last stage)
                                   (2000, 64, 6136), (2000, 128, 6136), (2000, 192, 6136), (2000, 320, 6136),
                                   # ping-pong kernel, 256 x 128 tiles (ragged M and N)
                                   (4000, 64, 2000), (4000, 128, 2000), (4000, 192, 2000)])
def test_hidden_integer_exact(M, H, F):
    """Small-integer inputs make X A_i exact in fp32, so Y must equal the
    RNE-to-bf16 rounding of the oracle's exact value, bit for bit."""
    announce(f"mlp hidden integer exact M={M} H={H} F={F}")
    X = inputs.small_ints((M, H), seed=101, lo=-4, hi=4, dtype="bf16")
    A = inputs.small_ints((H, F), seed=102, lo=-4, hi=4, dtype="bf16")
    B = inputs.small_ints((F, H), seed=103, lo=-4, hi=4, dtype="bf16")
    Y, _, _ = run_rank(X.cuda(), A.cuda(), B.cuda(), act=tp.TP_ACT_NONE)
    ref = _bf16_exact(O.hidden(X, A, O.GELU_NONE))
    assert np.array_equal(bits(Y), bits(ref))


def _one_hot_columns(H, F, seed):
    """A [H, F] with one small nonzero integer per column: X A stays a small
    integer, exactly representable in bf16."""
    g = torch.Generator().manual_seed(seed)
    rows = torch.randint(0, H, (F,), generator=g)
    vals = torch.randint(1, 5, (F,), generator=g) * (torch.randint(0, 2, (F,), generator=g) * 2 - 1)
    A = torch.zeros((H, F))
    A[rows, torch.arange(F)] = vals.float()
    return A.to(torch.bfloat16)


@pytest.mark.parametrize("M,H,F,Rc,Cc,P", [(512, 384, 256, 2, 3, 3), (93, 72, 40, 3, 2, 2),
                                            (50, 30, 22, 2, 3, 2), (1024, 1024, 512, 4, 4, 8),
                                            (515, 256, 96, 1, 2, 2), (1030, 640, 320, 2, 5, 4),
                                            # GEMM2 on the ping-pong kernel (fp32 out): 256 x 192, 256 x 256
                                            (2000, 6136, 128, 1, 1, 2), (4100, 6152, 64, 1, 1, 2),
                                            # GEMM2 on the ping-pong kernel, 256 x 128 tiles
                                            (4000, 2000, 64, 1, 1, 2)])
def test_chain_integer_exact(M, H, F, Rc, Cc, P):
    """Exact whole chain: Y small integers, fp32 sums exact, so Z_i and Z_out
    must equal the oracle bit for bit, chunked, on two streams."""
    announce(f"mlp chain integer exact M={M} H={H} F={F} R={Rc} C={Cc} P={P}")
    X = inputs.small_ints((M, H), seed=201, lo=-4, hi=4, dtype="bf16")
    A = _one_hot_columns(H, F, 202)
    B = inputs.small_ints((F, H), seed=203, lo=-4, hi=4, dtype="bf16")
    peers_cpu = [inputs.small_ints((M, H), seed=210 + p, lo=-512, hi=512) for p in range(P - 1)]
    Y, Z, Zo = run_rank(X.cuda(), A.cuda(), B.cuda(), R=Rc, C=Cc, peers=[p.cuda() for p in peers_cpu],
                        act=tp.TP_ACT_NONE, two_streams=True)
    z_ref = O.mlp_rank(X, A, B, O.GELU_NONE)
    assert np.array_equal(Z.numpy().astype(np.float64), z_ref)
    assert np.array_equal(Zo.numpy().astype(np.float64), R.reduce_full([z_ref] + peers_cpu))


# ------------------------------------------------------------ tolerance cases

@pytest.mark.parametrize("M,H,F,Rc,Cc", [(300, 264, 136, 3, 2), (77, 45, 51, 1, 1), (128, 4096, 64, 2, 4),
                                         (2050, 520, 776, 2, 1), (1, 1, 1, 1, 1), (333, 320, 200, 1, 1),
                                         (1500, 2048, 1024, 3, 2)])
def test_ragged_bf16(M, H, F, Rc, Cc):
    announce(f"mlp ragged bf16 M={M} H={H} F={F} R={Rc} C={Cc}")
    X = inputs.normal((M, H), 301, 1.0, "bf16")
    A = inputs.normal((H, F), 302, 1.0 / np.sqrt(H), "bf16")
    B = inputs.normal((F, H), 303, 1.0 / np.sqrt(F), "bf16")
    peers_cpu = [inputs.normal((M, H), 310 + p) for p in range(2)]
    Y, Z, Zo = run_rank(X.cuda(), A.cuda(), B.cuda(), R=Rc, C=Cc, peers=[p.cuda() for p in peers_cpu],
                        two_streams=True)
    y_ref = O.hidden(X, A)
    z_ref = O.mlp_rank(X, A, B)
    assert rel_err(Y.float(), y_ref) <= TOL_BF16
    assert rel_err(Z, z_ref) <= TOL_BF16
    assert rel_err(Zo, R.reduce_full([z_ref] + peers_cpu)) <= TOL_BF16


@pytest.mark.parametrize("M,H,F,Rc,Cc", [(77, 45, 51, 1, 1), (300, 264, 136, 3, 2), (1, 1, 1, 1, 1),
                                         (130, 129, 65, 2, 3), (33, 200, 97, 1, 2), (64, 256, 512, 2, 2)])
def test_ragged_fp32(M, H, F, Rc, Cc):
    """fp32 throughout: rows, columns and both contraction depths off the
    32 x 32 output tile and the 64-deep k slab, whole and chunked."""
    announce(f"mlp ragged fp32 M={M} H={H} F={F} R={Rc} C={Cc}")
    X = inputs.normal((M, H), 321, 1.0)
    A = inputs.normal((H, F), 322, 1.0 / np.sqrt(H))
    B = inputs.normal((F, H), 323, 1.0 / np.sqrt(F))
    peers_cpu = [inputs.normal((M, H), 330 + p) for p in range(2)]
    Y, Z, Zo = run_rank(X.cuda(), A.cuda(), B.cuda(), R=Rc, C=Cc, peers=[p.cuda() for p in peers_cpu],
                        two_streams=True)
    z_ref = O.mlp_rank(X, A, B)
    assert rel_err(Y, O.hidden(X, A)) <= TOL_F32
    assert rel_err(Z, z_ref) <= TOL_F32
    assert rel_err(Zo, R.reduce_full([z_ref] + peers_cpu)) <= TOL_F32


def test_tiny_fp32_two_ranks():
    """The tiny fp32 workload: X[64,256], A[256,1024] cut by columns into 2,
    B[1024,256] cut by rows into 2 (cut on the GPU), both ranks, summed."""
    w = TINY
    announce("mlp tiny fp32 P=2")
    X = inputs.normal((w.M, w.H), inputs.seed_for(1, inputs.SLOT_X), w.std_x)
    A = inputs.normal((w.H, w.P * w.F), inputs.seed_for(1, inputs.SLOT_A), w.std_a)
    B = inputs.normal((w.P * w.F, w.H), inputs.seed_for(1, inputs.SLOT_B), w.std_b)
    sa = {"device": [0, 1], "sharded_dim": [{"axis": 1, "num_shards": 2}]}
    sb = {"device": [0, 1], "sharded_dim": [{"axis": 0, "num_shards": 2}]}
    A_sh = {d: torch.empty((w.H, w.F), device="cuda") for d in range(2)}
    B_sh = {d: torch.empty((w.F, w.H), device="cuda") for d in range(2)}
    tp.tp_shard_materialize(A.cuda(), sa, A_sh)
    tp.tp_shard_materialize(B.cuda(), sb, B_sh)
    # both weights cut in one batched launch: same bits
    A_b = {d: torch.empty_like(A_sh[d]) for d in range(2)}
    B_b = {d: torch.empty_like(B_sh[d]) for d in range(2)}
    tp.tp_shard_materialize_batch([(A.cuda(), sa, A_b), (B.cuda(), sb, B_b)])
    torch.cuda.synchronize()
    for d in range(2):
        assert torch.equal(A_b[d].view(torch.int32), A_sh[d].view(torch.int32))
        assert torch.equal(B_b[d].view(torch.int32), B_sh[d].view(torch.int32))
    Xg = X.cuda()
    _, Z1, _ = run_rank(Xg, A_sh[1], B_sh[1])
    Y0, Z0, Zo = run_rank(Xg, A_sh[0], B_sh[0], peers=[Z1.cuda()], two_streams=True)
    oa, ob = L.split(A, sa), L.split(B, sb)
    assert rel_err(Y0, O.hidden(X, oa[0])) <= TOL_F32
    assert rel_err(Z0, O.mlp_rank(X, oa[0], ob[0])) <= TOL_F32
    assert rel_err(Zo, O.mlp_all_ranks(X, [oa[0], oa[1]], [ob[0], ob[1]])) <= TOL_F32
    assert rel_err(Zo, O.mlp_unsharded(X, A, B)) <= TOL_F32


def test_gpt2_small_tp4_full():
    """GPT-2-small MLP at TP=4, every element of every rank: weights cut on the
    GPU from the full A [768,3072] and B [3072,768]; ranks 1..3 first, then
    rank 0 reduces all four partials."""
    w = GPT2_SMALL
    announce("mlp gpt2-small tp4 full size")
    X = inputs.normal((w.M, w.H), inputs.seed_for(2, inputs.SLOT_X), w.std_x, "bf16")
    A = inputs.normal((w.H, w.P * w.F), inputs.seed_for(2, inputs.SLOT_A), w.std_a, "bf16")
    B = inputs.normal((w.P * w.F, w.H), inputs.seed_for(2, inputs.SLOT_B), w.std_b, "bf16")
    sa = {"device": list(range(4)), "sharded_dim": [{"axis": 1, "num_shards": 4}]}
    sb = {"device": list(range(4)), "sharded_dim": [{"axis": 0, "num_shards": 4}]}
    A_sh = {d: torch.empty((w.H, w.F), dtype=torch.bfloat16, device="cuda") for d in range(4)}
    B_sh = {d: torch.empty((w.F, w.H), dtype=torch.bfloat16, device="cuda") for d in range(4)}
    tp.tp_shard_materialize(A.cuda(), sa, A_sh)
    tp.tp_shard_materialize(B.cuda(), sb, B_sh)
    # the bench cuts both weights in one batched launch: same bits
    A_b = {d: torch.empty_like(A_sh[d]) for d in range(4)}
    B_b = {d: torch.empty_like(B_sh[d]) for d in range(4)}
    tp.tp_shard_materialize_batch([(A.cuda(), sa, A_b), (B.cuda(), sb, B_b)])
    torch.cuda.synchronize()
    for d in range(4):
        assert torch.equal(A_b[d].view(torch.int16), A_sh[d].view(torch.int16))
        assert torch.equal(B_b[d].view(torch.int16), B_sh[d].view(torch.int16))
    Xg = X.cuda()
    peers = [run_rank(Xg, A_sh[i], B_sh[i])[1].cuda() for i in range(1, 4)]
    Y0, Z0, Zo = run_rank(Xg, A_sh[0], B_sh[0], peers=peers, two_streams=True)
    oa, ob = L.split(A, sa), L.split(B, sb)
    assert rel_err(Y0.float(), O.hidden(X, oa[0])) <= TOL_BF16
    assert rel_err(Z0, O.mlp_rank(X, oa[0], ob[0])) <= TOL_BF16
    full = O.mlp_all_ranks(X, [oa[i] for i in range(4)], [ob[i] for i in range(4)])
    assert rel_err(Zo, full) <= TOL_BF16
    assert rel_err(Zo, O.mlp_unsharded(X, A, B)) <= TOL_BF16
    # the sum in place over the partial (the all-reduce's form, as timed): same bits
    Yg = torch.empty((w.M, w.F), dtype=torch.bfloat16, device="cuda")
    Zg = Guarded((w.M, w.H), torch.float32)
    tp.tp_colrow_mlp(Xg, A_sh[0], B_sh[0], Yg, Zg.t, peer_partials=peers, Z_out=Zg.t,
                     s_reduce=torch.cuda.Stream())
    torch.cuda.synchronize()
    assert Zg.guards_intact()
    assert np.array_equal(bits(Zg.t.cpu()), bits(Zo))


def _sample_rows(M, Rc, per_chunk):
    """Rows of each row chunk: its first and last row plus evenly spread ones."""
    Mr = M // Rc
    rows = []
    for r in range(Rc):
        rows += list(np.unique(np.linspace(r * Mr, (r + 1) * Mr - 1, per_chunk).astype(np.int64)))
    return np.array(rows)


def _large_case(w, per_chunk):
    announce(f"mlp {w.name}: inputs")
    X = inputs.normal((w.M, w.H), inputs.seed_for(w.cfg, inputs.SLOT_X), w.std_x, "bf16", device="cuda")
    As = [inputs.normal((w.H, w.F), inputs.seed_for(w.cfg, inputs.SLOT_A_SHARD + i), w.std_a, "bf16", device="cuda")
          for i in range(w.P)]
    Bs = [inputs.normal((w.F, w.H), inputs.seed_for(w.cfg, inputs.SLOT_B_SHARD + i), w.std_b, "bf16", device="cuda")
          for i in range(w.P)]
    announce(f"mlp {w.name}: ranks 1..{w.P - 1} (untimed peers)")
    peers = [run_rank(X, As[i], Bs[i])[1].cuda() for i in range(1, w.P)]
    announce(f"mlp {w.name}: rank 0, R={w.R} C={w.C}, two streams")
    Y0, Z0, Zo = run_rank(X, As[0], Bs[0], R=w.R, C=w.C, peers=peers, two_streams=True)
    announce(f"mlp {w.name}: rank 0 unchunked, one stream")
    Y0s, Z0s, Zos = run_rank(X, As[0], Bs[0], R=1, C=1, peers=peers, two_streams=False)
    # Chunking and stream overlap never change a bit.
    assert np.array_equal(bits(Y0), bits(Y0s))
    assert np.array_equal(bits(Z0), bits(Z0s))
    assert np.array_equal(bits(Zo), bits(Zos))
    announce(f"mlp {w.name}: rank 0, R={w.R} C={w.C}, two streams, sum in place over the partial")
    Yi = torch.empty((w.M, w.F), dtype=torch.bfloat16, device="cuda")
    Zi = Guarded((w.M, w.H), torch.float32)
    tp.tp_colrow_mlp(X, As[0], Bs[0], Yi, Zi.t, row_chunks=w.R, col_chunks=w.C, peer_partials=peers, Z_out=Zi.t,
                     s_reduce=torch.cuda.Stream())
    torch.cuda.synchronize()
    assert Zi.guards_intact()
    assert np.array_equal(bits(Zi.t.cpu()), bits(Zo))
    del Yi, Zi
    rows = _sample_rows(w.M, w.R, per_chunk)
    Xc = X.cpu()
    announce(f"mlp {w.name}: oracle on {len(rows)} sampled rows")
    z0_ref = O.mlp_rank_rows(Xc, As[0].cpu(), Bs[0].cpu(), rows)
    assert rel_err(Z0[rows], z0_ref) <= TOL_BF16
    assert rel_err(Y0[rows].float(), O.hidden(Xc[rows], As[0].cpu())) <= TOL_BF16
    acc = z0_ref.copy()
    for i in range(1, w.P):
        acc += O.mlp_rank_rows(Xc, As[i].cpu(), Bs[i].cpu(), rows)
    assert rel_err(Zo[rows], acc) <= TOL_BF16


def test_gpt3_6p7b_tp8_rowsplit():
    _large_case(GPT3_6P7B, per_chunk=64)


def test_gpt3_175b_tp8_2d():
    _large_case(GPT3_175B, per_chunk=64)


def test_error_leaves_outputs_untouched():
    announce("mlp error path")
    X = torch.zeros((30, 16), dtype=torch.bfloat16, device="cuda")
    A = torch.zeros((16, 8), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((8, 16), dtype=torch.bfloat16, device="cuda")
    Y = Guarded((30, 8), torch.bfloat16)
    Z = Guarded((30, 16), torch.float32)
    with pytest.raises(tp.TpError) as e:
        tp.tp_colrow_mlp(X, A, B, Y.t, Z.t, row_chunks=4)
    assert e.value.kind == "indivisible"
    torch.cuda.synchronize()
    assert Y.body_untouched() and Z.body_untouched()


@pytest.mark.parametrize("P", [4, 8])
def test_graph_replay_matches_eager(P):
    """The chunked call offered two streams, captured into a HIP graph: with 3
    peers every block's sum folds into its GEMM2 and the call keeps to one
    stream (one GEMM1 over all rows); with 7 the small blocks' sums run on the
    second stream beside the GEMMs.  Every replay, with eager work and host
    synchronisation in between, equals the eager call."""
    announce(f"mlp graph capture and replay P={P}")
    M, H, F, Rc, Cc = 1024, 512, 384, 2, 2
    X = inputs.normal((M, H), 401, 1.0, "bf16").cuda()
    A = inputs.normal((H, F), 402, 0.05, "bf16").cuda()
    B = inputs.normal((F, H), 403, 0.05, "bf16").cuda()
    peers = [inputs.normal((M, H), 410 + p).cuda() for p in range(P - 1)]
    Y = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    Z = torch.empty((M, H), device="cuda")
    Zo = torch.empty((M, H), device="cuda")
    s0, s1 = torch.cuda.Stream(), torch.cuda.Stream()

    def call():
        tp.tp_colrow_mlp(X, A, B, Y, Z, row_chunks=Rc, col_chunks=Cc, peer_partials=peers, Z_out=Zo,
                         s_compute=s0, s_reduce=s1)

    call()
    torch.cuda.synchronize()
    ref_y, ref_z, ref_zo = Y.clone(), Z.clone(), Zo.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s0):
        call()
    for rep in range(3):
        for t in (Y, Z, Zo):
            t.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(s0):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), ref_y.view(torch.int16)), rep
        assert torch.equal(Z.view(torch.int32), ref_z.view(torch.int32)), rep
        assert torch.equal(Zo.view(torch.int32), ref_zo.view(torch.int32)), rep
        peers[0].add_(0.0)   # eager work between replays


@pytest.mark.parametrize("M,H,F,Rc,Cc,P", [(515, 256, 96, 1, 1, 1), (512, 384, 256, 2, 3, 3), (1030, 640, 320, 2, 5, 4)])
def test_row_parallel_bias_integer_exact(M, H, F, Rc, Cc, P):
    """Z_out = Z_i + peers + bias ([CAI] section 5.2: the bias acts on the full
    output, added once); Z_i itself stays bias-free.  Integers: exact."""
    announce(f"mlp bias integer exact M={M} H={H} F={F} R={Rc} C={Cc} P={P}")
    X = inputs.small_ints((M, H), seed=251, lo=-4, hi=4, dtype="bf16")
    A = _one_hot_columns(H, F, 252)
    B = inputs.small_ints((F, H), seed=253, lo=-4, hi=4, dtype="bf16")
    bias_cpu = inputs.small_ints((H,), seed=254, lo=-64, hi=64)
    peers_cpu = [inputs.small_ints((M, H), seed=260 + p, lo=-512, hi=512) for p in range(P - 1)]
    Y = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    Z = torch.empty((M, H), device="cuda")
    Zo = torch.empty((M, H), device="cuda")
    tp.tp_colrow_mlp(X.cuda(), A.cuda(), B.cuda(), Y, Z, row_chunks=Rc, col_chunks=Cc,
                     peer_partials=[p.cuda() for p in peers_cpu], Z_out=Zo, act=tp.TP_ACT_NONE,
                     s_reduce=torch.cuda.Stream(), bias=bias_cpu.cuda())
    torch.cuda.synchronize()
    z_ref = O.mlp_rank(X, A, B, O.GELU_NONE)
    assert np.array_equal(Z.cpu().numpy().astype(np.float64), z_ref)
    assert np.array_equal(Zo.cpu().numpy().astype(np.float64), R.reduce_full([z_ref] + peers_cpu, "sum", bias_cpu))


def _run_fusion(X, A, B, peers, *, fusion, R=1, C=1, bias=None, z_out=True, in_place=False, x_next=False,
                two=False, noalloc=False):
    """One call into guarded outputs; returns the CPU copies of Y (None through
    the allocation-free entry point, which keeps Y to itself), Z, Z_out and X_next."""
    M, H = X.shape
    F = A.shape[1]
    Y = None if noalloc else Guarded((M, F), X.dtype)
    Z = Guarded((M, H), torch.float32)
    Zo = Guarded((M, H), torch.float32) if (z_out and not in_place) else None
    Xn = Guarded((M, H), X.dtype) if x_next else None
    s0 = torch.cuda.current_stream()
    kw = dict(row_chunks=R, col_chunks=C, peer_partials=list(peers),
              Z_out=Z.t if in_place else (Zo.t if Zo is not None else None), bias=bias,
              X_next=Xn.t if Xn is not None else None, reduce_fusion=fusion,
              s_compute=s0, s_reduce=torch.cuda.Stream() if two else s0)
    if noalloc:
        tp.tp_colrow_mlp_noalloc(X, A, B, Z.t, **kw)
    else:
        tp.tp_colrow_mlp(X, A, B, Y.t, Z.t, **kw)
    torch.cuda.synchronize()
    outs = [g for g in (Y, Z, Zo, Xn) if g is not None]
    assert all(g.guards_intact() for g in outs), "write outside an output buffer"
    return [g.t.cpu() if g is not None else None for g in (Y, Z, Zo, Xn)]


@pytest.mark.parametrize("M,H,F,P,Rc,Cc,opts", [
    (4096, 768, 768, 4, 1, 1, {}),                                  # the GPT-2-small rank at TP = 4
    (300, 264, 160, 3, 1, 1, {"bias": True, "x_next": True}),      # ragged rows, bias, bf16 next input
    (512, 384, 256, 4, 1, 1, {"in_place": True}),                  # Z_out = Z_i
    (512, 384, 256, 2, 1, 1, {"z_out": False, "x_next": True}),    # only the next layer's input
    (515, 256, 96, 1, 1, 1, {"bias": True}),                       # no peers: the bias alone
    (1000, 512, 256, 4, 2, 2, {"bias": True, "two": True}),        # only the final block folds
    (1000, 512, 256, 3, 2, 2, {"bias": True, "x_next": True}),     # one stream: one GEMM1, each block folds at its offsets
    (300, 264, 192, 4, 3, 3, {"x_next": True, "in_place": True}),  # the same, ragged rows, 3 x 3 blocks, in place
    # without a Y workspace every chunk keeps its GEMM1 as well
    (1000, 512, 256, 3, 2, 2, {"bias": True, "x_next": True, "noalloc": True}),
    (300, 264, 192, 4, 3, 3, {"x_next": True, "in_place": True, "noalloc": True}),
    (512, 384, 256, 5, 1, 1, {}),                                  # 4 peers: separate reduction
    (520, 392, 200, 3, 1, 1, {}),                                  # K % 32 != 0: separate reduction
    # the 256-row tiles, the tile staged through LDS in the epilogue: 256 x 128, 256 x 256 (in place),
    # 256 x 192 (bias and the bf16 next input), 15 peers with ragged rows, only the final block of a
    # two-stream schedule, and 16 peers (past the limit: separate reduction)
    (2048, 2048, 512, 8, 1, 1, {}),
    (4096, 4096, 256, 8, 1, 1, {"in_place": True}),
    (2048, 6144, 512, 8, 1, 1, {"bias": True, "x_next": True}),
    (2000, 4096, 256, 16, 1, 1, {"bias": True}),
    (4096, 4096, 256, 8, 2, 1, {"bias": True, "two": True}),
    (2048, 2048, 256, 17, 1, 1, {}),
    (2048, 2048, 512, 8, 2, 2, {"bias": True, "noalloc": True}),   # 256-row tiles, each block at its offsets
])
def test_reduce_fusion_same_bits(M, H, F, P, Rc, Cc, opts):
    """GEMM2 with the block's reduction folded into its epilogue writes the
    same bits as GEMM2 followed by the separate reduction kernel: Z_i, Z_out
    (or Z_i in place) and X_next; both against the oracle."""
    announce(f"mlp reduce fusion M={M} H={H} F={F} P={P} R={Rc} C={Cc} {sorted(opts)}")
    X = inputs.normal((M, H), 341, 1.0, "bf16")
    A = inputs.normal((H, F), 342, 1.0 / np.sqrt(H), "bf16")
    B = inputs.normal((F, H), 343, 1.0 / np.sqrt(F), "bf16")
    peers_cpu = [inputs.normal((M, H), 350 + p) for p in range(P - 1)]
    bias_cpu = inputs.normal((H,), 349) if opts.get("bias") else None
    kw = {k: v for k, v in opts.items() if k != "bias"}
    kw.update(R=Rc, C=Cc, bias=bias_cpu.cuda() if bias_cpu is not None else None)
    Xd, Ad, Bd, peers = X.cuda(), A.cuda(), B.cuda(), [p.cuda() for p in peers_cpu]
    fused = _run_fusion(Xd, Ad, Bd, peers, fusion=tp.TP_REDUCE_FUSION_AUTO, **kw)
    apart = _run_fusion(Xd, Ad, Bd, peers, fusion=tp.TP_REDUCE_FUSION_OFF, **kw)
    for a, b in zip(fused, apart):
        assert (a is None) == (b is None)
        if a is not None:
            assert np.array_equal(bits(a), bits(b))
    Y, Z, Zo, Xn = fused
    z_ref = O.mlp_rank(X, A, B)
    total = R.reduce_full([z_ref] + peers_cpu, "sum", bias_cpu)
    assert rel_err(Z, total if opts.get("in_place") else z_ref) <= TOL_BF16
    if Zo is not None:
        assert rel_err(Zo, total) <= TOL_BF16
    if Xn is not None:
        assert rel_err(Xn.float(), total) <= TOL_BF16


@pytest.mark.parametrize("M,H,F,P,Rc,Cc,opts", [
    (64, 256, 512, 2, 1, 1, {}),                                   # the tiny fp32 workload's rank
    (77, 45, 51, 3, 1, 1, {"bias": True, "x_next": True}),         # ragged everything, fp32 next input
    (130, 129, 65, 4, 1, 1, {"in_place": True}),                   # Z_out = Z_i
    (130, 128, 65, 3, 2, 2, {"bias": True}),                       # one stream: one GEMM1, every block folds
    (130, 128, 65, 3, 2, 2, {"bias": True, "noalloc": True}),      # every chunk's GEMM1 kept too
    (130, 128, 65, 3, 2, 2, {"bias": True, "two": True}),          # only the final block folds
])
def test_reduce_fusion_same_bits_fp32(M, H, F, P, Rc, Cc, opts):
    """fp32 throughout: the fp32 kernel's epilogue sum equals the separate
    reduction bit for bit, and the oracle within the fp32 tolerance."""
    announce(f"mlp reduce fusion fp32 M={M} H={H} F={F} P={P} R={Rc} C={Cc} {sorted(opts)}")
    X = inputs.normal((M, H), 381, 1.0)
    A = inputs.normal((H, F), 382, 1.0 / np.sqrt(H))
    B = inputs.normal((F, H), 383, 1.0 / np.sqrt(F))
    peers_cpu = [inputs.normal((M, H), 390 + p) for p in range(P - 1)]
    bias_cpu = inputs.normal((H,), 389) if opts.get("bias") else None
    kw = {k: v for k, v in opts.items() if k != "bias"}
    kw.update(R=Rc, C=Cc, bias=bias_cpu.cuda() if bias_cpu is not None else None)
    Xd, Ad, Bd, peers = X.cuda(), A.cuda(), B.cuda(), [p.cuda() for p in peers_cpu]
    fused = _run_fusion(Xd, Ad, Bd, peers, fusion=tp.TP_REDUCE_FUSION_AUTO, **kw)
    apart = _run_fusion(Xd, Ad, Bd, peers, fusion=tp.TP_REDUCE_FUSION_OFF, **kw)
    for a, b in zip(fused, apart):
        assert (a is None) == (b is None)
        if a is not None:
            assert np.array_equal(bits(a), bits(b))
    total = R.reduce_full([O.mlp_rank(X, A, B)] + peers_cpu, "sum", bias_cpu)
    out = fused[1] if opts.get("in_place") else (fused[2] if fused[2] is not None else fused[3])
    assert rel_err(out, total) <= TOL_F32


def test_timing_reports_the_fused_kernel():
    """With the reduction in GEMM2's epilogue the per-kernel timing sees one
    gemm2_reduce launch whose work is its algorithmic bytes (Y and B_i read,
    the peers' partials read, Z_i and Z_out written); with fusion off, a GEMM2
    and a reduce launch."""
    announce("mlp timing of the fused kernel")
    M, H, F, P = 512, 384, 256, 3
    X = inputs.normal((M, H), 361, 1.0, "bf16").cuda()
    A = inputs.normal((H, F), 362, 1.0 / np.sqrt(H), "bf16").cuda()
    B = inputs.normal((F, H), 363, 1.0 / np.sqrt(F), "bf16").cuda()
    peers = [inputs.normal((M, H), 370 + p).cuda() for p in range(P - 1)]
    Y = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    Z, Zo = torch.empty((M, H), device="cuda"), torch.empty((M, H), device="cuda")
    tp.tp_timing_enable(True)
    try:
        tp.tp_timing_read()
        tp.tp_colrow_mlp(X, A, B, Y, Z, peer_partials=peers, Z_out=Zo)
        fused = tp.tp_timing_read()
        tp.tp_colrow_mlp(X, A, B, Y, Z, peer_partials=peers, Z_out=Zo, reduce_fusion=tp.TP_REDUCE_FUSION_OFF)
        apart = tp.tp_timing_read()
    finally:
        tp.tp_timing_enable(False)
    assert fused["gemm2_reduce"]["launches"] == 1
    assert fused["gemm2"]["launches"] == 0 and fused["reduce"]["launches"] == 0
    assert fused["gemm2_reduce"]["work"] == 2 * (M * F + F * H) + 4 * (P - 1) * M * H + 2 * 4 * M * H
    assert fused["gemm2_reduce"]["total_ms"] > 0
    assert apart["gemm2_reduce"]["launches"] == 0
    assert apart["gemm2"]["launches"] == 1 and apart["reduce"]["launches"] == 1
    assert apart["gemm2"]["work"] == 2 * M * H * F


@pytest.mark.parametrize("M,H,F,P,fused", [(512, 384, 256, 4, True), (512, 384, 256, 5, False),
                                            (520, 392, 200, 3, False), (512, 384, 256, 1, False),
                                            (2048, 2048, 512, 8, True), (2048, 2048, 512, 16, True),
                                            (2048, 2048, 512, 17, False), (2048, 2048, 480, 8, False)])
def test_fusion_taken_where_the_rule_says(M, H, F, P, fused):
    """The reduction runs in GEMM2's epilogue for P <= 4 with F % 32 == 0 on a
    small block, and for P <= 16 with F % 64 == 0 on a block of the 256-row
    tiles; as its own kernel otherwise (P = 1 has nothing to sum)."""
    announce(f"mlp fusion rule M={M} H={H} F={F} P={P}")
    X = torch.zeros((M, H), dtype=torch.bfloat16, device="cuda")
    A = torch.zeros((H, F), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((F, H), dtype=torch.bfloat16, device="cuda")
    peers = [torch.zeros((M, H), device="cuda") for _ in range(P - 1)]
    Y = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    Z = torch.empty((M, H), device="cuda")
    tp.tp_timing_enable(True)
    try:
        tp.tp_timing_read()
        tp.tp_colrow_mlp(X, A, B, Y, Z, peer_partials=peers, Z_out=Z if P > 1 else None)
        st = tp.tp_timing_read()
    finally:
        tp.tp_timing_enable(False)
    assert st["gemm2_reduce"]["launches"] == (1 if fused else 0)
    assert st["gemm2"]["launches"] == (0 if fused else 1)
    assert st["reduce"]["launches"] == (1 if (P > 1 and not fused) else 0)


@pytest.mark.parametrize("two_streams", [True, False])
def test_timing_files_the_tail_reduction_apart(two_streams):
    """On the two-stream schedule (GEMM1 first over all rows, then each block's
    GEMM2 with its reduction beside the next) the last block's reduction, which
    no GEMM runs beside, is timed as reduce_tail and the earlier blocks' as
    reduce; on one stream, where no chunk's sum fits GEMM2's epilogue (7 peers
    on small blocks), the chunks run as one block: one GEMM1, one reduce."""
    announce(f"mlp timing of the tail reduction two_streams={two_streams}")
    M, H, F, P, Rc = 512, 384, 256, 8, 2
    X = torch.zeros((M, H), dtype=torch.bfloat16, device="cuda")
    A = torch.zeros((H, F), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((F, H), dtype=torch.bfloat16, device="cuda")
    peers = [torch.zeros((M, H), device="cuda") for _ in range(P - 1)]
    Y = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    Z = torch.empty((M, H), device="cuda")
    s0 = torch.cuda.current_stream()
    s1 = torch.cuda.Stream() if two_streams else s0
    tp.tp_timing_enable(True)
    try:
        tp.tp_timing_read()
        tp.tp_colrow_mlp(X, A, B, Y, Z, row_chunks=Rc, peer_partials=peers, Z_out=Z, s_compute=s0, s_reduce=s1)
        st = tp.tp_timing_read()
    finally:
        tp.tp_timing_enable(False)
    assert st["reduce"]["launches"] == (Rc - 1 if two_streams else 1)
    assert st["gemm1"]["launches"] == 1          # every chunk's rows in one GEMM1, on either schedule
    assert st["reduce_tail"]["launches"] == (1 if two_streams else 0)
    assert st["reduce_tail"]["work"] == (4.0 * (P + 1) * (M // Rc) * H if two_streams else 0.0)



@pytest.mark.parametrize("M,H,F,Rc,Cc,P,beside", [(4096, 2048, 512, 2, 1, 8, 0), (4096, 4096, 6144, 2, 2, 8, 3)])
def test_two_streams_fold_uncovered_reductions(M, H, F, Rc, Cc, P, beside):
    """On two streams a block's reduction runs beside the next GEMMs only where
    they are long enough to cover it; otherwise it goes into its GEMM2's
    epilogue, and where that leaves nothing for the second stream the schedule
    keeps to one, with one GEMM1 over all rows.  First case: chunk 0's sum of
    8 partials (151 MB) against the next chunk's 8.6 GFLOP, so both chunks
    fold; second: the GPT-3 175B block ratio (F = 6144), three reductions
    beside and the final one folded.  The sums are the same bits as with the
    separate reduction."""
    announce(f"mlp uncovered reductions M={M} H={H} F={F} R={Rc} C={Cc} P={P}")
    X = inputs.normal((M, H), 381, 1.0, "bf16").cuda()
    A = inputs.normal((H, F), 382, 1.0 / np.sqrt(H), "bf16").cuda()
    B = inputs.normal((F, H), 383, 1.0 / np.sqrt(F), "bf16").cuda()
    peers = [inputs.normal((M, H), 390 + p).cuda() for p in range(P - 1)]
    Y = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    Z, Zo = torch.empty((M, H), device="cuda"), torch.empty((M, H), device="cuda")
    Z2, Zo2 = torch.empty((M, H), device="cuda"), torch.empty((M, H), device="cuda")
    s0 = torch.cuda.current_stream()
    s1 = torch.cuda.Stream()
    tp.tp_timing_enable(True)
    try:
        tp.tp_timing_read()
        tp.tp_colrow_mlp(X, A, B, Y, Z, row_chunks=Rc, col_chunks=Cc, peer_partials=peers, Z_out=Zo,
                         s_compute=s0, s_reduce=s1)
        st = tp.tp_timing_read()
        tp.tp_colrow_mlp(X, A, B, Y, Z2, row_chunks=Rc, col_chunks=Cc, peer_partials=peers, Z_out=Zo2,
                         s_compute=s0, s_reduce=s1, reduce_fusion=tp.TP_REDUCE_FUSION_OFF)
        torch.cuda.synchronize()
    finally:
        tp.tp_timing_enable(False)
    assert st["reduce"]["launches"] == beside and st["reduce_tail"]["launches"] == 0
    assert st["gemm2_reduce"]["launches"] == Rc * Cc - beside
    assert st["gemm2"]["launches"] == beside
    assert st["gemm1"]["launches"] == 1          # GEMM1 first over all rows, on either schedule
    assert torch.equal(Zo, Zo2) and torch.equal(Z, Z2)

@pytest.mark.parametrize("Rc,Cc,act,h_out,folds", [(2, 1, tp.TP_ACT_GELU_ERF, True, 2), (2, 2, tp.TP_ACT_NONE, False, 1),
                                               (4, 1, tp.TP_ACT_GELU_ERF, False, 1)])
def test_one_stream_merges_the_chunks(Rc, Cc, act, h_out, folds):
    """Row chunks on one stream overlap nothing, so GEMM1 runs once over all
    rows; where each chunk's block folds its sum into GEMM2 (2048 x 2048, the
    256-row tiles) the blocks keep their GEMM2s, and where none does (7 peers
    on the small tiles) the layer runs as one block whose sum folds.  Y,
    H_out, Z_i and the sum are the same bits as the two-stream schedule (each
    block's separate reduction beside the next GEMM2) and as the allocation-free entry
    point, which keeps every chunk (Y holds one chunk), and match the oracle on
    sampled rows."""
    announce(f"mlp one stream, chunks merged R={Rc} C={Cc} act={act} h_out={h_out}")
    M, H, F, P = 4096, 2048, 512, 8
    X = inputs.normal((M, H), 461, 1.0, "bf16")
    A = inputs.normal((H, F), 462, 1.0 / np.sqrt(H), "bf16")
    B = inputs.normal((F, H), 463, 1.0 / np.sqrt(F), "bf16")
    peers_cpu = [inputs.normal((M, H), 470 + p) for p in range(P - 1)]
    Xd, Ad, Bd, peers = X.cuda(), A.cuda(), B.cuda(), [p.cuda() for p in peers_cpu]

    def run(two, fusion, noalloc=False):
        Y = Guarded((M, F), torch.bfloat16)
        Hs = Guarded((M, F), torch.bfloat16) if h_out else None
        Z, Zo = Guarded((M, H), torch.float32), Guarded((M, H), torch.float32)
        s0 = torch.cuda.current_stream()
        kw = dict(row_chunks=Rc, col_chunks=Cc, peer_partials=peers, Z_out=Zo.t, act=act, reduce_fusion=fusion,
                  H_out=Hs.t if h_out else None, s_compute=s0, s_reduce=torch.cuda.Stream() if two else s0)
        if noalloc:
            tp.tp_colrow_mlp_noalloc(Xd, Ad, Bd, Z.t, **kw)
        else:
            tp.tp_colrow_mlp(Xd, Ad, Bd, Y.t, Z.t, **kw)
        torch.cuda.synchronize()
        outs = [Y, Z, Zo] + ([Hs] if h_out else [])
        assert all(g.guards_intact() for g in outs), "write outside an output buffer"
        return [None if (noalloc and g is Y) else g.t.cpu() for g in outs]

    tp.tp_timing_enable(True)
    try:
        tp.tp_timing_read()
        got = run(False, tp.TP_REDUCE_FUSION_AUTO)
        st = tp.tp_timing_read()
        chunked = run(True, tp.TP_REDUCE_FUSION_OFF)
        st_chunked = tp.tp_timing_read()
        kept = run(False, tp.TP_REDUCE_FUSION_AUTO, noalloc=True)
        st_kept = tp.tp_timing_read()
    finally:
        tp.tp_timing_enable(False)
    assert st["gemm1"]["launches"] == 1 and st["gemm2_reduce"]["launches"] == folds
    assert st["gemm2"]["launches"] == 0 and st["reduce"]["launches"] == 0
    assert st_chunked["gemm1"]["launches"] == 1 and st_chunked["gemm2"]["launches"] == Rc * Cc
    # (at R = C = 2 each kept block takes the small tiles, whose epilogue sums at most 3 peers: separate reductions)
    assert st_kept["gemm1"]["launches"] == Rc
    assert st_kept["gemm2_reduce"]["launches"] + st_kept["gemm2"]["launches"] == Rc * Cc
    for a, b, c in zip(got, chunked, kept):
        assert np.array_equal(bits(a), bits(b))
        if c is not None:
            assert np.array_equal(bits(a), bits(c))
    rows = np.linspace(0, M - 1, 128).astype(np.int64)
    z0 = O.mlp_rank_rows(X, A, B, rows, act=O.GELU_ERF if act == tp.TP_ACT_GELU_ERF else O.GELU_NONE)
    assert rel_err(got[1][torch.from_numpy(rows)], z0) <= TOL_BF16
    total = z0 + sum(p[torch.from_numpy(rows)].double().numpy() for p in peers_cpu)
    assert rel_err(got[2][torch.from_numpy(rows)], total) <= TOL_BF16


def test_max_ranks_integer_exact():
    """P = 64 virtual ranks (63 peers), chunked, on two streams: exact."""
    announce("mlp P=64 integer exact")
    M, H, F, P = 256, 128, 64, 64
    X = inputs.small_ints((M, H), seed=281, lo=-4, hi=4, dtype="bf16")
    A = _one_hot_columns(H, F, 282)
    B = inputs.small_ints((F, H), seed=283, lo=-4, hi=4, dtype="bf16")
    peers_cpu = [inputs.small_ints((M, H), seed=300 + p, lo=-512, hi=512) for p in range(P - 1)]
    Y, Z, Zo = run_rank(X.cuda(), A.cuda(), B.cuda(), R=2, C=2, peers=[p.cuda() for p in peers_cpu],
                        act=tp.TP_ACT_NONE, two_streams=True)
    z_ref = O.mlp_rank(X, A, B, O.GELU_NONE)
    assert np.array_equal(Zo.numpy().astype(np.float64), R.reduce_full([z_ref] + peers_cpu))


def test_prepared_call_matches_direct_call():
    """A call marshalled once (prepare=True) and replayed gives the same bits as
    the direct call, on each replay."""
    announce("mlp prepared call")
    M, H, F = 512, 384, 256
    X = inputs.normal((M, H), seed=291, dtype="bf16").cuda()
    A = inputs.normal((H, F), seed=292, std=0.05, dtype="bf16").cuda()
    B = inputs.normal((F, H), seed=293, std=0.05, dtype="bf16").cuda()
    peer = inputs.normal((M, H), seed=294).cuda()
    Y = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    Z = torch.empty((M, H), device="cuda")
    Zo = torch.empty((M, H), device="cuda")
    tp.tp_colrow_mlp(X, A, B, Y, Z, row_chunks=2, peer_partials=[peer], Z_out=Zo)
    torch.cuda.synchronize()
    ref = Zo.clone()
    call = tp.tp_colrow_mlp(X, A, B, Y, Z, row_chunks=2, peer_partials=[peer], Z_out=Zo, prepare=True)
    s1 = torch.cuda.Stream()
    for _ in range(3):
        Zo.zero_()
        call(torch.cuda.current_stream(), s1)
        torch.cuda.synchronize()
        assert torch.equal(Zo.view(torch.int32), ref.view(torch.int32))
    # An output re-pointed to new storage: the replay refuses before launching anything.
    Zo.set_(torch.empty_like(Zo))
    with pytest.raises(tp.TpError, match="moved"):
        call()


@pytest.mark.parametrize("Rc,Cc,P,fusion", [(1, 1, 4, tp.TP_REDUCE_FUSION_AUTO), (2, 2, 3, tp.TP_REDUCE_FUSION_AUTO),
                                            (1, 1, 4, tp.TP_REDUCE_FUSION_OFF), (2, 1, 8, tp.TP_REDUCE_FUSION_AUTO)])
def test_column_shard_read_in_place(Rc, Cc, P, fusion):
    """A_i as a column slice of the full A (row stride P*F, A_ld) gives the bits
    of the copied shard, for the GPT-2 shape's small tiles and a ping-pong tile."""
    for M, H, F, dt in ((4096, 768, 768, "bf16"), (2048, 512, 2048, "bf16"), (64, 256, 512, "f32")):
        announce(f"mlp column shard in place M={M} H={H} F={F} {dt} R={Rc} C={Cc} P={P} fusion={fusion}")
        X = inputs.normal((M, H), 4501, 1.0, dt).cuda()
        A = inputs.normal((H, P * F), 4502, 0.02, dt).cuda()
        B = inputs.normal((P * F, H), 4503, 0.02, dt).cuda()
        peers = [inputs.normal((M, H), 4510 + p).cuda() for p in range(P - 1)]
        i = P - 1                                   # the last rank's shard: offset and stride both matter
        outs = []
        for A_i, B_i in ((A[:, i * F:(i + 1) * F].contiguous(), B[i * F:(i + 1) * F].contiguous()),
                         (A[:, i * F:(i + 1) * F], B[i * F:(i + 1) * F])):
            Y = Guarded((M, F), X.dtype)
            Z = Guarded((M, H), torch.float32)
            Zo = Guarded((M, H), torch.float32)
            tp.tp_colrow_mlp(X, A_i, B_i, Y.t, Z.t, row_chunks=Rc, col_chunks=Cc, peer_partials=peers, Z_out=Zo.t,
                             reduce_fusion=fusion, s_reduce=torch.cuda.Stream())
            torch.cuda.synchronize()
            assert Y.guards_intact() and Z.guards_intact() and Zo.guards_intact()
            outs.append([bits(g.t.cpu()) for g in (Y, Z, Zo)])
        for a, b in zip(*outs):
            assert np.array_equal(a, b)


def test_two_stream_gemm1_first_equals_one_block():
    """The headline's schedule shape (GEMM1 once over all rows, R = C = 2, three
    sums beside the next GEMM2 and the last in its epilogue: F = 6144 as in
    the 175B layer, so each block's sum is short enough to run beside the
    next block's GEMM2, and blocks of 2048 x 2048 take the 256-row tiles
    whose epilogue sums 7 peers) with every output the fused epilogue writes (the sum
    with the bias, the next layer's bf16 input, the pre-activation and Y)
    equals the same layer run as one block on one stream, bit for bit: chunking
    and the schedule change no result bit.  Guarded outputs catch stray
    writes."""
    M, H, F, P, Rc, Cc = 4096, 4096, 6144, 8, 2, 2
    announce(f"mlp two-stream GEMM1-first against one block M={M} H={H} F={F} P={P} R={Rc} C={Cc}")
    X = inputs.normal((M, H), 401, 1.0, "bf16").cuda()
    A = inputs.normal((H, F), 402, 1.0 / np.sqrt(H), "bf16").cuda()
    B = inputs.normal((F, H), 403, 1.0 / np.sqrt(F), "bf16").cuda()
    bias = inputs.normal((H,), 404, 0.1).cuda()
    peers = [inputs.normal((M, H), 410 + p).cuda() for p in range(P - 1)]
    outs = []
    for two in (True, False):
        Y, Hh = Guarded((M, F), torch.bfloat16), Guarded((M, F), torch.bfloat16)
        Z, Zo, Xn = Guarded((M, H), torch.float32), Guarded((M, H), torch.float32), Guarded((M, H), torch.bfloat16)
        s0 = torch.cuda.current_stream()
        s1 = torch.cuda.Stream() if two else s0
        tp.tp_timing_enable(True)
        try:
            tp.tp_timing_read()
            tp.tp_colrow_mlp(X, A, B, Y.t, Z.t, row_chunks=Rc if two else 1, col_chunks=Cc if two else 1,
                             peer_partials=peers, Z_out=Zo.t, bias=bias, X_next=Xn.t, H_out=Hh.t,
                             s_compute=s0, s_reduce=s1)
            st = tp.tp_timing_read()
        finally:
            tp.tp_timing_enable(False)
        torch.cuda.synchronize()
        for g in (Y, Hh, Z, Zo, Xn):
            assert g.guards_intact()
        if two:
            assert st["gemm1"]["launches"] == 1 and st["gemm2"]["launches"] == Rc * Cc - 1
            assert st["reduce"]["launches"] == Rc * Cc - 1 and st["gemm2_reduce"]["launches"] == 1
        outs.append([g.t.clone() for g in (Y, Hh, Zo, Xn)])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))
