"""Weights in a linear layer's [out, in] layout (TP_WEIGHTS_LINEAR): the
column-parallel shard A_i given as [F, H] and the row-parallel shard B_i as
[H, F], as ColossalAI's Linear1D_Col / Linear1D_Row hold them ([CAI] section
5.1).  The GEMMs read them k-contiguous instead of through the transposing LDS
read; every output must be the math layout's bits, and the full-size step must
match the oracle on sampled rows."""
import numpy as np
import pytest
import torch

import sharded_gemm_amd as tp
from sharded_gemm_amd import inputs
from sharded_gemm_amd.workloads import GPT3_175B
from oracle import mlp as O

from gpu_helpers import Guarded, announce, bits, rel_err, require_gpu

pytestmark = pytest.mark.gpu

TOL_BF16 = 1e-2


def setup_module(_):
    require_gpu()


def _forward(X, A, B, peers, *, layout, R=1, C=1, h_out=False, seq=0, bias=None, noalloc=False, one=False):
    """One forward call into guarded buffers (two streams); returns CPU copies
    of Y, Z_i, the sum (Z_out, or the concatenated Z_split blocks) and H_out.
    noalloc: through the allocation-free entry point, which keeps the row
    chunks (Y is then not returned).  one: s_reduce = s_compute."""
    M, H = X.shape
    F = A.shape[0] if layout == tp.TP_WEIGHTS_LINEAR else A.shape[1]
    Y = None if noalloc else Guarded((M, F), X.dtype)
    Z = Guarded((M, H), torch.float32)
    Zo = Guarded((M, H), torch.float32) if (peers and not seq) else None
    Hs = Guarded((M, F), X.dtype) if h_out else None
    Zs = [Guarded((M // seq, H), torch.float32) for _ in range(seq)] if seq else None
    kw = dict(row_chunks=R, col_chunks=C, peer_partials=list(peers), weight_layout=layout, bias=bias,
              s_compute=torch.cuda.current_stream(),
              s_reduce=torch.cuda.current_stream() if one else torch.cuda.Stream())
    if seq:
        kw["X_shards"] = [b.clone() for b in torch.chunk(X, seq)]
        kw["Z_split"] = [g.t for g in Zs]
        X = None
    kw.update(Z_out=Zo.t if Zo is not None else None, H_out=Hs.t if Hs is not None else None)
    if noalloc:
        tp.tp_colrow_mlp_noalloc(X, A, B, Z.t, **kw)
    else:
        tp.tp_colrow_mlp(X, A, B, Y.t, Z.t, **kw)
    torch.cuda.synchronize()
    outs = [Z] + ([Y] if Y is not None else []) + ([Zo] if Zo is not None else []) + \
        ([Hs] if Hs is not None else []) + (Zs or [])
    for g in outs:
        assert g.guards_intact(), "write outside an output buffer"
    total = Zo.t.cpu() if Zo is not None else (torch.cat([g.t.cpu() for g in Zs]) if seq else None)
    return (Y.t.cpu() if Y is not None else None), Z.t.cpu(), total, (Hs.t.cpu() if Hs is not None else None)


@pytest.mark.parametrize("M,H,F,R,C,P,opts", [
    (512, 384, 256, 2, 1, 3, {}),                      # small tiles, the sum in GEMM2's epilogue
    (300, 264, 136, 3, 2, 2, {}),                      # ragged: element-wise loads
    (4096, 768, 768, 1, 1, 4, {"h_out": True}),        # GPT-2-small shape, the saved pre-activation
    (2048, 2048, 512, 2, 1, 8, {}),                    # 256-row tiles, the last chunk's sum staged through LDS
    (2048, 4096, 1536, 2, 2, 8, {"bias": True}),       # column blocks of B_i^T rows, the bias
    (2048, 2048, 512, 2, 1, 8, {"seq": 8}),            # sequence parallel: reduce-scattered, blocks in place
    (1024, 512, 256, 2, 1, 4, {"seq": 4}),             # the same on the small tiles (separate reduce-scatter)
    (256, 96, 64, 2, 1, 2, {"f32": True}),             # fp32 throughout
    (4096, 2048, 512, 2, 1, 8, {"h_out": True, "one": True}),  # one stream: GEMM1 over all rows, each chunk's GEMM2 folds
])
def test_forward_linear_layout_same_bits(M, H, F, R, C, P, opts):
    """A_i^T and B_i^T given as [F, H] and [H, F]: Y, Z_i, the sum and H_out
    equal the math layout's bit for bit."""
    announce(f"linear weights forward M={M} H={H} F={F} R={R} C={C} P={P} {opts}")
    dt = "f32" if opts.get("f32") else "bf16"
    X = inputs.normal((M, H), 1101, 1.0, dt).cuda()
    A = inputs.normal((H, F), 1102, 1.0 / np.sqrt(H), dt).cuda()
    B = inputs.normal((F, H), 1103, 1.0 / np.sqrt(F), dt).cuda()
    peers = [inputs.normal((M, H), 1110 + p).cuda() for p in range(P - 1)]
    bias = inputs.normal((H,), 1109).cuda() if opts.get("bias") else None
    kw = dict(R=R, C=C, h_out=opts.get("h_out", False), seq=opts.get("seq", 0), bias=bias, one=opts.get("one", False))
    ref = _forward(X, A, B, peers, layout=tp.TP_WEIGHTS_MATH, **kw)
    got = _forward(X, A.t().contiguous(), B.t().contiguous(), peers, layout=tp.TP_WEIGHTS_LINEAR, **kw)
    for a, b in zip(got, ref):
        if b is not None:
            assert np.array_equal(bits(a), bits(b))
    if R * C > 1:
        # Every row chunk kept (one stream may merge their GEMM1s, or run the layer as one block):
        # each block's GEMM2 reads its rows of B_i^T at its offset.
        kept = _forward(X, A.t().contiguous(), B.t().contiguous(), peers, layout=tp.TP_WEIGHTS_LINEAR, noalloc=True,
                        **kw)
        for a, b in zip(kept[1:], ref[1:]):
            if b is not None:
                assert np.array_equal(bits(a), bits(b))


def test_forward_linear_shards_read_in_place():
    """Rank 1's shards read where they lie in the full linear weights: rows
    [F, 2F) of W1 [P*F, H] (contiguous) and columns [F, 2F) of W2 [H, P*F] (a
    row stride of P*F): the same bits as contiguous copies."""
    announce("linear weights forward, shards in place")
    M, H, F, P = 1024, 768, 768, 4
    X = inputs.normal((M, H), 1121, 1.0, "bf16").cuda()
    W1 = inputs.normal((P * F, H), 1122, 0.02, "bf16").cuda()
    W2 = inputs.normal((H, P * F), 1123, 0.02, "bf16").cuda()
    peers = [inputs.normal((M, H), 1130 + p).cuda() for p in range(P - 1)]
    A1, B1 = W1[F:2 * F], W2[:, F:2 * F]
    assert not B1.is_contiguous()
    ref = _forward(X, A1.contiguous(), B1.contiguous(), peers, layout=tp.TP_WEIGHTS_LINEAR)
    got = _forward(X, A1, B1, peers, layout=tp.TP_WEIGHTS_LINEAR)
    for a, b in zip(got, ref):
        if b is not None:
            assert np.array_equal(bits(a), bits(b))


def _backward(X, A, B, Hs, Y, dZ, peers, *, layout, R, act):
    M, H = X.shape
    F = Y.shape[1]
    wa, wb = ((F, H), (H, F)) if layout == tp.TP_WEIGHTS_LINEAR else ((H, F), (F, H))
    dH = Guarded((M, F), X.dtype)
    dX = Guarded((M, H), torch.float32)
    dXo = Guarded((M, H), torch.float32)
    dA = Guarded(wa, torch.float32)
    dB = Guarded(wb, torch.float32)
    tp.tp_colrow_mlp_backward(X, A, B, Hs, Y, dZ, dH.t, dX.t, dA.t, dB.t, row_chunks=R, peer_dX=list(peers),
                              dX_out=dXo.t, weight_layout=layout, act=act, s_compute=torch.cuda.current_stream(),
                              s_reduce=torch.cuda.Stream())
    torch.cuda.synchronize()
    for g in (dH, dX, dXo, dA, dB):
        assert g.guards_intact(), "write outside an output buffer"
    return dH.t.cpu(), dX.t.cpu(), dXo.t.cpu(), dA.t.cpu(), dB.t.cpu()


@pytest.mark.parametrize("M,H,F,R,P,ints", [
    (512, 384, 256, 2, 3, True), (4096, 768, 768, 1, 4, False), (2048, 2048, 512, 2, 8, True),
    (2048, 2048, 512, 2, 8, False), (300, 264, 136, 3, 2, False),
])
def test_backward_linear_layout(M, H, F, R, P, ints):
    """dH, dX and the summed dX equal the math layout's bits; dA_i and dB_i,
    now computed as dH^T X and dZ^T Y_i, are the math layout's transposes:
    exactly with small integers, and within the bf16 tolerance otherwise."""
    announce(f"linear weights backward M={M} H={H} F={F} R={R} P={P} ints={ints}")
    if ints:
        X = inputs.small_ints((M, H), seed=1141, lo=-4, hi=4, dtype="bf16").cuda()
        A = inputs.small_ints((H, F), seed=1142, lo=-2, hi=2, dtype="bf16").cuda()
        B = inputs.small_ints((F, H), seed=1143, lo=-2, hi=2, dtype="bf16").cuda()
        dZ = inputs.small_ints((M, H), seed=1144, lo=-4, hi=4, dtype="bf16").cuda()
        act = tp.TP_ACT_NONE
    else:
        X = inputs.normal((M, H), 1141, 1.0, "bf16").cuda()
        A = inputs.normal((H, F), 1142, 1.0 / np.sqrt(H), "bf16").cuda()
        B = inputs.normal((F, H), 1143, 1.0 / np.sqrt(F), "bf16").cuda()
        dZ = inputs.normal((M, H), 1144, 1.0, "bf16").cuda()
        act = tp.TP_ACT_GELU_ERF
    peers = [inputs.normal((M, H), 1150 + p).cuda() for p in range(P - 1)]
    Y = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    Hs = torch.empty((M, F), dtype=torch.bfloat16, device="cuda") if act == tp.TP_ACT_GELU_ERF else None
    tp.tp_colrow_mlp(X, A, B, Y, torch.empty((M, H), device="cuda"), act=act, H_out=Hs)
    torch.cuda.synchronize()
    ref = _backward(X, A, B, Hs, Y, dZ, peers, layout=tp.TP_WEIGHTS_MATH, R=R, act=act)
    got = _backward(X, A.t().contiguous(), B.t().contiguous(), Hs, Y, dZ, peers, layout=tp.TP_WEIGHTS_LINEAR, R=R,
                    act=act)
    for a, b in zip(got[:3], ref[:3]):
        assert np.array_equal(bits(a), bits(b))
    for a, b in zip(got[3:], ref[3:]):
        if ints:
            assert torch.equal(a, b.t())
        else:
            assert rel_err(a, b.t().double().numpy()) <= 1e-6


def test_forward_linear_gpt3_175b_sampled():
    """The GPT-3 175B per-rank step (R = 2, C = 2, two streams) with both
    shards in the linear layout, as the bench's --weights linear times it:
    128 sampled rows of the summed output match the oracle's."""
    w = GPT3_175B
    announce(f"linear weights forward {w.name} sampled")
    M, H, F, P = w.M, w.H, w.F, w.P
    X = inputs.normal((M, H), inputs.seed_for(w.cfg, inputs.SLOT_X), 1.0, "bf16", "cuda")
    At = inputs.normal((F, H), inputs.seed_for(w.cfg, inputs.SLOT_A), 0.02, "bf16", "cuda")
    Bt = inputs.normal((H, F), inputs.seed_for(w.cfg, inputs.SLOT_B), 0.02, "bf16", "cuda")
    peers = [inputs.normal((M, H), inputs.seed_for(w.cfg, inputs.SLOT_PARTIAL + p), 1.0, "f32", "cuda")
             for p in range(P - 1)]
    Y, Z, total, _ = _forward(X, At, Bt, peers, layout=tp.TP_WEIGHTS_LINEAR, R=w.R, C=w.C)
    rows = np.unique(np.concatenate([np.linspace(r * (M // w.R), (r + 1) * (M // w.R) - 1, 64).astype(np.int64)
                                     for r in range(w.R)]))
    announce(f"linear weights forward {w.name}: oracle on {len(rows)} rows")
    z0 = O.mlp_rank_rows(X.cpu(), At.t().cpu(), Bt.t().cpu(), rows)
    assert rel_err(Z[torch.from_numpy(rows)], z0) <= TOL_BF16
    ref = z0 + sum(p[torch.from_numpy(rows).cuda()].cpu().double().numpy() for p in peers)
    assert rel_err(total[torch.from_numpy(rows)], ref) <= TOL_BF16
