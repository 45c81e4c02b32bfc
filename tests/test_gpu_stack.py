"""GPU parity of tp_colrow_mlp_stack (layers chained through the reduce's
fused next-layer input, with the inter-layer overlap or one after another)
and of the X_next output, against the oracle's layer stack."""
import numpy as np
import pytest
import torch

import sharded_gemm_amd as tp
from sharded_gemm_amd import inputs
from sharded_gemm_amd.workloads import GPT3_175B, GPT3_6P7B
from oracle import mlp as O

from gpu_helpers import Guarded, announce, bits, rel_err, require_gpu

pytestmark = pytest.mark.gpu

TOL_BF16 = 1e-2


def setup_module(_):
    require_gpu()


def _pm1_one_hot(H, F, seed):
    """[H, F] with a single +-1 per column: X A picks (and maybe negates) one
    column of X, so Y is exactly representable whatever X holds."""
    g = torch.Generator().manual_seed(seed)
    rows = torch.randint(0, H, (F,), generator=g)
    sign = torch.randint(0, 2, (F,), generator=g) * 2 - 1
    A = torch.zeros((H, F))
    A[rows, torch.arange(F)] = sign.float()
    return A.to(torch.bfloat16)


def _layers_integer(M, H, Fs, P, seed):
    """Per layer: A (+-1 one-hot), B in {-1, 0, 1}, P-1 integer peers, a bias."""
    out = []
    for l, F in enumerate(Fs):
        s = seed + 100 * l
        out.append({"A_i": _pm1_one_hot(H, F, s),
                    "B_i": inputs.small_ints((F, H), seed=s + 1, lo=-1, hi=1, dtype="bf16"),
                    "peers": [inputs.small_ints((M, H), seed=s + 10 + p, lo=-64, hi=64) for p in range(P - 1)],
                    "bias": inputs.small_ints((H,), seed=s + 2, lo=-8, hi=8)})
    return out


def run_stack(X0, layers, *, R=1, C=1, act=tp.TP_ACT_NONE, two_streams=True, keep_z=True, prepared=False,
              fusion=tp.TP_REDUCE_FUSION_AUTO, linear=False):
    """The stack on the GPU into guarded buffers; returns per layer (Z_out, X_next)
    CPU copies.  prepared: marshal the call once and replay it twice, the
    outputs overwritten with NaN in between.  linear: the weights passed in a
    linear layer's [out, in] layout (A_i^T, B_i^T)."""
    M, H = X0.shape
    dt = X0.dtype
    xs = [X0.cuda()] + [Guarded((M, H), dt) for _ in layers]
    zs = [Guarded((M, H), torch.float32) for _ in layers] if keep_z else [None] * len(layers)
    Y = torch.empty((M, max(l["A_i"].shape[1] for l in layers)), dtype=dt, device="cuda")
    Zi = torch.empty((M, H), device="cuda")
    args = []
    for l, layer in enumerate(layers):
        F = layer["A_i"].shape[1]
        A_i, B_i = layer["A_i"].cuda(), layer["B_i"].cuda()
        if linear:
            A_i, B_i = A_i.t().contiguous(), B_i.t().contiguous()
        args.append(dict(X=xs[l] if l == 0 else xs[l].t, A_i=A_i, B_i=B_i,
                         weight_layout=tp.TP_WEIGHTS_LINEAR if linear else tp.TP_WEIGHTS_MATH,
                         Y_ws=Y[:, :F] if F == Y.shape[1] else torch.empty((M, F), dtype=dt, device="cuda"),
                         Z_i=Zi, row_chunks=R, col_chunks=C, peer_partials=[p.cuda() for p in layer["peers"]],
                         Z_out=zs[l].t if keep_z else None, act=act,
                         bias=layer["bias"].cuda() if layer.get("bias") is not None else None,
                         X_next=xs[l + 1].t, reduce_fusion=fusion))
    s0 = torch.cuda.current_stream()
    s1 = torch.cuda.Stream() if two_streams else s0
    if prepared:
        call = tp.tp_colrow_mlp_stack(args, s_compute=s0, s_reduce=s1, prepare=True)
        for _ in range(2):
            for t in xs[1:] + (zs if keep_z else []):
                t.t.fill_(float("nan"))
            call()
    else:
        tp.tp_colrow_mlp_stack(args, s_compute=s0, s_reduce=s1)
    torch.cuda.synchronize()
    res = []
    for l in range(len(layers)):
        assert xs[l + 1].guards_intact()
        if keep_z:
            assert zs[l].guards_intact()
        res.append((zs[l].t.cpu() if keep_z else None, xs[l + 1].t.cpu()))
    return res


@pytest.mark.parametrize("M,H,Fs,R,C,P,two", [
    # every block's sum folds (at most 3 peers on the small tiles): the layers one after another
    (512, 256, [128, 96], 2, 1, 4, True),
    (768, 384, [64, 64, 32], 3, 2, 3, True),
    (300, 264, [136, 64], 3, 2, 2, True),      # ragged tiles
    (256, 128, [64, 64], 1, 1, 2, True),       # one block: serial schedule
    (512, 256, [128, 128], 2, 2, 4, False),    # one stream
    (4096, 768, [768, 768], 2, 1, 4, True),    # GPT-2-small shape
    # 7 peers: the sums run beside the GEMMs, the inter-layer overlap over the row chunks
    (512, 256, [128, 96], 2, 1, 8, True),
    (768, 384, [64, 64, 32], 3, 2, 8, True),
    (300, 264, [136, 64], 3, 2, 8, True),      # ragged tiles
])
def test_stack_integer_exact(M, H, Fs, R, C, P, two):
    """Exact integers through every layer: each Z_out and each next-layer input
    (the sum rounded to bf16, RNE on both sides of the same exact value) equals
    the oracle's bit for bit."""
    announce(f"stack integer exact M={M} H={H} F={Fs} R={R} C={C} P={P} two={two}")
    X0 = inputs.small_ints((M, H), seed=1201, lo=-4, hi=4, dtype="bf16")
    layers = _layers_integer(M, H, Fs, P, 1300)
    got = run_stack(X0, layers, R=R, C=C, two_streams=two)
    ref = O.mlp_stack(X0, [dict(l, act=O.GELU_NONE) for l in layers], dtype="bf16")
    for l, ((z, xn), (zr, xr)) in enumerate(zip(got, ref)):
        assert np.array_equal(z.double().numpy(), zr), l
        assert np.array_equal(bits(xn), bits(torch.from_numpy(xr).to(torch.bfloat16))), l


@pytest.mark.parametrize("M,H,Fs,R,C,P", [(512, 256, [128, 96], 2, 1, 4), (4096, 768, [768, 768], 2, 1, 4),
                                           (2048, 2048, [512, 512], 2, 2, 8)])
def test_stack_linear_weights_same_bits(M, H, Fs, R, C, P):
    """The stack with every layer's weights in the [out, in] layout gives the
    math layout's bits in every Z_out and next-layer input."""
    announce(f"stack linear weights M={M} H={H} F={Fs} R={R} C={C} P={P}")
    X0 = inputs.normal((M, H), 1211, 1.0, "bf16")
    layers = [{"A_i": inputs.normal((H, F), 1220 + l, 1.0 / np.sqrt(H), "bf16"),
               "B_i": inputs.normal((F, H), 1230 + l, 1.0 / np.sqrt(F), "bf16"),
               "peers": [inputs.normal((M, H), 1240 + 10 * l + p) for p in range(P - 1)],
               "bias": inputs.normal((H,), 1290 + l)} for l, F in enumerate(Fs)]
    ref = run_stack(X0, layers, R=R, C=C, act=tp.TP_ACT_GELU_ERF)
    got = run_stack(X0, layers, R=R, C=C, act=tp.TP_ACT_GELU_ERF, linear=True)
    for l, ((z, xn), (zr, xr)) in enumerate(zip(got, ref)):
        assert np.array_equal(bits(z), bits(zr)), l
        assert np.array_equal(bits(xn), bits(xr)), l


def test_stack_layers_one_after_another():
    """Layers whose every block's sum folds into its GEMM2 (chunks of 2048 x 2048
    on the 256-row tiles, 7 peers, too much to sum beside the next GEMMs) run
    one after another, each with one GEMM1 over all rows: the same bits in
    every Z_out and next-layer input as the inter-layer overlap with the
    separate reductions."""
    announce("stack layer by layer")
    M, H, Fs, P, R = 4096, 2048, [512, 512], 8, 2
    X0 = inputs.normal((M, H), 1251, 1.0, "bf16")
    layers = [{"A_i": inputs.normal((H, F), 1260 + l, 1.0 / np.sqrt(H), "bf16"),
               "B_i": inputs.normal((F, H), 1270 + l, 1.0 / np.sqrt(F), "bf16"),
               "peers": [inputs.normal((M, H), 1280 + 10 * l + p) for p in range(P - 1)],
               "bias": inputs.normal((H,), 1295 + l)} for l, F in enumerate(Fs)]
    tp.tp_timing_enable(True)
    try:
        tp.tp_timing_read()
        got = run_stack(X0, layers, R=R, act=tp.TP_ACT_GELU_ERF)
        st = tp.tp_timing_read()
        ref = run_stack(X0, layers, R=R, act=tp.TP_ACT_GELU_ERF, fusion=tp.TP_REDUCE_FUSION_OFF)
        st_ref = tp.tp_timing_read()
    finally:
        tp.tp_timing_enable(False)
    assert st["gemm1"]["launches"] == len(Fs) and st["gemm2_reduce"]["launches"] == R * len(Fs)
    assert st["reduce"]["launches"] == 0 and st["gemm2"]["launches"] == 0
    assert st_ref["gemm1"]["launches"] == R * len(Fs) and st_ref["gemm2"]["launches"] == R * len(Fs)
    for l, ((z, xn), (zr, xr)) in enumerate(zip(got, ref)):
        assert np.array_equal(bits(z), bits(zr)), l
        assert np.array_equal(bits(xn), bits(xr)), l


@pytest.mark.parametrize("w", [GPT3_6P7B, GPT3_175B], ids=lambda w: w.name)
def test_stack_tp8_sampled(w):
    """Two layers of a GPT-3 per-rank shape at TP = 8, as the bench's 2-layer
    step runs them (R row chunks, C column blocks, two streams; the 175B layers
    with the inter-layer overlap, the 6.7B ones one after another, every
    chunk's sum folded): 128 rows of each layer's reduced output and of the next layer's
    bf16 input (64 per row chunk, each chunk's first and last among them)
    against the oracle's stack on those rows (rows stay independent through
    the stack).  The peers' partials of each layer are drawn, not computed."""
    announce(f"stack {w.name} sampled")
    M, H, F, P = w.M, w.H, w.F, w.P
    X0 = inputs.normal((M, H), inputs.seed_for(w.cfg, inputs.SLOT_X), 1.0, "bf16", "cuda")
    layers = []
    for l in range(2):
        s = inputs.seed_for(w.cfg, 0) + 7919 * (l + 1)
        layers.append({"A_i": inputs.normal((H, F), s + inputs.SLOT_A, 0.02, "bf16", "cuda"),
                       "B_i": inputs.normal((F, H), s + inputs.SLOT_B, 0.02, "bf16", "cuda"),
                       "peers": [inputs.normal((M, H), s + inputs.SLOT_PARTIAL + p, 1.0, "f32", "cuda")
                                 for p in range(P - 1)]})
    Y = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    Zi = torch.empty((M, H), device="cuda")
    xs = [Guarded((M, H), torch.bfloat16) for _ in layers]
    zs = [Guarded((M, H), torch.float32) for _ in layers]
    args = [dict(X=X0 if l == 0 else xs[l - 1].t, A_i=layer["A_i"], B_i=layer["B_i"], Y_ws=Y, Z_i=Zi,
                 row_chunks=w.R, col_chunks=w.C, peer_partials=layer["peers"], Z_out=zs[l].t, X_next=xs[l].t)
            for l, layer in enumerate(layers)]
    tp.tp_colrow_mlp_stack(args, s_compute=torch.cuda.current_stream(), s_reduce=torch.cuda.Stream())
    torch.cuda.synchronize()
    for g in xs + zs:
        assert g.guards_intact()
    rows = []
    Mr = M // w.R
    for r in range(w.R):
        rows += list(np.unique(np.linspace(r * Mr, (r + 1) * Mr - 1, 64).astype(np.int64)))
    ridx = torch.tensor(rows, device="cuda")
    announce(f"stack {w.name}: oracle on {len(rows)} rows")
    ref = O.mlp_stack(X0.index_select(0, ridx).cpu(),
                      [{"A_i": layer["A_i"].cpu(), "B_i": layer["B_i"].cpu(),
                        "peers": [p.index_select(0, ridx).cpu() for p in layer["peers"]]} for layer in layers],
                      dtype="bf16")
    for l, (zr, xr) in enumerate(ref):
        assert rel_err(zs[l].t.index_select(0, ridx), zr) <= TOL_BF16, l
        assert rel_err(xs[l].t.index_select(0, ridx).float(), xr) <= TOL_BF16, l


def test_stack_equals_layer_by_layer_calls_bitwise():
    """GeLU, random bf16: the stack gives the same bits as one tp_colrow_mlp call
    per layer (the overlap changes the schedule, not the arithmetic)."""
    announce("stack vs single-layer calls, gelu")
    M, H, F, P, R = 2048, 512, 384, 4, 2
    X0 = inputs.normal((M, H), seed=1401, dtype="bf16")
    layers = [{"A_i": inputs.normal((H, F), seed=1410 + l, std=0.05, dtype="bf16"),
               "B_i": inputs.normal((F, H), seed=1420 + l, std=0.05, dtype="bf16"),
               "peers": [inputs.normal((M, H), seed=1430 + 10 * l + p) for p in range(P - 1)],
               "bias": inputs.normal((H,), seed=1450 + l)} for l in range(3)]
    got = run_stack(X0, layers, R=R, act=tp.TP_ACT_GELU_ERF)
    x = X0.cuda()
    for l, layer in enumerate(layers):
        Y = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
        Zi = torch.empty((M, H), device="cuda")
        Zo = torch.empty((M, H), device="cuda")
        xn = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
        tp.tp_colrow_mlp(x, layer["A_i"].cuda(), layer["B_i"].cuda(), Y, Zi, row_chunks=R,
                         peer_partials=[p.cuda() for p in layer["peers"]], Z_out=Zo, bias=layer["bias"].cuda(),
                         X_next=xn, s_reduce=torch.cuda.Stream())
        torch.cuda.synchronize()
        assert np.array_equal(bits(got[l][0]), bits(Zo.cpu())), l
        assert np.array_equal(bits(got[l][1]), bits(xn.cpu())), l
        x = xn
    ref = O.mlp_stack(X0, layers, dtype="bf16")
    assert rel_err(got[-1][0], ref[-1][0]) <= TOL_BF16


@pytest.mark.parametrize("R,keep_z", [(1, True), (2, True), (1, False)])
def test_stack_reduce_fusion_same_bits(R, keep_z):
    """Layers whose reduction runs in GEMM2's epilogue (every layer with one
    block; the last block of the last layer with two row chunks) give the bits
    of the separate reduction kernel, Z_out and the bf16 next input alike."""
    announce(f"stack reduce fusion R={R} keep_z={keep_z}")
    M, H, F, P = 1024, 384, 256, 4
    X0 = inputs.normal((M, H), seed=1701, dtype="bf16")
    layers = [{"A_i": inputs.normal((H, F), seed=1710 + l, std=0.05, dtype="bf16"),
               "B_i": inputs.normal((F, H), seed=1720 + l, std=0.05, dtype="bf16"),
               "peers": [inputs.normal((M, H), seed=1730 + 10 * l + p) for p in range(P - 1)],
               "bias": inputs.normal((H,), seed=1750 + l)} for l in range(2)]
    fused = run_stack(X0, layers, R=R, act=tp.TP_ACT_GELU_ERF, keep_z=keep_z)
    apart = run_stack(X0, layers, R=R, act=tp.TP_ACT_GELU_ERF, keep_z=keep_z, fusion=tp.TP_REDUCE_FUSION_OFF)
    for (z, xn), (zr, xr) in zip(fused, apart):
        if keep_z:
            assert np.array_equal(bits(z), bits(zr))
        assert np.array_equal(bits(xn), bits(xr))
    ref = O.mlp_stack(X0, layers, dtype="bf16")
    assert rel_err(fused[-1][1].float(), ref[-1][0]) <= TOL_BF16


def test_prepared_stack_replays():
    """The stack marshalled once (prepare=True) and replayed gives the direct call's bits."""
    announce("stack prepared call")
    M, H, F, P = 1024, 256, 192, 3
    X0 = inputs.normal((M, H), seed=1601, dtype="bf16")
    layers = [{"A_i": inputs.normal((H, F), seed=1610 + l, std=0.05, dtype="bf16"),
               "B_i": inputs.normal((F, H), seed=1620 + l, std=0.05, dtype="bf16"),
               "peers": [inputs.normal((M, H), seed=1630 + 10 * l + p) for p in range(P - 1)],
               "bias": inputs.normal((H,), seed=1650 + l)} for l in range(2)]
    ref = run_stack(X0, layers, R=2, act=tp.TP_ACT_GELU_ERF)
    got = run_stack(X0, layers, R=2, act=tp.TP_ACT_GELU_ERF, prepared=True)
    for (z, xn), (zr, xr) in zip(got, ref):
        assert np.array_equal(bits(z), bits(zr))
        assert np.array_equal(bits(xn), bits(xr))


def test_x_next_only_and_fp32():
    """Z_out omitted (X_next alone); and the fp32 path, whose X_next is an fp32 copy."""
    announce("stack X_next only; fp32 stack")
    M, H, F, P = 512, 256, 128, 2
    X0 = inputs.small_ints((M, H), seed=1501, lo=-4, hi=4, dtype="bf16")
    layers = _layers_integer(M, H, [F, F], P, 1600)
    got = run_stack(X0, layers, R=2, keep_z=False)
    ref = O.mlp_stack(X0, [dict(l, act=O.GELU_NONE) for l in layers], dtype="bf16")
    for (_, xn), (_, xr) in zip(got, ref):
        assert np.array_equal(bits(xn), bits(torch.from_numpy(xr).to(torch.bfloat16)))
    X0f = inputs.normal((64, 256), seed=1701)
    lf = [{"A_i": inputs.normal((256, 512), seed=1710 + l, std=1 / 16), "B_i": inputs.normal((512, 256), seed=1720 + l, std=1 / 32),
           "peers": [inputs.normal((64, 256), seed=1730 + l)], "bias": None} for l in range(2)]
    got = run_stack(X0f, lf, R=2, act=tp.TP_ACT_GELU_ERF)
    ref = O.mlp_stack(X0f, lf, dtype="f32")
    assert rel_err(got[-1][0], ref[-1][0]) <= 1e-5
    assert np.array_equal(bits(got[0][0]), bits(got[0][1]))    # the fp32 copy is the fp32 sum


def test_broken_link_leaves_outputs_untouched():
    announce("stack error path")
    M, H, F = 64, 32, 16
    X = torch.zeros((M, H), dtype=torch.bfloat16, device="cuda")
    A = torch.zeros((H, F), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((F, H), dtype=torch.bfloat16, device="cuda")
    Y = Guarded((M, F), torch.bfloat16)
    Z = Guarded((M, H), torch.float32)
    Xn = Guarded((M, H), torch.bfloat16)
    other = torch.zeros((M, H), dtype=torch.bfloat16, device="cuda")
    layers = [dict(X=X, A_i=A, B_i=B, Y_ws=Y.t, Z_i=Z.t, X_next=Xn.t),
              dict(X=other, A_i=A, B_i=B, Y_ws=Y.t, Z_i=Z.t)]
    with pytest.raises(tp.TpError) as e:
        tp.tp_colrow_mlp_stack(layers)
    assert e.value.kind == "arg"
    torch.cuda.synchronize()
    for g in (Y, Z, Xn):
        assert g.body_untouched() and g.guards_intact()
