"""tp_colrow_mlp_noalloc, the forward for callers that cannot allocate: the
same outputs, bit for bit, as tp_colrow_mlp given a Y workspace, on two calls
in a row (the second smaller, so it runs over the first call's leftovers in
the library's scratch), through the C ABI."""
import numpy as np
import pytest
import torch

import sharded_gemm_amd as tp
from sharded_gemm_amd import inputs

from gpu_helpers import Guarded, announce, bits, require_gpu

pytestmark = pytest.mark.gpu


def setup_module(_):
    require_gpu()


def _case(M, H, F, R, C, P, dtype, seed):
    dt = "bf16" if dtype == torch.bfloat16 else "f32"
    X = inputs.normal((M, H), seed, 1.0, dt).cuda()
    A = inputs.normal((H, F), seed + 1, 0.05, dt).cuda()
    B = inputs.normal((F, H), seed + 2, 0.05, dt).cuda()
    peers = [inputs.normal((M, H), seed + 10 + p).cuda() for p in range(P - 1)]
    bias = inputs.normal((H,), seed + 3).cuda()
    return X, A, B, peers, bias


def _run(noalloc, X, A, B, peers, bias, R, C, two):
    M, H = X.shape
    F = A.shape[1]
    Z = Guarded((M, H), torch.float32)
    Zo = Guarded((M, H), torch.float32)
    Xn = Guarded((M, H), X.dtype)
    Hs = Guarded((M, F), X.dtype)
    s0 = torch.cuda.current_stream()
    s1 = torch.cuda.Stream() if two else s0
    kw = dict(row_chunks=R, col_chunks=C, peer_partials=peers, Z_out=Zo.t if peers else None,
              bias=bias if peers else None, X_next=Xn.t if peers else None, H_out=Hs.t, s_compute=s0, s_reduce=s1)
    if noalloc:
        tp.tp_colrow_mlp_noalloc(X, A, B, Z.t, **kw)
    else:
        Y = torch.empty((M, F), dtype=X.dtype, device="cuda")
        tp.tp_colrow_mlp(X, A, B, Y, Z.t, **kw)
    torch.cuda.synchronize()
    for g in (Z, Zo, Xn, Hs):
        assert g.guards_intact()
    return [g.t.cpu() for g in (Z, Zo, Xn, Hs)]


@pytest.mark.parametrize("first,second", [
    # bf16: two row chunks and two column blocks on two streams, then a single
    # block (the sum in GEMM2's epilogue) with fewer rows and columns
    ((1024, 512, 384, 2, 2, 3, torch.bfloat16, True), (256, 256, 128, 1, 1, 2, torch.bfloat16, True)),
    # the 175B row chunk's full Y (2048 x 6144 bf16, 24 MiB), then a ragged tile shape
    ((4096, 1024, 6144, 2, 1, 2, torch.bfloat16, True), (300, 264, 136, 3, 2, 2, torch.bfloat16, False)),
    # fp32 (the tiny workload's kernels), serial schedule
    ((512, 256, 512, 2, 1, 2, torch.float32, False), (64, 256, 512, 1, 1, 2, torch.float32, False)),
])
def test_noalloc_matches_workspace_entry_point(first, second):
    for k, (M, H, F, R, C, P, dtype, two) in enumerate((first, second)):
        announce(f"noalloc call {k}: M={M} H={H} F={F} R={R} C={C} P={P} {dtype} two={two}")
        X, A, B, peers, bias = _case(M, H, F, R, C, P, dtype, 4000 + 100 * k)
        ref = _run(False, X, A, B, peers, bias, R, C, two)
        got = _run(True, X, A, B, peers, bias, R, C, two)
        for name, a, b in zip(("Z_i", "Z_out", "X_next", "H_out"), got, ref):
            assert np.array_equal(bits(a), bits(b)), name


def test_noalloc_rejects_what_does_not_fit():
    """A row chunk of Y beyond the 32 MiB scratch, and a Y workspace passed in,
    are refused before anything is enqueued."""
    announce("noalloc rejections")
    M, H, F = 4096, 256, 8192          # 4096 x 8192 bf16 = 64 MiB in one chunk
    X = torch.zeros((M, H), dtype=torch.bfloat16, device="cuda")
    A = torch.zeros((H, F), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((F, H), dtype=torch.bfloat16, device="cuda")
    Z = Guarded((M, H), torch.float32)
    with pytest.raises(tp.TpError) as e:
        tp.tp_colrow_mlp_noalloc(X, A, B, Z.t)
    assert e.value.kind == "unsupported"
    tp.tp_colrow_mlp_noalloc(X, A, B, Z.t, row_chunks=2)   # 32 MiB per chunk: fits
    torch.cuda.synchronize()
    assert Z.guards_intact() and bool((Z.t == 0).all())
    from sharded_gemm_amd import _abi
    import ctypes as C
    args, keep = _abi._mlp_args(X, A, B, torch.empty((M, F), dtype=torch.bfloat16, device="cuda"), Z.t)
    assert _abi.load().tp_colrow_mlp_noalloc(C.byref(args), None, None) == _abi.TP_ERR_ARG
