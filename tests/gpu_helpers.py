"""Shared helpers of the GPU parity tests: canary-guarded buffers, oracle
comparison and seeded case names."""
import os
import sys

import numpy as np
import pytest
import torch

GUARD = 1024            # elements of sentinel before and after every output
SENTINEL_F32 = 0x7FC0DEAD
SENTINEL_BF16 = 0x7FC1


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sharded_gemm_amd import _abi
    if not os.path.exists(_abi.LIB_PATH):
        from sharded_gemm_amd import build
        build.build()
    _abi.load()


def announce(msg: str):
    """Name the case on stdout before a GPU step, so a crash log says which one."""
    sys.stdout.write(f"\n[case] {msg}\n")
    sys.stdout.flush()


class Guarded:
    """A device tensor of `shape` with sentinel bands on both sides."""

    def __init__(self, shape, dtype, device="cuda"):
        n = int(np.prod(shape)) if len(shape) else 1
        self.n = n
        self.shape = tuple(shape)
        self.dtype = dtype
        if dtype == torch.float32:
            self.base = torch.empty(n + 2 * GUARD, dtype=torch.int32, device=device)
            self.base.fill_(SENTINEL_F32)
            self.base = self.base.view(torch.float32)
        else:
            self.base = torch.empty(n + 2 * GUARD, dtype=torch.int16, device=device)
            self.base.fill_(SENTINEL_BF16)
            self.base = self.base.view(torch.bfloat16)
        self.t = self.base[GUARD:GUARD + n].view(self.shape)

    def fill_sentinel(self):
        ib = self.base.view(torch.int32 if self.dtype == torch.float32 else torch.int16)
        ib.fill_(SENTINEL_F32 if self.dtype == torch.float32 else SENTINEL_BF16)

    def guards_intact(self) -> bool:
        ib = self.base.view(torch.int32 if self.dtype == torch.float32 else torch.int16)
        s = SENTINEL_F32 if self.dtype == torch.float32 else SENTINEL_BF16
        head = ib[:GUARD]
        tail = ib[GUARD + self.n:]
        return bool((head == s).all().item()) and bool((tail == s).all().item())

    def body_untouched(self) -> bool:
        ib = self.base.view(torch.int32 if self.dtype == torch.float32 else torch.int16)
        s = SENTINEL_F32 if self.dtype == torch.float32 else SENTINEL_BF16
        return bool((ib[GUARD:GUARD + self.n] == s).all().item())


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit pattern of a CPU copy (bit-exact comparisons)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy()
    return t.numpy()


def rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| (the tolerance measure of the parity bar)."""
    g = got.detach().cpu().double().numpy() if isinstance(got, torch.Tensor) else np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    denom = np.max(np.abs(r)) if r.size else 0.0
    if denom == 0.0:
        return float(np.max(np.abs(g))) if g.size else 0.0
    return float(np.max(np.abs(g - r)) / denom)
