"""Seeded synthetic inputs shared by the tests, the bench and the oracle's callers.

This module only draws numbers; it holds none of the method's arithmetic.
Every tensor comes from a fresh CPU ``torch.Generator`` seeded with an integer,
so the same bytes can be fed to the CPU oracle and copied to the GPU.

Seed convention (per workload ``cfg`` = 1..5): ``seed = 1000 * cfg + slot`` with
slots X = 1, full A = 2, full B = 3, layout source = 4, A_i = 10 + i,
B_i = 30 + i, partial_p = 50 + p.
"""
from __future__ import annotations

import torch

SLOT_X = 1
SLOT_A = 2
SLOT_B = 3
SLOT_LAYOUT = 4
SLOT_A_SHARD = 10
SLOT_B_SHARD = 30
SLOT_PARTIAL = 50
SLOT_DZ = 5            # the output gradient of the backward workloads

_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def seed_for(cfg: int, slot: int) -> int:
    return 1000 * int(cfg) + int(slot)


def _gen(seed: int, device: str = "cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, seed: int, std: float = 1.0, dtype: str = "f32", device: str = "cpu") -> torch.Tensor:
    """N(0, std^2) samples drawn in fp32, then rounded (RNE) to ``dtype``.

    ``device="cuda"`` draws with torch's GPU generator (different numbers for
    the same seed, still deterministic); used only for large inputs whose CPU
    draw would be slow.  Copy the result to the host to feed the oracle the
    same bytes.
    """
    t = torch.randn(tuple(shape), generator=_gen(seed, device), dtype=torch.float32, device=device)
    if std != 1.0:
        t.mul_(float(std))
    return t.to(_DTYPES[dtype]).contiguous()


def small_ints(shape, seed: int, lo: int, hi: int, dtype: str = "f32") -> torch.Tensor:
    """Integers uniform in [lo, hi], stored as ``dtype`` (exact in bf16 for |v| <= 256)."""
    t = torch.randint(int(lo), int(hi) + 1, tuple(shape), generator=_gen(seed), dtype=torch.int64)
    return t.to(_DTYPES[dtype]).contiguous()


def arange_tensor(shape, dtype: str = "f32") -> torch.Tensor:
    """1, 2, 3, ... in row-major order (exact for small sizes); used for layout cases."""
    n = 1
    for d in shape:
        n *= int(d)
    return torch.arange(1, n + 1, dtype=torch.float64).reshape(tuple(shape)).to(_DTYPES[dtype]).contiguous()
