#!/usr/bin/env python3
"""Throughput of one rank's tensor-parallel MLP share and its layout kernels
on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-extras]
                    [--no-cpu-baseline]

A step is one pass of the whole hot path over one batch of synthetic input.
The headline workload is the GPT-3 175B per-rank MLP at TP = 8 with the
Domino 2D split (X in 2 row chunks, B_i in 2 column blocks): GEMM1 + GeLU
(over both row chunks in one launch where the library so schedules it), GEMM2
per block into the fp32 partial, and each block's 8-way partial sum on a
second stream beside the next block's GEMM2, the last block's in its GEMM2's
epilogue.  The value is
per-rank MLP TFLOP/s (2 GEMMs of 2*M*H*F flops) over K consecutive steps,
timed as eager launches, as K replays of a one-step HIP graph and as one
replay of a graph holding the K steps (the fastest counts, named in
"timed_as"; the last removes the host's per-step launch cost from steps
shorter than it).

Besides that, every workload reports per-step medians with p10/p90, warm
(steps back to back) and cold (512 MiB written between steps, so nothing of
the step's inputs is left in L2 or the MALL), the serial schedule's makespan
next to the two-stream one, and each kernel's rate from HIP events the
library records around its launches, as a fraction of its roofline.  The
other four workloads (tiny fp32, GPT-2 small, GPT-3 6.7B, the reshard) follow
under "configs" unless --no-extras.  The CPU oracle is timed on a row sample,
with all threads and with one.

Prints one JSON line (last line of stdout).
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import platform
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import sharded_gemm_amd as tp  # noqa: E402
from sharded_gemm_amd import _abi, inputs  # noqa: E402
from sharded_gemm_amd.workloads import (GPT2_SMALL, GPT3_175B, GPT3_6P7B, RESHARD, TINY,  # noqa: E402
                                        TINY_LAYOUT_SPECS)

METRIC = "per-rank TP-MLP TFLOP/s (% bf16 MFMA peak) + shard/reduce GB/s (% HBM)"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
# GEMM2 with the reduction in its epilogue moves far more bytes than its flops
# need time for (GPT-2 shape: about 70 MB against 4.8 GFLOP), so the library
# counts its work in bytes and it is priced against HBM.
BYTE_KERNELS = ("gemm2_reduce", "gemm_dgrad_reduce")


def log(msg):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


# --------------------------------------------------------------------------- workloads

# With --profile the peers' partials are drawn (seeded N(0,1)) instead of
# computed by the same path, so that a kernel trace of the run holds no GEMM
# launched outside the timed schedule.  The sums then mean nothing; the timing
# is the same (the kernels do not look at the values).
DRAWN_PEERS = False


def _peer(w, p, dev="cuda"):
    return inputs.normal((w.M, w.H), inputs.seed_for(w.cfg, inputs.SLOT_PARTIAL + p), 1.0, "f32", dev)


def _device_boxes(shape, spec):
    """{device: box} of a layout, from the library's host-only planner."""
    n, boxes, sod = tp.tp_layout_plan(shape, spec, num_dst=16)
    return {d: boxes[k] for d, k in enumerate(sod) if k >= 0}


class MlpStep:
    """Per-rank MLP step, optionally preceded by cutting the weights.  With
    ``seq`` the step is the sequence-parallel form: the input arrives as P
    sequence blocks that GEMM1 reads where they lie (or, with gather_input,
    that the call first all-gathers into X), and the output is
    reduce-scattered into P blocks."""

    serial = False
    reduce_wgs = 0
    reduce_fusion = tp.TP_REDUCE_FUSION_AUTO
    # The row-parallel all-reduce works in place on the partial output, as
    # torch.distributed.all_reduce does; separate_output keeps Z_i and writes
    # the sum to its own buffer instead.
    separate_output = False
    # Sequence parallel: all-gather the blocks into X before GEMM1 instead of
    # letting GEMM1 read them where they lie.
    gather_input = False
    # With full weights: rank 0 reads its column shard of A in place (a row
    # stride of P*F) and its row shard of B (contiguous rows), as the
    # column-parallel layer uses its shard; cut_weights copies both out of the
    # full weights at every step instead (one batched layout launch).
    cut_weights = False
    # Rank 0's weights in a linear layer's [out, in] layout (the same values,
    # transposed once at set-up): A_i^T [F, H] and B_i^T [H, F], with full
    # weights their row / column slices read in place.
    weights_linear = False

    def __init__(self, w, split_weights: bool, seq: bool = False):
        self.w = w
        self.seq = seq
        dev = "cuda"
        dt = "bf16" if w.dtype == "bf16" else "f32"
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        gen_dev = "cuda" if w.cfg in (3, 5) else "cpu"
        self.X = inputs.normal((w.M, w.H), inputs.seed_for(w.cfg, inputs.SLOT_X), w.std_x, dt, gen_dev).to(dev)
        self.split = split_weights
        if split_weights:
            self.A = inputs.normal((w.H, w.P * w.F), inputs.seed_for(w.cfg, inputs.SLOT_A), w.std_a, dt).to(dev)
            self.B = inputs.normal((w.P * w.F, w.H), inputs.seed_for(w.cfg, inputs.SLOT_B), w.std_b, dt).to(dev)
            self.sa = {"device": list(range(w.P)), "sharded_dim": [{"axis": 1, "num_shards": w.P}]}
            self.sb = {"device": list(range(w.P)), "sharded_dim": [{"axis": 0, "num_shards": w.P}]}
            self.As = {d: torch.empty((w.H, w.F), dtype=tdt, device=dev) for d in range(w.P)}
            self.Bs = {d: torch.empty((w.F, w.H), dtype=tdt, device=dev) for d in range(w.P)}
            tp.tp_shard_materialize(self.A, self.sa, self.As)
            tp.tp_shard_materialize(self.B, self.sb, self.Bs)
        else:
            self.As = {i: inputs.normal((w.H, w.F), inputs.seed_for(w.cfg, inputs.SLOT_A_SHARD + i), w.std_a, dt,
                                        gen_dev).to(dev) for i in range(w.P)}
            self.Bs = {i: inputs.normal((w.F, w.H), inputs.seed_for(w.cfg, inputs.SLOT_B_SHARD + i), w.std_b, dt,
                                        gen_dev).to(dev) for i in range(w.P)}
        self.Y = torch.empty((w.M, w.F), dtype=tdt, device=dev)
        self.Z = torch.empty((w.M, w.H), device=dev)
        self.Zo = torch.empty((w.M, w.H), device=dev)
        # peers' partials: computed once, untimed, by the same path
        self.peers = []
        for i in range(1, w.P):
            if DRAWN_PEERS:
                self.peers.append(_peer(w, i))
                continue
            z = torch.empty((w.M, w.H), device=dev)
            tp.tp_colrow_mlp(self.X, self.As[i], self.Bs[i], self.Y, z, row_chunks=w.R, col_chunks=w.C)
            self.peers.append(z)
        if seq:
            # every rank's sequence block as its own buffer; X becomes the gather workspace
            self.Xb = [b.clone() for b in torch.chunk(self.X, w.P)]
            self.Zs = [torch.empty((w.M // w.P, w.H), device=dev) for _ in range(w.P)]
        # The tiny workload's step also cuts the 2 x 2 tensor of the ShardingSpec
        # examples (axis 0, axis 1, both axes, broadcast, split + broadcast).
        self.layouts = None
        if w.cfg == 1:
            src = inputs.arange_tensor((2, 2)).to(dev)
            self.layouts = [(src, spec, {d: torch.empty(tuple(b - a for a, b in box), device=dev)
                                         for d, box in _device_boxes((2, 2), spec).items()})
                            for spec in TINY_LAYOUT_SPECS.values()]
        torch.cuda.synchronize()
        self.s0 = torch.cuda.Stream()     # a side stream: graph capture needs one
        self.s1 = torch.cuda.Stream()

    def _z_out(self):
        return self.Zo if self.separate_output else self.Z

    def result(self):
        return self.Zs[-1] if self.seq else self._z_out()

    def prepare(self):
        """Marshal the step's library calls once (the buffers never move)."""
        self.cut = None
        self.cut_layouts = None
        if self.layouts:
            self.cut_layouts = tp.tp_shard_materialize_batch(self.layouts, stream=self.s0, prepare=True)
        A0, B0 = self.As[0], self.Bs[0]
        if self.split and self.cut_weights:
            # rank 0's column shard of A and row shard of B in one batched call
            # (one launch): each rank materialises its own share
            self.cut = tp.tp_shard_materialize_batch([(self.A, self.sa, {0: self.As[0]}, 0),
                                                      (self.B, self.sb, {0: self.Bs[0]}, 0)],
                                                     stream=self.s0, prepare=True)
        elif self.split:
            A0, B0 = self.A[:, :self.w.F], self.B[:self.w.F]
        layout = tp.TP_WEIGHTS_MATH
        if self.weights_linear:
            if self.cut_weights:
                raise ValueError("--weights linear reads the shards in place; it does not combine with --cut-weights")
            layout = tp.TP_WEIGHTS_LINEAR
            if self.split:
                self.W1, self.W2 = self.A.t().contiguous(), self.B.t().contiguous()   # [P*F, H], [H, P*F]
                A0, B0 = self.W1[:self.w.F], self.W2[:, :self.w.F]
            else:
                A0, B0 = A0.t().contiguous(), B0.t().contiguous()
            torch.cuda.synchronize()
        X = None if (self.seq and not self.gather_input) else self.X
        self.mlp = tp.tp_colrow_mlp(X, A0, B0, self.Y, self.Z, row_chunks=self.w.R,
                                    col_chunks=self.w.C, peer_partials=self.peers,
                                    Z_out=None if self.seq else self._z_out(), s_compute=self.s0,
                                    s_reduce=self.s0 if self.serial else self.s1,
                                    reduce_workgroups=self.reduce_wgs, X_shards=self.Xb if self.seq else None,
                                    Z_split=self.Zs if self.seq else None, reduce_fusion=self.reduce_fusion,
                                    weight_layout=layout, prepare=True)

    def step(self):
        if self.cut_layouts is not None:
            self.cut_layouts()
        if self.cut is not None:
            self.cut()
        self.mlp()

    @property
    def work(self):
        return float(self.w.flops_per_rank)

    unit = "TFLOP/s"

    def config(self):
        w = self.w
        cfg = {"workload": w.name + ("-sp" if self.seq else ""), "tokens": w.M, "hidden": w.H, "ffn_per_rank": w.F,
               "tp": w.P, "row_chunks": w.R, "col_chunks": w.C,
               "weights": (("rank 0's shards of A and B copied out of the full weights each step" if self.cut_weights
                            else "rank 0's shards read in place: A's column slice with a row stride of P*F, B's row "
                                 "slice") if self.split else "per-rank shards drawn as such")
                          + (", stored [out, in] as a linear layer's (A_i^T [F, H], B_i^T [H, F])"
                             if self.weights_linear else ""),
               "reduce_stream": "compute" if self.serial else "second",
               "reduce_fusion": "auto" if self.reduce_fusion == tp.TP_REDUCE_FUSION_AUTO else "off",
               "reduce_output": ("reduce-scattered blocks" if self.seq else
                                 "separate buffer" if self.separate_output else "in place over the partial (all-reduce)"),
               "peers": "virtual ranks 1..P-1, partials precomputed by the same path"}
        if self.seq:
            cfg["sequence_parallel"] = {"blocks": w.P,
                                        "input": "all-gathered from P sequence blocks" if self.gather_input else
                                                 "read by GEMM1 from the P sequence blocks where they lie",
                                        "output": "reduce-scattered into P sequence blocks"}
        if self.layouts:
            cfg["layouts_cut_each_step"] = "the 2 x 2 tensor under the " + ", ".join(TINY_LAYOUT_SPECS) + " specs"
        return cfg

    def cpu_baseline(self, budget_s, rows=None):
        """The oracle on this step (sampled rows for the large shapes), fp64."""
        from threadpoolctl import threadpool_info
        from oracle import layout as L
        from oracle import mlp as O
        from oracle import reduce as R
        w = self.w
        Xc = self.X.cpu()
        A0, B0 = self.As[0].cpu(), self.Bs[0].cpu()
        if rows is None:
            rows = w.M if w.M * w.H * w.F <= 4096 * 768 * 768 else 256
        sample_rows = np.linspace(0, w.M - 1, rows).astype(np.int64)
        peers = [inputs.normal((rows, w.H), 99000 + p) for p in range(w.P - 1)]
        Ac = self.A.cpu() if self.split else None
        Bc = self.B.cpu() if self.split else None
        gspec = {"device": list(range(w.P)), "sharded_dim": [{"axis": 0, "num_shards": w.P}]}
        xblocks = dict(enumerate(np.split(Xc[sample_rows].float().numpy(), w.P))) if self.seq else None
        reps, t0 = 0, time.perf_counter()
        while True:
            if self.layouts:
                for src, spec, _ in self.layouts:
                    L.split(src.cpu(), spec)
            if self.split and self.cut_weights:
                L.split(Ac, self.sa)
                L.split(Bc, self.sb)
            if self.seq:
                L.gather(xblocks, (rows, w.H), gspec)
            z = O.mlp_rank_rows(Xc, A0, B0, sample_rows)
            if self.seq:
                R.reduce_split([z] + peers, w.P)
            else:
                R.reduce_full([z] + peers)
            reps += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = (time.perf_counter() - t0) / reps
        flops = 4.0 * rows * w.H * w.F
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
        return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
                "sample": (f"{rows} of {w.M} token rows of the per-rank MLP (fp64, numpy's BLAS), "
                           f"{'plus cutting the full weights into the shards of every rank (the oracle has no one-device form), ' if self.split and self.cut_weights else ''}"
                           f"{'plus the all-gather of those rows from P blocks, ' if self.seq else ''}"
                           f"plus the {w.P}-way partial sum of those rows; {reps} repetitions, "
                           f"{dt * 1e3:.1f} ms each; host {platform.processor() or platform.machine()}, "
                           f"os.cpu_count()={os.cpu_count()}")}


class BwdStep:
    """Backward of one rank's MLP share (dH, dX with its reduce over the ranks
    on the second stream, dA, dB), for the per-rank shape of an MLP workload."""

    serial = False
    reduce_wgs = 0
    reduce_fusion = tp.TP_REDUCE_FUSION_AUTO
    separate_output = False   # as in MlpStep: the input gradient's sum goes in place by default
    weights_linear = False    # as in MlpStep: rank 0's weights (and their gradients) stored [out, in]

    def __init__(self, w, seq: bool = False):
        self.w = w
        self.seq = seq
        dev = "cuda"
        dt = "bf16" if w.dtype == "bf16" else "f32"
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        gen_dev = "cuda" if w.cfg in (3, 5) else "cpu"
        self.X = inputs.normal((w.M, w.H), inputs.seed_for(w.cfg, inputs.SLOT_X), w.std_x, dt, gen_dev).to(dev)
        self.dZ = inputs.normal((w.M, w.H), inputs.seed_for(w.cfg, inputs.SLOT_DZ), 1.0, dt, gen_dev).to(dev)
        self.As = [inputs.normal((w.H, w.F), inputs.seed_for(w.cfg, inputs.SLOT_A_SHARD + i), w.std_a, dt,
                                 gen_dev).to(dev) for i in range(w.P)]
        self.Bs = [inputs.normal((w.F, w.H), inputs.seed_for(w.cfg, inputs.SLOT_B_SHARD + i), w.std_b, dt,
                                 gen_dev).to(dev) for i in range(w.P)]
        z = torch.empty((w.M, w.H), device=dev)
        self.Y = torch.empty((w.M, w.F), dtype=tdt, device=dev)
        self.Hs = torch.empty((w.M, w.F), dtype=tdt, device=dev)
        self.dH = torch.empty((w.M, w.F), dtype=tdt, device=dev)
        self.dX = torch.empty((w.M, w.H), device=dev)
        self.dXo = torch.empty((w.M, w.H), device=dev)
        self.dA = torch.empty((w.H, w.F), device=dev)
        self.dB = torch.empty((w.F, w.H), device=dev)
        # peers' input-gradient partials: their forward and backward, once, untimed, by the same path
        self.peers = []
        for i in range(1, w.P):
            if DRAWN_PEERS:
                self.peers.append(_peer(w, i))
                continue
            tp.tp_colrow_mlp(self.X, self.As[i], self.Bs[i], self.Y, z, row_chunks=w.R, H_out=self.Hs)
            dx = torch.empty((w.M, w.H), device=dev)
            tp.tp_colrow_mlp_backward(self.X, self.As[i], self.Bs[i], self.Hs, self.Y, self.dZ, self.dH, dx,
                                      self.dA, self.dB, row_chunks=w.R)
            self.peers.append(dx)
        tp.tp_colrow_mlp(self.X, self.As[0], self.Bs[0], self.Y, z, row_chunks=w.R, H_out=self.Hs)
        if seq:
            # dZ arrives as P sequence blocks (dZ becomes the gather workspace); dX leaves as P blocks
            self.dZb = [b.clone() for b in torch.chunk(self.dZ, w.P)]
            self.dXs = [torch.empty((w.M // w.P, w.H), device=dev) for _ in range(w.P)]
        torch.cuda.synchronize()
        self.s0 = torch.cuda.Stream()
        self.s1 = torch.cuda.Stream()

    def result(self):
        return self.dA

    def prepare(self):
        """Marshal the step's library call once (the buffers never move)."""
        A0, B0, layout = self.As[0], self.Bs[0], tp.TP_WEIGHTS_MATH
        if self.weights_linear:
            A0, B0, layout = A0.t().contiguous(), B0.t().contiguous(), tp.TP_WEIGHTS_LINEAR
            self.dA = torch.empty((self.w.F, self.w.H), device="cuda")
            self.dB = torch.empty((self.w.H, self.w.F), device="cuda")
            torch.cuda.synchronize()
        self.call = tp.tp_colrow_mlp_backward(
            self.X, A0, B0, self.Hs, self.Y, self.dZ, self.dH, self.dX, self.dA, self.dB,
            row_chunks=self.w.R, peer_dX=self.peers, weight_layout=layout,
            dX_out=None if self.seq else (self.dXo if self.separate_output else self.dX), s_compute=self.s0,
            s_reduce=self.s0 if self.serial else self.s1, reduce_workgroups=self.reduce_wgs,
            dZ_shards=self.dZb if self.seq else None, dX_split=self.dXs if self.seq else None,
            reduce_fusion=self.reduce_fusion, prepare=True)

    def step(self):
        self.call()

    @property
    def work(self):
        return 2.0 * self.w.flops_per_rank      # four GEMMs of 2 M H F each

    unit = "TFLOP/s"

    def config(self):
        w = self.w
        cfg = {"workload": w.name + ("-sp" if self.seq else "") + "-bwd", "pass": "backward", "tokens": w.M,
               "hidden": w.H, "ffn_per_rank": w.F, "tp": w.P, "row_chunks": w.R,
               "reduce_stream": "compute" if self.serial else "second",
               "reduce_fusion": "auto" if self.reduce_fusion == tp.TP_REDUCE_FUSION_AUTO else "off",
               "reduce_output": ("reduce-scattered blocks" if self.seq else
                                 "separate buffer" if self.separate_output else "in place over the partial (all-reduce)"),
               "peers": "virtual ranks 1..P-1, input-gradient partials precomputed by the same path"}
        if self.weights_linear:
            cfg["weights"] = "stored [out, in] as a linear layer's (A_i^T [F, H], B_i^T [H, F]), gradients likewise"
        if self.seq:
            cfg["sequence_parallel"] = {"blocks": w.P, "output_gradient": "all-gathered from P sequence blocks",
                                        "input_gradient": "reduce-scattered into P sequence blocks"}
        return cfg

    def cpu_baseline(self, budget_s):
        """The oracle's backward on a row sample (dH, dX of those rows and their
        contributions to dA, dB), fp64."""
        from threadpoolctl import threadpool_info
        from oracle import mlp as O
        from oracle import reduce as R
        w = self.w
        rows = w.M if w.M * w.H * w.F <= 4096 * 768 * 768 else 256
        sample_rows = np.linspace(0, w.M - 1, rows).astype(np.int64)
        Xs, dZs = self.X.cpu()[sample_rows], self.dZ.cpu()[sample_rows]
        A0, B0 = self.As[0].cpu(), self.Bs[0].cpu()
        peers = [inputs.normal((rows, w.H), 98000 + p) for p in range(w.P - 1)]
        reps, t0 = 0, time.perf_counter()
        while True:
            g = O.backward_rank(Xs, A0, B0, dZs)
            R.reduce_full([g["dX_i"]] + peers)
            reps += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = (time.perf_counter() - t0) / reps
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
        return {"value": 8.0 * rows * w.H * w.F / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
                "sample": (f"{rows} of {w.M} token rows of the per-rank MLP backward (fp64, numpy BLAS: "
                           f"dH, dX and those rows' share of dA and dB), plus the {w.P}-way sum of dX; "
                           f"{reps} repetitions, {dt * 1e3:.1f} ms each; host "
                           f"{platform.processor() or platform.machine()}, os.cpu_count()={os.cpu_count()}")}


class StackStep:
    """Two forward layers of an MLP workload's per-rank shape chained with
    tp_colrow_mlp_stack: layer 2 reads layer 1's reduced output (rounded to
    bf16 by the reduce), and layer 1's later row chunks reduce beside layer
    2's earlier GEMMs (the inter-layer overlap)."""

    serial = False
    reduce_wgs = 0
    reduce_fusion = tp.TP_REDUCE_FUSION_AUTO
    L = 2

    def __init__(self, w):
        self.w = w
        dev = "cuda"
        gen_dev = "cuda" if w.cfg in (3, 5) else "cpu"
        self.X = inputs.normal((w.M, w.H), inputs.seed_for(w.cfg, inputs.SLOT_X), w.std_x, "bf16", gen_dev).to(dev)
        self.layers = []
        self.Y = torch.empty((w.M, w.F), dtype=torch.bfloat16, device=dev)
        self.Z = torch.empty((w.M, w.H), device=dev)
        x = self.X
        for l in range(self.L):
            As = [inputs.normal((w.H, w.F), inputs.seed_for(w.cfg, inputs.SLOT_A_SHARD + i) + 7919 * l, w.std_a,
                                "bf16", gen_dev).to(dev) for i in range(w.P)]
            Bs = [inputs.normal((w.F, w.H), inputs.seed_for(w.cfg, inputs.SLOT_B_SHARD + i) + 7919 * l, w.std_b,
                                "bf16", gen_dev).to(dev) for i in range(w.P)]
            # peers' partials of this layer's input: computed once, untimed, by the same path
            peers = []
            for i in range(1, w.P):
                if DRAWN_PEERS:
                    peers.append(_peer(w, i + 100 * l))
                    continue
                z = torch.empty((w.M, w.H), device=dev)
                tp.tp_colrow_mlp(x, As[i], Bs[i], self.Y, z, row_chunks=w.R)
                peers.append(z)
            xn = torch.empty((w.M, w.H), dtype=torch.bfloat16, device=dev)
            zo = torch.empty((w.M, w.H), device=dev)
            if DRAWN_PEERS:
                xn.copy_(inputs.normal((w.M, w.H), inputs.seed_for(w.cfg, inputs.SLOT_X) + 7919 * (l + 1), 1.0, "bf16",
                                       dev))
            else:
                tp.tp_colrow_mlp(x, As[0], Bs[0], self.Y, self.Z, row_chunks=w.R, peer_partials=peers, Z_out=zo,
                                 X_next=xn)
            self.layers.append(dict(X=x, A_i=As[0], B_i=Bs[0], Y_ws=self.Y, Z_i=self.Z, row_chunks=w.R, col_chunks=w.C,
                                    peer_partials=peers, Z_out=zo, X_next=xn))
            x = xn
        torch.cuda.synchronize()
        self.s0 = torch.cuda.Stream()
        self.s1 = torch.cuda.Stream()

    def result(self):
        return self.layers[-1]["Z_out"]

    def prepare(self):
        """Marshal the step's library call once (the buffers never move)."""
        self.call = tp.tp_colrow_mlp_stack([dict(l, reduce_workgroups=self.reduce_wgs, reduce_fusion=self.reduce_fusion)
                                            for l in self.layers],
                                           s_compute=self.s0, s_reduce=self.s0 if self.serial else self.s1,
                                           prepare=True)

    def step(self):
        self.call()

    @property
    def work(self):
        return float(self.L * self.w.flops_per_rank)

    unit = "TFLOP/s"

    def config(self):
        w = self.w
        return {"workload": f"{w.name}-{self.L}layer", "layers": self.L, "tokens": w.M, "hidden": w.H,
                "ffn_per_rank": w.F, "tp": w.P, "row_chunks": w.R, "col_chunks": w.C,
                "reduce_stream": "compute" if self.serial else "second",
                "overlap": "inter-layer (layer l+1 chunk r waits only for layer l chunk r)",
                "peers": "virtual ranks 1..P-1, partials of each layer's input precomputed by the same path"}

    def cpu_baseline(self, budget_s):
        """The oracle's stack on a row sample (rows are independent through the stack)."""
        from threadpoolctl import threadpool_info
        from oracle import mlp as O
        w = self.w
        rows = 256
        sample_rows = np.linspace(0, w.M - 1, rows).astype(np.int64)
        idx = torch.from_numpy(sample_rows).cuda()
        layers = [{"A_i": l["A_i"].cpu(), "B_i": l["B_i"].cpu(),
                   "peers": [p.index_select(0, idx).cpu() for p in l["peer_partials"]]} for l in self.layers]
        Xs = self.X.index_select(0, idx).cpu()
        reps, t0 = 0, time.perf_counter()
        while True:
            O.mlp_stack(Xs, layers)
            reps += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = (time.perf_counter() - t0) / reps
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
        return {"value": self.L * 4.0 * rows * w.H * w.F / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
                "kind": "oracle",
                "sample": (f"{rows} of {w.M} token rows through the {self.L}-layer stack (fp64, numpy BLAS), with "
                           f"the {w.P}-way sums; {reps} repetitions, {dt * 1e3:.1f} ms each")}


class ReshardStep:
    """The 2x4-mesh layout workload: fused split+replicate, then split reduce."""

    def __init__(self, w):
        self.w = w
        self.src = inputs.normal(w.src_shape, inputs.seed_for(4, inputs.SLOT_LAYOUT), device="cuda")
        self.spec = {"device": [-(k + 1) for k in range(8)],
                     "device_map": {-(k + 1): [2 * k, 2 * k + 1] for k in range(8)},
                     "sharded_dim": [{"axis": 0, "num_shards": 2}, {"axis": 2, "num_shards": 4}]}
        self.dst = {d: torch.empty((4, 2048, 2048), device="cuda") for d in range(16)}
        self.parts = [inputs.normal(w.partial_shape, inputs.seed_for(4, inputs.SLOT_PARTIAL + p), device="cuda")
                      for p in range(w.num_partials)]
        rows = w.partial_shape[0] // w.num_splits
        self.outs = [torch.empty((rows, w.partial_shape[1]), device="cuda") for _ in range(w.num_splits)]
        torch.cuda.synchronize()
        self.s0 = torch.cuda.Stream()

    def result(self):
        return self.outs[-1]

    def step(self):
        tp.tp_shard_materialize(self.src, self.spec, self.dst, stream=self.s0)
        tp.tp_partial_reduce(self.parts, self.outs, tp.TP_REDUCE_SPLIT, stream=self.s0)

    @property
    def work(self):
        src = self.src.numel() * 4
        parts = sum(p.numel() for p in self.parts) * 4
        return float(src + 2 * src + parts + parts / self.w.num_partials)

    unit = "GB/s"

    def config(self):
        w = self.w
        return {"workload": w.name, "src_shape": list(w.src_shape), "mesh": list(w.mesh_shape),
                "dims_mapping": list(w.dims_mapping), "replicas": w.group_size,
                "partials": w.num_partials, "partial_shape": list(w.partial_shape), "splits": w.num_splits}

    def cpu_baseline(self, budget_s):
        from oracle import layout as L
        from oracle import reduce as R
        w = self.w
        rows = 256   # a row sample of every tensor (the full 2.5 GiB would take minutes)
        src = self.src[:, :rows // 8].cpu()
        parts = [p[:rows].cpu() for p in self.parts]
        spec = {"device": self.spec["device"], "device_map": self.spec["device_map"],
                "sharded_dim": self.spec["sharded_dim"]}
        reps, t0 = 0, time.perf_counter()
        while True:
            L.split(src, spec)
            R.reduce_split(parts, w.num_splits)
            reps += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = (time.perf_counter() - t0) / reps
        nbytes = src.numel() * 4 * 3 + sum(p.numel() for p in parts) * 4 * (1 + 1 / w.num_partials)
        return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"{rows // 8} of 2048 S-rows of the source and {rows} of 8192 rows of each partial; "
                          f"{reps} repetitions"}


class ShortRunStep:
    """Short runs: an fp32 [16777216, 8] tensor (512 MiB) cut into 8 shards on
    axis 0 (2) and axis 1 (4), so every run is 2 elements (8 bytes), then the
    shards gathered back into the full tensor.  The pages' axis-1 example at
    memory-bound size: the split and the gather both go through whole-row
    blocks with 16-byte accesses."""

    SHAPE = (16777216, 8)
    SPEC = {"device": list(range(8)), "sharded_dim": [{"axis": 0, "num_shards": 2}, {"axis": 1, "num_shards": 4}]}

    def __init__(self):
        self.w = None
        self.src = inputs.normal(self.SHAPE, 7001, device="cuda")
        self.dst = {d: torch.empty((self.SHAPE[0] // 2, 2), device="cuda") for d in range(8)}
        self.full = torch.empty(self.SHAPE, device="cuda")
        torch.cuda.synchronize()
        self.s0 = torch.cuda.Stream()

    def result(self):
        return self.full

    def step(self):
        tp.tp_shard_materialize(self.src, self.SPEC, self.dst, stream=self.s0)
        tp.tp_shard_gather(self.dst, self.SPEC, [self.full], self.SHAPE, stream=self.s0)

    @property
    def work(self):
        return float(4 * self.src.numel() * 4)      # split: read + write; gather: read + write

    unit = "GB/s"

    def config(self):
        return {"workload": "shortrun-split-gather", "shape": list(self.SHAPE), "dtype": "f32",
                "sharded_dim": [[0, 2], [1, 4]], "run_bytes": 8, "shards": 8,
                "step": "split into the 8 shards, then gather them back"}

    def cpu_baseline(self, budget_s):
        from oracle import layout as L
        rows = 65536
        src = self.src[:rows].cpu()
        reps, t0 = 0, time.perf_counter()
        while True:
            pieces = L.split(src, self.SPEC)
            L.gather(pieces, (rows, 8), self.SPEC)
            reps += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = (time.perf_counter() - t0) / reps
        return {"value": 4 * rows * 8 * 4 / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"{rows} of {self.SHAPE[0]} rows split and gathered back; {reps} repetitions"}


WORKLOADS = {
    GPT2_SMALL.name: lambda: MlpStep(GPT2_SMALL, split_weights=True),
    GPT3_6P7B.name: lambda: MlpStep(GPT3_6P7B, split_weights=False),
    GPT3_175B.name: lambda: MlpStep(GPT3_175B, split_weights=False),
    TINY.name: lambda: MlpStep(TINY, split_weights=True),
    RESHARD.name: lambda: ReshardStep(RESHARD),
    GPT2_SMALL.name + "-bwd": lambda: BwdStep(GPT2_SMALL),
    GPT3_6P7B.name + "-bwd": lambda: BwdStep(GPT3_6P7B),
    GPT3_175B.name + "-bwd": lambda: BwdStep(GPT3_175B),
    GPT2_SMALL.name + "-sp": lambda: MlpStep(GPT2_SMALL, split_weights=True, seq=True),
    GPT3_6P7B.name + "-sp": lambda: MlpStep(GPT3_6P7B, split_weights=False, seq=True),
    GPT3_175B.name + "-sp": lambda: MlpStep(GPT3_175B, split_weights=False, seq=True),
    GPT3_6P7B.name + "-sp-bwd": lambda: BwdStep(GPT3_6P7B, seq=True),
    GPT2_SMALL.name + "-2layer": lambda: StackStep(GPT2_SMALL),
    GPT3_6P7B.name + "-2layer": lambda: StackStep(GPT3_6P7B),
    GPT3_175B.name + "-2layer": lambda: StackStep(GPT3_175B),
    GPT3_175B.name + "-sp-bwd": lambda: BwdStep(GPT3_175B, seq=True),
    "shortrun-split-gather": ShortRunStep,
}


# --------------------------------------------------------------------------- roofline

COPY_CALIBRATION_BYTES = 256 << 20


def copy_calibration():
    """A plain 256 MiB copy through the layout kernel (a one-device broadcast):
    its FETCH_SIZE / WRITE_SIZE readings calibrate the traffic counters."""
    src = torch.empty(COPY_CALIBRATION_BYTES // 4, device="cuda")
    src.fill_(1.0)
    dst = torch.empty_like(src)
    spec = {"device": [-1], "device_map": {-1: [0]}, "sharded_dim": []}
    for _ in range(3):
        tp.tp_shard_materialize(src, spec, {0: dst})
    torch.cuda.synchronize()


def _code_only(text):
    """C++ source with comments removed and whitespace collapsed (string literals
    in these kernels hold no comment markers)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash():
    """Hash of the kernel sources' code (device code and its launch dispatch;
    comments and layout do not count); traffic figures taken on other code are
    stale."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "sharded_gemm_amd", "csrc", "*.hip")))
    for f in files:
        with open(f, encoding="utf-8") as fh:
            code = _code_only(fh.read())
        if "__global__" not in code:      # no kernel in it (device data only)
            continue
        h.update(os.path.basename(f).encode())
        h.update(code.encode())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None when there is none or it was taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic__{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def _peak(unit, dtype):
    if unit == "GB/s":
        return "hbm", PEAK_HBM_GBS
    return ("mfma", PEAK_BF16_TFLOPS) if dtype == "bf16" else ("alu", PEAK_F32_TFLOPS)


def kernel_table(stats, steps, dtype):
    """Per library kernel: launches per step, average duration (HIP events on
    the launching stream) and the algorithmic rate with its roofline fraction."""
    out = {}
    for name, st in stats.items():
        if st["launches"] == 0:
            continue
        is_gemm = name.startswith("gemm") and name not in BYTE_KERNELS
        avg_ms = st["total_ms"] / st["launches"]
        rate = st["work"] / (st["total_ms"] * 1e-3)
        unit = "TFLOP/s" if is_gemm else "GB/s"
        bound, peak = _peak(unit, dtype)
        achieved = rate / (1e12 if is_gemm else 1e9)
        out[name] = {"launches_per_step": st["launches"] / steps, "avg_ms": avg_ms,
                     "ms_per_step": st["total_ms"] / steps, "work_per_launch": st["work"] / st["launches"],
                     "achieved": achieved, "unit": unit, "bound": bound, "peak": peak, "frac": achieved / peak}
    return out


def schedule_label(kernels, row_chunks, serial):
    """What the library made of the row chunks, read off its launch counts:
    None while every chunk keeps its own GEMM1 (the schedule as configured)."""
    g1 = kernels.get("gemm1", {}).get("launches_per_step")
    if g1 is None or g1 >= row_chunks:
        return None
    if "reduce" in kernels and not serial:
        return ("two streams: GEMM1 once over all rows, then each block's GEMM2 with the previous block's sum "
                "beside it on the second stream" +
                ("; the last block's sum in its GEMM2's epilogue" if "gemm2_reduce" in kernels else ""))
    one = "one stream" + ("" if serial else " (the second offered, unused)")
    if "gemm2_reduce" in kernels and "reduce" not in kernels:
        return one + (": every row chunk's sum folds into its GEMM2's epilogue, so GEMM1 runs once over all rows "
                      "and each chunk keeps its GEMM2")
    return one + ": the row chunks run as one block"


def roofline(kernels, dtype, workload, default_schedule=True, timing="cold", kernels_warm=None):
    """Roofline entry of the dominant kernel: the kernel with the most time per
    step among the GEMMs (together most of an MLP step), GEMM2 counting with
    the reduction when that runs in its epilogue; elsewhere the kernel with the
    most time.  `frac` is the cold figure; the same kernel's rate with the
    steps back to back (as the value's timed steps run) rides along as
    `warm`."""
    if not kernels:
        return None
    pool = [k for k in kernels if k.startswith("gemm")] or list(kernels)
    name = max(pool, key=lambda k: kernels[k]["ms_per_step"])
    k = kernels[name]
    # The counters were taken with the default schedule and outputs; another
    # schedule moves other bytes.
    traffic = measured_traffic(workload, name) if default_schedule else None
    out = {"kernel": name, "bound": k["bound"], "achieved": k["achieved"], "peak": k["peak"], "unit": k["unit"],
           "frac": k["frac"], "traffic": traffic, "avg_ms": k["avg_ms"],
           "work_per_launch": k["work_per_launch"], "timing": timing}
    kw = (kernels_warm or {}).get(name)
    if kw:
        out["warm"] = {"achieved": kw["achieved"], "frac": kw["frac"], "avg_ms": kw["avg_ms"]}
    return out


# --------------------------------------------------------------------------- torch context

def torch_context(wl, reps=20):
    """torch.matmul (hipBLASLt) on the step's GEMM shapes and a torch sum of the
    P partials of one reduce block, timed with events on one stream.  Context
    only: these are library calls, not part of the path."""
    w = wl.w
    s = torch.cuda.Stream()
    Mr, Hc = w.M // w.R, w.H // w.C
    X = wl.X[:Mr]
    A, B = wl.As[0], wl.Bs[0]
    Y = torch.empty((Mr, w.F), dtype=X.dtype, device="cuda")
    parts = [wl.Z[:Mr]] + [p[:Mr] for p in wl.peers]

    def t(fn):
        with torch.cuda.stream(s):
            for _ in range(3):
                fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            for _ in range(reps):
                fn()
            e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    out = {}
    ms = t(lambda: torch.matmul(X, A, out=Y))
    out["gemm1_matmul"] = {"shape": [Mr, w.F, w.H], "ms": ms, "TFLOP/s": 2.0 * Mr * w.F * w.H / ms / 1e9}
    if w.R > 1:
        # The library's schedules may run GEMM1 once over every row.
        Yall = torch.empty((w.M, w.F), dtype=X.dtype, device="cuda")
        ms = t(lambda: torch.matmul(wl.X, A, out=Yall))
        out["gemm1_matmul_all_rows"] = {"shape": [w.M, w.F, w.H], "ms": ms,
                                        "TFLOP/s": 2.0 * w.M * w.F * w.H / ms / 1e9}
        del Yall
    Bc = B[:, :Hc].contiguous()
    Z = torch.empty((Mr, Hc), dtype=X.dtype, device="cuda")
    ms = t(lambda: torch.matmul(Y, Bc, out=Z))
    out["gemm2_matmul"] = {"shape": [Mr, Hc, w.F], "ms": ms, "TFLOP/s": 2.0 * Mr * Hc * w.F / ms / 1e9,
                           "note": "bf16 output (torch.matmul has no fp32 output for bf16 inputs)"}
    if len(parts) > 1:
        acc = torch.empty_like(parts[0])

        def tsum():
            torch.add(parts[0], parts[1], out=acc)
            for p in parts[2:]:
                acc.add_(p)
        ms = t(tsum)
        nbytes = 4.0 * (len(parts) + 1) * Mr * w.H
        rb = 4.0 * (3 * (len(parts) - 1)) * Mr * w.H
        out["reduce_torch_add"] = {"partials": len(parts), "ms": ms, "GB/s_algorithmic": nbytes / ms / 1e6,
                                   "GB/s_moved": rb / ms / 1e6}
    for k, v in out.items():
        log(f"[bench] torch context {k}: {v}")
    return out


# --------------------------------------------------------------------------- timing

FLUSH_BYTES = 512 << 20
HEADLINE = GPT3_175B.name
EXTRAS = (TINY.name, GPT2_SMALL.name, GPT3_6P7B.name, RESHARD.name, "shortrun-split-gather")


class Flusher:
    """512 MiB read and written on a stream between timed steps: twice the
    256 MB MALL, so a step timed after it finds none of its inputs in L2 or
    the MALL (cold-cache timing)."""

    def __init__(self):
        self.buf = torch.zeros(FLUSH_BYTES // 4, device="cuda")

    def __call__(self, stream):
        with torch.cuda.stream(stream):
            self.buf.add_(1.0)


def spread(ms):
    """Median, p10 and p90 of per-step times (ms)."""
    a = np.asarray(ms, dtype=np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)), "p90": float(np.percentile(a, 90)),
            "n": int(a.size)}


def capture(wl, n=1):
    """n consecutive steps captured into one HIP graph on the workload's compute
    stream, or None when capture fails or a replay differs from the eager
    result."""
    try:
        eager_out = wl.result().clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=wl.s0):
            for _ in range(n):
                wl.step()
        with torch.cuda.stream(wl.s0):
            for _ in range(3):
                graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(eager_out.view(torch.int32), wl.result().view(torch.int32)):
            raise RuntimeError("graph replay differs from the eager step")
        return graph
    except Exception as e:  # report and time eagerly
        log(f"[bench] graph capture unavailable ({e}); timing eager steps")
        return None


def measure(wl, steps, warmup, flusher, kernel_tables=True, profile=False):
    """Time one workload: K consecutive steps (eager and graph replay; the
    faster gives ms_per_step), per-step times warm and cold in that mode, and
    the library's per-kernel events, warm and cold (eager launches).  With
    profile, only cold steps run (warm-up included), eagerly: the per-kernel
    events of the cold steps and their per-step times, so that every kernel
    launch of the process is one the cold table times."""
    if hasattr(wl, "prepare"):
        wl.prepare()
    dtype = "bf16" if getattr(getattr(wl, "w", None), "dtype", "f32") == "bf16" else "f32"
    if profile:
        for _ in range(warmup):
            flusher(wl.s0)
            wl.step()
        torch.cuda.synchronize()
        return measure_profile(wl, steps, flusher, dtype)
    # One eager step gives the result a graph replay must reproduce; the W
    # warm-up steps come after the capture, right before the timed ones: the
    # capture leaves the GPU idle for a while, and the first 5-10 ms of work
    # after an idle spell run up to 10% slower (MI355X: 175B step 1,343 against
    # 1,145 us over the first ten steps after 2 s idle; once GPT-2's 20 timed
    # steps came out at 84 us each against 28).
    wl.step()
    torch.cuda.synchronize()
    graph = capture(wl)
    # The K timed steps as one graph: one launch for all of them.
    block = capture(wl, steps) if graph is not None and steps > 1 else None
    # W steps, repeated until they have kept the GPU busy for 20 ms: a short
    # step (GPT-2's 28 us) would otherwise be timed inside that ramp.
    t0 = time.perf_counter()
    while True:
        for _ in range(warmup):
            wl.step()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= 0.02 or warmup == 0:
            break
    s0 = wl.s0

    def one(use_graph):
        if use_graph:
            with torch.cuda.stream(s0):
                graph.replay()
        else:
            wl.step()

    def all_k(mode):
        if mode == "block":
            with torch.cuda.stream(s0):
                block.replay()
        else:
            for _ in range(steps):
                one(mode == "graph")

    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def consecutive(mode):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(s0)
        all_k(mode)
        stop.record(s0)
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / steps, (time.perf_counter() - t0) / steps

    ms_eager, _ = consecutive("eager")
    ms_graph = consecutive("graph")[0] if graph is not None else None
    ms_block = consecutive("block")[0] if block is not None else None
    # per-step figures (and the flushes between cold steps) need one launch per step
    use_graph = ms_graph is not None and ms_graph < ms_eager
    timed = {"eager launches": ms_eager, "hip graph replay": ms_graph, f"one hip graph of the {steps} steps": ms_block}
    timed_as = min((k for k in timed if timed[k] is not None), key=lambda k: timed[k])
    ms = timed[timed_as]

    def per_step(cold, use_graph):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        for e0, e1 in evs:
            if cold:
                flusher(s0)
            e0.record(s0)
            one(use_graph)
            e1.record(s0)
        torch.cuda.synchronize()
        return [e0.elapsed_time(e1) for e0, e1 in evs]

    warm = per_step(False, use_graph)
    cold = per_step(True, use_graph)

    def kernels(cold):
        tp.tp_timing_enable(True)
        for _ in range(2):            # creates the timing events outside the measured steps
            wl.step()
        torch.cuda.synchronize()
        tp.tp_timing_read()
        for _ in range(steps):
            if cold:
                flusher(s0)
            wl.step()
        torch.cuda.synchronize()
        tp.tp_timing_enable(False)
        return kernel_table(tp.tp_timing_read(), steps, dtype)

    out = {"ms_per_step": ms, "timed_as": timed_as,
           "ms_per_step_eager": ms_eager, "ms_per_step_graph": ms_graph, "ms_per_step_graph_k": ms_block,
           "step_ms": {"warm": spread(warm), "cold": spread(cold)}, "dtype": dtype}
    if kernel_tables:
        out["kernels_cold"] = kernels(True)
        out["kernels_warm"] = kernels(False)
    return out


def measure_profile(wl, steps, flusher, dtype):
    """Cold eager steps with the library's per-kernel events (--profile)."""
    tp.tp_timing_enable(True)
    tp.tp_timing_read()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        flusher(wl.s0)
        e0.record(wl.s0)
        wl.step()
        e1.record(wl.s0)
    torch.cuda.synchronize()
    tp.tp_timing_enable(False)
    table = kernel_table(tp.tp_timing_read(), steps, dtype)
    cold = spread([e0.elapsed_time(e1) for e0, e1 in evs])
    return {"ms_per_step": cold["median"], "timed_as": "eager launches, cold, with per-kernel events (profile mode)",
            "ms_per_step_eager": cold["median"], "ms_per_step_graph": None, "step_ms": {"cold": cold},
            "dtype": dtype, "kernels_cold": table, "kernels_warm": {}}


def rate(wl, ms):
    return wl.work / (ms * 1e-3) / (1e12 if wl.unit == "TFLOP/s" else 1e9)


def run_workload(name, steps, warmup, flusher, args, serial_too=True):
    """Set up, time and summarise one workload (and, for a chunked MLP, its
    serial schedule); returns (workload object, summary dict)."""
    log(f"[bench] workload {name}: setting up")
    wl = WORKLOADS[name]()
    wl.serial, wl.reduce_wgs = args.serial, args.reduce_wgs
    if args.no_reduce_fusion:
        wl.reduce_fusion = tp.TP_REDUCE_FUSION_OFF
    wl.separate_output = args.separate_output
    wl.cut_weights = args.cut_weights
    wl.gather_input = args.gather_input
    wl.weights_linear = args.weights == "linear"
    log(f"[bench] workload {name}: timing")
    m = measure(wl, steps, warmup, flusher, profile=args.profile)
    default_schedule = not (args.serial or args.reduce_wgs or args.no_reduce_fusion or args.separate_output or
                            args.gather_input or args.weights != "math")
    summ = {"config": wl.config(), "value": rate(wl, m["ms_per_step"]), "unit": wl.unit,
            "ms_per_step": m["ms_per_step"], "timed_as": m["timed_as"],
            "ms_per_step_eager": m["ms_per_step_eager"], "ms_per_step_graph": m["ms_per_step_graph"],
            "ms_per_step_graph_k": m.get("ms_per_step_graph_k"),
            "step_ms": m["step_ms"], "value_cold_median": rate(wl, m["step_ms"]["cold"]["median"]),
            "peers": "drawn N(0,1) (profile mode)" if DRAWN_PEERS else "computed by the same path",
            "roofline": roofline(m["kernels_cold"], m["dtype"], name, default_schedule,
                                 kernels_warm=m["kernels_warm"]),
            "kernels": m["kernels_cold"], "kernels_warm": m["kernels_warm"], "dtype": m["dtype"]}
    label = schedule_label(m["kernels_cold"], wl.w.R, wl.serial) if isinstance(wl, MlpStep) else None
    if label:
        summ["config"]["schedule"] = label
    for k, v in m["kernels_cold"].items():
        log(f"[bench]   {k:18s} {v['launches_per_step']:.0f}/step  avg {v['avg_ms'] * 1e3:9.1f} us  "
            f"{v['achieved']:9.1f} {v['unit']}  ({100 * v['frac']:.1f}% of {v['peak']:.0f}, cold)")
    log(f"[bench]   step {m['ms_per_step'] * 1e3:.1f} us ({m['timed_as']}); per step cold median "
        f"{m['step_ms']['cold']['median'] * 1e3:.1f} us")
    two_blocks = isinstance(wl, (MlpStep, BwdStep, StackStep)) and wl.w.R * getattr(wl.w, "C", 1) > 1
    if serial_too and two_blocks and not args.serial and not args.profile:
        log(f"[bench] workload {name}: serial schedule")
        wl.serial = True
        ms = measure(wl, steps, warmup, flusher, kernel_tables=False)
        wl.serial = False
        summ["serial"] = {"ms_per_step": ms["ms_per_step"], "timed_as": ms["timed_as"], "step_ms": ms["step_ms"],
                          "value": rate(wl, ms["ms_per_step"])}
        summ["overlap_saves"] = {"warm_median_ms": ms["step_ms"]["warm"]["median"] - m["step_ms"]["warm"]["median"],
                                 "cold_median_ms": ms["step_ms"]["cold"]["median"] - m["step_ms"]["cold"]["median"]}
        log(f"[bench]   serial {ms['ms_per_step'] * 1e3:.1f} us against {m['ms_per_step'] * 1e3:.1f} us on two streams")
        if hasattr(wl, "prepare"):
            wl.prepare()
    return wl, summ


def cpu_baselines(wl, budget_s, single_thread=True):
    """The oracle timed with every BLAS thread, and with one (fewer sampled rows)."""
    from threadpoolctl import threadpool_limits
    log("[bench] timing the CPU oracle (all threads)")
    cpu = wl.cpu_baseline(budget_s)
    if single_thread:
        log("[bench] timing the CPU oracle (one thread)")
        with threadpool_limits(limits=1):
            kw = {"rows": 32} if isinstance(wl, MlpStep) and wl.w.M * wl.w.H * wl.w.F > 4096 * 768 * 768 else {}
            one = wl.cpu_baseline(budget_s, **kw)
        cpu["single_thread"] = {k: one[k] for k in ("value", "unit", "cores", "sample")}
    return cpu


# --------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(WORKLOADS))
    ap.add_argument("--no-extras", action="store_true",
                    help="time only --workload (the default run also times the other four configurations)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle timing per thread setting")
    ap.add_argument("--serial", action="store_true", help="run the reduce on the compute stream")
    ap.add_argument("--separate-output", action="store_true",
                    help="write the reduced output to its own buffer instead of in place over the partial")
    ap.add_argument("--weights", choices=("math", "linear"), default="math",
                    help="forward MLP workloads: rank 0's weight shards in the math layout (A_i [H, F], B_i [F, H]) "
                         "or a linear layer's [out, in] (A_i^T, B_i^T)")
    ap.add_argument("--gather-input", action="store_true",
                    help="sequence-parallel workloads: all-gather the input blocks into X before GEMM1 instead of "
                         "reading them in place")
    ap.add_argument("--cut-weights", action="store_true",
                    help="copy rank 0's weight shards out of the full weights each step (workloads with full weights) "
                         "instead of reading them in place")
    ap.add_argument("--no-reduce-fusion", action="store_true",
                    help="always run the forward's reduction as its own kernel, never in GEMM2's epilogue")
    ap.add_argument("--reduce-wgs", type=int, default=0,
                    help="cap on the reduce kernel's workgroups beside the GEMMs (0 = library default)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a 256 MiB plain copy (for calibrating traffic counters)")
    ap.add_argument("--profile", action="store_true",
                    help="for kernel traces and counters: draw the peers' partials instead of computing them, and "
                         "run only cold eager steps (warm-up included) with per-kernel events; implies --no-extras")
    ap.add_argument("--no-torch-context", action="store_true",
                    help="skip timing torch.matmul (hipBLASLt) and a torch sum on the headline's shapes")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the partial sum over ranks runs over virtual shards on one device).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if not os.path.exists(_abi.LIB_PATH):
        from sharded_gemm_amd import build
        build.build()
    tp.load()

    if args.profile:
        global DRAWN_PEERS
        DRAWN_PEERS = True
        args.no_extras = True
        args.no_torch_context = True
    if args.copy_calibration:
        log("[bench] 256 MiB copy for counter calibration")
        copy_calibration()
    flusher = Flusher()
    wl, head = run_workload(args.workload, args.steps, args.warmup, flusher, args)
    cpu = None if args.no_cpu_baseline else cpu_baselines(wl, args.cpu_budget)
    context = (torch_context(wl) if not args.no_torch_context and isinstance(wl, MlpStep) and wl.w.dtype == "bf16"
               else None)
    del wl
    torch.cuda.empty_cache()

    configs = {}
    if not args.no_extras and args.workload == HEADLINE:
        for name in EXTRAS:
            w2, summ = run_workload(name, args.steps, args.warmup, flusher, args)
            if not args.no_cpu_baseline:
                summ["cpu_baseline"] = cpu_baselines(w2, min(3.0, args.cpu_budget), single_thread=False)
            configs[name] = summ
            del w2
            torch.cuda.empty_cache()

    rec = {"metric": METRIC, "value": head["value"], "unit": head["unit"], "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": head["dtype"], "data": "synthetic (seeded N(0,1)/N(0,0.02) tensors)",
           "config": head["config"], "roofline": head["roofline"], "cpu_baseline": cpu}
    for k in ("timed_as", "ms_per_step_eager", "ms_per_step_graph", "ms_per_step_graph_k", "step_ms",
              "value_cold_median", "serial",
              "overlap_saves", "kernels", "kernels_warm"):
        if k in head:
            rec[k] = head[k]
    rec["timing"] = ("value: K consecutive steps (the fastest of eager launches, K replays of a one-step HIP graph "
                     "and one replay of a graph of the K steps); step_ms: "
                     "per-step HIP events, warm = back to back, cold = after 512 MiB written; kernels: the "
                     "library's HIP events around each launch on its stream, cold; roofline: the dominant "
                     "kernel of the cold table")
    if context is not None:
        rec["torch_context"] = context
    if configs:
        rec["configs"] = configs
    rec["device"] = torch.cuda.get_device_name(0)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
