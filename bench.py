#!/usr/bin/env python3
"""Throughput of one rank's tensor-parallel MLP share and its layout kernels
on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one pass of the whole hot path over one batch of synthetic input.
It is timed both as eager launches and as a captured HIP graph replay; the
faster mode gives the value and is named in "timed_as".
Default workload (GPT-2-small MLP at TP=4, 4096 tokens): cut this rank's
A_i/B_i out of the full weights (split along columns / rows into 4 shards
each), run GEMM1 + GeLU and GEMM2 on the compute stream, and sum the 4 fp32
partials (this rank's and 3 peers' computed beforehand by the same path) on a
second stream.  The value is per-rank MLP TFLOP/s (2 GEMMs, 2*M*H*F flops
each) over the whole step.  Per-kernel durations come from HIP events that
the library records around each of its launches inside the timed region.

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
from sharded_gemm_amd.workloads import GPT2_SMALL, GPT3_175B, GPT3_6P7B, RESHARD, TINY  # noqa: E402

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

class MlpStep:
    """Per-rank MLP step, optionally preceded by cutting the weights.  With
    ``seq`` the step is the sequence-parallel form: the input arrives as P
    sequence blocks that the call all-gathers, and the output is
    reduce-scattered into P blocks."""

    serial = False
    reduce_wgs = 0
    reduce_fusion = tp.TP_REDUCE_FUSION_AUTO
    # The row-parallel all-reduce works in place on the partial output, as
    # torch.distributed.all_reduce does; separate_output keeps Z_i and writes
    # the sum to its own buffer instead.
    separate_output = False

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
            z = torch.empty((w.M, w.H), device=dev)
            tp.tp_colrow_mlp(self.X, self.As[i], self.Bs[i], self.Y, z, row_chunks=w.R, col_chunks=w.C)
            self.peers.append(z)
        if seq:
            # every rank's sequence block as its own buffer; X becomes the gather workspace
            self.Xb = [b.clone() for b in torch.chunk(self.X, w.P)]
            self.Zs = [torch.empty((w.M // w.P, w.H), device=dev) for _ in range(w.P)]
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
        if self.split:
            # rank 0's column shard of A and row shard of B in one batched call
            # (one launch): each rank materialises its own share
            self.cut = tp.tp_shard_materialize_batch([(self.A, self.sa, {0: self.As[0]}, 0),
                                                      (self.B, self.sb, {0: self.Bs[0]}, 0)],
                                                     stream=self.s0, prepare=True)
        self.mlp = tp.tp_colrow_mlp(self.X, self.As[0], self.Bs[0], self.Y, self.Z, row_chunks=self.w.R,
                                    col_chunks=self.w.C, peer_partials=self.peers,
                                    Z_out=None if self.seq else self._z_out(), s_compute=self.s0,
                                    s_reduce=self.s0 if self.serial else self.s1,
                                    reduce_workgroups=self.reduce_wgs, X_shards=self.Xb if self.seq else None,
                                    Z_split=self.Zs if self.seq else None, reduce_fusion=self.reduce_fusion,
                                    prepare=True)

    def step(self):
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
               "weights_cut_each_step": "rank 0's shards of A and B" if self.split else False,
               "reduce_stream": "compute" if self.serial else "second",
               "reduce_fusion": "auto" if self.reduce_fusion == tp.TP_REDUCE_FUSION_AUTO else "off",
               "reduce_output": ("reduce-scattered blocks" if self.seq else
                                 "separate buffer" if self.separate_output else "in place over the partial (all-reduce)"),
               "peers": "virtual ranks 1..P-1, partials precomputed by the same path"}
        if self.seq:
            cfg["sequence_parallel"] = {"blocks": w.P, "input": "all-gathered from P sequence blocks",
                                        "output": "reduce-scattered into P sequence blocks"}
        return cfg

    def cpu_baseline(self, budget_s):
        """The oracle on this step (sampled rows for the large shapes), fp64."""
        from threadpoolctl import threadpool_info
        from oracle import layout as L
        from oracle import mlp as O
        from oracle import reduce as R
        w = self.w
        Xc = self.X.cpu()
        A0, B0 = self.As[0].cpu(), self.Bs[0].cpu()
        rows = w.M if w.M * w.H * w.F <= 4096 * 768 * 768 else 256
        sample_rows = np.linspace(0, w.M - 1, rows).astype(np.int64)
        peers = [inputs.normal((rows, w.H), 99000 + p) for p in range(w.P - 1)]
        Ac = self.A.cpu() if self.split else None
        Bc = self.B.cpu() if self.split else None
        gspec = {"device": list(range(w.P)), "sharded_dim": [{"axis": 0, "num_shards": w.P}]}
        xblocks = dict(enumerate(np.split(Xc[sample_rows].float().numpy(), w.P))) if self.seq else None
        reps, t0 = 0, time.perf_counter()
        while True:
            if self.split:
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
                "sample": (f"{rows} of {w.M} token rows of the per-rank MLP (fp64, numpy BLAS), "
                           f"{'plus cutting the full weights into the shards of every rank (the oracle has no one-device form), ' if self.split else ''}"
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
        self.call = tp.tp_colrow_mlp_backward(
            self.X, self.As[0], self.Bs[0], self.Hs, self.Y, self.dZ, self.dH, self.dX, self.dA, self.dB,
            row_chunks=self.w.R, peer_dX=self.peers,
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
                z = torch.empty((w.M, w.H), device=dev)
                tp.tp_colrow_mlp(x, As[i], Bs[i], self.Y, z, row_chunks=w.R)
                peers.append(z)
            xn = torch.empty((w.M, w.H), dtype=torch.bfloat16, device=dev)
            zo = torch.empty((w.M, w.H), device=dev)
            tp.tp_colrow_mlp(x, As[0], Bs[0], self.Y, self.Z, row_chunks=w.R, peer_partials=peers, Z_out=zo, X_next=xn)
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
            h.update(os.path.basename(f).encode())
            h.update(_code_only(fh.read()).encode())
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


def kernel_table(stats, steps):
    out = {}
    for name, st in stats.items():
        if st["launches"] == 0:
            continue
        is_gemm = name.startswith("gemm") and name not in BYTE_KERNELS
        avg_ms = st["total_ms"] / st["launches"]
        rate = st["work"] / (st["total_ms"] * 1e-3)
        out[name] = {"launches_per_step": st["launches"] / steps, "avg_ms": avg_ms,
                     "ms_per_step": st["total_ms"] / steps,
                     "achieved": rate / (1e12 if is_gemm else 1e9),
                     "unit": "TFLOP/s" if is_gemm else "GB/s"}
    return out


def roofline(kernels, dtype, workload, default_schedule=True):
    """Roofline entry of the dominant kernel.  In an MLP step that is the slower
    of the two GEMMs (together more than half the step; the weight cuts are two
    short launches whose per-launch event overhead would otherwise let them
    overtake a GEMM from run to run), GEMM2 counting with the reduction when
    that runs in its epilogue; elsewhere the kernel with the most time."""
    if not kernels:
        return None
    pool = [k for k in kernels if k.startswith("gemm")] or list(kernels)
    name = max(pool, key=lambda k: kernels[k]["ms_per_step"])
    k = kernels[name]
    # The counters were taken with the default schedule and outputs; another
    # schedule moves other bytes.
    traffic = measured_traffic(workload, name) if default_schedule else None
    if k["unit"] == "TFLOP/s":
        peak = PEAK_BF16_TFLOPS if dtype == "bf16" else PEAK_F32_TFLOPS
        return {"kernel": name, "bound": "mfma" if dtype == "bf16" else "alu", "achieved": k["achieved"],
                "peak": peak, "unit": "TFLOP/s", "frac": k["achieved"] / peak, "traffic": traffic}
    return {"kernel": name, "bound": "hbm", "achieved": k["achieved"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": k["achieved"] / PEAK_HBM_GBS, "traffic": traffic}


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


# --------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=GPT2_SMALL.name, choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle timing")
    ap.add_argument("--serial", action="store_true", help="run the reduce on the compute stream")
    ap.add_argument("--separate-output", action="store_true",
                    help="write the reduced output to its own buffer instead of in place over the partial")
    ap.add_argument("--no-reduce-fusion", action="store_true",
                    help="always run the forward's reduction as its own kernel, never in GEMM2's epilogue")
    ap.add_argument("--reduce-wgs", type=int, default=0,
                    help="cap on the reduce kernel's workgroups beside the GEMMs (0 = library default)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a 256 MiB plain copy (for calibrating traffic counters)")
    ap.add_argument("--torch-context", action="store_true",
                    help="also time torch.matmul (hipBLASLt) and a torch sum of the partials on the same shapes "
                         "(context only; MLP workloads)")
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

    if args.copy_calibration:
        log("[bench] 256 MiB copy for counter calibration")
        copy_calibration()
    log(f"[bench] workload {args.workload}: setting up")
    wl = WORKLOADS[args.workload]()
    wl.serial, wl.reduce_wgs = args.serial, args.reduce_wgs
    if args.no_reduce_fusion:
        wl.reduce_fusion = tp.TP_REDUCE_FUSION_OFF
    wl.separate_output = args.separate_output
    if hasattr(wl, "prepare"):
        wl.prepare()
    dtype = "bf16" if getattr(getattr(wl, "w", None), "dtype", "f32") == "bf16" else "f32"
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        wl.step()
    torch.cuda.synchronize()

    # The step is captured once into a HIP graph (the hot path is launch-bound
    # at these sizes) and the timed region replays it; a second timed region
    # runs the same steps eagerly with per-kernel HIP events for the table.
    graph = None
    try:
        eager_out = wl.result().clone()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=wl.s0):
            wl.step()
        with torch.cuda.stream(wl.s0):
            for _ in range(3):
                graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(eager_out.view(torch.int32), wl.result().view(torch.int32)):
            raise RuntimeError("graph replay differs from the eager step")
    except Exception as e:  # report and time eagerly
        log(f"[bench] graph capture unavailable ({e}); timing eager steps")
        graph = None

    def run(k):
        if graph is None:
            for _ in range(k):
                wl.step()
        else:
            with torch.cuda.stream(wl.s0):
                for _ in range(k):
                    graph.replay()

    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)

    def timed(use_graph):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(wl.s0)
        if use_graph:
            run(args.steps)
        else:
            for _ in range(args.steps):
                wl.step()
        stop.record(wl.s0)
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / args.steps, (time.perf_counter() - t0) / args.steps

    # Both execution modes run the same kernels on the same data; the faster is
    # the value (a captured graph removes host launch gaps, but its replay does
    # not overlap the two streams the way eager launches do).
    log(f"[bench] timing {args.steps} eager steps")
    ms_eager_plain, wall_eager_plain = timed(False)
    ms_graph = None
    if graph is not None:
        log(f"[bench] timing {args.steps} graph replays")
        ms_graph, wall_graph = timed(True)
    use_graph = ms_graph is not None and ms_graph < ms_eager_plain
    ms_per_step = ms_graph if use_graph else ms_eager_plain
    wall = wall_graph if use_graph else wall_eager_plain

    log(f"[bench] timing {args.steps} eager steps with per-kernel events")
    tp.tp_timing_enable(True)
    for _ in range(args.steps):      # creates the timing events outside the timed region
        wl.step()
    torch.cuda.synchronize()
    tp.tp_timing_read()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    start.record(wl.s0)
    for _ in range(args.steps):
        wl.step()
    stop.record(wl.s0)
    torch.cuda.synchronize()
    wall_eager = time.perf_counter() - t1
    tp.tp_timing_enable(False)
    stats = tp.tp_timing_read()
    ms_eager = start.elapsed_time(stop) / args.steps

    value = wl.work / (ms_per_step * 1e-3) / (1e12 if wl.unit == "TFLOP/s" else 1e9)
    kernels = kernel_table(stats, args.steps)
    for name, k in kernels.items():
        log(f"[bench] {name:12s} {k['launches_per_step']:.0f}/step  avg {k['avg_ms'] * 1e3:9.1f} us  "
            f"{k['achieved']:9.1f} {k['unit']}")
    log(f"[bench] step {ms_per_step * 1e3:.1f} us ({'graph replay' if use_graph else 'eager'}; eager "
        f"{ms_eager_plain * 1e3:.1f} us, graph {ms_graph * 1e3 if ms_graph else float('nan'):.1f} us; "
        f"eager with kernel events {ms_eager * 1e3:.1f} us)")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        cpu = wl.cpu_baseline(args.cpu_budget)

    context = torch_context(wl) if args.torch_context and isinstance(wl, MlpStep) else None

    rec = {"metric": METRIC, "value": value, "unit": wl.unit, "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": dtype, "data": "synthetic (seeded N(0,1)/N(0,0.02) tensors)",
           "config": wl.config(), "roofline": roofline(kernels, dtype, args.workload, default_schedule=not (
               args.serial or args.reduce_wgs or args.no_reduce_fusion or args.separate_output)), "cpu_baseline": cpu,
           "kernels": kernels, "timed_as": "hip graph replay" if use_graph else "eager launches",
           "ms_per_step_eager": ms_eager_plain, "ms_per_step_graph": ms_graph,
           "ms_per_step_eager_with_kernel_events": ms_eager,
           "device": torch.cuda.get_device_name(0)}
    if context is not None:
        rec["torch_context"] = context
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
