"""The five synthetic workloads: shapes, value scales, chunk counts and seeds.

Pure data.  Each MLP workload is one rank's share of a column->row tensor-parallel
MLP: X[M,H] times A_i[H,F] (a column slice of A[H,P*F]), GeLU, times B_i[F,H]
(a row slice of B[P*F,H]), giving an fp32 partial [M,H] that is summed over the
P virtual ranks.  R is the number of independent row chunks of X and C the
number of column blocks of B_i (the Domino splits).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field


@dataclass(frozen=True)
class MlpWorkload:
    cfg: int
    name: str
    dtype: str          # "f32" or "bf16": storage type of X, A_i, B_i (and Y)
    M: int              # tokens
    H: int              # hidden
    F: int              # per-rank FFN width
    P: int              # tensor-parallel degree (virtual ranks)
    R: int = 1          # row chunks of X
    C: int = 1          # column blocks of B_i
    std_x: float = 1.0
    std_a: float = 0.02
    std_b: float = 0.02
    split_full_weights: bool = False   # draw full A, B and cut them (else per-rank draws)

    @property
    def flops_per_rank(self) -> int:
        return 2 * 2 * self.M * self.H * self.F


@dataclass(frozen=True)
class LayoutWorkload:
    cfg: int
    name: str
    src_shape: tuple
    mesh_shape: tuple
    process_ids: tuple
    dims_mapping: tuple
    group_size: int             # replication factor of each shard through a device map
    partial_shape: tuple        # shape of each partial buffer for the split reduce
    num_partials: int
    num_splits: int


TINY = MlpWorkload(cfg=1, name="tiny-fp32-p2", dtype="f32", M=64, H=256, F=512, P=2,
                   std_x=1.0, std_a=1.0 / math.sqrt(256), std_b=1.0 / math.sqrt(1024),
                   split_full_weights=True)
GPT2_SMALL = MlpWorkload(cfg=2, name="gpt2-small-tp4", dtype="bf16", M=4096, H=768, F=768, P=4,
                         split_full_weights=True)
GPT3_6P7B = MlpWorkload(cfg=3, name="gpt3-6.7b-tp8-rowsplit2", dtype="bf16", M=8192, H=4096, F=2048,
                        P=8, R=2)
GPT3_175B = MlpWorkload(cfg=5, name="gpt3-175b-tp8-2d-r2c2", dtype="bf16", M=4096, H=12288, F=6144,
                        P=8, R=2, C=2)
RESHARD = LayoutWorkload(cfg=4, name="reshard-2x4-mesh", src_shape=(8, 2048, 8192), mesh_shape=(2, 4),
                         process_ids=tuple(range(8)), dims_mapping=(0, -1, 1), group_size=2,
                         partial_shape=(8192, 8192), num_partials=8, num_splits=8)

MLP_WORKLOADS = {w.cfg: w for w in (TINY, GPT2_SMALL, GPT3_6P7B, GPT3_175B)}

# The 2x2 layout cases of the tiny workload: the tensor [[1,2],[3,4]] under the
# ONNX ShardingSpec examples (axis 0, axis 1, both axes, broadcast, mixed).
TINY_LAYOUT_SPECS = {
    "axis0": {"device": [0, 1], "sharded_dim": [{"axis": 0, "num_shards": 2}]},
    "axis1": {"device": [0, 1], "sharded_dim": [{"axis": 1, "num_shards": 2}]},
    "both": {"device": [0, 1, 2, 3],
             "sharded_dim": [{"axis": 0, "num_shards": 2}, {"axis": 1, "num_shards": 2}]},
    "broadcast": {"device": [-1], "device_map": {-1: [0, 1]}, "sharded_dim": []},
    "mixed": {"device": [-1, -2], "device_map": {-1: [0, 1], -2: [2, 3]},
              "sharded_dim": [{"axis": 0, "num_shards": 2}]},
}
