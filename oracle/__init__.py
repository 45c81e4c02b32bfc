"""CPU oracle for the tensor-parallel MLP and shard-layout path.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, obviously-correct
float64 restatement of what the pages define.  Only the tests, the smoke check
in ``__graft_entry__`` and the bench's ``cpu_baseline`` leg may import it; the
product path (``sharded_gemm_amd``) never does, and the two share no code.

Modules
  layout  -- ShardingSpec split / broadcast / device-map replication and
             ProcessMesh + dims_mapping shards  (ONNX multi-device proposal;
             OneFlow SBP article; Paddle SPMD-rules page)
  reduce  -- partial-sum -> full and partial-sum -> split reduction
             (OneFlow SBP "partial"; ColossalAI 1D-TP all-reduce)
  mlp     -- GeLU and one rank's column->row MLP share, plus the all-rank sum
             (ColossalAI 1D tensor parallelism, sections 2 and 2.1), and its
             backward (section 2.2; DeepSpeed-Domino, backward)

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against the pages' worked examples, closed forms, invariants, library special
cases or brute force.  No function is "parity unpinned".
"""
from . import layout, mlp, reduce  # noqa: F401

__all__ = ["layout", "reduce", "mlp"]
