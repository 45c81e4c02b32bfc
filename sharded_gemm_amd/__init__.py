"""MI355X-native tensor-parallel MLP share and shard-layout kernels.

The compute lives in ``libtpshard.so`` (hand-written HIP for gfx950, C ABI in
``include/tpshard.h``); ``sharded_gemm_amd._abi`` is its thin ctypes binding.
``inputs`` and ``workloads`` hold the seeded synthetic inputs and the
workload table.  Importing this package does not load the library; the first
call into the binding does, and raises if it was not built.
"""
from ._abi import (  # noqa: F401
    TP_ACT_GELU_ERF, TP_ACT_NONE, TP_BF16, TP_F32, TP_REDUCE_FULL, TP_REDUCE_OP_MAX, TP_REDUCE_OP_MIN,
    TP_REDUCE_FUSION_AUTO, TP_REDUCE_FUSION_OFF, TP_REDUCE_OP_SUM, TP_REDUCE_SPLIT, TP_WEIGHTS_LINEAR,
    TP_WEIGHTS_MATH, TpError, load,
    tp_check_broadcast_binary, tp_colrow_mlp, tp_colrow_mlp_backward, tp_colrow_mlp_noalloc, tp_colrow_mlp_stack, tp_infer_matmul_dims_mapping, tp_layout_plan, tp_partial_reduce, tp_shard_gather, tp_shard_materialize, tp_shard_materialize_batch, tp_timing_enable,
    tp_timing_read, version,
)
