/*
 * tpshard: one rank's share of a column->row tensor-parallel MLP block and the
 * shard-layout kernels around it, for AMD Instinct MI355X (gfx950).
 *
 * Plain C ABI.  Every pointer argument is either a host pointer (specs, shapes,
 * pointer tables: read during the call only) or a device pointer (tensor data:
 * caller-owned, e.g. allocated by PyTorch).  The library never allocates device
 * memory.  Every call validates all of its arguments before it enqueues any
 * work, so a call that returns an error has left every output untouched.
 * Work is enqueued asynchronously on the caller's HIP stream(s); results are
 * valid once those streams have completed.
 *
 * Pages cited (by title and section):
 *   [ONNX]  "ONNX multi-device proposal: tensor- and pipeline-parallel
 *           annotations based on ShardingSpec" (ONNX 多设备执行提案解析)
 *   [SBP]   OneFlow global tensor article (placement, SBP, 2D SBP)
 *   [CAI]   "ColossalAI 1D Tensor Parallelism: principles and Shardformer"
 *   [SPMD]  Paddle "SPMD derivation rules and pipeline scheduling"
 *   [DOM]   "DeepSpeed-Domino in depth"
 */
#ifndef TPSHARD_H
#define TPSHARD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
/* Every entry point returns TP_OK (0) or one of the negative codes below.   */
enum {
  TP_OK = 0,
  TP_ERR_ARG = -1,         /* null pointer, bad size, bad dtype/mode, aliasing */
  TP_ERR_SPEC = -2,        /* ill-formed layout (axis range, device counts, map keys) */
  TP_ERR_INDIVISIBLE = -3, /* a dim is not a multiple of its shard / chunk count */
  TP_ERR_UNSUPPORTED = -4, /* well-formed but outside what this library does */
  TP_ERR_HIP = -5          /* a HIP runtime call failed (message has hipGetErrorString) */
};

/* Message describing the last failing call on the calling thread ("" if none).
 * The string stays valid until the next call on the same thread. */
const char *tp_last_error(void);

/* Library version, e.g. "tpshard 0.1 gfx950". */
const char *tp_version(void);

/* A hipStream_t passed as an opaque pointer; NULL means the null stream. */
typedef void *tp_stream_t;

/* Element types. */
enum { TP_F32 = 0, TP_BF16 = 1 };

/* ---- layout description ------------------------------------------------ */
/* Mirror of ShardingSpecProto / ShardedDimProto / SimpleShardedDimProto
 * ([ONNX] "Proto definitions").  tensor_name is not needed here.            */
typedef struct {
  int64_t dim_value;  /* size of the sharded dim if known; 0 = absent (not checked) */
  int64_t num_shards; /* >= 1, must divide the dim ([ONNX] "note on divisibility":
                         the backend decides; this one rejects, TP_ERR_INDIVISIBLE) */
} tp_simple_sharding;

typedef struct {
  int64_t axis;                              /* in [-r, r-1]; negative counts from the back */
  const tp_simple_sharding *simple_sharding; /* exactly 1 entry (else TP_ERR_UNSUPPORTED) */
  int64_t num_simple_sharding;
} tp_sharded_dim;

typedef struct {
  int64_t key;            /* negative: the value that stands for this group in `device` */
  const int64_t *devices; /* physical device ids (>= 0), in replication order */
  int64_t num_devices;    /* >= 1 */
} tp_device_group;

typedef struct {
  /* device[k] receives shard k: a physical id (>= 0) or a negative key into
   * device_map whose whole group receives a copy ([ONNX] "Sharding as a
   * Broadcast", "mixing split and broadcast").  num_device must equal the
   * product of num_shards over sharded_dim. */
  const int64_t *device;
  int64_t num_device;
  const tp_device_group *device_map; /* = index_to_device_group_map; may be NULL if unused */
  int64_t num_groups;
  /* Shards are enumerated with the FIRST listed sharded_dim outermost ([ONNX]
   * "index rule for multi-axis sharding": axis0 outer, axis1 inner). */
  const tp_sharded_dim *sharded_dim;
  int64_t num_sharded_dim; /* 0 = pure replication */
} tp_sharding_spec;

/* [SPMD] "ProcessMesh": mesh shape and process ids laid out row-major. */
typedef struct {
  const int64_t *shape;       /* mesh dims, each >= 1 */
  int64_t ndim;
  const int64_t *process_ids; /* prod(shape) distinct ids >= 0 */
} tp_process_mesh;

enum { TP_LAYOUT_SPEC = 0, TP_LAYOUT_DIMS_MAPPING = 1 };

typedef struct {
  int32_t kind;          /* TP_LAYOUT_SPEC or TP_LAYOUT_DIMS_MAPPING */
  tp_sharding_spec spec; /* used when kind == TP_LAYOUT_SPEC */
  tp_process_mesh mesh;  /* used when kind == TP_LAYOUT_DIMS_MAPPING */
  /* [SPMD] "dims_mapping": length = tensor rank; dims_mapping[i] = j >= 0 cuts
   * tensor axis i into mesh.shape[j] blocks, the process at mesh coordinate c
   * holding block c[j]; -1 keeps axis i whole.  A mesh dim may be used once. */
  const int64_t *dims_mapping;
} tp_layout;

/* ---- host-only planning ------------------------------------------------ */
/*
 * Normalise a layout of a tensor of shape[ndim] into its list of distinct
 * shards.  Host only: launches nothing, needs no GPU.
 *   *num_shards_out     number of distinct shards S
 *   boxes[s*2*ndim ...] for s < min(S, max_shards): per axis (start, stop)
 *   shard_of_device[d]  for d < num_dst: the shard device d receives, or -1
 * boxes and shard_of_device may be NULL.  Under TP_LAYOUT_DIMS_MAPPING the
 * processes holding the same block form one shard (replicated mesh dims).
 * Errors: TP_ERR_ARG (null shape/layout, ndim < 0 or > 8, negative dims),
 *         TP_ERR_SPEC, TP_ERR_INDIVISIBLE, TP_ERR_UNSUPPORTED as above.
 */
int tp_layout_plan(const int64_t *shape, int64_t ndim, const tp_layout *layout,
                   int64_t *num_shards_out, int64_t *boxes, int64_t max_shards,
                   int64_t *shard_of_device, int64_t num_dst);

/* ---- host sharding checker ---------------------------------------------- */
/*
 * Output sharding of a broadcasting binary elementwise operator (Add, Mul, ...)
 * whose inputs of shape1[ndim1] and shape2[ndim2] carry layout1 and layout2
 * ([ONNX] sharding formalism, "validity check" and the broadcasting n-ary
 * group; its composition example Add([M,1], [1,N])).  Host only.
 * Inputs align on their trailing axes (output rank r = max(ndim1, ndim2)).  An
 * axis where both inputs have the full size must be cut into the same number
 * of pieces by both; an axis of size 1 is broadcast.  Output shards are listed
 * row-major over the output axes; shard k lives on the devices that hold both
 * input shards it is computed from.
 *   out_shape[r]          the broadcast output shape
 *   *num_shards_out       S, the number of output shards
 *   boxes[(k*r + a)*2 ..] (start, stop) on axis a, for k < min(S, max_shards)
 *   dev_offsets[k]        for k <= min(S, max_shards): shard k's devices are
 *                         devices[dev_offsets[k] .. dev_offsets[k+1]), sorted;
 *                         entries at or beyond max_devices are not written
 * boxes, dev_offsets and devices may be NULL.
 * Errors: TP_ERR_ARG (NULL outputs, shapes that do not broadcast), everything
 *         tp_layout_plan reports for either layout, TP_ERR_SPEC (a
 *         non-broadcast axis cut differently; an output shard whose input
 *         shards share no device).
 */
int tp_check_broadcast_binary(const int64_t *shape1, int64_t ndim1, const tp_layout *layout1,
                              const int64_t *shape2, int64_t ndim2, const tp_layout *layout2,
                              int64_t *out_shape, int64_t *num_shards_out, int64_t *boxes, int64_t max_shards,
                              int64_t *dev_offsets, int64_t *devices, int64_t max_devices);

/*
 * dims_mapping of Z = matmul(X[..., M, K], Y[..., K, N]) on a mesh of mesh_ndim
 * dims ([SPMD] rules for computing operators: einsum ...mk,...kn->...mn, merge
 * the inputs' mappings per axis, read the output's off the merged axes).  Host
 * only.  x_map and y_map have ndim >= 2 entries (leading batch axes, then the
 * matrix axes); values in [-1, mesh_ndim-1].  On success z_map[ndim] holds the
 * output mapping and *partial_mesh_dim the mesh dim that cuts the contracted
 * axis K (the output is then a partial sum over it), or -1.
 * Errors: TP_ERR_ARG (NULL pointers, ndim or mesh_ndim out of range),
 *         TP_ERR_SPEC (a value out of range, a mesh dim used twice in one
 *         mapping, an axis the two inputs cut by different mesh dims, which
 *         needs a reshard, or one mesh dim cutting two einsum axes).
 */
int tp_infer_matmul_dims_mapping(const int64_t *x_map, const int64_t *y_map, int64_t ndim, int64_t mesh_ndim,
                                 int64_t *z_map, int64_t *partial_mesh_dim);

/* ---- shard materialisation ------------------------------------------- */
/*
 * Split and replicate a row-major tensor src[shape] (dtype TP_F32 or TP_BF16;
 * bits are copied, never converted) into per-device row-major buffers:
 * dst[d] receives device d's shard, for every device d named by the layout
 * ([ONNX] "Sharding as a Split"; [SBP] "SBP": split pieces concatenate back to
 * the tensor, broadcast pieces equal it; [SPMD] "dims_mapping").  Each shard
 * is read once and written to every device of its group.
 *   dst: host array of num_dst device pointers, indexed by physical device
 *        id; num_dst must exceed every id the layout names; entries of ids the
 *        layout does not name are ignored (may be NULL); named ones must be
 *        non-NULL and must not overlap src or each other.
 * Errors: as tp_layout_plan, plus TP_ERR_ARG for a null src, a bad dtype, a
 *         too-small num_dst or a NULL dst of a named device; TP_ERR_HIP.
 */
int tp_shard_materialize(const void *src, int32_t dtype, const int64_t *shape, int64_t ndim,
                         const tp_layout *layout, void *const *dst, int64_t num_dst,
                         tp_stream_t stream);

/* One tensor of tp_shard_materialize_batch: the arguments of
 * tp_shard_materialize, and optionally one device's share alone. */
typedef struct {
  const void *src;
  int32_t dtype;
  const int64_t *shape;
  int64_t ndim;
  const tp_layout *layout;
  void *const *dst;
  int64_t num_dst;
  int32_t local_only;    /* 0 (a zero-initialised item): every device the layout names
                            receives its shard, as tp_shard_materialize.  1: only
                            local_device's shard is read and written, the share one
                            process materialises for its own device in SPMD execution
                            ([SPMD] "dims_mapping": each process holds its own slice);
                            the other dst entries are ignored (may be NULL) */
  int64_t local_device;  /* with local_only: a device id the layout names, < num_dst */
} tp_materialize_item;

/*
 * tp_shard_materialize for several tensors (each with its own layout and
 * destinations), e.g. the column and row cuts of both weights of a layer.
 * Every item is validated before anything is enqueued; the shards are then
 * packed into as few launches as possible (shards of up to four tensors share
 * one), which saves the fixed cost of a launch per tensor.  No destination
 * may overlap another destination or any item's source.  num_items = 0 is a
 * no-op.
 * Errors: as tp_shard_materialize, the message naming the item.
 */
int tp_shard_materialize_batch(const tp_materialize_item *items, int64_t num_items, tp_stream_t stream);

/* ---- gather (the inverse of materialisation) ------------------------- */
/*
 * Assemble the full row-major tensor of shape[ndim] from its per-device shards
 * and write it to each of num_out outputs: the all-gather of a layout ([SBP]
 * "SBP": split pieces concatenate back to the logical tensor, broadcast pieces
 * are copies of it; [CAI] section 5.1, gather_output: the column layer's
 * split outputs all-gathered along the last axis; section 5.3: the
 * sequence-parallel input all-gathered along the sequence axis).
 *   src: host array of num_src device pointers, indexed by physical device id
 *        as in tp_shard_materialize; src[d] holds device d's shard row-major.
 *        Each distinct shard is read once, from the first device its group
 *        lists (replicas are copies by definition and are not compared);
 *        entries of other devices are not read and may be NULL.
 *   out: host array of num_out >= 1 device pointers, each receiving the whole
 *        tensor; outputs must not overlap each other or a shard that is read.
 * Bits are copied, never converted (dtype TP_F32 or TP_BF16).
 * Errors: as tp_layout_plan, plus TP_ERR_ARG for a null or too-short src, a
 *         NULL src of a read device, num_out < 1, a NULL or overlapping
 *         output, a bad dtype; TP_ERR_HIP.
 */
int tp_shard_gather(const void *const *src, int64_t num_src, int32_t dtype, const int64_t *shape,
                    int64_t ndim, const tp_layout *layout, void *const *out, int64_t num_out,
                    tp_stream_t stream);

/* ---- partial-sum reduction ------------------------------------------- */
enum { TP_REDUCE_FULL = 0, TP_REDUCE_SPLIT = 1 };
/*
 * Sum P fp32 partial buffers elementwise ([SBP] "SBP": partial-sum pieces add
 * up to the tensor; [CAI] section 2.1: the row-parallel output is summed by
 * one all-reduce; sections 3 and 5.3: reduce-scatter leaves rank j block j).
 * The sum is taken in fp32 in ascending p: ((p0 + p1) + p2) + ...
 *   partials: host array of P device pointers, each a [rows, cols] matrix with
 *             row stride ld_in (elements, >= cols).
 *   TP_REDUCE_FULL : num_splits must be 1; out[0] is [rows, cols], stride ld_out.
 *                    out[0] may equal partials[0] (in place); no other overlap.
 *   TP_REDUCE_SPLIT: num_splits = S must divide rows; out[j] (j < S) receives
 *                    rows [j*rows/S, (j+1)*rows/S) of the sum, stride ld_out;
 *                    outputs must not overlap inputs.
 *   1 <= P <= 64, 1 <= S <= 64; rows, cols >= 0 (0 = nothing to do).
 * Errors: TP_ERR_ARG, TP_ERR_INDIVISIBLE, TP_ERR_UNSUPPORTED (P or S > 64), TP_ERR_HIP.
 */
int tp_partial_reduce(const float *const *partials, int64_t P, int64_t rows, int64_t cols,
                      int64_t ld_in, int32_t mode, int64_t num_splits, float *const *out,
                      int64_t ld_out, tp_stream_t stream);

/* Reduction operator of a partial tensor ([SBP] "SBP": besides sum, min and
 * max also apply to partial values). */
enum { TP_REDUCE_OP_SUM = 0, TP_REDUCE_OP_MAX = 1, TP_REDUCE_OP_MIN = 2 };

/*
 * tp_partial_reduce with a choice of operator and an optional bias:
 *   out = op over p of partials[p]  (+ bias[col], added once to the reduced value)
 * MAX / MIN take fmaxf / fminf (a NaN element loses to a number); SUM is the
 * fp32 sum in ascending p.  bias: NULL or a device array of `cols` fp32 values,
 * the row-parallel layer's bias, which acts on the full output ([CAI] section
 * 5.2), so it is added after the reduction and not per partial.  bias must not
 * overlap any output.  Other arguments, conventions and errors as
 * tp_partial_reduce; TP_ERR_ARG for an unknown op.
 */
int tp_partial_reduce_ex(const float *const *partials, int64_t P, int64_t rows, int64_t cols,
                         int64_t ld_in, int32_t mode, int64_t num_splits, float *const *out,
                         int64_t ld_out, int32_t op, const float *bias, tp_stream_t stream);

/* ---- one rank's column->row MLP ------------------------------------ */
enum { TP_ACT_NONE = 0, TP_ACT_GELU_ERF = 1 };

typedef struct {
  int32_t dtype;     /* TP_BF16: X, A_i, B_i, Y_ws bf16 (fp32 accumulate);
                        TP_F32 : all fp32 */
  int32_t act;       /* TP_ACT_GELU_ERF: GeLU(x) = x/2 (1 + erf(x/sqrt 2)) applied to
                        the fp32 accumulator of X A_i (the pages never define GeLU;
                        the exact erf form is the reading taken); TP_ACT_NONE */
  int64_t M, H, F;   /* X[M,H], A_i[H,F], B_i[F,H]; all >= 1 */
  const void *X;     /* [M, H] row-major, replicated input of every rank (NULL only
                        with X_shards, below) */
  const void *A_i;   /* [H, F] row-major: this rank's column slice of A ([CAI] section 2) */
  const void *B_i;   /* [F, H] row-major: this rank's row slice of B ([CAI] section 2.1) */
  void *Y_ws;        /* [M, F] caller-owned workspace; on completion holds
                        act(X A_i) rounded to dtype (RNE) */
  float *Z_i;        /* [M, H] fp32: this rank's partial Y B_i (no communication,
                        [DOM] RowParallelLinearNoComm) */
  int64_t row_chunks;/* R >= 1, divides M: independent row chunks of X ([DOM] "row-wise
                        split of inputs X") */
  int64_t col_chunks;/* C >= 1, divides H: column blocks of B_i ([DOM] "column-wise split
                        of weights B") */
  int64_t P;         /* tensor-parallel degree, 1..64; 1 = no reduction */
  const float *const *peer_partials; /* host array of P-1 device pointers, each [M,H]
                        fp32: the partials of virtual ranks 1..P-1 */
  float *Z_out;      /* [M,H] fp32, required when P > 1: Z_i + sum of peers, written
                        block (r,c) by block on s_reduce; may equal Z_i */
  int64_t reduce_workgroups; /* upper bound on the reduce kernel's workgroups when it runs
                        beside the GEMMs on s_reduce (it then shares the CUs with
                        them); 0 = library default: 256 beside a GEMM, a one-shot
                        grid for the final block, which nothing follows; >= 0 */
  void *H_out;       /* optional [M, F] (dtype): X A_i before the activation, rounded to
                        dtype (RNE), kept for the backward pass; NULL = not stored.
                        Must be NULL when act = TP_ACT_NONE (H would equal Y). */
  const float *bias; /* optional [H] fp32: the row-parallel layer's bias, added once to the
                        full sum ([CAI] section 5.2), so Z_out = sum of partials + bias;
                        NULL = none.  Needs Z_out or Z_split (for any P); Z_i stays
                        bias-free. */
  /* Sequence parallelism ([CAI] section 5.3: the column layer all-gathers its
   * input along the sequence axis, the row layer reduce-scatters its output
   * instead of all-reducing it).  X and Z are [M, H] with the token (sequence)
   * axis outermost, so sequence block j is rows [j*M/S, (j+1)*M/S). */
  int64_t seq_splits;/* S: 0 or 1 = off; else 2..64, divides M, and the row chunks and
                        the sequence blocks nest (M/R divides M/S or M/S divides M/R) */
  const void *const *X_shards; /* optional host array of S device pointers, each [M/S, H]
                        (dtype): sequence block j of the input.  When set the call
                        all-gathers them into X, which is then a caller-owned
                        [M, H] workspace the call writes, chunk r on s_reduce before
                        chunk r's first GEMM on s_compute reads it; or X is NULL and
                        GEMM1 reads the blocks where they lie (the all-gather folded
                        into its operand loads; nothing is gathered).  That needs
                        each row chunk inside one block, or, where a chunk spans
                        blocks, bf16, 16-byte aligned blocks of a multiple of 256
                        rows, at most 8 per chunk, H a multiple of 32 (else
                        TP_ERR_UNSUPPORTED) */
  float *const *Z_split; /* optional host array of S device pointers, each [M/S, H] fp32:
                        the reduce-scattered output, block j = rows [j*M/S, (j+1)*M/S)
                        of Z_i + peers (+ bias).  Replaces Z_out, which must be NULL. */
  void *X_next;      /* optional [M, H] in dtype: the full sum (+ bias) rounded to dtype
                        (RNE for bf16), written by the same reduction, i.e. the next
                        layer's input; Z_out may then be NULL.  Not with Z_split. */
  int32_t reduce_fusion; /* TP_REDUCE_FUSION_AUTO (0): where a block's reduction would
                        run with nothing beside it (the serial schedule, or the final
                        block of the two-stream one), or beside GEMMs too short to
                        cover it (bf16, tp_colrow_mlp only: its bytes at 6 TB/s take
                        more than 3/4 of the next block's GEMM2, or of the next
                        chunk's GEMM1 and first GEMM2, at 1.2 PFLOP/s), GEMM2 adds
                        the peers' partials and the bias in its epilogue and writes
                        Z_out / X_next itself.
                        Taken for P <= 4 and Z_out or a Z_split whose chunk spans at
                        most 4 sequence blocks on blocks of fewer than 256 output
                        tiles of 128 x 128 (bf16: 16-byte aligned rows, F a multiple
                        of 32), and for bf16 blocks of at least that many tiles with
                        P <= 16, the same outputs, 16-byte aligned rows and F a
                        multiple of 64; otherwise, and
                        always with TP_REDUCE_FUSION_OFF (1), a separate reduction
                        kernel runs.  Both give the same bits. */
  int64_t A_ld;      /* row stride of A_i in elements; 0 = contiguous.  TP_WEIGHTS_MATH:
                        with A_ld = P*F, A_i may point into the full A [H, P*F] at
                        column i*F: the rank consumes its column shard in place, as
                        the column-parallel layer uses its weight shard ([CAI]
                        section 5.1), with no copy.  Must be >= F (MATH) or >= H
                        (LINEAR). */
  int32_t weight_layout; /* TP_WEIGHTS_MATH (0): A_i is [H, F] and B_i [F, H] (Y = X A_i,
                        Z_i = Y B_i).  TP_WEIGHTS_LINEAR (1): both as a linear layer
                        stores its weight, [out, in]: A_i is [F, H] (A_i^T) and B_i
                        [H, F] (B_i^T); the GEMMs read them k-contiguous, with no
                        transpose pass.  Same results, bit for bit. */
  int64_t B_ld;      /* row stride of B_i in elements; 0 = contiguous.  TP_WEIGHTS_LINEAR:
                        with B_ld = P*F, B_i may point into the full [H, P*F] weight
                        at column i*F (the row-parallel layer's shard, in place).
                        Must be >= H (MATH) or >= F (LINEAR). */
} tp_mlp_args;

enum { TP_WEIGHTS_MATH = 0, TP_WEIGHTS_LINEAR = 1 };

enum { TP_REDUCE_FUSION_AUTO = 0, TP_REDUCE_FUSION_OFF = 1 };

/*
 * Enqueue one rank's MLP share: for each row chunk r, Y[r] = act(X[r] A_i) on
 * s_compute; for each column block c, Z_i[r,c] = Y[r] B_i[:,c] on s_compute;
 * when P > 1, s_reduce waits for block (r,c) and reduces it into Z_out while
 * s_compute moves on to the next block ([DOM] "forward": the all-reduce of one
 * micro-batch hides behind the next one's GeMM-GeLU-GeMM).  Before returning,
 * s_compute is made to wait for s_reduce, so completion of s_compute means the
 * whole call is done.  s_reduce may equal s_compute (serial schedule); with a
 * single block (R = C = 1) the reduce runs on s_compute, as nothing could
 * overlap it, and so it does (in GEMM2's epilogue, reduce_fusion AUTO) for a
 * block whose reduction the next GEMMs are too short to cover; where that
 * leaves s_reduce nothing to do the call keeps to s_compute.  GEMM1 runs
 * once over all M rows (larger tiles, and no sum beside it) ahead of the
 * blocks' GEMM2s wherever that leaves every block's sum where it would be
 * with a GEMM1 per chunk; on s_compute alone the chunks overlap nothing, so
 * each keeps its GEMM2 where its sum folds into that GEMM2, and otherwise the
 * layer runs as the single block (R = C = 1).  The
 * calls are capturable into a HIP graph (no memsets, no allocation, no host
 * synchronisation).
 * Chunking never changes a result bit: each output element is accumulated in
 * the same order whatever R and C are.  With sequence parallelism (S > 1) the
 * gather of chunk r+1's input rows runs on s_reduce beside chunk r's GEMMs,
 * and each block's reduction is written to the sequence blocks it covers.
 * Errors: TP_ERR_ARG (null or overlapping buffers, bad dtype/act, sizes < 1,
 *         P or S out of range, X_shards or Z_split without S > 1, Z_out with
 *         Z_split), TP_ERR_INDIVISIBLE (R does not divide M, C does not divide
 *         H, S does not divide M), TP_ERR_UNSUPPORTED (row chunks and sequence
 *         blocks that do not nest), TP_ERR_HIP.
 */
int tp_colrow_mlp(const tp_mlp_args *args, tp_stream_t s_compute, tp_stream_t s_reduce);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * tp_colrow_mlp with args->Y_ws = NULL, the hidden activations Y kept instead
 * in a fixed 32 MiB device array of the library, one per GPU (held from module
 * load until the process ends), which every row chunk reuses in turn.  Y is
 * therefore not returned; every other argument, output and result bit is as in
 * tp_colrow_mlp.  The call allocates nothing (no hipMalloc, no hipFree); the
 * first call on a device looks up that device's array, and the first call that
 * needs two streams creates the thread's reusable HIP events, as tp_colrow_mlp
 * does.  All calls on one GPU share its array: calls that overlap on one GPU
 * (other streams, other threads) race.
 * Errors: those of tp_colrow_mlp; TP_ERR_ARG for a non-NULL Y_ws;
 *         TP_ERR_UNSUPPORTED when one row chunk of Y, (M/R) * F elements of the
 *         dtype, exceeds 32 MiB (then nothing is enqueued).
 */
int tp_colrow_mlp_noalloc(const tp_mlp_args *args, tp_stream_t s_compute, tp_stream_t s_reduce);

/*
 * Enqueue num_layers forward layers, layer l+1 reading layer l's output
 * (layers[l].X_next == layers[l+1].X, same dtype, M, H and row_chunks), with
 * Domino's inter-layer overlap ([DOM] "row-wise split of inputs X": no data
 * dependency across row chunks, so the reduction of layer l's chunk r runs on
 * s_reduce beside the GEMMs of layer l+1's earlier chunks; DominoTransformer's
 * inter_layer_overlap_forward).  Chunk r of layer l+1 waits only for chunk r
 * of layer l.  Layers that would each keep to s_compute alone (every block's
 * sum folded into its GEMM2's epilogue, as tp_colrow_mlp decides) have nothing
 * to overlap and run one after another, each as tp_colrow_mlp runs it on one
 * stream.  Each layer is validated as by tp_colrow_mlp (sequence
 * parallelism is not supported inside a stack); buffers other than a layer's
 * own inputs and outputs may be shared between layers (one Y_ws for all, X
 * buffers used in turn), since each chunk's reuse is ordered by the schedule.
 * The result of every layer equals what tp_colrow_mlp gives it, bit for bit.
 * Errors: as tp_colrow_mlp, prefixed with the layer; TP_ERR_ARG for a broken
 *         link between layers; TP_ERR_UNSUPPORTED for seq_splits > 1.
 */
int tp_colrow_mlp_stack(const tp_mlp_args *layers, int64_t num_layers, tp_stream_t s_compute, tp_stream_t s_reduce);

/* ---- backward of one rank's column->row MLP ------------------------- */
typedef struct {
  int32_t dtype;     /* as in the forward: TP_BF16 (X, A_i, B_i, H_i, Y_i, dZ, dH_ws bf16,
                        fp32 accumulate) or TP_F32 (all fp32) */
  int32_t act;       /* the forward's activation */
  int64_t M, H, F;   /* X[M,H], A_i[H,F], B_i[F,H]; all >= 1 */
  const void *X;     /* [M, H] the forward's input */
  const void *A_i;   /* [H, F] this rank's column slice of A */
  const void *B_i;   /* [F, H] this rank's row slice of B */
  const void *H_i;   /* [M, F] the forward's pre-activation X A_i (its H_out); required for
                        TP_ACT_GELU_ERF, ignored for TP_ACT_NONE */
  const void *Y_i;   /* [M, F] the forward's Y = act(X A_i) (its Y_ws) */
  const void *dZ;    /* [M, H] gradient of the loss with respect to the MLP output Z (the
                        sum over ranks, so the same on every rank) */
  void *dH_ws;       /* [M, F] caller-owned workspace; on completion holds the gradient at
                        the pre-activation, (dZ B_i^T) * act'(H_i), rounded to dtype */
  float *dX_i;       /* [M, H] fp32: this rank's partial input gradient dH A_i^T ([CAI]
                        section 2.2: the column-parallel layer's input gradient is a
                        partial that must be summed over ranks) */
  float *dA_i;       /* [H, F] fp32 weight gradient X^T dH */
  float *dB_i;       /* [F, H] fp32 weight gradient Y_i^T dZ */
  int32_t accumulate;/* 1: dA_i and dB_i are added to (gradient accumulation across
                        micro-batches); 0: overwritten */
  int64_t row_chunks;/* R >= 1, divides M: independent row chunks ([DOM] micro-batches) */
  int64_t P;         /* tensor-parallel degree, 1..64; 1 = no reduction of dX */
  const float *const *peer_dX; /* host array of P-1 device pointers, each [M,H] fp32: the
                        input-gradient partials of virtual ranks 1..P-1 */
  float *dX_out;     /* [M,H] fp32, required when P > 1: dX_i + sum of peers, written chunk
                        by chunk on s_reduce; may equal dX_i */
  int64_t reduce_workgroups; /* as in the forward; 0 = library default; >= 0 */
  /* Sequence parallelism ([CAI] section 5.3: in the backward the row layer
   * all-gathers the output gradient and the column layer reduce-scatters the
   * input gradient).  X is the forward's gathered [M, H] input. */
  int64_t seq_splits;/* S: 0 or 1 = off; else as in the forward */
  const void *const *dZ_shards; /* optional host array of S device pointers, each [M/S, H]
                        (dtype): sequence block j of dZ.  When set the call all-gathers
                        them into dZ, which is then a caller-owned [M, H] workspace */
  float *const *dX_split; /* optional host array of S device pointers, each [M/S, H] fp32:
                        the reduce-scattered input gradient (replaces dX_out, which
                        must be NULL) */
  int32_t reduce_fusion; /* TP_REDUCE_FUSION_AUTO (0): the dX GEMM adds the peers' input
                        gradients in its epilogue and writes dX_out itself, and the
                        call runs on s_compute alone, when every chunk qualifies:
                        bf16, P <= 4, dX_out (not dX_split), 16-byte aligned rows,
                        F a multiple of 32 and fewer than 256 output tiles of
                        128 x 128 per chunk (small layers, whose GEMMs are too short
                        for the hand-off to s_reduce to pay); otherwise, and always
                        with TP_REDUCE_FUSION_OFF (1), the reduction runs on
                        s_reduce beside the later GEMMs.  Same bits. */
  int32_t weight_layout; /* TP_WEIGHTS_MATH (0): A_i [H, F], B_i [F, H], and dA_i, dB_i
                        written in that layout.  TP_WEIGHTS_LINEAR (1): A_i [F, H],
                        B_i [H, F] (a linear layer's [out, in]), and dA_i [F, H],
                        dB_i [H, F] likewise.  All contiguous. */
} tp_mlp_bwd_args;

/*
 * Enqueue the backward of one rank's MLP share ([CAI] section 2.2; [DOM]
 * "backward": each gradient GEMM splits into an input-gradient GEMM and an
 * independent weight-gradient GEMM, so the reduction of an input gradient hides
 * behind GEMMs that do not depend on it).  For each row chunk r, on s_compute:
 * dH[r] = (dZ[r] B_i^T) * act'(H_i[r]) (one GEMM, the derivative applied to its
 * fp32 accumulator), dX_i[r] = dH[r] A_i^T; then, when P > 1, s_reduce waits
 * for chunk r and reduces dX[r] into dX_out while s_compute moves on to chunk
 * r+1, and after the last chunk to dA_i (+)= X^T dH and dB_i (+)= Y_i^T dZ over
 * all M rows, one pass each.  Each weight-gradient element is accumulated over
 * the rows in the same order whatever R is, so the result does not depend on R.
 * Small layers instead sum dX over the ranks in the dX GEMM's epilogue on
 * s_compute (reduce_fusion), with the same bits.
 * Before returning, s_compute waits for s_reduce.  Capturable into a HIP graph.
 * With sequence parallelism, chunk r's rows of dZ are gathered on s_reduce
 * ahead of chunk r's GEMMs and dX is reduce-scattered into dX_split.
 * Errors: TP_ERR_ARG (null or overlapping buffers, bad dtype/act, sizes < 1,
 *         P or S out of range, dZ_shards or dX_split without S > 1, dX_out with
 *         dX_split), TP_ERR_INDIVISIBLE (R or S does not divide M),
 *         TP_ERR_UNSUPPORTED (row chunks and sequence blocks that do not nest),
 *         TP_ERR_HIP.
 */
int tp_colrow_mlp_backward(const tp_mlp_bwd_args *args, tp_stream_t s_compute, tp_stream_t s_reduce);

/* ---- per-kernel timing (measurement support) ---------------------------- */
/* Kernel families timed by the optional instrumentation below: the forward's
 * GEMMs, the backward's input-gradient GEMMs (dH and dX) and its
 * weight-gradient GEMMs (dA and dB), the gather kernel, GEMM2 with the
 * reduction folded into its epilogue and the dX GEMM with the input gradient's
 * reduction folded into its epilogue (both memory-bound: their work counts
 * bytes, the operands and the peers' partials read once and each output
 * written once).  TP_KERNEL_REDUCE_TAIL is the forward's last-block reduction
 * on a chunked two-stream schedule, which no GEMM runs beside (a one-shot
 * grid over the whole chip); every other reduction is TP_KERNEL_REDUCE. */
enum { TP_KERNEL_MATERIALIZE = 0, TP_KERNEL_GEMM1 = 1, TP_KERNEL_GEMM2 = 2, TP_KERNEL_REDUCE = 3,
       TP_KERNEL_GEMM_DGRAD = 4, TP_KERNEL_GEMM_WGRAD = 5, TP_KERNEL_GATHER = 6,
       TP_KERNEL_GEMM2_REDUCE = 7, TP_KERNEL_GEMM_DGRAD_REDUCE = 8, TP_KERNEL_REDUCE_TAIL = 9,
       TP_KERNEL_KINDS = 10 };

typedef struct {
  int64_t launches;  /* kernel launches timed since the last read */
  double total_ms;   /* sum of their durations (HIP events on the launching stream) */
  double min_ms, max_ms;
  double work;       /* algorithmic work of those launches: flops for GEMMs
                        (2 M N K), bytes for copies and reductions (each input
                        element read once plus each output element written once) */
} tp_kernel_stat;

/* Turn per-kernel timing on (1) or off (0) for calls made on the calling
 * thread.  While on, every kernel the library launches is bracketed by two
 * timing events recorded on its own stream.  Returns TP_OK. */
int tp_timing_enable(int32_t on);

/* Wait for every timed launch of the calling thread to finish, fold the
 * durations into stats[kind] for kind < TP_KERNEL_KINDS (stats must hold
 * TP_KERNEL_KINDS entries) and reset the counters.
 * Errors: TP_ERR_ARG (stats NULL), TP_ERR_HIP. */
int tp_timing_read(tp_kernel_stat *stats);

#ifdef __cplusplus
}
#endif

#endif /* TPSHARD_H */
