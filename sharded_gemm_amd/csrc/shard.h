// Launch interfaces of the layout and reduction kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.h"

namespace tpshard {

// Copies every shard of `plan` from src into dst[device] for each receiving
// device.  Arguments already validated.  Returns TP_OK or a negative status.
int shard_materialize_launch(const ShardPlan& plan, const void *src, int64_t esize, void *const *dst,
                             hipStream_t stream);

// One tensor of a batched materialisation.
struct MatJob {
  const ShardPlan *plan;
  const void *src;
  int64_t esize;
  void *const *dst;
};

// shard_materialize_launch for several tensors at once, packed into as few
// launches as the argument tables allow (shards of up to 4 tensors share one).
int shard_materialize_batch_launch(const MatJob *jobs, int njobs, hipStream_t stream);

// Writes the full tensor of `plan` into each of out[0..nout) from the shards:
// shard k is read from src[first device of its group].  Arguments already
// validated.  Returns TP_OK or a negative status.
int shard_gather_launch(const ShardPlan& plan, const void *const *src, int64_t esize, void *const *out, int64_t nout,
                        hipStream_t stream);

// out_row_block(row) <- op over p of partials[p][row, :] (+ bias[:]), ascending
// p, fp32; op 0 sum, 1 max, 2 min.  rows_per_out rows go to each out[j]; out[j]
// has row stride ld_out.  Arguments already validated (1 <= P <= 64,
// 1 <= nout <= 64).  max_wgs > 0 caps the grid (the kernel strides over the rest).
// lo (sum only, nout = 1): also write the result to lo[row * ld_lo + col] in
// lo_dtype (TP_BF16, rounded to nearest even, or TP_F32); out[0] may then be
// NULL to write lo alone.
int partial_reduce_launch(const float *const *partials, int P, int64_t rows, int64_t cols, int64_t ld_in,
                          float *const *out, int nout, int64_t rows_per_out, int64_t ld_out,
                          hipStream_t stream, int64_t max_wgs = 0, int op = 0, const float *bias = nullptr,
                          void *lo = nullptr, int lo_dtype = 0, int64_t ld_lo = 0);

}  // namespace tpshard
