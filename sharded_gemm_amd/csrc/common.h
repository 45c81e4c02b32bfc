// Internal helpers shared by the library's translation units: thread-local
// error reporting and small argument checks.  Host code only.
#pragma once

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/tpshard.h"

namespace tpshard {

// Records a printf-style message as the calling thread's last error and
// returns `code`, so call sites can write `return fail(TP_ERR_ARG, "...")`.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// true iff [a, a+na) and [b, b+nb) (bytes) overlap; empty ranges never overlap.
inline bool overlaps(const void *a, int64_t na, const void *b, int64_t nb) {
  if (na <= 0 || nb <= 0) return false;
  auto pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + static_cast<uintptr_t>(nb) && pb < pa + static_cast<uintptr_t>(na);
}

inline int64_t dtype_size(int32_t dtype) {
  return dtype == TP_F32 ? 4 : dtype == TP_BF16 ? 2 : 0;
}

constexpr int kMaxRank = 8;

// tp_colrow_mlp's validation and enqueue.  With y_scratch, args->Y_ws must be
// NULL: once every argument has passed validation, y_scratch is asked for a
// device buffer of `bytes` (one row chunk of Y, [M/R, F]) that every chunk
// then reuses in turn (GEMM1 and GEMM2 of every chunk run in order on
// s_compute, so chunk r+1's GEMM1 only starts after chunk r's GEMM2 has read
// it); a status other than TP_OK from it is returned as is.
int colrow_mlp_run(const tp_mlp_args *a, tp_stream_t s_compute, tp_stream_t s_reduce,
                   int (*y_scratch)(int64_t bytes, void **out));

}  // namespace tpshard
