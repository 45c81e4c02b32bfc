// GEMM launch interface used by the MLP scheduler.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tpshard {

// C[M,N] = epilogue(A[M,K] * W[K,N]); all row-major with the given row strides
// (in elements).  A, W are bf16 for the bf16 epilogues and fp32 for the fp32 ones.
struct GemmArgs {
  const void *a;
  const void *w;
  void *c;
  int64_t M, N, K;
  int64_t lda, ldw, ldc;
};

enum {
  kEpiGeluBf16 = 0,   // bf16 inputs, C = bf16(GeLU(acc))
  kEpiIdentBf16 = 1,  // bf16 inputs, C = bf16(acc)
  kEpiF32 = 2,        // bf16 inputs, C = acc (fp32)
  kEpiGeluF32 = 3,    // fp32 inputs, C = GeLU(acc) (fp32)
  kEpiPlainF32 = 4,   // fp32 inputs, C = acc (fp32)
};

// Enqueues the GEMM on stream s; returns the launch status.
hipError_t gemm_launch(const GemmArgs& p, int epi, hipStream_t s);

}  // namespace tpshard
