// GEMM launch interface used by the MLP scheduler.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace tpshard {

// C[M,N] = epilogue(A[M,K] * W[K,N]) with row strides in elements.
//   a_t = 0: A is stored [M][lda] (k contiguous);   a_t = 1: A is stored [K][lda] (m contiguous), i.e. A^T is given.
//   w_t = 0: W is stored [K][ldw] (n contiguous);   w_t = 1: W is stored [N][ldw] (k contiguous), i.e. W^T is given.
// C is stored [M][ldc].  A, W are bf16 for the bf16 epilogues and fp32 for the fp32 ones.
// The partial sum folded into an fp32-output epilogue (kEpiF32Red): with v the
// tile's result as stored in C, out = (((v + peer[0]) + peer[1]) + ...) + bias[n],
// the order of the separate reduction kernel, so the two agree bit for bit.
// Peers and lo are [M][ldc] like C; bias is indexed by column.  The fp32 sum
// goes to out[0] ([M][ldc]), or, reduce-scattered, row m to out[m / rows_per_out]
// at row m % rows_per_out (each [rows_per_out][ldc]).
// Two forms: on the small-tile path the peers' vectors stream in during the
// k loop (at most kMaxFusedPeers peers: their vectors sit beside the
// accumulators); on the 256-row tiles the epilogue stages each half tile
// through LDS and reads the peers' rows whole (at most kMaxEpiPeers peers).
constexpr int kMaxFusedPeers = 3;
constexpr int kMaxEpiPeers = 15;
constexpr int kMaxFusedOuts = 4;
struct EpiReduce {
  const float *peer[kMaxEpiPeers];
  float *out[kMaxFusedOuts];   // fp32 sum, or out[0] null for none; a single out may equal C
                               // (then C receives the sum only)
  const float *bias;           // or null
  void *lo;                    // copy of the sum in bf16 (RNE) or fp32, or null (single out only)
  int32_t np;                  // peers used (see the two forms above)
  int32_t lo_bf16;             // lo holds bf16 (else fp32)
  int32_t nout;                // outputs, 1..kMaxFusedOuts
  int32_t rows_per_out;        // rows of each output when nout > 1
};

// A (not transposed) may come as row blocks held apart, e.g. the sequence
// blocks of an all-gathered input read where they lie.
constexpr int kMaxABlocks = 8;

struct GemmArgs {
  const void *a;
  const void *w;
  void *c;
  int64_t M, N, K;
  int64_t lda, ldw, ldc;
  int a_t = 0, w_t = 0;
  // Second tensor of the epilogue, stored [M][ldaux] like C: the pre-activation
  // written by the saving GeLU epilogues, read by the GeLU-derivative ones.
  void *aux = nullptr;
  int64_t ldaux = 0;
  // fp32 outputs only: the accumulator starts from C's current contents
  // (C += A W, continuing the same k order), else from zero.
  int acc_init = 0;
  // kEpiF32Red only.
  EpiReduce red{};
  // a_blk_rows > 0: A's rows [j * a_blk_rows, (j + 1) * a_blk_rows) are the
  // rows of a_blk[j] ([a_blk_rows][lda] each) and `a` is unused.  DMA paths
  // only, A not transposed, a_blk_rows a multiple of 256 so that no tile
  // straddles two blocks (gemm_blocks_ok).
  const void *a_blk[kMaxABlocks] = {};
  int64_t a_blk_rows = 0;
};

enum {
  kEpiGeluBf16 = 0,      // bf16 inputs, C = bf16(GeLU(acc))
  kEpiIdentBf16 = 1,     // bf16 inputs, C = bf16(acc)
  kEpiF32 = 2,           // bf16 inputs, C = acc (fp32)
  kEpiGeluF32 = 3,       // fp32 inputs, C = GeLU(acc) (fp32)
  kEpiPlainF32 = 4,      // fp32 inputs, C = acc (fp32)
  kEpiGeluSaveBf16 = 5,  // bf16 inputs, C = bf16(GeLU(acc)), aux = bf16(acc)
  kEpiDGeluBf16 = 6,     // bf16 inputs, C = bf16(acc * GeLU'(aux)), aux bf16
  kEpiGeluSaveF32 = 7,   // fp32 inputs, C = GeLU(acc), aux = acc (fp32)
  kEpiDGeluF32 = 8,      // fp32 inputs, C = acc * GeLU'(aux), aux fp32
  kEpiF32Red = 9,        // bf16 inputs, C = acc (fp32) and the partial sum of red (A not transposed)
  kEpiF32RedSplit = 10,  // kEpiF32Red's reduce-scattered form (red.nout > 1); chosen inside gemm_launch
  kEpiPlainF32Red = 11,  // fp32 inputs, C = acc (fp32) and the partial sum of red (forward layout)
};

// Enqueues the GEMM on stream s; returns the launch status.
hipError_t gemm_launch(const GemmArgs& p, int epi, hipStream_t s);

// Whether gemm_launch takes p with kEpiF32Red: A not transposed, whole
// 16-byte vectors along every row of C, the peers, out, bias and lo; either
// on the small-tile path (fewer 128 x 128 tiles than CUs, K % 32 == 0, at most
// kMaxFusedPeers peers, a single output when W is transposed), where the
// peers' loads fit beside the accumulators without costing occupancy, or on
// the 256-row tiles (K % 64 == 0, operands within 32-bit offsets, at most
// kMaxEpiPeers peers), where the epilogue stages the tile through LDS.
bool gemm_red_ok(const GemmArgs& p);
// The same for kEpiPlainF32Red (the fp32 kernel, any alignment and size).
bool gemm_red_ok_f32(const GemmArgs& p);

// Up to 4 independent GEMMs in one launch (same results as one gemm_launch
// call each), for groups gemm_group_ok accepts: small weight-gradient problems
// that would each leave CUs idle.  gemm_launch_group returns
// hipErrorInvalidValue otherwise.
bool gemm_group_ok(const GemmArgs *ps, int n, int epi);
// Whether gemm_launch takes p's A as row blocks (a_blk_rows > 0) with epilogue
// epi: bf16 operands on the DMA paths (16-byte aligned blocks and rows, K a
// multiple of 32), A not transposed, a_blk_rows a multiple of 256, at most
// kMaxABlocks blocks.
bool gemm_blocks_ok(const GemmArgs& p, int epi);
hipError_t gemm_launch_group(const GemmArgs *ps, int n, int epi, hipStream_t s);

}  // namespace tpshard
