// The C ABI: argument validation, then enqueue.  Every entry point checks all
// of its arguments before it launches anything, so an error leaves outputs
// untouched.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <map>
#include <string>
#include <vector>

#include "common.h"
#include "gemm.h"
#include "plan.h"
#include "shard.h"
#include "timing.h"

namespace tpshard {

namespace {
thread_local std::string g_last_error;
}

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

void clear_error() { g_last_error.clear(); }

namespace {

constexpr int64_t kMaxP = 64;
constexpr int64_t kMaxSplits = 64;
constexpr int64_t kMaxLayers = 1024;
// Workgroups of a reduce that runs beside the GEMMs.  The large GEMM tiles fill
// every SIMD's register file, so the reduce mostly takes CUs between GEMM
// workgroups; one workgroup per CU back-fills those gaps without crowding out
// the next GEMM (measured on MI355X against 32 ... 16384).
constexpr int64_t kReduceBesideGemm = 256;
// GEMMs of fewer 128 x 128 output tiles than this (the CU count) are "small".
constexpr int64_t kSmallTiles = 256;
// Rates for weighing a block's reduction against the GEMMs it would run
// beside (MI355X, measured in the step: bf16 GEMMs at about 1.2 PFLOP/s, a
// reduction alone at about 6 TB/s), and the share of those GEMMs' time the
// reduction may take and still run beside them.
constexpr double kGemmFlopRate = 1.2e15, kReduceByteRate = 6.0e12, kBesideShare = 0.75;

int hip_fail(hipError_t e, const char *what) {
  return fail(TP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Events for the two-stream schedule, kept per device and reused across calls
// (a stream wait captures the event's state when it is enqueued, so an event
// may be re-recorded as soon as the wait that consumes it has been enqueued).
struct EventPool {
  std::map<int, std::vector<hipEvent_t>> by_device;
  ~EventPool() {
    for (auto& kv : by_device)
      for (hipEvent_t e : kv.second) (void)hipEventDestroy(e);
  }
};
thread_local EventPool g_events;

int get_events(size_t n, hipEvent_t **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  auto& v = g_events.by_device[dev];
  while (v.size() < n) {
    hipEvent_t ev;
    // Hand-offs between two streams of one device need a device-scope release
    // only (the partial is read by the next kernel on this device).
    e = hipEventCreateWithFlags(&ev, hipEventDisableTiming | hipEventReleaseToDevice);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreateWithFlags");
    v.push_back(ev);
  }
  *out = v.data();
  return TP_OK;
}

int64_t matrix_bytes(int64_t rows, int64_t cols, int64_t ld, int64_t esize) {
  if (rows <= 0 || cols <= 0) return 0;
  return ((rows - 1) * ld + cols) * esize;
}

struct Buf { const void *p; int64_t n; const char *name; };

// Every output is disjoint from every input and from every other output.
int check_disjoint(const std::vector<Buf>& ins, const std::vector<Buf>& outs) {
  for (size_t i = 0; i < outs.size(); ++i) {
    for (const Buf& in : ins)
      if (overlaps(outs[i].p, outs[i].n, in.p, in.n)) return fail(TP_ERR_ARG, "%s overlaps %s", outs[i].name, in.name);
    for (size_t j = 0; j < i; ++j)
      if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return fail(TP_ERR_ARG, "%s overlaps %s", outs[i].name, outs[j].name);
  }
  return TP_OK;
}

// Sequence blocks of an [M, .] tensor with the token axis outermost: S blocks
// of Ms rows.  S = 1 means sequence parallelism is off.
struct SeqSplit {
  int64_t S = 1, Ms = 0;
};

int check_seq(int64_t seq_splits, int64_t M, int64_t R, const void *shards, const void *split, const void *full_out,
              const char *shards_name, const char *split_name, const char *full_name, SeqSplit *sq) {
  if (seq_splits < 0 || seq_splits > kMaxSplits)
    return fail(TP_ERR_ARG, "seq_splits = %lld outside [0, %lld]", (long long)seq_splits, (long long)kMaxSplits);
  sq->S = seq_splits > 1 ? seq_splits : 1;
  sq->Ms = M / sq->S;
  if (sq->S == 1) {
    if (shards || split) return fail(TP_ERR_ARG, "%s and %s need seq_splits > 1", shards_name, split_name);
    return TP_OK;
  }
  if (M % sq->S) return fail(TP_ERR_INDIVISIBLE, "seq_splits %lld does not divide M = %lld", (long long)sq->S, (long long)M);
  const int64_t Mr = M / R;
  if (sq->Ms % Mr && Mr % sq->Ms)
    return fail(TP_ERR_UNSUPPORTED, "row chunks of %lld rows and sequence blocks of %lld rows do not nest", (long long)Mr, (long long)sq->Ms);
  if (split && full_out) return fail(TP_ERR_ARG, "%s and %s are exclusive", split_name, full_name);
  return TP_OK;
}

// Rows [r0, r0 + rows) of the full [M, H] tensor `full`, gathered from its
// sequence blocks of Ms rows.  The row range and the blocks nest, so it is
// max(1, rows / Ms) equal contiguous pieces: the gather of a [rows, H] tensor
// split along its first axis, piece k coming from block (r0 + k*seg) / Ms.
int gather_rows(const void *const *blocks, int64_t Ms, int64_t r0, int64_t rows, int64_t H, int64_t es, void *full,
                hipStream_t s) {
  const int64_t seg = std::min(rows, Ms), nseg = rows / seg;
  ShardPlan plan;
  plan.ndim = 2;
  plan.shape[0] = rows;
  plan.shape[1] = H;
  plan.extent[0] = seg;
  plan.extent[1] = H;
  std::vector<const void *> src(static_cast<size_t>(nseg));
  for (int64_t k = 0; k < nseg; ++k) {
    const int64_t g = r0 + k * seg, j = g / Ms;
    src[k] = static_cast<const char *>(blocks[j]) + (g - j * Ms) * H * es;
    plan.offset.push_back(k * seg);
    plan.offset.push_back(0);
    plan.devices.push_back({k});
  }
  plan.max_device = nseg - 1;
  void *dst = static_cast<char *>(full) + r0 * H * es;
  return shard_gather_launch(plan, src.data(), es, &dst, 1, s);
}

// Reduce rows [r0, r0 + rows) x columns [c0, c0 + cols) of the P partials
// (row stride ld) into the full output, or into the sequence blocks of Ms rows
// the row range covers (the reduce-scatter).  `full` may be NULL when `lo`
// (the same rows of a second full-size output in lo_dtype, row stride ld) takes
// the result instead.
int reduce_rows(const float *const *parts, int64_t P, int64_t r0, int64_t rows, int64_t c0, int64_t cols, int64_t ld,
                float *full, float *const *split, int64_t Ms, hipStream_t s, int64_t max_wgs, const float *bias,
                void *lo = nullptr, int lo_dtype = 0, int kind = TP_KERNEL_REDUCE) {
  std::vector<float *> dst;
  int64_t per = rows;
  if (!split) {
    dst.push_back(full ? full + r0 * ld + c0 : nullptr);
  } else {
    per = std::min(rows, Ms);
    for (int64_t k = 0; k < rows / per; ++k) {
      const int64_t g = r0 + k * per, j = g / Ms;
      dst.push_back(split[j] + (g - j * Ms) * ld + c0);
    }
  }
  void *lo_at = lo ? static_cast<char *>(lo) + (r0 * ld + c0) * dtype_size(lo_dtype) : nullptr;
  hipEvent_t t1 = timing_begin(s);
  const int rc = partial_reduce_launch(parts, static_cast<int>(P), rows, cols, ld, dst.data(), static_cast<int>(dst.size()),
                                       per, ld, s, max_wgs, TP_REDUCE_OP_SUM, bias, lo_at, lo_dtype, ld);
  if (rc != TP_OK) return rc;
  const double out_bytes = (full || split ? 4.0 : 0.0) + (lo ? static_cast<double>(dtype_size(lo_dtype)) : 0.0);
  timing_end(t1, s, kind, (4.0 * P + out_bytes) * rows * cols);
  return TP_OK;
}

// One forward layer, validated: sizes, the chunking and what the call writes.
struct MlpPlan {
  int64_t es = 0, M = 0, H = 0, F = 0, R = 1, C = 1, Mr = 0, Hc = 0;
  bool gather = false, reduce = false;
  // X is NULL and GEMM1 reads the sequence blocks X_shards where they lie.
  bool x_in_place = false;
  // TP_WEIGHTS_LINEAR: A_i, B_i stored [out, in] (k-contiguous for the GEMMs);
  // their row strides.
  bool w_linear = false;
  int64_t lda = 0, ldb = 0;
  // Y_ws holds one row chunk ([M/R, F]) that every chunk reuses in turn.
  bool y_chunk = false;
  int epi1 = 0, epi2 = 0;
  SeqSplit sq;
};

// Chunk r's Y: its own rows of Y_ws, or the one chunk-sized Y_ws, which
// chunk r+1's GEMM1 may overwrite once chunk r's GEMM2 (earlier on s0) has read it.
char *chunk_y(const tp_mlp_args *a, const MlpPlan& pl, int64_t r) {
  return static_cast<char *>(a->Y_ws) + (pl.y_chunk ? 0 : r * pl.Mr * pl.F * pl.es);
}

// GEMM1 of row chunk r: Y[r] = act(X[r] A_i).  X[r] is rows of X, or, with X
// NULL, the sequence blocks where they lie: at an offset into the one block
// that holds the chunk, or the chunk's blocks as A's row blocks.
GemmArgs chunk_gemm1(const tp_mlp_args *a, const MlpPlan& pl, int64_t r) {
  const int64_t es = pl.es, H = pl.H, F = pl.F, Mr = pl.Mr;
  GemmArgs g1{nullptr, a->A_i, chunk_y(a, pl, r), Mr, F, H, H, pl.lda, F};
  g1.w_t = pl.w_linear ? 1 : 0;
  if (!pl.x_in_place) {
    g1.a = static_cast<const char *>(a->X) + r * Mr * H * es;
  } else {
    const int64_t Ms = pl.sq.Ms, g0 = r * Mr, j0 = g0 / Ms;
    if (Mr <= Ms) {
      g1.a = static_cast<const char *>(a->X_shards[j0]) + (g0 - j0 * Ms) * H * es;
    } else {
      g1.a_blk_rows = Ms;
      for (int64_t k = 0; k < Mr / Ms && k < kMaxABlocks; ++k) g1.a_blk[k] = a->X_shards[j0 + k];
    }
  }
  if (a->H_out) {
    g1.aux = static_cast<char *>(a->H_out) + r * Mr * F * es;
    g1.ldaux = F;
  }
  return g1;
}

int validate_mlp(const tp_mlp_args *a, MlpPlan *pl, bool y_chunk = false) {
  if (!a) return fail(TP_ERR_ARG, "args is NULL");
  const int64_t es = dtype_size(a->dtype);
  if (!es) return fail(TP_ERR_ARG, "unknown dtype %d", a->dtype);
  if (a->act != TP_ACT_NONE && a->act != TP_ACT_GELU_ERF) return fail(TP_ERR_ARG, "unknown act %d", a->act);
  if (a->M < 1 || a->H < 1 || a->F < 1) return fail(TP_ERR_ARG, "M, H, F must be >= 1");
  if (!a->A_i || !a->B_i || !a->Z_i) return fail(TP_ERR_ARG, "A_i, B_i and Z_i must be non-NULL");
  if (!a->X && !a->X_shards)
    return fail(TP_ERR_ARG, "X must be non-NULL (or NULL with X_shards: GEMM1 then reads the blocks where they lie)");
  if (y_chunk && a->Y_ws) return fail(TP_ERR_ARG, "Y_ws must be NULL: this entry point keeps Y in its own scratch");
  if (!y_chunk && !a->Y_ws) return fail(TP_ERR_ARG, "Y_ws must be non-NULL");
  if (a->row_chunks < 1 || a->col_chunks < 1) return fail(TP_ERR_ARG, "row_chunks and col_chunks must be >= 1");
  if (a->M % a->row_chunks) return fail(TP_ERR_INDIVISIBLE, "row_chunks %lld does not divide M = %lld", (long long)a->row_chunks, (long long)a->M);
  if (a->H % a->col_chunks) return fail(TP_ERR_INDIVISIBLE, "col_chunks %lld does not divide H = %lld", (long long)a->col_chunks, (long long)a->H);
  if (a->P < 1 || a->P > kMaxP) return fail(TP_ERR_ARG, "P = %lld outside [1, %lld]", (long long)a->P, (long long)kMaxP);
  SeqSplit sq;
  int rc = check_seq(a->seq_splits, a->M, a->row_chunks, a->X_shards, a->Z_split, a->Z_out, "X_shards", "Z_split", "Z_out", &sq);
  if (rc != TP_OK) return rc;
  if (a->X_next && a->Z_split) return fail(TP_ERR_UNSUPPORTED, "X_next with a reduce-scattered output (Z_split)");
  const bool has_out = a->Z_out || a->Z_split || a->X_next;
  if (a->P > 1 && (!a->peer_partials || !has_out)) return fail(TP_ERR_ARG, "P > 1 needs peer_partials and Z_out (or Z_split, or X_next)");
  if (a->bias && !has_out) return fail(TP_ERR_ARG, "a bias needs Z_out, Z_split or X_next (it is added to the full sum)");
  if (a->reduce_workgroups < 0) return fail(TP_ERR_ARG, "reduce_workgroups < 0");
  if (a->reduce_fusion != TP_REDUCE_FUSION_AUTO && a->reduce_fusion != TP_REDUCE_FUSION_OFF)
    return fail(TP_ERR_ARG, "unknown reduce_fusion %d", a->reduce_fusion);
  if (a->H_out && a->act == TP_ACT_NONE) return fail(TP_ERR_ARG, "H_out needs an activation (it would equal Y)");
  const int64_t M = a->M, H = a->H, F = a->F;
  if (M >= (int64_t(1) << 31) || H >= (int64_t(1) << 31) || F >= (int64_t(1) << 31) ||
      (M / a->row_chunks) * (H / a->col_chunks) >= (int64_t(1) << 31))
    return fail(TP_ERR_UNSUPPORTED, "sizes exceed the 32-bit index range of the kernels");
  if (a->weight_layout != TP_WEIGHTS_MATH && a->weight_layout != TP_WEIGHTS_LINEAR)
    return fail(TP_ERR_ARG, "unknown weight_layout %d", a->weight_layout);
  const bool linear = a->weight_layout == TP_WEIGHTS_LINEAR;
  // A_i: [H][lda >= F] or, linear, [F][lda >= H]; B_i: [F][ldb >= H] or [H][ldb >= F].
  const int64_t a_rows = linear ? F : H, a_cols = linear ? H : F, b_rows = linear ? H : F, b_cols = linear ? F : H;
  if (a->A_ld != 0 && a->A_ld < a_cols)
    return fail(TP_ERR_ARG, "A_ld = %lld < %lld (the row length of A_i)", (long long)a->A_ld, (long long)a_cols);
  if (a->B_ld != 0 && a->B_ld < b_cols)
    return fail(TP_ERR_ARG, "B_ld = %lld < %lld (the row length of B_i)", (long long)a->B_ld, (long long)b_cols);
  const int64_t lda_w = a->A_ld ? a->A_ld : a_cols, ldb_w = a->B_ld ? a->B_ld : b_cols;
  if (lda_w >= (int64_t(1) << 31) || ldb_w >= (int64_t(1) << 31))
    return fail(TP_ERR_UNSUPPORTED, "A_ld or B_ld exceeds the 32-bit index range of the kernels");
  const int64_t bx = M * H * es, ba = matrix_bytes(a_rows, a_cols, lda_w, es), bb = matrix_bytes(b_rows, b_cols, ldb_w, es),
                by = M * F * es, bz = M * H * 4;
  const bool gather = a->X_shards != nullptr && a->X;
  std::vector<Buf> ins = {{a->A_i, ba, "A_i"}, {a->B_i, bb, "B_i"}};
  // (The library's own scratch, which replaces Y_ws when y_chunk, is disjoint
  // from every caller buffer.)
  std::vector<Buf> outs = {{a->Z_i, bz, "Z_i"}};
  if (!y_chunk) outs.push_back({a->Y_ws, by, "Y_ws"});
  if (a->X) (gather ? outs : ins).push_back({a->X, bx, "X"});
  if (a->X_shards) {
    for (int64_t j = 0; j < sq.S; ++j) {
      if (!a->X_shards[j]) return fail(TP_ERR_ARG, "X_shards[%lld] is NULL", (long long)j);
      ins.push_back({a->X_shards[j], sq.Ms * H * es, "X shard"});
    }
  }
  for (int64_t p = 1; p < a->P; ++p) {
    if (!a->peer_partials[p - 1]) return fail(TP_ERR_ARG, "peer_partials[%lld] is NULL", (long long)(p - 1));
    ins.push_back({a->peer_partials[p - 1], bz, "peer partial"});
  }
  if (a->bias) ins.push_back({a->bias, H * 4, "bias"});
  const bool reduce = a->P > 1 || a->bias || a->Z_split || a->X_next;
  if (reduce && a->Z_out && a->Z_out != a->Z_i) outs.push_back({a->Z_out, bz, "Z_out"});
  if (a->Z_split) {
    for (int64_t j = 0; j < sq.S; ++j) {
      if (!a->Z_split[j]) return fail(TP_ERR_ARG, "Z_split[%lld] is NULL", (long long)j);
      outs.push_back({a->Z_split[j], sq.Ms * H * 4, "Z_split block"});
    }
  }
  if (a->X_next) outs.push_back({a->X_next, bx, "X_next"});
  if (a->H_out) outs.push_back({a->H_out, by, "H_out"});
  if ((rc = check_disjoint(ins, outs)) != TP_OK) return rc;

  const bool bf16 = a->dtype == TP_BF16;
  const bool save = a->H_out != nullptr;
  pl->es = es;
  pl->M = M;
  pl->H = H;
  pl->F = F;
  pl->R = a->row_chunks;
  pl->C = a->col_chunks;
  pl->Mr = M / pl->R;
  pl->Hc = H / pl->C;
  pl->gather = gather;
  pl->reduce = reduce;
  pl->y_chunk = y_chunk;
  pl->sq = sq;
  pl->epi1 = bf16 ? (a->act == TP_ACT_GELU_ERF ? (save ? kEpiGeluSaveBf16 : kEpiGeluBf16) : kEpiIdentBf16)
                  : (a->act == TP_ACT_GELU_ERF ? (save ? kEpiGeluSaveF32 : kEpiGeluF32) : kEpiPlainF32);
  pl->epi2 = bf16 ? kEpiF32 : kEpiPlainF32;
  pl->w_linear = linear;
  pl->lda = lda_w;
  pl->ldb = ldb_w;
  pl->x_in_place = !a->X;
  if (pl->x_in_place) {
    // A row chunk inside one block is read at an offset; one that spans
    // blocks needs them as whole tiles' worth of rows on the DMA paths.
    for (int64_t r = 0; r < pl->R; ++r) {
      const GemmArgs g1 = chunk_gemm1(a, *pl, r);
      if (g1.a_blk_rows == 0) continue;
      if (pl->Mr / sq.Ms > kMaxABlocks || !gemm_blocks_ok(g1, pl->epi1))
        return fail(TP_ERR_UNSUPPORTED,
                    "X = NULL: row chunks of %lld rows span sequence blocks of %lld rows, which GEMM1 reads in place "
                    "only for bf16, 16-byte aligned blocks of a multiple of 256 rows, at most %d per chunk, and "
                    "H a multiple of 32",
                    (long long)pl->Mr, (long long)sq.Ms, kMaxABlocks);
    }
  }
  return TP_OK;
}

// GEMM2 of block (r, c): Z_i[r, c] = Y[r] B_i[:, c] (columns c of B_i; with
// linear weights the same block is rows c of B_i^T).
GemmArgs block_gemm2(const tp_mlp_args *a, const MlpPlan& pl, int64_t r, int64_t c) {
  const int64_t zoff = r * pl.Mr * pl.H + c * pl.Hc;
  const int64_t woff = pl.w_linear ? c * pl.Hc * pl.ldb : c * pl.Hc;
  GemmArgs g{chunk_y(a, pl, r), static_cast<const char *>(a->B_i) + woff * pl.es, a->Z_i + zoff,
             pl.Mr, pl.Hc, pl.F, pl.F, pl.ldb, pl.H};
  g.w_t = pl.w_linear ? 1 : 0;
  return g;
}

// Whether block (r, c)'s reduction folds into its GEMM2's epilogue, and if so
// that GEMM2 (*gr).  It does where the reduction would run with nothing beside
// it anyway (one stream, or the final block: `last` says nothing follows chunk
// r on s0): one launch fewer and no second read of the partial just written.
// It does so too on two streams where the GEMMs that s0 issues next (the next
// block's GEMM2, or the next chunk's GEMM1 and first GEMM2) are too short to
// cover it: beside them it would slow them by about its own length and still
// run past them (GPT-3 6.7B at TP = 8, R = 2: 604 MB of reduction beside
// 137 GFLOP; that step took 417 us on two streams against 388 us with each
// chunk's sum in GEMM2's epilogue).  Only where `weigh`: a stack of layers
// keeps every reduction it can beside the GEMMs (GPT-3 6.7B, two layers:
// 866 us so against 884-897 us with each chunk folded, whose epilogue then
// also writes the next layer's input).  The kernel must take the block as well
// (gemm_red_ok).
bool fused_block(const tp_mlp_args *a, const MlpPlan& pl, int64_t r, int64_t c, bool two, bool last, bool weigh,
                 GemmArgs *gr, bool g1_done = false) {
  const int64_t H = pl.H, F = pl.F, Mr = pl.Mr, Hc = pl.Hc;
  const bool f32 = pl.epi2 == kEpiPlainF32;
  if (!pl.reduce || a->reduce_fusion != TP_REDUCE_FUSION_AUTO || !(pl.epi2 == kEpiF32 || f32) ||
      a->P - 1 > kMaxEpiPeers)
    return false;
  const bool final_block = last && c + 1 == pl.C;
  if (two && !final_block) {
    if (f32 || !weigh) return false;
    // (with every GEMM1 already done, the next block's GEMM2 alone)
    const double next_flops = 2.0 * Mr * F * (c + 1 < pl.C || g1_done ? Hc : H + Hc);
    const double red_bytes = 4.0 * (a->P + 1) * Mr * Hc;
    if (red_bytes / kReduceByteRate <= kBesideShare * next_flops / kGemmFlopRate) return false;
  }
  const int64_t zoff = r * Mr * H + c * Hc;
  *gr = block_gemm2(a, pl, r, c);
  gr->red.np = static_cast<int32_t>(a->P - 1);
  for (int64_t p = 1; p < a->P; ++p) gr->red.peer[p - 1] = a->peer_partials[p - 1] + zoff;
  gr->red.nout = 1;
  gr->red.rows_per_out = static_cast<int32_t>(Mr);
  if (a->Z_split) {
    // Reduce-scattered: the chunk lies in one sequence block, or covers
    // whole ones (the two nest).
    const int64_t Ms = pl.sq.Ms, g0 = r * Mr, j0 = g0 / Ms;
    if (Mr <= Ms) {
      gr->red.out[0] = a->Z_split[j0] + (g0 - j0 * Ms) * H + c * Hc;
    } else if (Mr / Ms <= kMaxFusedOuts) {
      gr->red.nout = static_cast<int32_t>(Mr / Ms);
      gr->red.rows_per_out = static_cast<int32_t>(Ms);
      for (int64_t k = 0; k < Mr / Ms; ++k) gr->red.out[k] = a->Z_split[j0 + k] + c * Hc;
    } else {
      return false;
    }
  } else {
    gr->red.out[0] = a->Z_out ? a->Z_out + zoff : nullptr;
  }
  gr->red.bias = a->bias ? a->bias + c * Hc : nullptr;
  gr->red.lo = a->X_next ? static_cast<char *>(a->X_next) + zoff * pl.es : nullptr;
  gr->red.lo_bf16 = a->dtype == TP_BF16;
  return f32 ? gemm_red_ok_f32(*gr) : gemm_red_ok(*gr);
}

// Whether any block of the layer hands its reduction to s1 on a two-stream
// schedule; `last_chunk_last`: nothing follows the layer's last chunk on s0.
bool any_block_beside(const tp_mlp_args *a, const MlpPlan& pl, bool last_chunk_last, bool weigh,
                      bool g1_done = false) {
  if (!pl.reduce) return false;
  GemmArgs gr{};
  for (int64_t r = 0; r < pl.R; ++r)
    for (int64_t c = 0; c < pl.C; ++c)
      if (!fused_block(a, pl, r, c, true, last_chunk_last && r + 1 == pl.R, weigh, &gr, g1_done)) return true;
  return false;
}

// Whether every block of the layer takes the same place on two streams
// (beside the next GEMMs, or folded) when every GEMM1 runs first as when each
// chunk's GEMM1 runs ahead of its GEMM2s.
bool same_places_with_gemm1_first(const tp_mlp_args *a, const MlpPlan& pl) {
  GemmArgs gr{};
  for (int64_t r = 0; r < pl.R; ++r)
    for (int64_t c = 0; c < pl.C; ++c) {
      const bool last = r + 1 == pl.R;
      if (fused_block(a, pl, r, c, true, last, true, &gr, false) != fused_block(a, pl, r, c, true, last, true, &gr, true))
        return false;
    }
  return true;
}

// The layer as a single block (R = C = 1).
MlpPlan one_block(const MlpPlan& pl) {
  MlpPlan w = pl;
  w.R = w.C = 1;
  w.Mr = pl.M;
  w.Hc = pl.H;
  return w;
}

// Whether GEMM1 can run over every row of the layer in one launch: the
// kernels' 32-bit index range, and X read in place as at most kMaxABlocks
// blocks of whole tiles.
bool gemm1_spans_layer(const tp_mlp_args *a, const MlpPlan& w) {
  if (w.M * w.F >= (int64_t(1) << 31) || w.M * w.H >= (int64_t(1) << 31)) return false;
  if (!w.x_in_place) return true;
  const GemmArgs g1 = chunk_gemm1(a, w, 0);
  return g1.a_blk_rows == 0 || (w.M / w.sq.Ms <= kMaxABlocks && gemm_blocks_ok(g1, w.epi1));
}

int launch_gemm1(const tp_mlp_args *a, const MlpPlan& pl, int64_t r, hipStream_t s0) {
  const GemmArgs g1 = chunk_gemm1(a, pl, r);
  hipEvent_t t0 = timing_begin(s0);
  const hipError_t e = gemm_launch(g1, pl.epi1, s0);
  if (e != hipSuccess) return hip_fail(e, "GEMM1 launch");
  timing_end(t0, s0, TP_KERNEL_GEMM1, 2.0 * pl.Mr * pl.F * pl.H);
  return TP_OK;
}

// Row chunk r of one forward layer: GEMM1 and, per column block, GEMM2 and its
// reduction (in GEMM2's epilogue, or handed to s1 through ev_blocks[c] when
// `two`).  `last`: nothing follows this chunk on s0, so its final block's
// reduction runs alone and takes the whole chip (a one-shot grid) instead of
// the share sized to run beside a GEMM.  `weigh`: as in fused_block.
// `gemm1`: false where one earlier GEMM1 launch already covered every row.
int enqueue_chunk(const tp_mlp_args *a, const MlpPlan& pl, int64_t r, hipStream_t s0, hipStream_t s1, bool two,
                  hipEvent_t *ev_blocks, bool last, bool weigh, bool gemm1 = true) {
  const int64_t es = pl.es, H = pl.H, F = pl.F, Mr = pl.Mr, Hc = pl.Hc;
  int rc0 = gemm1 ? launch_gemm1(a, pl, r, s0) : TP_OK;
  if (rc0 != TP_OK) return rc0;
  hipEvent_t t0 = nullptr;
  hipError_t e;
  std::vector<const float *> parts(static_cast<size_t>(a->P));
  for (int64_t c = 0; c < pl.C; ++c) {
    const int64_t zoff = r * Mr * H + c * Hc;
    const bool final_block = last && c + 1 == pl.C;
    GemmArgs gr{};
    if (fused_block(a, pl, r, c, two, last, weigh, &gr, !gemm1)) {
      const bool f32 = pl.epi2 == kEpiPlainF32;
      t0 = timing_begin(s0);
      e = gemm_launch(gr, f32 ? kEpiPlainF32Red : kEpiF32Red, s0);
      if (e != hipSuccess) return hip_fail(e, "GEMM2 launch");
      // Memory-bound: its work is bytes (Y rows and B columns, the peers'
      // blocks and the bias read once, every output written once).
      const double cells = static_cast<double>(Mr) * Hc;
      const double bytes = es * (static_cast<double>(Mr) * F + static_cast<double>(F) * Hc) +
                           4.0 * gr.red.np * cells + (gr.red.out[0] != gr.c ? 4.0 * cells : 0.0) +
                           (gr.red.out[0] ? 4.0 * cells : 0.0) + (gr.red.lo ? es * cells : 0.0) +
                           (gr.red.bias ? 4.0 * Hc : 0.0);
      timing_end(t0, s0, TP_KERNEL_GEMM2_REDUCE, bytes);
      continue;
    }
    const GemmArgs g2 = block_gemm2(a, pl, r, c);
    t0 = timing_begin(s0);
    e = gemm_launch(g2, pl.epi2, s0);
    if (e != hipSuccess) return hip_fail(e, "GEMM2 launch");
    timing_end(t0, s0, TP_KERNEL_GEMM2, 2.0 * Mr * Hc * F);
    if (!pl.reduce) continue;
    hipStream_t sr = s0;
    if (two) {
      if ((e = hipEventRecord(ev_blocks[c], s0)) != hipSuccess) return hip_fail(e, "hipEventRecord");
      if ((e = hipStreamWaitEvent(s1, ev_blocks[c], 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
      sr = s1;
    }
    parts[0] = a->Z_i + zoff;
    for (int64_t p = 1; p < a->P; ++p) parts[p] = a->peer_partials[p - 1] + zoff;
    const bool beside = two && !final_block;
    const int64_t wgs = a->reduce_workgroups ? a->reduce_workgroups : (beside ? kReduceBesideGemm : 0);
    const int rc = reduce_rows(parts.data(), a->P, r * Mr, Mr, c * Hc, Hc, H, a->Z_out, a->Z_split, pl.sq.Ms, sr,
                               two ? wgs : 0,
                               a->bias ? a->bias + c * Hc : nullptr, a->X_next, a->dtype,
                               two && final_block ? TP_KERNEL_REDUCE_TAIL : TP_KERNEL_REDUCE);
    if (rc != TP_OK) return rc;
  }
  return TP_OK;
}

}  // namespace

}  // namespace tpshard

using namespace tpshard;

extern "C" {

const char *tp_last_error(void) { return g_last_error.c_str(); }

const char *tp_version(void) { return "tpshard 0.1 gfx950"; }

int tp_layout_plan(const int64_t *shape, int64_t ndim, const tp_layout *layout, int64_t *num_shards_out,
                   int64_t *boxes, int64_t max_shards, int64_t *shard_of_device, int64_t num_dst) {
  clear_error();
  if (!num_shards_out) return fail(TP_ERR_ARG, "num_shards_out is NULL");
  if (max_shards < 0 || num_dst < 0) return fail(TP_ERR_ARG, "negative output capacity");
  ShardPlan plan;
  const int rc = build_plan(shape, ndim, layout, &plan);
  if (rc != TP_OK) return rc;
  *num_shards_out = plan.nshards();
  if (boxes) {
    const int64_t n = std::min(max_shards, plan.nshards());
    for (int64_t k = 0; k < n; ++k)
      for (int i = 0; i < plan.ndim; ++i) {
        boxes[(k * plan.ndim + i) * 2] = plan.offset[k * plan.ndim + i];
        boxes[(k * plan.ndim + i) * 2 + 1] = plan.offset[k * plan.ndim + i] + plan.extent[i];
      }
  }
  if (shard_of_device) {
    for (int64_t d = 0; d < num_dst; ++d) shard_of_device[d] = -1;
    for (int64_t k = 0; k < plan.nshards(); ++k)
      for (int64_t d : plan.devices[k])
        if (d < num_dst) shard_of_device[d] = k;
  }
  return TP_OK;
}

int tp_shard_materialize(const void *src, int32_t dtype, const int64_t *shape, int64_t ndim,
                         const tp_layout *layout, void *const *dst, int64_t num_dst, tp_stream_t stream) {
  const tp_materialize_item item{src, dtype, shape, ndim, layout, dst, num_dst};
  return tp_shard_materialize_batch(&item, 1, stream);
}

int tp_shard_materialize_batch(const tp_materialize_item *items, int64_t num_items, tp_stream_t stream) {
  clear_error();
  if (num_items < 0 || (num_items > 0 && !items)) return fail(TP_ERR_ARG, "need num_items >= 0 and an item array");
  std::vector<ShardPlan> plans(static_cast<size_t>(num_items));
  std::vector<MatJob> jobs;
  std::vector<Buf> ins, outs;
  for (int64_t i = 0; i < num_items; ++i) {
    const tp_materialize_item& it = items[i];
    const int64_t esize = dtype_size(it.dtype);
    if (!esize) return fail(TP_ERR_ARG, "item %lld: unknown dtype %d", (long long)i, it.dtype);
    ShardPlan& plan = plans[i];
    int rc = build_plan(it.shape, it.ndim, it.layout, &plan);
    if (rc != TP_OK) {
      if (num_items == 1) return rc;
      const std::string msg = tp_last_error();
      return fail(rc, "item %lld: %s", (long long)i, msg.c_str());
    }
    int64_t numel = 1, shard_elems = 1;
    for (int a = 0; a < plan.ndim; ++a) {
      numel *= plan.shape[a];
      shard_elems *= plan.extent[a];
    }
    if (!it.src && numel > 0) return fail(TP_ERR_ARG, "item %lld: src is NULL", (long long)i);
    if (it.local_only != 0 && it.local_only != 1)
      return fail(TP_ERR_ARG, "item %lld: local_only must be 0 or 1", (long long)i);
    if (it.local_only) {
      // One device's share: keep the shards whose group holds it, written to it alone.
      if (it.local_device < 0 || it.local_device >= it.num_dst)
        return fail(TP_ERR_ARG, "item %lld: local_device %lld outside [0, num_dst)", (long long)i,
                    (long long)it.local_device);
      ShardPlan mine;
      mine.ndim = plan.ndim;
      for (int a = 0; a < plan.ndim; ++a) {
        mine.shape[a] = plan.shape[a];
        mine.extent[a] = plan.extent[a];
      }
      for (int64_t k = 0; k < plan.nshards(); ++k)
        for (int64_t d : plan.devices[k])
          if (d == it.local_device) {
            mine.offset.insert(mine.offset.end(), plan.offset.begin() + k * plan.ndim,
                               plan.offset.begin() + (k + 1) * plan.ndim);
            mine.devices.push_back({d});
            mine.max_device = d;
            break;
          }
      if (mine.devices.empty())
        return fail(TP_ERR_ARG, "item %lld: the layout does not name local_device %lld", (long long)i,
                    (long long)it.local_device);
      plan = std::move(mine);
    }
    if (plan.max_device >= it.num_dst)
      return fail(TP_ERR_ARG, "item %lld: num_dst = %lld but the layout names device %lld", (long long)i,
                  (long long)it.num_dst, (long long)plan.max_device);
    if (plan.max_device >= 0 && !it.dst) return fail(TP_ERR_ARG, "item %lld: dst is NULL", (long long)i);
    for (const auto& grp : plan.devices)
      for (int64_t d : grp) {
        if (!it.dst[d] && shard_elems > 0) return fail(TP_ERR_ARG, "item %lld: dst[%lld] is NULL", (long long)i, (long long)d);
        outs.push_back({it.dst[d], shard_elems * esize, "a destination"});
      }
    ins.push_back({it.src, numel * esize, "a source"});
    jobs.push_back({&plan, it.src, esize, it.dst});
  }
  const int rc = check_disjoint(ins, outs);
  if (rc != TP_OK) return rc;
  return shard_materialize_batch_launch(jobs.data(), static_cast<int>(jobs.size()), static_cast<hipStream_t>(stream));
}

int tp_shard_gather(const void *const *src, int64_t num_src, int32_t dtype, const int64_t *shape, int64_t ndim,
                    const tp_layout *layout, void *const *out, int64_t num_out, tp_stream_t stream) {
  clear_error();
  const int64_t esize = dtype_size(dtype);
  if (!esize) return fail(TP_ERR_ARG, "unknown dtype %d", dtype);
  ShardPlan plan;
  int rc = build_plan(shape, ndim, layout, &plan);
  if (rc != TP_OK) return rc;
  int64_t numel = 1, shard_elems = 1;
  for (int i = 0; i < plan.ndim; ++i) {
    numel *= plan.shape[i];
    shard_elems *= plan.extent[i];
  }
  if (num_out < 1 || !out) return fail(TP_ERR_ARG, "need num_out >= 1 outputs");
  if (plan.max_device >= num_src)
    return fail(TP_ERR_ARG, "num_src = %lld but the layout names device %lld", (long long)num_src, (long long)plan.max_device);
  if (plan.max_device >= 0 && !src) return fail(TP_ERR_ARG, "src is NULL");
  const int64_t full_bytes = numel * esize, shard_bytes = shard_elems * esize;
  std::vector<Buf> ins, outs;
  for (const auto& grp : plan.devices) {
    if (!src[grp[0]] && shard_bytes > 0) return fail(TP_ERR_ARG, "src[%lld] is NULL", (long long)grp[0]);
    ins.push_back({src[grp[0]], shard_bytes, "a shard"});
  }
  for (int64_t j = 0; j < num_out; ++j) {
    if (!out[j] && full_bytes > 0) return fail(TP_ERR_ARG, "out[%lld] is NULL", (long long)j);
    outs.push_back({out[j], full_bytes, "an output"});
  }
  if ((rc = check_disjoint(ins, outs)) != TP_OK) return rc;
  return shard_gather_launch(plan, src, esize, out, num_out, static_cast<hipStream_t>(stream));
}

int tp_partial_reduce(const float *const *partials, int64_t P, int64_t rows, int64_t cols, int64_t ld_in,
                      int32_t mode, int64_t num_splits, float *const *out, int64_t ld_out, tp_stream_t stream) {
  return tp_partial_reduce_ex(partials, P, rows, cols, ld_in, mode, num_splits, out, ld_out, TP_REDUCE_OP_SUM,
                              nullptr, stream);
}

int tp_partial_reduce_ex(const float *const *partials, int64_t P, int64_t rows, int64_t cols, int64_t ld_in,
                         int32_t mode, int64_t num_splits, float *const *out, int64_t ld_out, int32_t op,
                         const float *bias, tp_stream_t stream) {
  clear_error();
  if (op != TP_REDUCE_OP_SUM && op != TP_REDUCE_OP_MAX && op != TP_REDUCE_OP_MIN)
    return fail(TP_ERR_ARG, "unknown reduce op %d", op);
  if (P < 1) return fail(TP_ERR_ARG, "P = %lld < 1", (long long)P);
  if (P > kMaxP) return fail(TP_ERR_UNSUPPORTED, "P = %lld > %lld", (long long)P, (long long)kMaxP);
  if (!partials) return fail(TP_ERR_ARG, "partials is NULL");
  if (rows < 0 || cols < 0) return fail(TP_ERR_ARG, "negative size");
  if (ld_in < cols || ld_out < cols || ld_in < 1 || ld_out < 1) return fail(TP_ERR_ARG, "row stride smaller than cols");
  if (mode != TP_REDUCE_FULL && mode != TP_REDUCE_SPLIT) return fail(TP_ERR_ARG, "unknown mode %d", mode);
  if (num_splits < 1) return fail(TP_ERR_ARG, "num_splits = %lld < 1", (long long)num_splits);
  if (mode == TP_REDUCE_FULL && num_splits != 1) return fail(TP_ERR_ARG, "FULL mode needs num_splits = 1");
  if (num_splits > kMaxSplits) return fail(TP_ERR_UNSUPPORTED, "num_splits = %lld > %lld", (long long)num_splits, (long long)kMaxSplits);
  if (rows % num_splits) return fail(TP_ERR_INDIVISIBLE, "%lld rows not divisible by %lld splits", (long long)rows, (long long)num_splits);
  if (!out) return fail(TP_ERR_ARG, "out is NULL");
  const int64_t rps = rows / num_splits;
  const int64_t in_bytes = matrix_bytes(rows, cols, ld_in, 4), out_bytes = matrix_bytes(rps, cols, ld_out, 4);
  for (int64_t p = 0; p < P; ++p)
    if (!partials[p] && in_bytes) return fail(TP_ERR_ARG, "partials[%lld] is NULL", (long long)p);
  for (int64_t j = 0; j < num_splits; ++j) {
    if (!out[j] && out_bytes) return fail(TP_ERR_ARG, "out[%lld] is NULL", (long long)j);
    for (int64_t p = 0; p < P; ++p) {
      const bool in_place = mode == TP_REDUCE_FULL && p == 0 && out[j] == partials[0] && ld_out == ld_in;
      if (!in_place && overlaps(out[j], out_bytes, partials[p], in_bytes))
        return fail(TP_ERR_ARG, "out[%lld] overlaps partials[%lld]", (long long)j, (long long)p);
    }
    for (int64_t i = 0; i < j; ++i)
      if (overlaps(out[j], out_bytes, out[i], out_bytes)) return fail(TP_ERR_ARG, "out[%lld] overlaps out[%lld]", (long long)j, (long long)i);
    if (bias && overlaps(out[j], out_bytes, bias, cols * 4)) return fail(TP_ERR_ARG, "out[%lld] overlaps bias", (long long)j);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t t0 = timing_begin(s);
  const int rc = partial_reduce_launch(partials, static_cast<int>(P), rows, cols, ld_in, out,
                                       static_cast<int>(num_splits), rps, ld_out, s, 0, op, bias);
  if (rc == TP_OK) timing_end(t0, s, TP_KERNEL_REDUCE, 4.0 * (P + 1) * rows * cols);
  return rc;
}

int tp_colrow_mlp(const tp_mlp_args *a, tp_stream_t s_compute, tp_stream_t s_reduce) {
  clear_error();
  return colrow_mlp_run(a, s_compute, s_reduce, nullptr);
}

}  // extern "C"

int tpshard::colrow_mlp_run(const tp_mlp_args *a, tp_stream_t s_compute, tp_stream_t s_reduce,
                            int (*y_scratch)(int64_t bytes, void **out)) {
  MlpPlan pl;
  int rc = validate_mlp(a, &pl, y_scratch != nullptr);
  if (rc != TP_OK) return rc;
  tp_mlp_args own;
  if (y_scratch) {
    // Everything is valid: only now ask for one row chunk's worth of Y.
    void *y = nullptr;
    if ((rc = y_scratch(pl.Mr * pl.F * pl.es, &y)) != TP_OK) return rc;
    own = *a;
    own.Y_ws = y;
    a = &own;
  }
  hipStream_t s0 = static_cast<hipStream_t>(s_compute), s1 = static_cast<hipStream_t>(s_reduce);
  const bool gather = pl.gather;
  // The reduce stream only pays when a later block's GEMMs can run beside an
  // earlier block's reduce or gather; with a single block, or where every
  // block's reduction goes into GEMM2's epilogue and nothing is gathered
  // beside, the hand-off (an event record and a cross-queue wait, about 10 us
  // each way on MI355X) is pure latency.
  const bool two = (s0 != s1) && pl.R * pl.C > 1 && ((gather && pl.R > 1) || any_block_beside(a, pl, true, true));
  // On one stream the row chunks overlap nothing: they only cut GEMM1 into
  // smaller launches with smaller tiles.  Where every chunk's sum goes into
  // its GEMM2's epilogue, GEMM1 therefore runs once over all rows and each
  // chunk keeps its GEMM2 (GPT-3 6.7B at TP = 8, R = 2: GEMM1 over 8192 rows
  // in 103 us against two 4096-row launches of 67 us, step 371-372 against
  // 389 us; as one block, 385-387 us, its 8192-row GEMM2 with the sum taking
  // 295 us against 2 x 137).  Where no chunk's sum folds (too many peers for
  // a small block's epilogue, or fusion off) or there is nothing to sum, the
  // layer runs as one block, whose sum may still fold.  A row's result is
  // the same bits however the rows and columns are cut.
  const MlpPlan whole = one_block(pl);
  const MlpPlan *run = &pl;
  bool gemm1_whole = false;
  // On two streams, too, GEMM1 runs first over all rows where that moves no
  // block's sum off the second stream: each sum then runs beside the next
  // block's GEMM2 and none beside a GEMM1 (GPT-3 175B, R = 2, C = 2: the
  // second chunk's GEMM1 ran 15-22 us slower beside the first chunk's last
  // sum).
  if (two && pl.R > 1 && !gather && !pl.y_chunk && gemm1_spans_layer(a, whole) &&
      same_places_with_gemm1_first(a, pl))
    gemm1_whole = true;
  if (!two && pl.R * pl.C > 1 && !pl.y_chunk && gemm1_spans_layer(a, whole)) {
    GemmArgs gr{};
    if (pl.reduce && fused_block(a, pl, pl.R - 1, pl.C - 1, false, true, true, &gr))
      gemm1_whole = pl.R > 1;
    else
      run = &whole;
  }
  const int64_t R = run->R, C = run->C, Mr = run->Mr, H = pl.H, es = pl.es;
  hipEvent_t *ev = nullptr;
  if (two) {
    if ((rc = get_events(static_cast<size_t>(R * C + R + 2), &ev)) != TP_OK) return rc;
  }
  hipEvent_t *ev_red = ev, *ev_gat = two ? ev + R * C : nullptr;
  hipEvent_t ev_fork = two ? ev[R * C + R] : nullptr, ev_join = two ? ev[R * C + R + 1] : nullptr;
  hipError_t e;
  // Chunk 0's rows are needed before anything can compute, so they are
  // gathered on s_compute itself; later chunks travel on s_reduce beside the
  // GEMMs, after chunk 0's gather (the two would only split the bandwidth)
  // and after whatever the caller enqueued on s_compute (the shards, and the
  // end of any earlier use of X).
  auto gather_chunk = [&](int64_t r) -> int {
    const bool side = two && r > 0;
    const int grc = gather_rows(a->X_shards, pl.sq.Ms, r * Mr, Mr, H, es, const_cast<void *>(a->X), side ? s1 : s0);
    if (grc != TP_OK) return grc;
    if (side) {
      hipError_t ge = hipEventRecord(ev_gat[r], s1);
      if (ge != hipSuccess) return hip_fail(ge, "hipEventRecord");
    }
    return TP_OK;
  };
  if (gather && gemm1_whole) {
    if ((rc = gather_rows(a->X_shards, pl.sq.Ms, 0, pl.M, H, es, const_cast<void *>(a->X), s0)) != TP_OK) return rc;
  } else if (gather && (rc = gather_chunk(0)) != TP_OK) {
    return rc;
  }
  if (two && gather && R > 1) {
    if ((e = hipEventRecord(ev_fork, s0)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    if ((e = hipStreamWaitEvent(s1, ev_fork, 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  }
  if (gemm1_whole && (rc = launch_gemm1(a, whole, 0, s0)) != TP_OK) return rc;
  for (int64_t r = 0; r < R; ++r) {
    // The next chunk's input rows travel on s_reduce while this chunk computes.
    if (gather && !gemm1_whole && r + 1 < R && (rc = gather_chunk(r + 1)) != TP_OK) return rc;
    if (gather && two && r > 0 && (e = hipStreamWaitEvent(s0, ev_gat[r], 0)) != hipSuccess)
      return hip_fail(e, "hipStreamWaitEvent");
    if ((rc = enqueue_chunk(a, *run, r, s0, s1, two, two ? ev_red + r * C : nullptr, r + 1 == R, true,
                            !gemm1_whole)) != TP_OK)
      return rc;
  }
  if (two) {
    if ((e = hipEventRecord(ev_join, s1)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    if ((e = hipStreamWaitEvent(s0, ev_join, 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  }
  return TP_OK;
}

extern "C" {

int tp_colrow_mlp_stack(const tp_mlp_args *layers, int64_t num_layers, tp_stream_t s_compute, tp_stream_t s_reduce) {
  clear_error();
  if (!layers || num_layers < 1 || num_layers > kMaxLayers)
    return fail(TP_ERR_ARG, "need 1 <= num_layers <= %lld and a non-NULL layer array", (long long)kMaxLayers);
  std::vector<MlpPlan> pl(static_cast<size_t>(num_layers));
  int rc;
  for (int64_t l = 0; l < num_layers; ++l) {
    if ((rc = validate_mlp(&layers[l], &pl[l])) != TP_OK) {
      const std::string msg = tp_last_error();
      return fail(rc, "layer %lld: %s", (long long)l, msg.c_str());
    }
    if (layers[l].seq_splits > 1) return fail(TP_ERR_UNSUPPORTED, "layer %lld: sequence parallelism inside a stack", (long long)l);
  }
  for (int64_t l = 0; l + 1 < num_layers; ++l) {
    const tp_mlp_args &cur = layers[l], &nxt = layers[l + 1];
    if (!cur.X_next || cur.X_next != nxt.X)
      return fail(TP_ERR_ARG, "layer %lld must write the next layer's input (X_next == layer %lld's X)", (long long)l,
                  (long long)(l + 1));
    if (cur.dtype != nxt.dtype || cur.M != nxt.M || cur.H != nxt.H || cur.row_chunks != nxt.row_chunks)
      return fail(TP_ERR_ARG, "layers %lld and %lld differ in dtype, M, H or row_chunks", (long long)l, (long long)(l + 1));
  }
  hipStream_t s0 = static_cast<hipStream_t>(s_compute), s1 = static_cast<hipStream_t>(s_reduce);
  // Layers that would each keep to s_compute on their own (every block's sum
  // too long for the GEMMs after it, so it folds into its GEMM2's epilogue,
  // which also writes the next layer's input) run one after another, each
  // with its row chunks sharing one GEMM1 (GPT-3 6.7B, two layers: 823-824 us
  // against 839-843 us with the inter-layer overlap, one box).
  bool alone = true;
  for (int64_t l = 0; l < num_layers && alone; ++l)
    alone = !any_block_beside(&layers[l], pl[l], true, true);
  if (alone) {
    for (int64_t l = 0; l < num_layers; ++l)
      if ((rc = colrow_mlp_run(&layers[l], s_compute, s_compute, nullptr)) != TP_OK) return rc;
    return TP_OK;
  }
  const int64_t R = pl[0].R;
  bool any_reduce = false, any_split = R > 1;
  int64_t nev = 1;
  for (const MlpPlan& p : pl) {
    any_reduce = any_reduce || p.reduce;
    any_split = any_split || p.C > 1;
    nev += R * p.C + R;
  }
  // [DOM] inter-layer overlap: chunk r of layer l+1 needs only chunk r of
  // layer l's reduced output, so the reduction of layer l's later chunks runs
  // on s_reduce beside layer l+1's GEMMs of the earlier ones (unless every
  // block's reduction goes into its GEMM2's epilogue).
  bool beside = false;
  for (int64_t l = 0; l < num_layers; ++l)
    beside = beside || any_block_beside(&layers[l], pl[l], l + 1 == num_layers, false);
  const bool two = (s0 != s1) && any_reduce && any_split && beside;
  hipEvent_t *ev = nullptr;
  if (two && (rc = get_events(static_cast<size_t>(nev), &ev)) != TP_OK) return rc;
  hipError_t e;
  int64_t at = 0;
  hipEvent_t *prev_done = nullptr;
  for (int64_t l = 0; l < num_layers; ++l) {
    hipEvent_t *blocks = two ? ev + at : nullptr;
    hipEvent_t *done = two ? ev + at + R * pl[l].C : nullptr;
    at += R * pl[l].C + R;
    for (int64_t r = 0; r < R; ++r) {
      if (two && prev_done && (e = hipStreamWaitEvent(s0, prev_done[r], 0)) != hipSuccess)
        return hip_fail(e, "hipStreamWaitEvent");
      const bool last = l + 1 == num_layers && r + 1 == R;
      if ((rc = enqueue_chunk(&layers[l], pl[l], r, s0, s1, two, two ? blocks + r * pl[l].C : nullptr, last,
                              false)) != TP_OK)
        return rc;
      if (two && pl[l].reduce && (e = hipEventRecord(done[r], s1)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    }
    prev_done = two ? done : nullptr;
  }
  if (two) {
    hipEvent_t joined = ev[nev - 1];
    if ((e = hipEventRecord(joined, s1)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    if ((e = hipStreamWaitEvent(s0, joined, 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  }
  return TP_OK;
}

int tp_colrow_mlp_backward(const tp_mlp_bwd_args *a, tp_stream_t s_compute, tp_stream_t s_reduce) {
  clear_error();
  if (!a) return fail(TP_ERR_ARG, "args is NULL");
  const int64_t es = dtype_size(a->dtype);
  if (!es) return fail(TP_ERR_ARG, "unknown dtype %d", a->dtype);
  if (a->act != TP_ACT_NONE && a->act != TP_ACT_GELU_ERF) return fail(TP_ERR_ARG, "unknown act %d", a->act);
  if (a->M < 1 || a->H < 1 || a->F < 1) return fail(TP_ERR_ARG, "M, H, F must be >= 1");
  if (!a->X || !a->A_i || !a->B_i || !a->Y_i || !a->dZ || !a->dH_ws || !a->dX_i || !a->dA_i || !a->dB_i)
    return fail(TP_ERR_ARG, "X, A_i, B_i, Y_i, dZ, dH_ws, dX_i, dA_i and dB_i must be non-NULL");
  const bool gelu = a->act == TP_ACT_GELU_ERF;
  if (gelu && !a->H_i) return fail(TP_ERR_ARG, "H_i (the forward's pre-activation) is needed for the GeLU derivative");
  if (a->accumulate != 0 && a->accumulate != 1) return fail(TP_ERR_ARG, "accumulate must be 0 or 1");
  if (a->row_chunks < 1) return fail(TP_ERR_ARG, "row_chunks must be >= 1");
  if (a->M % a->row_chunks) return fail(TP_ERR_INDIVISIBLE, "row_chunks %lld does not divide M = %lld", (long long)a->row_chunks, (long long)a->M);
  if (a->P < 1 || a->P > kMaxP) return fail(TP_ERR_ARG, "P = %lld outside [1, %lld]", (long long)a->P, (long long)kMaxP);
  SeqSplit sq;
  int rc = check_seq(a->seq_splits, a->M, a->row_chunks, a->dZ_shards, a->dX_split, a->dX_out, "dZ_shards", "dX_split", "dX_out", &sq);
  if (rc != TP_OK) return rc;
  if (a->P > 1 && (!a->peer_dX || !(a->dX_out || a->dX_split))) return fail(TP_ERR_ARG, "P > 1 needs peer_dX and dX_out (or dX_split)");
  if (a->reduce_workgroups < 0) return fail(TP_ERR_ARG, "reduce_workgroups < 0");
  if (a->reduce_fusion != TP_REDUCE_FUSION_AUTO && a->reduce_fusion != TP_REDUCE_FUSION_OFF)
    return fail(TP_ERR_ARG, "unknown reduce_fusion %d", a->reduce_fusion);
  if (a->weight_layout != TP_WEIGHTS_MATH && a->weight_layout != TP_WEIGHTS_LINEAR)
    return fail(TP_ERR_ARG, "unknown weight_layout %d", a->weight_layout);
  const bool linear = a->weight_layout == TP_WEIGHTS_LINEAR;
  const int64_t M = a->M, H = a->H, F = a->F;
  if (M >= (int64_t(1) << 31) || H >= (int64_t(1) << 31) || F >= (int64_t(1) << 31) || (M / a->row_chunks) * H >= (int64_t(1) << 31))
    return fail(TP_ERR_UNSUPPORTED, "sizes exceed the 32-bit index range of the kernels");
  const int64_t bx = M * H * es, ba = H * F * es, bb = F * H * es, by = M * F * es, bz = M * H * 4;
  const bool gather = a->dZ_shards != nullptr;
  std::vector<Buf> ins = {{a->X, bx, "X"}, {a->A_i, ba, "A_i"}, {a->B_i, bb, "B_i"}, {a->Y_i, by, "Y_i"}};
  std::vector<Buf> outs = {{a->dH_ws, by, "dH_ws"}, {a->dX_i, bz, "dX_i"}, {a->dA_i, H * F * 4, "dA_i"},
                           {a->dB_i, F * H * 4, "dB_i"}};
  (gather ? outs : ins).push_back({a->dZ, bx, "dZ"});
  if (gather) {
    for (int64_t j = 0; j < sq.S; ++j) {
      if (!a->dZ_shards[j]) return fail(TP_ERR_ARG, "dZ_shards[%lld] is NULL", (long long)j);
      ins.push_back({a->dZ_shards[j], sq.Ms * H * es, "dZ shard"});
    }
  }
  if (gelu) ins.push_back({a->H_i, by, "H_i"});
  for (int64_t p = 1; p < a->P; ++p) {
    if (!a->peer_dX[p - 1]) return fail(TP_ERR_ARG, "peer_dX[%lld] is NULL", (long long)(p - 1));
    ins.push_back({a->peer_dX[p - 1], bz, "peer dX"});
  }
  const bool reduce = a->P > 1 || a->dX_split;
  if (reduce && a->dX_out && a->dX_out != a->dX_i) outs.push_back({a->dX_out, bz, "dX_out"});
  if (a->dX_split) {
    for (int64_t j = 0; j < sq.S; ++j) {
      if (!a->dX_split[j]) return fail(TP_ERR_ARG, "dX_split[%lld] is NULL", (long long)j);
      outs.push_back({a->dX_split[j], sq.Ms * H * 4, "dX_split block"});
    }
  }
  if ((rc = check_disjoint(ins, outs)) != TP_OK) return rc;

  hipStream_t s0 = static_cast<hipStream_t>(s_compute), s1 = static_cast<hipStream_t>(s_reduce);
  const int64_t R = a->row_chunks, Mr = M / R;
  const bool bf16 = a->dtype == TP_BF16;
  // dX_i[r] = dH[r] A_i^T: A_i is [H][F], i.e. W^T for W = A_i^T.  With the
  // reduction folded in, the epilogue also sums the peers' dX[r] into dX_out.
  auto dx_gemm = [&](int64_t r, bool fused) {
    // A_i^T: A_i [H][F] read transposed, or the linear layout's [F][H] as is.
    GemmArgs gx{static_cast<const char *>(a->dH_ws) + r * Mr * F * es, a->A_i, a->dX_i + r * Mr * H, Mr, H, F, F,
                linear ? H : F, H};
    gx.w_t = linear ? 0 : 1;
    if (fused) {
      gx.red.np = static_cast<int32_t>(a->P - 1);
      for (int64_t p = 1; p < a->P; ++p) gx.red.peer[p - 1] = a->peer_dX[p - 1] + r * Mr * H;
      gx.red.out[0] = a->dX_out + r * Mr * H;
      gx.red.nout = 1;
    }
    return gx;
  };
  // Small layers sum dX in the dX GEMM's epilogue: their GEMMs are too short
  // for the hand-off to s_reduce and back to pay for the overlap it buys.
  bool fuse = reduce && a->reduce_fusion == TP_REDUCE_FUSION_AUTO && bf16 && !a->dX_split && a->dX_out &&
              a->P - 1 <= kMaxFusedPeers && ((Mr + 127) / 128) * ((H + 127) / 128) < kSmallTiles;
  for (int64_t r = 0; fuse && r < R; ++r) fuse = gemm_red_ok(dx_gemm(r, true));
  // As in the forward: a second stream only pays when its work can run beside
  // GEMMs: a chunk's reduce beside that chunk's weight-gradient GEMMs, the
  // next chunk's gather beside this chunk's GEMMs.
  const bool two = (s0 != s1) && ((reduce && !fuse) || (gather && R > 1));
  hipEvent_t *ev = nullptr;
  if (two) {
    if ((rc = get_events(static_cast<size_t>(2 * R + 2), &ev)) != TP_OK) return rc;
  }
  hipEvent_t *ev_red = ev, *ev_gat = two ? ev + R : nullptr;
  hipEvent_t ev_fork = two ? ev[2 * R] : nullptr, ev_join = two ? ev[2 * R + 1] : nullptr;
  hipError_t e;
  if (two && gather && R > 1) {
    if ((e = hipEventRecord(ev_fork, s0)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    if ((e = hipStreamWaitEvent(s1, ev_fork, 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  }
  auto gather_chunk = [&](int64_t r) -> int {
    const bool side = two && r > 0;
    const int grc = gather_rows(a->dZ_shards, sq.Ms, r * Mr, Mr, H, es, const_cast<void *>(a->dZ), side ? s1 : s0);
    if (grc != TP_OK) return grc;
    if (side) {
      hipError_t ge = hipEventRecord(ev_gat[r], s1);
      if (ge != hipSuccess) return hip_fail(ge, "hipEventRecord");
    }
    return TP_OK;
  };
  if (gather && (rc = gather_chunk(0)) != TP_OK) return rc;

  const int epi_dh = bf16 ? (gelu ? kEpiDGeluBf16 : kEpiIdentBf16) : (gelu ? kEpiDGeluF32 : kEpiPlainF32);
  const int epi_f32 = bf16 ? kEpiF32 : kEpiPlainF32;
  const char *X = static_cast<const char *>(a->X), *Yi = static_cast<const char *>(a->Y_i);
  const char *dZ = static_cast<const char *>(a->dZ);
  char *dH = static_cast<char *>(a->dH_ws);
  std::vector<const float *> parts(static_cast<size_t>(a->P));
  for (int64_t r = 0; r < R; ++r) {
    if (gather && r + 1 < R && (rc = gather_chunk(r + 1)) != TP_OK) return rc;
    if (gather && two && r > 0 && (e = hipStreamWaitEvent(s0, ev_gat[r], 0)) != hipSuccess)
      return hip_fail(e, "hipStreamWaitEvent");
    // dH[r] = (dZ[r] B_i^T) * act'(H_i[r]): B_i is [F][H], i.e. W^T for W = B_i^T.
    // (With linear weights B_i is stored [H][F], B_i^T as is.)
    GemmArgs gd{dZ + r * Mr * H * es, a->B_i, dH + r * Mr * F * es, Mr, F, H, H, linear ? F : H, F};
    gd.w_t = linear ? 0 : 1;
    if (gelu) {
      gd.aux = const_cast<char *>(static_cast<const char *>(a->H_i)) + r * Mr * F * es;
      gd.ldaux = F;
    }
    hipEvent_t t0 = timing_begin(s0);
    e = gemm_launch(gd, epi_dh, s0);
    if (e != hipSuccess) return hip_fail(e, "dH GEMM launch");
    timing_end(t0, s0, TP_KERNEL_GEMM_DGRAD, 2.0 * Mr * F * H);
    if (fuse) {
      const GemmArgs gx = dx_gemm(r, true);
      t0 = timing_begin(s0);
      e = gemm_launch(gx, kEpiF32Red, s0);
      if (e != hipSuccess) return hip_fail(e, "dX GEMM launch");
      const double cells = static_cast<double>(Mr) * H;
      timing_end(t0, s0, TP_KERNEL_GEMM_DGRAD_REDUCE,
                 es * (static_cast<double>(Mr) * F + static_cast<double>(F) * H) + 4.0 * gx.red.np * cells +
                     (gx.red.out[0] != gx.c ? 4.0 * cells : 0.0) + 4.0 * cells);
    } else {
      t0 = timing_begin(s0);
      e = gemm_launch(dx_gemm(r, false), epi_f32, s0);
      if (e != hipSuccess) return hip_fail(e, "dX GEMM launch");
      timing_end(t0, s0, TP_KERNEL_GEMM_DGRAD, 2.0 * Mr * H * F);
    }
    if (reduce && !fuse) {
      hipStream_t sr = s0;
      if (two) {
        if ((e = hipEventRecord(ev_red[r], s0)) != hipSuccess) return hip_fail(e, "hipEventRecord");
        if ((e = hipStreamWaitEvent(s1, ev_red[r], 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
        sr = s1;
      }
      parts[0] = a->dX_i + r * Mr * H;
      for (int64_t p = 1; p < a->P; ++p) parts[p] = a->peer_dX[p - 1] + r * Mr * H;
      rc = reduce_rows(parts.data(), a->P, r * Mr, Mr, 0, H, H, a->dX_out, a->dX_split, sq.Ms, sr,
                       two ? (a->reduce_workgroups ? a->reduce_workgroups : kReduceBesideGemm) : 0, nullptr);
      if (rc != TP_OK) return rc;
    }
  }
  // Weight gradients over all rows in one pass each, once every chunk's dH is
  // there: dA_i (+)= X^T dH, dB_i (+)= Y_i^T dZ.  The same bits as one pass per
  // chunk continuing the previous chunk's sum (each element is accumulated over
  // the rows in the same order), without reading and rewriting the fp32
  // gradients once per further chunk (the 175B shapes: 302 MB each way per
  // weight and chunk).  The last chunk's dX reduction runs beside them.
  {
    // Linear weights take their gradients in the same layout: dA_i^T = dH^T X
    // ([F][H]) and dB_i^T = dZ^T Y_i ([H][F]), each element the same sum over
    // the rows.
    const int cont = a->accumulate ? 1 : 0;
    GemmArgs ga = linear ? GemmArgs{dH, X, a->dA_i, F, H, M, F, H, H} : GemmArgs{X, dH, a->dA_i, H, F, M, H, F, F};
    ga.a_t = 1;
    ga.acc_init = cont;
    GemmArgs gb = linear ? GemmArgs{dZ, Yi, a->dB_i, H, F, M, H, F, F} : GemmArgs{Yi, dZ, a->dB_i, F, H, M, F, H, H};
    gb.a_t = 1;
    gb.acc_init = cont;
    const GemmArgs pair[2] = {ga, gb};
    hipEvent_t t0;
    if (gemm_group_ok(pair, 2, epi_f32)) {
      // Both too small to fill the chip alone: one grouped launch.
      t0 = timing_begin(s0);
      e = gemm_launch_group(pair, 2, epi_f32, s0);
      if (e != hipSuccess) return hip_fail(e, "dA/dB GEMM launch");
      timing_end(t0, s0, TP_KERNEL_GEMM_WGRAD, 2.0 * H * F * M * 2);
    } else {
      t0 = timing_begin(s0);
      e = gemm_launch(ga, epi_f32, s0);
      if (e != hipSuccess) return hip_fail(e, "dA GEMM launch");
      timing_end(t0, s0, TP_KERNEL_GEMM_WGRAD, 2.0 * H * F * M);
      t0 = timing_begin(s0);
      e = gemm_launch(gb, epi_f32, s0);
      if (e != hipSuccess) return hip_fail(e, "dB GEMM launch");
      timing_end(t0, s0, TP_KERNEL_GEMM_WGRAD, 2.0 * F * H * M);
    }
  }
  if (two) {
    if ((e = hipEventRecord(ev_join, s1)) != hipSuccess) return hip_fail(e, "hipEventRecord");
    if ((e = hipStreamWaitEvent(s0, ev_join, 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  }
  return TP_OK;
}

}  // extern "C"
