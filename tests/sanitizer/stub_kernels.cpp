// Host stand-ins for the library's kernel launchers, for a CPU build of the
// host code (planning, checking, validation and scheduling) under
// AddressSanitizer and UndefinedBehaviorSanitizer.  Nothing runs on a GPU:
// each launcher checks that every byte range its kernel would touch lies
// inside one allocation the test registered, and aborts otherwise, so the
// scheduler's pointer arithmetic is verified for every call it makes.
#include <cstdint>
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../sharded_gemm_amd/csrc/gemm.h"
#include "../../sharded_gemm_amd/csrc/shard.h"
#include "stub_registry.h"

namespace {

struct Range {
  uintptr_t lo, hi;
};
std::vector<Range> g_allocs;
long g_launches = 0;

void need(const void *p, int64_t rows, int64_t cols, int64_t ld, int64_t es, const char *what) {
  if (rows <= 0 || cols <= 0) return;
  if (!p || ld < cols) {
    std::fprintf(stderr, "launch check: %s null or stride %lld < %lld\n", what, (long long)ld, (long long)cols);
    std::abort();
  }
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  const uintptr_t hi = lo + static_cast<uintptr_t>(((rows - 1) * ld + cols) * es);
  for (const Range& r : g_allocs)
    if (lo >= r.lo && hi <= r.hi) return;
  std::fprintf(stderr, "launch check: %s [%#lx, %#lx) outside every allocation\n", what, (unsigned long)lo,
               (unsigned long)hi);
  std::abort();
}

bool f32_epi(int epi) {
  using namespace tpshard;
  return epi == kEpiGeluF32 || epi == kEpiPlainF32 || epi == kEpiGeluSaveF32 || epi == kEpiDGeluF32 ||
         epi == kEpiPlainF32Red;
}

}  // namespace

void stub_register(const void *p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  g_allocs.push_back({lo, lo + static_cast<uintptr_t>(bytes)});
}
void stub_reset() { g_allocs.clear(); }
long stub_launches() { return g_launches; }

namespace tpshard {

hipError_t gemm_launch(const GemmArgs& p, int epi, hipStream_t) {
  ++g_launches;
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  const int64_t in_es = f32_epi(epi) ? 4 : 2;
  const bool out_f32 = f32_epi(epi) || epi == kEpiF32 || epi == kEpiF32Red;
  if (p.a_blk_rows > 0) {
    if (!gemm_blocks_ok(p, epi)) return hipErrorInvalidValue;
    for (int64_t j = 0; j * p.a_blk_rows < p.M; ++j)
      need(p.a_blk[j], std::min(p.a_blk_rows, p.M - j * p.a_blk_rows), p.K, p.lda, in_es, "GEMM A block");
  } else if (p.a_t) {
    need(p.a, p.K, p.M, p.lda, in_es, "GEMM A^T");
  } else {
    need(p.a, p.M, p.K, p.lda, in_es, "GEMM A");
  }
  if (p.w_t) need(p.w, p.N, p.K, p.ldw, in_es, "GEMM W^T"); else need(p.w, p.K, p.N, p.ldw, in_es, "GEMM W");
  need(p.c, p.M, p.N, p.ldc, out_f32 ? 4 : 2, "GEMM C");
  if (epi == kEpiGeluSaveBf16 || epi == kEpiDGeluBf16) need(p.aux, p.M, p.N, p.ldaux, 2, "GEMM aux");
  if (epi == kEpiGeluSaveF32 || epi == kEpiDGeluF32) need(p.aux, p.M, p.N, p.ldaux, 4, "GEMM aux");
  if (epi == kEpiF32Red || epi == kEpiPlainF32Red) {
    const EpiReduce& r = p.red;
    for (int q = 0; q < r.np; ++q) need(r.peer[q], p.M, p.N, p.ldc, 4, "GEMM peer");
    if (r.nout > 1) {
      for (int j = 0; j < r.nout; ++j) need(r.out[j], r.rows_per_out, p.N, p.ldc, 4, "GEMM split out");
    } else if (r.out[0]) {
      need(r.out[0], p.M, p.N, p.ldc, 4, "GEMM out");
    }
    if (r.bias) need(r.bias, 1, p.N, p.N, 4, "GEMM bias");
    if (r.lo) need(r.lo, p.M, p.N, p.ldc, r.lo_bf16 ? 2 : 4, "GEMM lo");
  }
  return hipSuccess;
}

// The real rules depend on alignment and tile counts; the stand-ins accept
// what the kernels' own conditions would, minus alignment, so both the fused
// and the separate reduction paths get exercised.
bool gemm_red_ok(const GemmArgs& p) {
  if (p.a_t || p.acc_init || p.red.np < 0 || p.K % 32 != 0 || p.K <= 0) return false;
  if (((p.M + 127) / 128) * ((p.N + 127) / 128) >= 256)   // the 256-row tiles: the epilogue stages the tile
    return p.red.np <= kMaxEpiPeers && p.K % 64 == 0 && p.red.nout >= 1 && p.red.nout <= kMaxFusedOuts &&
           (p.red.nout == 1 || (!p.red.lo && p.red.rows_per_out * p.red.nout == p.M)) &&
           p.M * p.lda * 2 < (int64_t{1} << 31) && (p.w_t ? p.N : p.K) * p.ldw * 2 < (int64_t{1} << 31);
  return p.red.np <= kMaxFusedPeers && p.red.nout >= 1 && p.red.nout <= kMaxFusedOuts &&
         !(p.w_t && p.red.nout > 1) && (p.red.nout == 1 || (!p.red.lo && p.red.rows_per_out * p.red.nout == p.M));
}
bool gemm_red_ok_f32(const GemmArgs& p) {
  return !p.a_t && !p.w_t && !p.acc_init && p.red.np >= 0 && p.red.np <= kMaxFusedPeers && p.red.nout >= 1 &&
         p.red.nout <= kMaxFusedOuts && (p.red.nout == 1 || (!p.red.lo && p.red.rows_per_out * p.red.nout == p.M));
}
bool gemm_blocks_ok(const GemmArgs& p, int epi) {
  if (p.a_blk_rows <= 0 || p.a_blk_rows % 256 != 0 || p.a_t || p.K % 32 != 0 || p.K <= 0) return false;
  if (epi != kEpiGeluBf16 && epi != kEpiIdentBf16 && epi != kEpiF32 && epi != kEpiGeluSaveBf16 && epi != kEpiF32Red)
    return false;
  const int64_t nblk = (p.M + p.a_blk_rows - 1) / p.a_blk_rows;
  if (nblk > kMaxABlocks) return false;
  for (int64_t j = 0; j < nblk; ++j)
    if (!p.a_blk[j]) return false;
  return true;
}
bool gemm_group_ok(const GemmArgs *ps, int n, int epi) {
  if (n < 1 || n > 4 || epi != kEpiF32) return false;
  for (int q = 0; q < n; ++q)
    if (!ps[q].a_t || ps[q].w_t || ps[q].K % 32 || ((ps[q].M + 127) / 128) * ((ps[q].N + 127) / 128) >= 256)
      return false;
  return true;
}
hipError_t gemm_launch_group(const GemmArgs *ps, int n, int epi, hipStream_t s) {
  for (int q = 0; q < n; ++q)
    if (gemm_launch(ps[q], epi, s) != hipSuccess) return hipErrorInvalidValue;
  return hipSuccess;
}

int shard_materialize_batch_launch(const MatJob *jobs, int njobs, hipStream_t) {
  ++g_launches;
  for (int i = 0; i < njobs; ++i) {
    const ShardPlan& pl = *jobs[i].plan;
    int64_t numel = 1, shard = 1;
    for (int a = 0; a < pl.ndim; ++a) {
      numel *= pl.shape[a];
      shard *= pl.extent[a];
    }
    need(jobs[i].src, 1, numel, numel, jobs[i].esize, "materialize src");
    for (const auto& grp : pl.devices)
      for (int64_t d : grp) need(jobs[i].dst[d], 1, shard, shard, jobs[i].esize, "materialize dst");
  }
  return TP_OK;
}

int shard_materialize_launch(const ShardPlan& plan, const void *src, int64_t esize, void *const *dst, hipStream_t s) {
  const MatJob j{&plan, src, esize, dst};
  return shard_materialize_batch_launch(&j, 1, s);
}

int shard_gather_launch(const ShardPlan& pl, const void *const *src, int64_t esize, void *const *out, int64_t nout,
                        hipStream_t) {
  ++g_launches;
  int64_t numel = 1, shard = 1;
  for (int a = 0; a < pl.ndim; ++a) {
    numel *= pl.shape[a];
    shard *= pl.extent[a];
  }
  for (const auto& grp : pl.devices) need(src[grp[0]], 1, shard, shard, esize, "gather src");
  for (int64_t j = 0; j < nout; ++j) need(out[j], 1, numel, numel, esize, "gather out");
  return TP_OK;
}

int partial_reduce_launch(const float *const *partials, int P, int64_t rows, int64_t cols, int64_t ld_in,
                          float *const *out, int nout, int64_t rows_per_out, int64_t ld_out, hipStream_t, int64_t,
                          int, const float *bias, void *lo, int lo_dtype, int64_t ld_lo) {
  ++g_launches;
  for (int p = 0; p < P; ++p) need(partials[p], rows, cols, ld_in, 4, "reduce partial");
  for (int j = 0; j < nout; ++j)
    if (out[j] || !lo) need(out[j], rows_per_out, cols, ld_out, 4, "reduce out");
  if (bias) need(bias, 1, cols, cols, 4, "reduce bias");
  if (lo) need(lo, rows, cols, ld_lo, lo_dtype == TP_BF16 ? 2 : 4, "reduce lo");
  return TP_OK;
}

}  // namespace tpshard
