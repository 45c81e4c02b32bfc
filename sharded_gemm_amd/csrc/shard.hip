// Shard materialisation (split + replicate in one pass) and its inverse, the
// gather of every shard into full copies of the tensor ([ONNX] "Sharding as a
// Split", "Sharding as a Broadcast", "mixing split and broadcast"; [SBP] "SBP";
// [SPMD] "dims_mapping"; [CAI] sections 5.1 and 5.3: gather_output and the
// sequence-parallel all-gather).
//
// All shards of a layout have the same extents, so a shard is a set of
// equal-length runs that are contiguous in the full tensor (the innermost
// sharded axis and every axis after it) separated by fixed strides on the
// outer axes, while each device holds its shard as one contiguous buffer.  The
// split reads the runs and writes each element to every device of the shard's
// group; the gather reads each shard's contiguous buffer once (from the first
// device its group lists) and writes it into its box of every output.  A
// workgroup streams a slice of one shard with the widest vector the alignment
// allows (16, 8, 4 or 2 bytes per lane).  Every byte is read once and written
// once per destination: loads are non-temporal, and so are the stores of
// large copies; a copy of at most 64 MiB keeps its output in the caches for
// the kernel that reads it next.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <vector>

#include "common.h"
#include "plan.h"
#include "shard.h"
#include "timing.h"

namespace tpshard {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxShardsPerLaunch = 32;
constexpr int kMaxDstPerLaunch = 64;
constexpr int kMaxWalksPerLaunch = 4;   // tensors (shard geometries) per materialize launch

// Where the elements of one shard sit in the full tensor.
struct BoxWalk {
  uint32_t run_v;                 // vectors per contiguous run
  uint32_t total_v;               // vectors per shard (= nruns * run_v)
  int32_t nouter;                 // outer dims after merging, innermost last
  uint32_t oext[kMaxRank];
  int64_t ostride_b[kMaxRank];    // outer strides in bytes
};

// Byte offset, from the box origin in the full tensor, of vector idx of the
// shard's contiguous buffer.
template <int VB>
__device__ __forceinline__ int64_t box_offset(const BoxWalk& w, uint32_t idx) {
  uint32_t r = idx / w.run_v;
  const uint32_t c = idx - r * w.run_v;
  int64_t off = static_cast<int64_t>(c) * VB;
  for (int i = w.nouter - 1; i >= 0; --i) {
    const uint32_t q = r / w.oext[i];
    off += static_cast<int64_t>(r - q * w.oext[i]) * w.ostride_b[i];
    r = q;
  }
  return off;
}

struct MatArgs {
  BoxWalk w[kMaxWalksPerLaunch];             // one per tensor in the launch
  const char *src[kMaxShardsPerLaunch];      // each shard's box origin in its tensor
  int32_t walk[kMaxShardsPerLaunch];         // which of w each shard follows
  int32_t dst_begin[kMaxShardsPerLaunch + 1];
  char *dst[kMaxDstPerLaunch];
};

struct GatherArgs {
  BoxWalk w;
  const char *shard[kMaxShardsPerLaunch];    // each shard's contiguous buffer
  int64_t dst_base_b[kMaxShardsPerLaunch];   // byte offset of each shard's box origin
  int32_t nout;
  char *out[kMaxDstPerLaunch];               // full-tensor outputs
};

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <int VB> struct VecOf;
template <> struct VecOf<16> { typedef u32x4_t T; };
template <> struct VecOf<8> { typedef u32x2_t T; };
template <> struct VecOf<4> { typedef uint32_t T; };
template <> struct VecOf<2> { typedef uint16_t T; };

// NT: non-temporal stores (large copies); otherwise the copy stays in the
// caches for the kernel that reads it next (a weight cut feeding a GEMM).
template <int VB, bool NT>
__device__ __forceinline__ void store_vec(typename VecOf<VB>::T v, char *p) {
  typedef typename VecOf<VB>::T V;
  if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<V *>(p));
  else *reinterpret_cast<V *>(p) = v;
}

// Workgroup -> (shard, slice): consecutive workgroups take the same slice of
// consecutive shards, so the shards advance together through the tensor (the
// runs side by side in the full tensor are read at the same time): 8% faster
// than shard after shard on the reshard's split (283 -> 261 us, MI355X, cold).
__device__ __forceinline__ void shard_slice(int *s, uint32_t *xb) {
  const uint32_t lin = blockIdx.y * gridDim.x + blockIdx.x;
  *s = static_cast<int>(lin % gridDim.y);
  *xb = lin / gridDim.y;
}

template <int VB, bool NT>
__global__ void __launch_bounds__(kThreads) materialize_kernel(MatArgs a) {
  typedef typename VecOf<VB>::T V;
  int s;
  uint32_t xb;
  shard_slice(&s, &xb);
  const char *src = a.src[s];
  const BoxWalk& w = a.w[a.walk[s]];
  const int d0 = a.dst_begin[s], d1 = a.dst_begin[s + 1];
  const uint32_t stride = gridDim.x * kThreads;
  for (uint32_t idx = xb * kThreads + threadIdx.x; idx < w.total_v; idx += stride) {
    const V v = __builtin_nontemporal_load(reinterpret_cast<const V *>(src + box_offset<VB>(w, idx)));
    for (int d = d0; d < d1; ++d)
      store_vec<VB, NT>(v, a.dst[d] + static_cast<int64_t>(idx) * VB);
  }
}

template <int VB, bool NT>
__global__ void __launch_bounds__(kThreads) gather_kernel(GatherArgs a) {
  typedef typename VecOf<VB>::T V;
  int s;
  uint32_t xb;
  shard_slice(&s, &xb);
  const char *src = a.shard[s];
  const int64_t base = a.dst_base_b[s];
  const uint32_t stride = gridDim.x * kThreads;
  for (uint32_t idx = xb * kThreads + threadIdx.x; idx < a.w.total_v; idx += stride) {
    const V v = __builtin_nontemporal_load(reinterpret_cast<const V *>(src + static_cast<int64_t>(idx) * VB));
    const int64_t off = base + box_offset<VB>(a.w, idx);
    for (int d = 0; d < a.nout; ++d) store_vec<VB, NT>(v, a.out[d] + off);
  }
}

// Short runs.  When the innermost cut axis leaves runs of under 16 bytes, a
// shard's elements lie a few bytes apart through the whole tensor and the
// per-shard kernels above read one element per lane from a different row:
// nothing coalesces, and every shard's workgroups pull the same cache lines.
// Here the tensor is viewed as rows of n runs of L elements (n shards along
// the innermost cut axis; the row index runs over every axis before it), and a
// workgroup takes a block of RB consecutive rows that lie in one box of the
// outer cut axes, so they are RB consecutive rows of each of the n shards it
// touches.  The split loads the block with 16-byte loads into LDS and writes
// each shard's RB x L elements with 16-byte stores assembled from LDS; the
// gather does the reverse.  Every HBM access is a full 16-byte vector, in
// order across the lanes.  In LDS each row is padded to an odd number of
// dwords: the lanes assembling consecutive output vectors read rows a fixed
// number apart, which with unpadded power-of-two rows would put most of them
// on a few banks.
constexpr int kRowsMaxShards = 64;
// 20 KiB of LDS holds a 16 KiB block of 8-element fp32 rows with their
// padding and lets 8 workgroups share a CU (the wave limit), against 5 at
// 32 KiB: 13% faster split + gather on MI355X.
constexpr int kRowsLdsBytes = 20 * 1024;
constexpr int kRowsPer = kRowsLdsBytes / 16 / 256;   // 16-byte vectors per lane per block, at most

struct RowsArgs {
  int32_t nax;                        // axes before the innermost cut axis
  int64_t shape[kMaxRank];            // their full extents
  int64_t ext[kMaxRank];              // their box extents
  int32_t dweight[kMaxRank];          // weight of each axis's shard digit in the digit index (0: not cut)
  int32_t sweight;                    // weight of the innermost cut axis's digit
  int32_t n, L, rb;                   // shards along the innermost cut axis, run length, rows per block
  int32_t pitch;                      // elements per row in LDS (the row, padded)
  int64_t rows;                       // rows of the full tensor (a multiple of rb)
  int32_t slot[kRowsMaxShards];       // digit index -> shard slot, or -1 (not in this call)
  int32_t dst_begin[kRowsMaxShards + 1];
  char *dst[kMaxDstPerLaunch];        // split: the devices of slot k at dst_begin[k] ..; gather: the outputs
  const char *src[kRowsMaxShards];    // gather: slot k's buffer
  const char *full;                   // split: the full tensor
  int32_t nout;                       // gather: outputs
};

// Digit index (shard of the outer cut axes) and local row of full-tensor row r0.
__device__ __forceinline__ void rows_box(const RowsArgs& a, int64_t r0, int32_t *dig, int64_t *lr) {
  int64_t rem = r0, l = 0, lstride = 1;
  int32_t d = 0;
  for (int i = a.nax - 1; i >= 0; --i) {
    const int64_t c = rem % a.shape[i];
    rem /= a.shape[i];
    d += static_cast<int32_t>(c / a.ext[i]) * a.dweight[i];
    l += (c % a.ext[i]) * lstride;
    lstride *= a.ext[i];
  }
  *dig = d;
  *lr = l;
}

template <int ES>
struct ElemOf;
template <> struct ElemOf<2> { typedef uint16_t T; };
template <> struct ElemOf<4> { typedef uint32_t T; };

// Lane-side index walks: one division per 16-byte vector, then the next
// element's row and column by increment.
template <int ES, bool NT>
__global__ void __launch_bounds__(kThreads) rows_split_kernel(RowsArgs a) {
  typedef typename ElemOf<ES>::T E;
  constexpr int EPV = 16 / ES;                       // elements per 16-byte vector
  static_assert(kThreads == 256, "kRowsPer assumes 256 lanes");
  __shared__ __attribute__((aligned(16))) E lds[kRowsLdsBytes / ES];
  const int wrow = a.n * a.L;
  const int blk_vec = a.rb * wrow * ES / 16;         // <= kRowsPer * kThreads (host: rb * pitch * ES <= LDS)
  const int shard_vec = a.rb * a.L * ES / 16;        // output vectors per shard per block
  const int64_t nblk = a.rows / a.rb;
  u32x4_t buf[kRowsPer];
  // The block's rows, 16-byte loads in order; the next block's are in flight
  // while this one is written out.
  auto load = [&](int64_t b) {
    const u32x4_t *in = reinterpret_cast<const u32x4_t *>(a.full + b * a.rb * wrow * ES);
#pragma unroll
    for (int q = 0; q < kRowsPer; ++q) {
      const int i = threadIdx.x + q * kThreads;
      if (i < blk_vec) buf[q] = __builtin_nontemporal_load(in + i);
    }
  };
  int64_t b = blockIdx.x;
  if (b < nblk) load(b);
  for (; b < nblk; b += gridDim.x) {
#pragma unroll
    for (int q = 0; q < kRowsPer; ++q) {
      const int i = threadIdx.x + q * kThreads;
      if (i >= blk_vec) break;
      const E *e = reinterpret_cast<const E *>(&buf[q]);
      int r = i * EPV / wrow, j = i * EPV - r * wrow;
#pragma unroll
      for (int t = 0; t < EPV; ++t) {
        lds[r * a.pitch + j] = e[t];
        if (++j == wrow) { j = 0; ++r; }
      }
    }
    int32_t dig;
    int64_t lr;
    rows_box(a, b * a.rb, &dig, &lr);
    __syncthreads();
    if (b + gridDim.x < nblk) load(b + gridDim.x);
    for (int u = threadIdx.x; u < a.n * shard_vec; u += kThreads) {
      const int s = u / shard_vec, v = u - s * shard_vec;
      const int k = a.slot[dig + s * a.sweight];
      if (k < 0) continue;
      E e[EPV];
      int r = v * EPV / a.L, c = v * EPV - r * a.L;
      const int base = s * a.L;
#pragma unroll
      for (int t = 0; t < EPV; ++t) {
        e[t] = lds[r * a.pitch + base + c];
        if (++c == a.L) { c = 0; ++r; }
      }
      const u32x4_t vec = __builtin_bit_cast(u32x4_t, e);
      const int64_t off = lr * a.L * ES + static_cast<int64_t>(v) * 16;
      for (int d = a.dst_begin[k]; d < a.dst_begin[k + 1]; ++d) store_vec<16, NT>(vec, a.dst[d] + off);
    }
    __syncthreads();
  }
}

template <int ES, bool NT>
__global__ void __launch_bounds__(kThreads) rows_gather_kernel(RowsArgs a) {
  typedef typename ElemOf<ES>::T E;
  constexpr int EPV = 16 / ES;
  __shared__ __attribute__((aligned(16))) E lds[kRowsLdsBytes / ES];
  const int wrow = a.n * a.L;
  const int blk_vec = a.rb * wrow * ES / 16;
  const int shard_vec = a.rb * a.L * ES / 16;
  const int nvec = a.n * shard_vec;                  // = blk_vec
  const int64_t nblk = a.rows / a.rb;
  u32x4_t buf[kRowsPer];
  // Each shard's run of the block, 16-byte loads in order; the next block's
  // are in flight while this one is written out.
  auto load = [&](int64_t b) {
    int32_t dig;
    int64_t lr;
    rows_box(a, b * a.rb, &dig, &lr);
#pragma unroll
    for (int q = 0; q < kRowsPer; ++q) {
      const int u = threadIdx.x + q * kThreads;
      if (u < nvec) {
        const int s = u / shard_vec, v = u - s * shard_vec;
        const int k = a.slot[dig + s * a.sweight];
        buf[q] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4_t *>(a.src[k] + lr * a.L * ES + static_cast<int64_t>(v) * 16));
      }
    }
  };
  int64_t b = blockIdx.x;
  if (b < nblk) load(b);
  for (; b < nblk; b += gridDim.x) {
#pragma unroll
    for (int q = 0; q < kRowsPer; ++q) {
      const int u = threadIdx.x + q * kThreads;
      if (u >= nvec) break;
      const int s = u / shard_vec, v = u - s * shard_vec;
      const E *e = reinterpret_cast<const E *>(&buf[q]);
      int r = v * EPV / a.L, c = v * EPV - r * a.L;
      const int base = s * a.L;
#pragma unroll
      for (int t = 0; t < EPV; ++t) {
        lds[r * a.pitch + base + c] = e[t];
        if (++c == a.L) { c = 0; ++r; }
      }
    }
    __syncthreads();
    const int64_t r0 = b * a.rb;
    if (b + gridDim.x < nblk) load(b + gridDim.x);
    for (int i = threadIdx.x; i < blk_vec; i += kThreads) {
      E e[EPV];
      int r = i * EPV / wrow, j = i * EPV - r * wrow;
#pragma unroll
      for (int t = 0; t < EPV; ++t) {
        e[t] = lds[r * a.pitch + j];
        if (++j == wrow) { j = 0; ++r; }
      }
      const u32x4_t vec = __builtin_bit_cast(u32x4_t, e);
      for (int d = 0; d < a.nout; ++d)
        store_vec<16, NT>(vec, a.dst[d] + r0 * wrow * ES + static_cast<int64_t>(i) * 16);
    }
    __syncthreads();
  }
}

// Run/stride decomposition of a plan's (common) shard box.
struct Geometry {
  int64_t shard_elems = 1;
  int64_t run = 1;                 // elements per contiguous run
  int64_t stride[kMaxRank] = {};   // element strides of the full tensor
  std::vector<int64_t> oext, ostr; // merged outer extents and element strides
};

Geometry geometry(const ShardPlan& plan) {
  Geometry g;
  const int r = plan.ndim;
  for (int i = 0; i < r; ++i) g.shard_elems *= plan.extent[i];
  // Contiguous run: from the innermost axis out to the last one that is cut.
  int jstar = -1;
  for (int i = 0; i < r; ++i)
    if (plan.extent[i] < plan.shape[i]) jstar = i;
  int64_t s = 1;
  for (int i = r - 1; i >= 0; --i) {
    g.stride[i] = s;
    s *= plan.shape[i];
  }
  if (jstar < 0) {
    g.run = g.shard_elems;
  } else {
    for (int i = jstar; i < r; ++i) g.run *= (i == jstar ? plan.extent[i] : plan.shape[i]);
  }
  // Outer axes 0..jstar-1, merged where the inner neighbour is whole.
  for (int i = 0; i < jstar; ++i) {
    if (plan.extent[i] == 1) continue;
    if (!g.oext.empty() && g.ostr.back() == plan.extent[i] * g.stride[i] && plan.extent[i] == plan.shape[i]) {
      g.oext.back() *= plan.extent[i];
      g.ostr.back() = g.stride[i];
    } else {
      g.oext.push_back(plan.extent[i]);
      g.ostr.push_back(g.stride[i]);
    }
  }
  return g;
}

int64_t box_origin(const ShardPlan& plan, const Geometry& g, int64_t k) {
  int64_t off = 0;
  for (int i = 0; i < plan.ndim; ++i) off += plan.offset[k * plan.ndim + i] * g.stride[i];
  return off;
}

// Widest vector (bytes) that every address of the copy is aligned to.  `full`
// is the full tensor's base, `pieces` the per-device buffers actually touched.
int vector_bytes(const ShardPlan& plan, const Geometry& g, int64_t esize, const void *full,
                 const std::vector<const void *>& pieces) {
  auto aligned = [&](int vb) {
    if ((g.run * esize) % vb) return false;
    for (int64_t s2 : g.ostr)
      if ((s2 * esize) % vb) return false;
    if (reinterpret_cast<uintptr_t>(full) % vb) return false;
    for (int64_t k = 0; k < plan.nshards(); ++k)
      if ((box_origin(plan, g, k) * esize) % vb) return false;
    for (const void *p : pieces)
      if (reinterpret_cast<uintptr_t>(p) % vb) return false;
    return true;
  };
  for (int cand : {16, 8, 4})
    if (cand >= esize && aligned(cand)) return cand;
  return static_cast<int>(esize);
}

int fill_walk(const Geometry& g, int64_t esize, int vb, BoxWalk *w) {
  const int64_t total_v = g.shard_elems * esize / vb;
  if (total_v >= (int64_t(1) << 31))
    return fail(TP_ERR_UNSUPPORTED, "shard of %lld bytes exceeds the 32-bit index range", (long long)(g.shard_elems * esize));
  w->run_v = static_cast<uint32_t>(g.run * esize / vb);
  w->total_v = static_cast<uint32_t>(total_v);
  w->nouter = static_cast<int32_t>(g.oext.size());
  for (size_t i = 0; i < g.oext.size(); ++i) {
    w->oext[i] = static_cast<uint32_t>(g.oext[i]);
    w->ostride_b[i] = g.ostr[i] * esize;
  }
  return TP_OK;
}

// Copies writing up to this many bytes keep their output in the caches (the
// kernel that consumes it, e.g. the GEMM reading a freshly cut weight, runs
// next); larger ones stream past the caches.
constexpr int64_t kCachedCopyBytes = int64_t(64) << 20;

template <class K, class Args>
void launch_vb(K k_nt, K k_cached, bool nt, dim3 grid, hipStream_t s, const Args& a) {
  if (nt) hipLaunchKernelGGL(k_nt, grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(k_cached, grid, dim3(kThreads), 0, s, a);
}

dim3 copy_grid(uint32_t total_v, int nshards) {
  const int64_t want = (static_cast<int64_t>(total_v) + kThreads - 1) / kThreads;
  const int64_t cap = std::max<int64_t>(1, (1 << 20) / nshards);
  return dim3(static_cast<unsigned>(std::min(want, cap)), static_cast<unsigned>(nshards));
}

// The row-block geometry of a plan whose innermost cut leaves runs of under
// 16 bytes, or false when the short-run kernels do not apply (long runs; an
// element size other than 2 or 4; more than kRowsMaxShards shard positions;
// no block of at least 8 rows that stays inside one box and fits the LDS).
bool rows_plan(const ShardPlan& plan, int64_t esize, RowsArgs *a) {
  if (esize != 2 && esize != 4) return false;
  const int r = plan.ndim;
  int jstar = -1;
  for (int i = 0; i < r; ++i)
    if (plan.extent[i] < plan.shape[i]) jstar = i;
  if (jstar < 1) return false;
  int64_t L = plan.extent[jstar];
  for (int i = jstar + 1; i < r; ++i) L *= plan.shape[i];
  if (L * esize >= 16) return false;
  const int64_t n = plan.shape[jstar] / plan.extent[jstar];
  // Digit index: the shard digits of the cut axes, row-major, the innermost cut axis last.
  int64_t combos = n, rows = 1;
  a->sweight = 1;
  for (int i = jstar - 1; i >= 0; --i) {
    const int64_t ni = plan.shape[i] / plan.extent[i];
    a->dweight[i] = ni > 1 ? static_cast<int32_t>(combos) : 0;
    if (ni > 1) combos *= ni;
    rows *= plan.shape[i];
    if (combos > kRowsMaxShards) return false;
  }
  if (combos > kRowsMaxShards || plan.nshards() > kRowsMaxShards) return false;
  // Consecutive rows that stay in one box: the innermost outer cut axis's box
  // extent times the axes inside it, or every row when no outer axis is cut.
  int64_t G = rows;
  for (int i = jstar - 1; i >= 0; --i)
    if (plan.extent[i] < plan.shape[i]) {
      G = plan.extent[i];
      for (int q = i + 1; q < jstar; ++q) G *= plan.shape[q];
      break;
    }
  // LDS row: the row padded to an odd number of dwords (an even number of
  // elements for 2-byte ones, so that rows stay dword-aligned).
  int64_t pitch = n * L;
  while ((pitch * esize) % 4 != 0 || ((pitch * esize) / 4) % 2 == 0) ++pitch;
  int64_t rb = 1;
  while (rb * 2 <= G && G % (rb * 2) == 0 && rb * 2 * pitch * esize <= kRowsLdsBytes) rb *= 2;
  if (rb < 8) return false;
  a->nax = jstar;
  for (int i = 0; i < jstar; ++i) {
    a->shape[i] = plan.shape[i];
    a->ext[i] = plan.extent[i];
  }
  a->n = static_cast<int32_t>(n);
  a->L = static_cast<int32_t>(L);
  a->rb = static_cast<int32_t>(rb);
  a->pitch = static_cast<int32_t>(pitch);
  a->rows = rows;
  for (int q = 0; q < kRowsMaxShards; ++q) a->slot[q] = -1;
  for (int64_t k = 0; k < plan.nshards(); ++k) {
    int32_t idx = static_cast<int32_t>(plan.offset[k * r + jstar] / plan.extent[jstar]) * a->sweight;
    for (int i = 0; i < jstar; ++i) idx += static_cast<int32_t>(plan.offset[k * r + i] / plan.extent[i]) * a->dweight[i];
    a->slot[idx] = static_cast<int32_t>(k);
  }
  return true;
}

bool aligned16p(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Blocks per workgroup: the split runs one (a one-shot grid), the gather two,
// the second block's loads in flight while the first is written out (measured
// best of 1, 2 and 4 for each, and of a 4096-workgroup grid-stride loop).
unsigned rows_grid(const RowsArgs& a, int64_t per_wg) {
  return static_cast<unsigned>(std::min<int64_t>(std::max<int64_t>(1, a.rows / a.rb / per_wg), 1 << 20));
}

// The short-run split of one tensor, or 1 when it does not apply (the caller
// then uses the per-shard kernel).
int rows_split(const MatJob& jb, hipStream_t stream) {
  RowsArgs a{};
  if (!rows_plan(*jb.plan, jb.esize, &a) || !aligned16p(jb.src)) return 1;
  int nd = 0;
  a.dst_begin[0] = 0;
  int64_t ndev = 0;
  for (int64_t k = 0; k < jb.plan->nshards(); ++k) {
    const auto& grp = jb.plan->devices[k];
    if (nd + static_cast<int>(grp.size()) > kMaxDstPerLaunch) return 1;
    for (int64_t d : grp) {
      if (!aligned16p(jb.dst[d])) return 1;
      a.dst[nd++] = static_cast<char *>(jb.dst[d]);
    }
    a.dst_begin[k + 1] = nd;
    ndev += static_cast<int64_t>(grp.size());
  }
  a.full = static_cast<const char *>(jb.src);
  // Algorithmic bytes: the full tensor read once (every element of it belongs
  // to some shard), each device's shard written once.
  const int64_t elems = a.rows * a.n * a.L;
  int64_t per_shard = 1;
  for (int i = 0; i < jb.plan->ndim; ++i) per_shard *= jb.plan->extent[i];
  const double bytes = static_cast<double>(elems) * jb.esize + static_cast<double>(ndev) * per_shard * jb.esize;
  const bool nt = static_cast<double>(ndev) * per_shard * jb.esize > static_cast<double>(kCachedCopyBytes);
  hipEvent_t t0 = timing_begin(stream);
  const dim3 grid(rows_grid(a, 1));
  if (jb.esize == 4) launch_vb(rows_split_kernel<4, true>, rows_split_kernel<4, false>, nt, grid, stream, a);
  else launch_vb(rows_split_kernel<2, true>, rows_split_kernel<2, false>, nt, grid, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TP_ERR_HIP, "materialize launch: %s", hipGetErrorString(e));
  timing_end(t0, stream, TP_KERNEL_MATERIALIZE, bytes);
  return TP_OK;
}

}  // namespace

int shard_materialize_batch_launch(const MatJob *jobs, int njobs, hipStream_t stream) {
  std::vector<Geometry> geo;
  std::vector<int> live;
  int vb = 16;
  int64_t written = 0;
  for (int j = 0; j < njobs; ++j) {
    const MatJob& jb = jobs[j];
    geo.push_back(geometry(*jb.plan));
    if (geo.back().shard_elems == 0 || jb.plan->nshards() == 0) continue;
    // Short runs: the row-block kernel, a launch of its own.
    const int rc = rows_split(jb, stream);
    if (rc == TP_OK) continue;
    if (rc < 0) return rc;
    std::vector<const void *> pieces;
    for (const auto& grp : jb.plan->devices)
      for (int64_t d : grp) pieces.push_back(jb.dst[d]);
    vb = std::min(vb, vector_bytes(*jb.plan, geo.back(), jb.esize, jb.src, pieces));
    written += static_cast<int64_t>(pieces.size()) * geo.back().shard_elems * jb.esize;
    live.push_back(j);
  }
  if (live.empty()) return TP_OK;
  std::vector<BoxWalk> walks(static_cast<size_t>(njobs));
  for (int j : live) {
    const int rc = fill_walk(geo[j], jobs[j].esize, vb, &walks[j]);
    if (rc != TP_OK) return rc;
  }
  const bool nt = written > kCachedCopyBytes;

  // Pack shards (of one or several tensors) into launches bounded by the argument tables.
  MatArgs a{};
  int ns = 0, nd = 0, nw = 0, walk_job[kMaxWalksPerLaunch] = {};
  uint32_t max_v = 0;
  double bytes = 0;
  auto flush = [&]() -> int {
    if (ns == 0) return TP_OK;
    const dim3 grid = copy_grid(max_v, ns);
    hipEvent_t t0 = timing_begin(stream);
    switch (vb) {
      case 16: launch_vb(materialize_kernel<16, true>, materialize_kernel<16, false>, nt, grid, stream, a); break;
      case 8: launch_vb(materialize_kernel<8, true>, materialize_kernel<8, false>, nt, grid, stream, a); break;
      case 4: launch_vb(materialize_kernel<4, true>, materialize_kernel<4, false>, nt, grid, stream, a); break;
      default: launch_vb(materialize_kernel<2, true>, materialize_kernel<2, false>, nt, grid, stream, a); break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TP_ERR_HIP, "materialize launch: %s", hipGetErrorString(e));
    timing_end(t0, stream, TP_KERNEL_MATERIALIZE, bytes);
    ns = nd = nw = 0;
    max_v = 0;
    bytes = 0;
    a.dst_begin[0] = 0;
    return TP_OK;
  };
  a.dst_begin[0] = 0;
  for (int j : live) {
    const MatJob& jb = jobs[j];
    const ShardPlan& plan = *jb.plan;
    const int64_t shard_bytes = geo[j].shard_elems * jb.esize;
    for (int64_t k = 0; k < plan.nshards(); ++k) {
      const auto& grp = plan.devices[k];
      if (static_cast<int>(grp.size()) > kMaxDstPerLaunch)
        return fail(TP_ERR_UNSUPPORTED, "a shard is replicated to more than %d devices", kMaxDstPerLaunch);
      int wi = -1;
      for (int q = 0; q < nw; ++q)
        if (walk_job[q] == j) wi = q;
      if (ns == kMaxShardsPerLaunch || nd + static_cast<int>(grp.size()) > kMaxDstPerLaunch ||
          (wi < 0 && nw == kMaxWalksPerLaunch)) {
        const int rc = flush();
        if (rc != TP_OK) return rc;
        wi = -1;
      }
      if (wi < 0) {
        wi = nw++;
        walk_job[wi] = j;
        a.w[wi] = walks[j];
        max_v = std::max(max_v, walks[j].total_v);
      }
      a.src[ns] = static_cast<const char *>(jb.src) + box_origin(plan, geo[j], k) * jb.esize;
      a.walk[ns] = wi;
      for (int64_t d : grp) a.dst[nd++] = static_cast<char *>(jb.dst[d]);
      a.dst_begin[++ns] = nd;
      bytes += static_cast<double>(1 + grp.size()) * shard_bytes;
    }
  }
  return flush();
}

int shard_materialize_launch(const ShardPlan& plan, const void *src, int64_t esize, void *const *dst,
                             hipStream_t stream) {
  const MatJob job{&plan, src, esize, dst};
  return shard_materialize_batch_launch(&job, 1, stream);
}

int shard_gather_launch(const ShardPlan& plan, const void *const *src, int64_t esize, void *const *out, int64_t nout,
                        hipStream_t stream) {
  const Geometry g = geometry(plan);
  if (g.shard_elems == 0 || plan.nshards() == 0 || nout == 0) return TP_OK;
  // Short runs: the row-block kernel (every shard position present, every
  // pointer 16-byte aligned, the outputs in one launch).
  {
    RowsArgs a{};
    bool ok = nout <= kMaxDstPerLaunch && rows_plan(plan, esize, &a);
    if (ok) {
      // The gather reads every shard position.
      int64_t combos = a.n;
      for (int i = 0; i < a.nax; ++i)
        if (a.dweight[i]) combos *= plan.shape[i] / plan.extent[i];
      ok = combos == plan.nshards();
    }
    for (int64_t k = 0; ok && k < plan.nshards(); ++k) {
      a.src[k] = static_cast<const char *>(src[plan.devices[k][0]]);
      ok = aligned16p(a.src[k]);
    }
    for (int64_t j = 0; ok && j < nout; ++j) {
      a.dst[j] = static_cast<char *>(out[j]);
      ok = aligned16p(out[j]);
    }
    if (ok) {
      a.nout = static_cast<int32_t>(nout);
      const double full_bytes = static_cast<double>(a.rows) * a.n * a.L * esize;
      const bool nt = nout * full_bytes > static_cast<double>(kCachedCopyBytes);
      hipEvent_t t0 = timing_begin(stream);
      const dim3 grid(rows_grid(a, 2));
      if (esize == 4) launch_vb(rows_gather_kernel<4, true>, rows_gather_kernel<4, false>, nt, grid, stream, a);
      else launch_vb(rows_gather_kernel<2, true>, rows_gather_kernel<2, false>, nt, grid, stream, a);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return fail(TP_ERR_HIP, "gather launch: %s", hipGetErrorString(e));
      timing_end(t0, stream, TP_KERNEL_GATHER, (1.0 + nout) * full_bytes);
      return TP_OK;
    }
  }
  std::vector<const void *> pieces;
  for (const auto& grp : plan.devices) pieces.push_back(src[grp[0]]);
  for (int64_t j = 1; j < nout; ++j) pieces.push_back(out[j]);
  const int vb = vector_bytes(plan, g, esize, out[0], pieces);
  GatherArgs a{};
  int rc = fill_walk(g, esize, vb, &a.w);
  if (rc != TP_OK) return rc;
  const bool nt = nout * plan.nshards() * g.shard_elems * esize > kCachedCopyBytes;

  // Outputs in groups of kMaxDstPerLaunch (a shard is re-read per group),
  // shards in groups of kMaxShardsPerLaunch.
  for (int64_t j0 = 0; j0 < nout; j0 += kMaxDstPerLaunch) {
    a.nout = static_cast<int32_t>(std::min<int64_t>(kMaxDstPerLaunch, nout - j0));
    for (int j = 0; j < a.nout; ++j) a.out[j] = static_cast<char *>(out[j0 + j]);
    for (int64_t k0 = 0; k0 < plan.nshards(); k0 += kMaxShardsPerLaunch) {
      const int ns = static_cast<int>(std::min<int64_t>(kMaxShardsPerLaunch, plan.nshards() - k0));
      for (int s = 0; s < ns; ++s) {
        a.shard[s] = static_cast<const char *>(src[plan.devices[k0 + s][0]]);
        a.dst_base_b[s] = box_origin(plan, g, k0 + s) * esize;
      }
      const dim3 grid = copy_grid(a.w.total_v, ns);
      hipEvent_t t0 = timing_begin(stream);
      switch (vb) {
        case 16: launch_vb(gather_kernel<16, true>, gather_kernel<16, false>, nt, grid, stream, a); break;
        case 8: launch_vb(gather_kernel<8, true>, gather_kernel<8, false>, nt, grid, stream, a); break;
        case 4: launch_vb(gather_kernel<4, true>, gather_kernel<4, false>, nt, grid, stream, a); break;
        default: launch_vb(gather_kernel<2, true>, gather_kernel<2, false>, nt, grid, stream, a); break;
      }
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return fail(TP_ERR_HIP, "gather launch: %s", hipGetErrorString(e));
      timing_end(t0, stream, TP_KERNEL_GATHER, static_cast<double>(ns) * (1 + a.nout) * g.shard_elems * esize);
    }
  }
  return TP_OK;
}

}  // namespace tpshard
