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

template <int VB, bool NT>
__global__ void __launch_bounds__(kThreads) materialize_kernel(MatArgs a) {
  typedef typename VecOf<VB>::T V;
  const int s = blockIdx.y;
  const char *src = a.src[s];
  const BoxWalk& w = a.w[a.walk[s]];
  const int d0 = a.dst_begin[s], d1 = a.dst_begin[s + 1];
  const uint32_t stride = gridDim.x * kThreads;
  for (uint32_t idx = blockIdx.x * kThreads + threadIdx.x; idx < w.total_v; idx += stride) {
    const V v = __builtin_nontemporal_load(reinterpret_cast<const V *>(src + box_offset<VB>(w, idx)));
    for (int d = d0; d < d1; ++d)
      store_vec<VB, NT>(v, a.dst[d] + static_cast<int64_t>(idx) * VB);
  }
}

template <int VB, bool NT>
__global__ void __launch_bounds__(kThreads) gather_kernel(GatherArgs a) {
  typedef typename VecOf<VB>::T V;
  const int s = blockIdx.y;
  const char *src = a.shard[s];
  const int64_t base = a.dst_base_b[s];
  const uint32_t stride = gridDim.x * kThreads;
  for (uint32_t idx = blockIdx.x * kThreads + threadIdx.x; idx < a.w.total_v; idx += stride) {
    const V v = __builtin_nontemporal_load(reinterpret_cast<const V *>(src + static_cast<int64_t>(idx) * VB));
    const int64_t off = base + box_offset<VB>(a.w, idx);
    for (int d = 0; d < a.nout; ++d) store_vec<VB, NT>(v, a.out[d] + off);
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
