// Shard materialisation: split + replicate in one pass ([ONNX] "Sharding as a
// Split", "Sharding as a Broadcast", "mixing split and broadcast"; [SBP]
// "SBP"; [SPMD] "dims_mapping").
//
// All shards of a layout have the same extents, so a shard is a set of
// equal-length runs that are contiguous in the source (the innermost sharded
// axis and every axis after it) separated by fixed strides on the outer axes.
// The destination of a shard is one contiguous buffer per receiving device.
// A workgroup streams a slice of one shard with the widest vector the
// alignment allows (16, 8, 4 or 2 bytes per lane) and writes each element to
// every device of the shard's group, so the source is read exactly once.
// The source is read once and destinations written once, so both use
// non-temporal accesses.
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
constexpr int kUnroll = 1;   // one vector per lane, one-shot grid: measured best on MI355X
constexpr int kMaxShardsPerLaunch = 32;
constexpr int kMaxDstPerLaunch = 64;

struct MatArgs {
  const char *src;
  uint32_t run_v;                 // vectors per run
  uint32_t total_v;               // vectors per shard (= nruns * run_v)
  int32_t nouter;                 // outer dims after merging, innermost last
  uint32_t oext[kMaxRank];
  int64_t ostride_b[kMaxRank];    // outer strides in bytes
  int64_t src_base_b[kMaxShardsPerLaunch];   // byte offset of each shard's box origin
  int32_t dst_begin[kMaxShardsPerLaunch + 1];
  char *dst[kMaxDstPerLaunch];
};

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <int VB> struct VecOf;
template <> struct VecOf<16> { typedef u32x4_t T; };
template <> struct VecOf<8> { typedef u32x2_t T; };
template <> struct VecOf<4> { typedef uint32_t T; };
template <> struct VecOf<2> { typedef uint16_t T; };

template <int VB>
__global__ void __launch_bounds__(kThreads) materialize_kernel(MatArgs a) {
  typedef typename VecOf<VB>::T V;
  const int s = blockIdx.y;
  const char *src = a.src + a.src_base_b[s];
  const int d0 = a.dst_begin[s], d1 = a.dst_begin[s + 1];
  const uint32_t stride = gridDim.x * kThreads;
  for (uint32_t base = blockIdx.x * kThreads + threadIdx.x; base < a.total_v; base += stride * kUnroll) {
    V v[kUnroll];
    uint32_t idx[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      idx[u] = base + u * stride;
      if (idx[u] < a.total_v) {
        uint32_t r = idx[u] / a.run_v;
        const uint32_t c = idx[u] - r * a.run_v;
        int64_t off = static_cast<int64_t>(c) * VB;
        for (int i = a.nouter - 1; i >= 0; --i) {
          const uint32_t q = r / a.oext[i];
          off += static_cast<int64_t>(r - q * a.oext[i]) * a.ostride_b[i];
          r = q;
        }
        v[u] = __builtin_nontemporal_load(reinterpret_cast<const V *>(src + off));
      }
    }
    for (int d = d0; d < d1; ++d) {
      char *dst = a.dst[d];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        if (idx[u] < a.total_v)
          __builtin_nontemporal_store(v[u], reinterpret_cast<V *>(dst + static_cast<int64_t>(idx[u]) * VB));
    }
  }
}

}  // namespace

int shard_materialize_launch(const ShardPlan& plan, const void *src, int64_t esize, void *const *dst,
                             hipStream_t stream) {
  const int r = plan.ndim;
  int64_t shard_elems = 1;
  for (int i = 0; i < r; ++i) shard_elems *= plan.extent[i];
  if (shard_elems == 0 || plan.nshards() == 0) return TP_OK;

  // Contiguous run: from the innermost axis out to the last one that is cut.
  int jstar = -1;
  for (int i = 0; i < r; ++i)
    if (plan.extent[i] < plan.shape[i]) jstar = i;
  int64_t stride[kMaxRank];
  {
    int64_t s = 1;
    for (int i = r - 1; i >= 0; --i) {
      stride[i] = s;
      s *= plan.shape[i];
    }
  }
  int64_t run = 1;
  for (int i = std::max(jstar, 0); i < r; ++i) run *= (i == jstar ? plan.extent[i] : plan.shape[i]);
  if (jstar < 0) run = shard_elems;
  // Outer axes 0..jstar-1, merged where the inner neighbour is whole.
  std::vector<int64_t> oext, ostr;
  for (int i = 0; i < jstar; ++i) {
    if (plan.extent[i] == 1) continue;
    if (!oext.empty() && ostr.back() == plan.extent[i] * stride[i] && plan.extent[i] == plan.shape[i]) {
      oext.back() *= plan.extent[i];
      ostr.back() = stride[i];
    } else {
      oext.push_back(plan.extent[i]);
      ostr.push_back(stride[i]);
    }
  }

  // Widest vector that every address of the copy is aligned to.
  auto aligned = [&](int vb) {
    if ((run * esize) % vb) return false;
    if (reinterpret_cast<uintptr_t>(src) % vb) return false;
    for (int64_t s2 : ostr)
      if ((s2 * esize) % vb) return false;
    for (int64_t k = 0; k < plan.nshards(); ++k) {
      int64_t off = 0;
      for (int i = 0; i < r; ++i) off += plan.offset[k * r + i] * stride[i];
      if ((off * esize) % vb) return false;
      for (int64_t d : plan.devices[k])
        if (reinterpret_cast<uintptr_t>(dst[d]) % vb) return false;
    }
    return true;
  };
  int vb = static_cast<int>(esize);
  for (int cand : {16, 8, 4})
    if (cand >= esize && aligned(cand)) {
      vb = cand;
      break;
    }
  const int64_t run_v = run * esize / vb;
  const int64_t total_v = shard_elems * esize / vb;
  if (total_v >= (int64_t(1) << 31))
    return fail(TP_ERR_UNSUPPORTED, "shard of %lld bytes exceeds the 32-bit index range", (long long)(shard_elems * esize));

  MatArgs a{};
  a.src = static_cast<const char *>(src);
  a.run_v = static_cast<uint32_t>(run_v);
  a.total_v = static_cast<uint32_t>(total_v);
  a.nouter = static_cast<int32_t>(oext.size());
  for (size_t i = 0; i < oext.size(); ++i) {
    a.oext[i] = static_cast<uint32_t>(oext[i]);
    a.ostride_b[i] = ostr[i] * esize;
  }

  // Batch shards into launches bounded by the argument tables.
  int64_t k = 0;
  while (k < plan.nshards()) {
    int ns = 0, nd = 0;
    a.dst_begin[0] = 0;
    while (k < plan.nshards() && ns < kMaxShardsPerLaunch) {
      const auto& grp = plan.devices[k];
      if (nd + static_cast<int>(grp.size()) > kMaxDstPerLaunch) {
        if (ns > 0) break;
        return fail(TP_ERR_UNSUPPORTED, "a shard is replicated to more than %d devices", kMaxDstPerLaunch);
      }
      int64_t off = 0;
      for (int i = 0; i < r; ++i) off += plan.offset[k * r + i] * stride[i];
      a.src_base_b[ns] = off * esize;
      for (int64_t d : grp) a.dst[nd++] = static_cast<char *>(dst[d]);
      a.dst_begin[++ns] = nd;
      ++k;
    }
    const int64_t want = (total_v + kThreads * kUnroll - 1) / (kThreads * kUnroll);
    const int64_t cap = std::max<int64_t>(1, (1 << 20) / ns);
    const dim3 grid(static_cast<unsigned>(std::min(want, cap)), static_cast<unsigned>(ns));
    hipEvent_t t0 = timing_begin(stream);
    switch (vb) {
      case 16: hipLaunchKernelGGL(materialize_kernel<16>, grid, dim3(kThreads), 0, stream, a); break;
      case 8: hipLaunchKernelGGL(materialize_kernel<8>, grid, dim3(kThreads), 0, stream, a); break;
      case 4: hipLaunchKernelGGL(materialize_kernel<4>, grid, dim3(kThreads), 0, stream, a); break;
      default: hipLaunchKernelGGL(materialize_kernel<2>, grid, dim3(kThreads), 0, stream, a); break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TP_ERR_HIP, "materialize launch: %s", hipGetErrorString(e));
    timing_end(t0, stream, TP_KERNEL_MATERIALIZE, static_cast<double>(ns + nd) * shard_elems * esize);
  }
  return TP_OK;
}

}  // namespace tpshard
