// The forward entry point for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation): tp_colrow_mlp with its one workspace, the hidden activations Y,
// in a fixed device array of this library instead of a caller's buffer.
//
// The array is a file-scope device variable, so every GPU the library runs on
// holds its own copy from module load until the process ends.  Host code may
// only use the address hipGetSymbolAddress returns for the current device
// (the variable's own name is a host-side stand-in); it is looked up once per
// device, with that device current, on the entry point's first call there.
// Every call on a GPU shares that GPU's array: calls that overlap on one GPU
// (on different streams, or from different threads) race on it.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <mutex>

#include "common.h"

namespace tpshard {
namespace {

constexpr size_t kScratchBytes = size_t{32} << 20;   // one row chunk of Y: 32 MiB
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// This device's copy of the array, for `bytes` of it.  Called by the
// validated forward (colrow_mlp_run) before anything is enqueued.
int scratch_for(int64_t bytes, void **out) {
  if (bytes < 0 || static_cast<uint64_t>(bytes) > kScratchBytes)
    return fail(TP_ERR_UNSUPPORTED, "one row chunk of Y (%lld bytes) exceeds the %zu-byte scratch", (long long)bytes,
                kScratchBytes);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TP_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(TP_ERR_UNSUPPORTED, "device %d beyond the %d this library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail(TP_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    if (!p) return fail(TP_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TP_OK;
}

}  // namespace
}  // namespace tpshard

using namespace tpshard;

extern "C" int tp_colrow_mlp_noalloc(const tp_mlp_args *a, tp_stream_t s_compute, tp_stream_t s_reduce) {
  clear_error();
  if (!a) return fail(TP_ERR_ARG, "args is NULL");
  return colrow_mlp_run(a, s_compute, s_reduce, scratch_for);
}
