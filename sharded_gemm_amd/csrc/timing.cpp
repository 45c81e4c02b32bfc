// Per-kernel timing instrumentation (see tpshard.h, tp_timing_enable).
#include "timing.h"

#include <vector>

namespace tpshard {

namespace {

struct Pending {
  hipEvent_t start, stop;
  int kind;
  double work;
};

struct Timing {
  bool on = false;
  std::vector<hipEvent_t> free_events;
  std::vector<Pending> pending;
  ~Timing() {
    for (hipEvent_t e : free_events) (void)hipEventDestroy(e);
  }
};
thread_local Timing g_timing;

hipEvent_t take_event() {
  if (!g_timing.free_events.empty()) {
    hipEvent_t e = g_timing.free_events.back();
    g_timing.free_events.pop_back();
    return e;
  }
  // Timing-only events: no system-scope fence, so recording one neither
  // writes back nor invalidates caches around the kernel being timed.
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

bool timing_on() { return g_timing.on; }

hipEvent_t timing_begin(hipStream_t s) {
  if (!g_timing.on) return nullptr;
  hipEvent_t e = take_event();
  if (!e) return nullptr;
  if (hipEventRecord(e, s) != hipSuccess) {
    g_timing.free_events.push_back(e);
    return nullptr;
  }
  return e;
}

void timing_end(hipEvent_t start, hipStream_t s, int kind, double work) {
  if (!start) return;
  hipEvent_t stop = take_event();
  if (!stop || hipEventRecord(stop, s) != hipSuccess) {
    g_timing.free_events.push_back(start);
    return;
  }
  g_timing.pending.push_back({start, stop, kind, work});
}

}  // namespace tpshard

using namespace tpshard;

extern "C" {

int tp_timing_enable(int32_t on) {
  g_timing.on = on != 0;
  return TP_OK;
}

int tp_timing_read(tp_kernel_stat *stats) {
  clear_error();
  if (!stats) return fail(TP_ERR_ARG, "stats is NULL");
  for (int k = 0; k < TP_KERNEL_KINDS; ++k) stats[k] = tp_kernel_stat{0, 0.0, 0.0, 0.0, 0.0};
  int rc = TP_OK;
  for (const Pending& p : g_timing.pending) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(p.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, p.start, p.stop);
    if (e != hipSuccess && rc == TP_OK) rc = fail(TP_ERR_HIP, "timing event: %s", hipGetErrorString(e));
    if (e == hipSuccess && p.kind >= 0 && p.kind < TP_KERNEL_KINDS) {
      tp_kernel_stat& st = stats[p.kind];
      st.min_ms = st.launches ? (ms < st.min_ms ? ms : st.min_ms) : ms;
      st.max_ms = st.launches ? (ms > st.max_ms ? ms : st.max_ms) : ms;
      st.launches += 1;
      st.total_ms += ms;
      st.work += p.work;
    }
    g_timing.free_events.push_back(p.start);
    g_timing.free_events.push_back(p.stop);
  }
  g_timing.pending.clear();
  return rc;
}

}  // extern "C"
