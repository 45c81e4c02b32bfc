// Optional per-kernel timing: HIP timing events around each launch, folded
// into per-kind statistics on request.  Thread-local; off by default.
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace tpshard {

bool timing_on();

// Records a start event on s if timing is on; returns it (nullptr when off).
hipEvent_t timing_begin(hipStream_t s);
// Records the end event on s and files the launch under kind/work.
void timing_end(hipEvent_t start, hipStream_t s, int kind, double work);

}  // namespace tpshard
