// Host-side layout planning: a ShardingSpec or (ProcessMesh, dims_mapping)
// pair becomes a list of distinct shard boxes, each with the devices that
// receive it.  Pure C++ (no HIP), so it is testable without a GPU.
#pragma once

#include <cstdint>
#include <vector>

#include "common.h"

namespace tpshard {

struct ShardPlan {
  int ndim = 0;
  int64_t shape[kMaxRank] = {};
  int64_t extent[kMaxRank] = {};     // every shard has the same extents
  std::vector<int64_t> offset;       // nshards * ndim box origins
  std::vector<std::vector<int64_t>> devices;  // per shard, receiving device ids
  int64_t max_device = -1;           // largest device id named
  int64_t nshards() const { return static_cast<int64_t>(devices.size()); }
};

// Returns TP_OK or a negative status (message recorded via fail()).
int build_plan(const int64_t *shape, int64_t ndim, const tp_layout *layout, ShardPlan *plan);

}  // namespace tpshard
