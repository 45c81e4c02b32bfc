// Layout planning (host only).
//
// ShardingSpec form ([ONNX] "Proto definitions", "Sharding as a Split",
// "index rule for multi-axis sharding", "Sharding as a Broadcast", "mixing
// split and broadcast"): every listed axis is cut into num_shards equal
// pieces; shard k is the box whose per-axis piece indices are the mixed-radix
// digits of k, the first listed axis being the most significant digit; the
// k-th `device` entry (a device, or a negative key naming a device group)
// receives it.
//
// ProcessMesh form ([SPMD] "ProcessMesh", "dims_mapping"; [SBP] "2D SBP"):
// axis i with dims_mapping[i] = j is cut into mesh.shape[j] pieces and the
// process at mesh coordinate c holds piece c[j]; processes that agree on every
// used mesh coordinate hold the same box and form one shard's device group.
#include "plan.h"

#include <algorithm>
#include <set>

namespace tpshard {

namespace {

int check_shape(const int64_t *shape, int64_t ndim) {
  if (ndim < 0 || ndim > kMaxRank) return fail(TP_ERR_ARG, "ndim %lld outside [0, %d]", (long long)ndim, kMaxRank);
  if (ndim > 0 && !shape) return fail(TP_ERR_ARG, "shape is NULL");
  for (int64_t i = 0; i < ndim; ++i)
    if (shape[i] < 0) return fail(TP_ERR_ARG, "shape[%lld] = %lld is negative", (long long)i, (long long)shape[i]);
  return TP_OK;
}

// Fills plan->offset for shards enumerated in mixed radix over (axes, counts),
// the first entry being the most significant digit.
void enumerate_boxes(const std::vector<int>& axes, const std::vector<int64_t>& counts, ShardPlan *plan) {
  int64_t total = 1;
  for (int64_t n : counts) total *= n;
  plan->offset.assign(static_cast<size_t>(total * plan->ndim), 0);
  for (int64_t k = 0; k < total; ++k) {
    int64_t rest = k;
    for (int m = static_cast<int>(axes.size()) - 1; m >= 0; --m) {
      const int64_t digit = rest % counts[m];
      rest /= counts[m];
      plan->offset[k * plan->ndim + axes[m]] = digit * plan->extent[axes[m]];
    }
  }
}

int plan_spec(const tp_sharding_spec& spec, ShardPlan *plan) {
  const int r = plan->ndim;
  if (spec.num_sharded_dim < 0) return fail(TP_ERR_ARG, "num_sharded_dim < 0");
  if (spec.num_sharded_dim > 0 && !spec.sharded_dim) return fail(TP_ERR_ARG, "sharded_dim is NULL");
  for (int64_t m = 0; m < spec.num_sharded_dim; ++m) {
    const tp_sharded_dim& sd = spec.sharded_dim[m];
    if (sd.num_simple_sharding != 1)
      return fail(TP_ERR_UNSUPPORTED, "sharded_dim[%lld] has %lld simple_sharding entries (exactly 1 supported)",
                  (long long)m, (long long)sd.num_simple_sharding);
    if (!sd.simple_sharding) return fail(TP_ERR_ARG, "sharded_dim[%lld].simple_sharding is NULL", (long long)m);
  }
  std::vector<int> axes;
  std::vector<int64_t> counts;
  for (int64_t m = 0; m < spec.num_sharded_dim; ++m) {
    const tp_sharded_dim& sd = spec.sharded_dim[m];
    if (sd.axis < -r || sd.axis > r - 1)
      return fail(TP_ERR_SPEC, "axis %lld outside [-%d, %d]", (long long)sd.axis, r, r - 1);
    const int a = static_cast<int>(sd.axis < 0 ? sd.axis + r : sd.axis);
    if (std::find(axes.begin(), axes.end(), a) != axes.end())
      return fail(TP_ERR_SPEC, "axis %d is sharded twice", a);
    const int64_t n = sd.simple_sharding[0].num_shards;
    const int64_t dv = sd.simple_sharding[0].dim_value;
    if (n < 1) return fail(TP_ERR_SPEC, "num_shards %lld < 1", (long long)n);
    if (dv != 0 && dv != plan->shape[a])
      return fail(TP_ERR_SPEC, "dim_value %lld != dim %lld of axis %d", (long long)dv, (long long)plan->shape[a], a);
    if (plan->shape[a] % n != 0)
      return fail(TP_ERR_INDIVISIBLE, "dim %lld of axis %d is not divisible by num_shards %lld",
                  (long long)plan->shape[a], a, (long long)n);
    axes.push_back(a);
    counts.push_back(n);
  }
  int64_t total = 1;
  for (int64_t n : counts) total *= n;
  if (spec.num_device != total)
    return fail(TP_ERR_SPEC, "%lld device entries for %lld shards", (long long)spec.num_device, (long long)total);
  if (total > 0 && !spec.device) return fail(TP_ERR_ARG, "device is NULL");
  if (spec.num_groups < 0) return fail(TP_ERR_ARG, "num_groups < 0");
  if (spec.num_groups > 0 && !spec.device_map) return fail(TP_ERR_ARG, "device_map is NULL");
  for (int64_t g = 0; g < spec.num_groups; ++g) {
    const tp_device_group& grp = spec.device_map[g];
    if (grp.key >= 0) return fail(TP_ERR_SPEC, "device_map key %lld must be negative", (long long)grp.key);
    for (int64_t h = 0; h < g; ++h)
      if (spec.device_map[h].key == grp.key) return fail(TP_ERR_SPEC, "device_map key %lld repeated", (long long)grp.key);
    if (grp.num_devices < 1) return fail(TP_ERR_SPEC, "device group %lld is empty", (long long)grp.key);
    if (!grp.devices) return fail(TP_ERR_ARG, "device group %lld has NULL devices", (long long)grp.key);
    for (int64_t i = 0; i < grp.num_devices; ++i)
      if (grp.devices[i] < 0) return fail(TP_ERR_SPEC, "device group %lld lists id %lld", (long long)grp.key, (long long)grp.devices[i]);
  }
  plan->devices.assign(static_cast<size_t>(total), {});
  for (int64_t k = 0; k < total; ++k) {
    const int64_t e = spec.device[k];
    if (e >= 0) {
      plan->devices[k].push_back(e);
      continue;
    }
    const tp_device_group *hit = nullptr;
    for (int64_t g = 0; g < spec.num_groups; ++g)
      if (spec.device_map[g].key == e) hit = &spec.device_map[g];
    if (!hit) return fail(TP_ERR_SPEC, "device key %lld is not in device_map", (long long)e);
    plan->devices[k].assign(hit->devices, hit->devices + hit->num_devices);
  }
  std::set<int64_t> seen;
  for (const auto& grp : plan->devices)
    for (int64_t d : grp) {
      if (!seen.insert(d).second) return fail(TP_ERR_SPEC, "device %lld receives more than one shard", (long long)d);
      plan->max_device = std::max(plan->max_device, d);
    }
  for (int i = 0; i < r; ++i) plan->extent[i] = plan->shape[i];
  for (size_t m = 0; m < axes.size(); ++m) plan->extent[axes[m]] = plan->shape[axes[m]] / counts[m];
  enumerate_boxes(axes, counts, plan);
  return TP_OK;
}

int plan_mesh(const tp_process_mesh& mesh, const int64_t *dims_mapping, ShardPlan *plan) {
  const int r = plan->ndim;
  if (mesh.ndim < 1 || mesh.ndim > kMaxRank) return fail(TP_ERR_SPEC, "mesh rank %lld outside [1, %d]", (long long)mesh.ndim, kMaxRank);
  if (!mesh.shape) return fail(TP_ERR_ARG, "mesh.shape is NULL");
  const int q = static_cast<int>(mesh.ndim);
  int64_t count = 1;
  for (int j = 0; j < q; ++j) {
    if (mesh.shape[j] < 1) return fail(TP_ERR_SPEC, "mesh dim %d is %lld", j, (long long)mesh.shape[j]);
    count *= mesh.shape[j];
  }
  if (!mesh.process_ids) return fail(TP_ERR_ARG, "mesh.process_ids is NULL");
  std::set<int64_t> ids;
  for (int64_t p = 0; p < count; ++p) {
    if (mesh.process_ids[p] < 0 || !ids.insert(mesh.process_ids[p]).second)
      return fail(TP_ERR_SPEC, "process ids must be distinct and >= 0 (id %lld)", (long long)mesh.process_ids[p]);
    plan->max_device = std::max(plan->max_device, mesh.process_ids[p]);
  }
  if (r > 0 && !dims_mapping) return fail(TP_ERR_ARG, "dims_mapping is NULL");
  std::vector<int> used(q, 0);
  std::vector<int> axes;
  std::vector<int64_t> counts;
  for (int i = 0; i < r; ++i) {
    const int64_t j = dims_mapping[i];
    if (j < -1 || j > q - 1) return fail(TP_ERR_SPEC, "dims_mapping[%d] = %lld outside [-1, %d]", i, (long long)j, q - 1);
    if (j < 0) continue;
    if (used[j]) return fail(TP_ERR_SPEC, "mesh dim %lld is used by two tensor axes", (long long)j);
    used[j] = 1;
    if (plan->shape[i] % mesh.shape[j] != 0)
      return fail(TP_ERR_INDIVISIBLE, "dim %lld of axis %d is not divisible by mesh dim %lld",
                  (long long)plan->shape[i], i, (long long)mesh.shape[j]);
    axes.push_back(i);
    counts.push_back(mesh.shape[j]);
  }
  for (int i = 0; i < r; ++i) plan->extent[i] = plan->shape[i];
  for (size_t m = 0; m < axes.size(); ++m) plan->extent[axes[m]] = plan->shape[axes[m]] / counts[m];
  enumerate_boxes(axes, counts, plan);
  int64_t total = 1;
  for (int64_t n : counts) total *= n;
  plan->devices.assign(static_cast<size_t>(total), {});
  // Walk the mesh row-major; a process's shard index is the mixed-radix
  // number formed by its coordinates on the used mesh dims, in tensor-axis order.
  std::vector<int64_t> coord(q, 0);
  for (int64_t p = 0; p < count; ++p) {
    int64_t rest = p;
    for (int j = q - 1; j >= 0; --j) {
      coord[j] = rest % mesh.shape[j];
      rest /= mesh.shape[j];
    }
    int64_t k = 0;
    for (size_t m = 0; m < axes.size(); ++m) k = k * counts[m] + coord[dims_mapping[axes[m]]];
    plan->devices[k].push_back(mesh.process_ids[p]);
  }
  return TP_OK;
}

}  // namespace

int build_plan(const int64_t *shape, int64_t ndim, const tp_layout *layout, ShardPlan *plan) {
  int rc = check_shape(shape, ndim);
  if (rc != TP_OK) return rc;
  if (!layout) return fail(TP_ERR_ARG, "layout is NULL");
  *plan = ShardPlan{};
  plan->ndim = static_cast<int>(ndim);
  for (int64_t i = 0; i < ndim; ++i) plan->shape[i] = shape[i];
  if (layout->kind == TP_LAYOUT_SPEC) return plan_spec(layout->spec, plan);
  if (layout->kind == TP_LAYOUT_DIMS_MAPPING) return plan_mesh(layout->mesh, layout->dims_mapping, plan);
  return fail(TP_ERR_ARG, "unknown layout kind %d", layout->kind);
}

}  // namespace tpshard
