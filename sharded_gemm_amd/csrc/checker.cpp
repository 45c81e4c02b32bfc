// Host sharding checker (no GPU work).
//
// Broadcasting binary elementwise operators ([ONNX] sharding formalism,
// "validity check" and the broadcasting n-ary group): inputs align on their
// trailing axes; an axis on which both inputs have the full size must be cut
// into the same number of pieces by both; an axis of size 1 in one input is
// broadcast.  The output is cut like the input(s) that carry each axis, and
// an output shard lives on the devices that hold both input shards it is
// computed from (the intersection of their groups); an empty intersection
// makes the specs incompatible.
//
// Matmul dims_mapping ([SPMD] rules for computing operators): the einsum
// notation of matmul(X[..., M, K], Y[..., K, N]) is ...mk,...kn->...mn; the
// inputs' mappings merge axis by axis (equal, or -1 against a value; two
// different mesh dims need a reshard); the output takes the merged mapping of
// its axes, and a cut contracted axis k leaves the output partial over that
// mesh dim ([ONNX] reduction group: local reduction, then a collective one).
#include <algorithm>
#include <iterator>
#include <map>
#include <vector>

#include "common.h"
#include "plan.h"

namespace tpshard {
namespace {

// A shard's box origin, padded with leading zeros to rank r.
std::vector<int64_t> padded_origin(const ShardPlan& p, int64_t k, int r) {
  std::vector<int64_t> o(static_cast<size_t>(r), 0);
  const int pad = r - p.ndim;
  for (int i = 0; i < p.ndim; ++i) o[pad + i] = p.offset[k * p.ndim + i];
  return o;
}

}  // namespace
}  // namespace tpshard

using namespace tpshard;

extern "C" {

int tp_check_broadcast_binary(const int64_t *shape1, int64_t ndim1, const tp_layout *layout1,
                              const int64_t *shape2, int64_t ndim2, const tp_layout *layout2,
                              int64_t *out_shape, int64_t *num_shards_out, int64_t *boxes, int64_t max_shards,
                              int64_t *dev_offsets, int64_t *devices, int64_t max_devices) {
  clear_error();
  if (!out_shape || !num_shards_out) return fail(TP_ERR_ARG, "out_shape and num_shards_out must be non-NULL");
  if (max_shards < 0 || max_devices < 0) return fail(TP_ERR_ARG, "negative output capacity");
  ShardPlan p1, p2;
  int rc = build_plan(shape1, ndim1, layout1, &p1);
  if (rc != TP_OK) return rc;
  rc = build_plan(shape2, ndim2, layout2, &p2);
  if (rc != TP_OK) return rc;
  const int r = std::max(p1.ndim, p2.ndim);
  int64_t s1[kMaxRank], s2[kMaxRank], n1[kMaxRank], n2[kMaxRank], nout[kMaxRank], oshape[kMaxRank];
  for (int a = 0; a < r; ++a) {
    const int i1 = a - (r - p1.ndim), i2 = a - (r - p2.ndim);
    s1[a] = i1 >= 0 ? p1.shape[i1] : 1;
    s2[a] = i2 >= 0 ? p2.shape[i2] : 1;
    n1[a] = (i1 >= 0 && p1.extent[i1] > 0) ? p1.shape[i1] / p1.extent[i1] : 1;
    n2[a] = (i2 >= 0 && p2.extent[i2] > 0) ? p2.shape[i2] / p2.extent[i2] : 1;
    if (s1[a] != s2[a] && s1[a] != 1 && s2[a] != 1)
      return fail(TP_ERR_ARG, "axis %d: dims %lld and %lld do not broadcast", a, (long long)s1[a], (long long)s2[a]);
    oshape[a] = std::max(s1[a], s2[a]);
    if (s1[a] != 1 && s2[a] != 1 && n1[a] != n2[a])
      return fail(TP_ERR_SPEC, "axis %d is not broadcast, yet the inputs cut it into %lld and %lld pieces", a,
                  (long long)n1[a], (long long)n2[a]);
    nout[a] = s1[a] != 1 ? n1[a] : (s2[a] != 1 ? n2[a] : 1);
  }
  // Device groups of each input's shards, keyed by padded box origin.
  std::map<std::vector<int64_t>, std::vector<int64_t>> g1, g2;
  for (int64_t k = 0; k < p1.nshards(); ++k) {
    auto d = p1.devices[k];
    std::sort(d.begin(), d.end());
    g1[padded_origin(p1, k, r)] = d;
  }
  for (int64_t k = 0; k < p2.nshards(); ++k) {
    auto d = p2.devices[k];
    std::sort(d.begin(), d.end());
    g2[padded_origin(p2, k, r)] = d;
  }
  int64_t total = 1;
  for (int a = 0; a < r; ++a) total *= nout[a];
  // Output shards row-major over the output axes (axis 0 outermost).
  std::vector<std::vector<int64_t>> devs(static_cast<size_t>(total));
  std::vector<int64_t> origin(static_cast<size_t>(r)), need1(static_cast<size_t>(r)), need2(static_cast<size_t>(r));
  for (int64_t k = 0; k < total; ++k) {
    int64_t rest = k;
    for (int a = r - 1; a >= 0; --a) {
      const int64_t idx = rest % nout[a];
      rest /= nout[a];
      origin[a] = idx * (oshape[a] / nout[a]);
      need1[a] = s1[a] != 1 ? origin[a] : 0;
      need2[a] = s2[a] != 1 ? origin[a] : 0;
    }
    auto h1 = g1.find(need1), h2 = g2.find(need2);
    if (h1 == g1.end() || h2 == g2.end()) return fail(TP_ERR_SPEC, "output shard %lld reads no single input shard", (long long)k);
    std::set_intersection(h1->second.begin(), h1->second.end(), h2->second.begin(), h2->second.end(),
                          std::back_inserter(devs[k]));
    if (devs[k].empty())
      return fail(TP_ERR_SPEC, "output shard %lld: no device holds both input shards it is computed from", (long long)k);
    if (k < max_shards && boxes)
      for (int a = 0; a < r; ++a) {
        boxes[(k * r + a) * 2] = origin[a];
        boxes[(k * r + a) * 2 + 1] = origin[a] + oshape[a] / nout[a];
      }
  }
  for (int a = 0; a < r; ++a) out_shape[a] = oshape[a];
  *num_shards_out = total;
  if (dev_offsets) {
    int64_t off = 0;
    for (int64_t k = 0; k <= std::min(total, max_shards); ++k) {
      dev_offsets[k] = off;
      if (k == total) break;
      for (int64_t d : devs[k]) {
        if (devices && off < max_devices) devices[off] = d;
        ++off;
      }
    }
  }
  return TP_OK;
}

int tp_infer_matmul_dims_mapping(const int64_t *x_map, const int64_t *y_map, int64_t ndim, int64_t mesh_ndim,
                                 int64_t *z_map, int64_t *partial_mesh_dim) {
  clear_error();
  if (!x_map || !y_map || !z_map || !partial_mesh_dim) return fail(TP_ERR_ARG, "NULL argument");
  if (ndim < 2 || ndim > kMaxRank) return fail(TP_ERR_ARG, "ndim %lld outside [2, %d]", (long long)ndim, kMaxRank);
  if (mesh_ndim < 1 || mesh_ndim > kMaxRank) return fail(TP_ERR_ARG, "mesh_ndim %lld outside [1, %d]", (long long)mesh_ndim, kMaxRank);
  for (const int64_t *m : {x_map, y_map}) {
    bool used[kMaxRank] = {};
    for (int64_t i = 0; i < ndim; ++i) {
      if (m[i] < -1 || m[i] >= mesh_ndim) return fail(TP_ERR_SPEC, "dims_mapping value %lld outside [-1, %lld]", (long long)m[i], (long long)(mesh_ndim - 1));
      if (m[i] >= 0) {
        if (used[m[i]]) return fail(TP_ERR_SPEC, "mesh dim %lld used twice in one dims_mapping", (long long)m[i]);
        used[m[i]] = true;
      }
    }
  }
  auto merge = [](int64_t a, int64_t b, int64_t *out) {
    if (a >= 0 && b >= 0 && a != b) return false;
    *out = a >= 0 ? a : b;
    return true;
  };
  // einsum axes: batch..., m, k, n
  std::vector<int64_t> axis_map;
  for (int64_t i = 0; i + 2 < ndim; ++i) {
    int64_t v;
    if (!merge(x_map[i], y_map[i], &v))
      return fail(TP_ERR_SPEC, "batch axis %lld is cut by mesh dims %lld and %lld: needs a reshard", (long long)i,
                  (long long)x_map[i], (long long)y_map[i]);
    axis_map.push_back(v);
  }
  const int64_t m = x_map[ndim - 2], n = y_map[ndim - 1];
  int64_t k;
  if (!merge(x_map[ndim - 1], y_map[ndim - 2], &k))
    return fail(TP_ERR_SPEC, "contracted axis k is cut by mesh dims %lld and %lld: needs a reshard",
                (long long)x_map[ndim - 1], (long long)y_map[ndim - 2]);
  bool used[kMaxRank] = {};
  std::vector<int64_t> all = axis_map;
  all.push_back(m);
  all.push_back(k);
  all.push_back(n);
  for (int64_t v : all)
    if (v >= 0) {
      if (used[v]) return fail(TP_ERR_SPEC, "mesh dim %lld cuts two einsum axes", (long long)v);
      used[v] = true;
    }
  for (size_t i = 0; i < axis_map.size(); ++i) z_map[i] = axis_map[i];
  z_map[ndim - 2] = m;
  z_map[ndim - 1] = n;
  *partial_mesh_dim = k;
  return TP_OK;
}

}  // extern "C"
