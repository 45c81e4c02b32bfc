// Drives the host code of the library (layout planning, the sharding
// checker, argument validation and the stream scheduler) through brute-force
// layouts, every error path and many valid MLP configurations, built with
// AddressSanitizer and UndefinedBehaviorSanitizer and linked against the
// stand-in launchers of stub_kernels.cpp.  Device buffers are fake addresses
// the host code only computes with; the stand-ins check every range a kernel
// would touch against them.  Prints one summary line; any sanitizer report or
// failed check aborts with a non-zero status.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <vector>

#include "../../include/tpshard.h"
#include "stub_registry.h"

namespace {

std::map<int, long> g_codes;
long g_calls = 0;

int note(int rc) {
  ++g_calls;
  ++g_codes[rc];
  if (rc != TP_OK && tp_last_error()[0] == '\0') {
    std::fprintf(stderr, "status %d without a message\n", rc);
    std::abort();
  }
  return rc;
}

void expect(bool ok, const char *what) {
  if (!ok) {
    std::fprintf(stderr, "check failed: %s (last error: %s)\n", what, tp_last_error());
    std::abort();
  }
}

// Fake device allocations: disjoint, 4 KiB aligned, 1 MiB apart.
uintptr_t g_next = uintptr_t{1} << 44;
void *dev(int64_t bytes) {
  void *p = reinterpret_cast<void *>(g_next);
  stub_register(p, bytes);
  g_next += ((static_cast<uintptr_t>(bytes) + 4095) & ~uintptr_t{4095}) + (uintptr_t{1} << 20);
  return p;
}

// ---- layouts ----------------------------------------------------------------

struct SpecBuf {
  std::vector<tp_simple_sharding> ss;
  std::vector<tp_sharded_dim> sd;
  std::vector<int64_t> device;
  std::vector<std::vector<int64_t>> groups;
  std::vector<tp_device_group> map;
  tp_layout lay{};

  void finish() {
    sd.clear();
    for (size_t i = 0; i < ss.size(); ++i) sd.push_back({axes[i], &ss[i], 1});
    map.clear();
    for (size_t g = 0; g < groups.size(); ++g)
      map.push_back({-static_cast<int64_t>(g) - 1, groups[g].data(), static_cast<int64_t>(groups[g].size())});
    lay.kind = TP_LAYOUT_SPEC;
    lay.spec.device = device.data();
    lay.spec.num_device = static_cast<int64_t>(device.size());
    lay.spec.device_map = map.empty() ? nullptr : map.data();
    lay.spec.num_groups = static_cast<int64_t>(map.size());
    lay.spec.sharded_dim = sd.data();
    lay.spec.num_sharded_dim = static_cast<int64_t>(sd.size());
  }
  std::vector<int64_t> axes;
};

// Plan twice (count, then exact-size outputs) and check the boxes tile the
// tensor: every shard has the same extent and the shard count times the
// shard volume is the tensor's volume.
void plan_exact(const std::vector<int64_t>& shape, const tp_layout& lay) {
  int64_t n = -1;
  const int rc = note(tp_layout_plan(shape.data(), static_cast<int64_t>(shape.size()), &lay, &n, nullptr, 0, nullptr, 0));
  if (rc != TP_OK) return;
  const int64_t r = static_cast<int64_t>(shape.size());
  std::vector<int64_t> boxes(static_cast<size_t>(2 * r * n + (n == 0)));
  const int64_t num_dst = 64;
  std::vector<int64_t> sod(num_dst);
  expect(tp_layout_plan(shape.data(), r, &lay, &n, boxes.data(), n, sod.data(), num_dst) == TP_OK, "second plan");
  int64_t vol = 1, svol = 1;
  for (int64_t a = 0; a < r; ++a) {
    vol *= shape[a];
    svol *= boxes[2 * a + 1] - boxes[2 * a];
  }
  expect(n * svol == vol || vol == 0, "shards tile the tensor");
  for (int64_t k = 0; k < n; ++k)
    for (int64_t a = 0; a < r; ++a) {
      expect(boxes[(k * r + a) * 2] >= 0 && boxes[(k * r + a) * 2 + 1] <= shape[a], "box inside the tensor");
      expect(boxes[(k * r + a) * 2 + 1] - boxes[(k * r + a) * 2] == boxes[2 * a + 1] - boxes[2 * a], "equal extents");
    }
}

void brute_force_specs() {
  const int64_t dims[] = {1, 2, 3, 4, 6};
  std::vector<std::vector<int64_t>> shapes;
  for (int64_t a : dims) {
    shapes.push_back({a});
    for (int64_t b : dims) {
      shapes.push_back({a, b});
      for (int64_t c : dims) shapes.push_back({a, b, c});
    }
  }
  for (const auto& shape : shapes) {
    const int r = static_cast<int>(shape.size());
    // ordered subsets of the axes, as given and counted from the back
    std::vector<std::vector<int64_t>> orders = {{}};
    for (int a = 0; a < r; ++a) orders.push_back({a});
    for (int a = 0; a < r; ++a)
      for (int b = 0; b < r; ++b)
        if (a != b) orders.push_back({a, b});
    if (r == 3)
      for (int a = 0; a < 3; ++a)
        for (int b = 0; b < 3; ++b)
          for (int c = 0; c < 3; ++c)
            if (a != b && b != c && a != c) orders.push_back({a, b, c});
    orders.push_back({0, 0});           // duplicate axis
    orders.push_back({r});              // out of range
    orders.push_back({-r - 1});
    for (const auto& ord : orders) {
      const size_t m = ord.size();
      size_t combos = 1;
      for (size_t i = 0; i < m; ++i) combos *= 4;
      for (size_t code = 0; code < combos; ++code) {
        std::vector<int64_t> ns(m);
        size_t c = code;
        int64_t total = 1;
        for (size_t i = 0; i < m; ++i) {
          ns[i] = 1 + static_cast<int64_t>(c % 4);
          c /= 4;
          total *= ns[i];
        }
        for (int form = 0; form < 7; ++form) {
          SpecBuf sb;
          for (size_t i = 0; i < m; ++i) {
            sb.axes.push_back(form == 1 && ord[i] >= 0 ? ord[i] - r : ord[i]);   // negative form
            sb.ss.push_back({form == 2 ? 5 : 0, ns[i]});                          // wrong dim_value
          }
          if (form == 3) {                                                         // groups of two
            for (int64_t k = 0; k < total; ++k) {
              sb.device.push_back(-k - 1);
              sb.groups.push_back({2 * k, 2 * k + 1});
            }
          } else {
            for (int64_t k = 0; k < total; ++k) sb.device.push_back(k);
          }
          if (form == 4 && !sb.device.empty()) sb.device.pop_back();               // too few devices
          if (form == 5 && total > 1) sb.device[1] = sb.device[0];                 // a device twice
          if (form == 6) sb.device[0] = -7;                                        // key without a group
          sb.finish();
          plan_exact(shape, sb.lay);
        }
      }
    }
  }
}

void brute_force_meshes() {
  const std::vector<std::vector<int64_t>> meshes = {{2}, {4}, {2, 2}, {2, 3}, {3, 2, 2}};
  const std::vector<std::vector<int64_t>> shapes = {{4}, {6, 4}, {4, 6}, {12, 2, 6}, {2, 2, 2}};
  for (const auto& mesh : meshes) {
    const int64_t q = static_cast<int64_t>(mesh.size());
    int64_t np = 1;
    for (int64_t d : mesh) np *= d;
    std::vector<int64_t> ids(np);
    for (int64_t i = 0; i < np; ++i) ids[i] = np - 1 - i;
    for (const auto& shape : shapes) {
      const size_t r = shape.size();
      size_t combos = 1;
      for (size_t i = 0; i < r; ++i) combos *= static_cast<size_t>(q + 3);
      for (size_t code = 0; code < combos; ++code) {
        std::vector<int64_t> dm(r);
        size_t c = code;
        for (size_t i = 0; i < r; ++i) {
          dm[i] = static_cast<int64_t>(c % (q + 3)) - 2;   // -2 .. q
          c /= (q + 3);
        }
        tp_layout lay{};
        lay.kind = TP_LAYOUT_DIMS_MAPPING;
        lay.mesh = {mesh.data(), q, ids.data()};
        lay.dims_mapping = dm.data();
        plan_exact(shape, lay);
      }
    }
  }
}

void checker() {
  // broadcasting binary ops: layouts of [4,1] / [1,4] / [4,4] / [4] pairs
  const std::vector<std::vector<int64_t>> shapes = {{4, 1}, {1, 4}, {4, 4}, {4}, {2, 4, 4}};
  const int64_t mesh[] = {2, 2}, ids[] = {0, 1, 2, 3};
  for (const auto& s1 : shapes)
    for (const auto& s2 : shapes)
      for (int d1 = -2; d1 < 9; ++d1)
        for (int d2 = -2; d2 < 9; ++d2) {
          std::vector<int64_t> m1(s1.size(), -1), m2(s2.size(), -1);
          if (d1 >= 0) m1[static_cast<size_t>(d1) % m1.size()] = d1 % 3 - 1;
          if (d2 >= 0) m2[static_cast<size_t>(d2) % m2.size()] = d2 % 3 - 1;
          tp_layout l1{}, l2{};
          l1.kind = l2.kind = TP_LAYOUT_DIMS_MAPPING;
          l1.mesh = l2.mesh = {mesh, 2, ids};
          l1.dims_mapping = m1.data();
          l2.dims_mapping = m2.data();
          int64_t out_shape[3], n = 0;
          const int rc = note(tp_check_broadcast_binary(s1.data(), (int64_t)s1.size(), &l1, s2.data(), (int64_t)s2.size(),
                                                        &l2, out_shape, &n, nullptr, 0, nullptr, nullptr, 0));
          if (rc != TP_OK) continue;
          const int64_t r = static_cast<int64_t>(std::max(s1.size(), s2.size()));
          std::vector<int64_t> boxes(static_cast<size_t>(2 * r * n + 1)), offs(static_cast<size_t>(n + 1));
          expect(tp_check_broadcast_binary(s1.data(), (int64_t)s1.size(), &l1, s2.data(), (int64_t)s2.size(), &l2,
                                           out_shape, &n, boxes.data(), n, offs.data(), nullptr, 0) == TP_OK,
                 "checker boxes");
          std::vector<int64_t> devs(static_cast<size_t>(offs[n] + 1));
          expect(tp_check_broadcast_binary(s1.data(), (int64_t)s1.size(), &l1, s2.data(), (int64_t)s2.size(), &l2,
                                           out_shape, &n, boxes.data(), n, offs.data(), devs.data(), offs[n]) == TP_OK,
                 "checker devices");
          // smaller capacities truncate (documented): exact-size buffers, so a
          // write past the capacity is a sanitizer report
          if (offs[n] > 0) {
            std::vector<int64_t> few(static_cast<size_t>(offs[n] - 1));
            expect(tp_check_broadcast_binary(s1.data(), (int64_t)s1.size(), &l1, s2.data(), (int64_t)s2.size(), &l2,
                                             out_shape, &n, boxes.data(), n, offs.data(), few.data(),
                                             offs[n] - 1) == TP_OK, "checker device capacity");
          }
          if (n > 1) {
            std::vector<int64_t> fewb(static_cast<size_t>(2 * r * (n - 1))), fewo(static_cast<size_t>(n));
            expect(tp_check_broadcast_binary(s1.data(), (int64_t)s1.size(), &l1, s2.data(), (int64_t)s2.size(), &l2,
                                             out_shape, &n, fewb.data(), n - 1, fewo.data(), nullptr, 0) == TP_OK,
                   "checker shard capacity");
          }
        }
  // matmul dims_mapping merge
  for (int64_t nd = 2; nd <= 3; ++nd)
    for (int64_t q = 1; q <= 3; ++q) {
      size_t combos = 1;
      for (int64_t i = 0; i < 2 * nd; ++i) combos *= static_cast<size_t>(q + 2);
      for (size_t code = 0; code < combos; ++code) {
        std::vector<int64_t> x(nd), y(nd), z(nd);
        size_t c = code;
        for (int64_t i = 0; i < nd; ++i, c /= (q + 2)) x[i] = static_cast<int64_t>(c % (q + 2)) - 1;
        for (int64_t i = 0; i < nd; ++i, c /= (q + 2)) y[i] = static_cast<int64_t>(c % (q + 2)) - 1;
        int64_t part = 0;
        note(tp_infer_matmul_dims_mapping(x.data(), y.data(), nd, q, z.data(), &part));
      }
    }
  int64_t z[2], part;
  const int64_t x[2] = {0, -1};
  note(tp_infer_matmul_dims_mapping(nullptr, x, 2, 2, z, &part));
  note(tp_infer_matmul_dims_mapping(x, x, 9, 2, z, &part));
}

// ---- entry points with fake device buffers -----------------------------------

void layout_calls() {
  const int64_t shape[3] = {8, 6, 4};
  SpecBuf sb;
  sb.axes = {0, 2};
  sb.ss = {{0, 2}, {0, 2}};
  for (int64_t k = 0; k < 4; ++k) {
    sb.device.push_back(-k - 1);
    sb.groups.push_back({2 * k, 2 * k + 1});
  }
  sb.finish();
  void *src = dev(8 * 6 * 4 * 4);
  std::vector<void *> dst(8);
  for (auto& p : dst) p = dev(4 * 6 * 2 * 4);
  expect(note(tp_shard_materialize(src, TP_F32, shape, 3, &sb.lay, dst.data(), 8, nullptr)) == TP_OK, "materialize");
  expect(note(tp_shard_materialize(src, TP_F32, shape, 3, &sb.lay, dst.data(), 7, nullptr)) == TP_ERR_ARG, "num_dst");
  expect(note(tp_shard_materialize(src, 9, shape, 3, &sb.lay, dst.data(), 8, nullptr)) == TP_ERR_ARG, "dtype");
  expect(note(tp_shard_materialize(nullptr, TP_F32, shape, 3, &sb.lay, dst.data(), 8, nullptr)) == TP_ERR_ARG, "src");
  std::vector<void *> bad = dst;
  bad[3] = static_cast<char *>(src) + 16;
  expect(note(tp_shard_materialize(src, TP_F32, shape, 3, &sb.lay, bad.data(), 8, nullptr)) == TP_ERR_ARG, "overlap");
  bad = dst;
  bad[5] = nullptr;
  expect(note(tp_shard_materialize(src, TP_F32, shape, 3, &sb.lay, bad.data(), 8, nullptr)) == TP_ERR_ARG, "null dst");
  // one device's share, and a batch of two items
  tp_materialize_item items[2] = {{src, TP_F32, shape, 3, &sb.lay, dst.data(), 8, 1, 5},
                                  {src, TP_F32, shape, 3, &sb.lay, dst.data(), 8, 0, 0}};
  expect(note(tp_shard_materialize_batch(items, 1, nullptr)) == TP_OK, "local share");
  items[0].local_device = 9;
  expect(note(tp_shard_materialize_batch(items, 1, nullptr)) == TP_ERR_ARG, "local device");
  items[0].local_device = 5;
  expect(note(tp_shard_materialize_batch(items, 2, nullptr)) == TP_ERR_ARG, "batch outputs overlap");
  expect(note(tp_shard_materialize_batch(nullptr, 2, nullptr)) == TP_ERR_ARG, "no items");
  // gather back into two outputs
  void *out[2] = {dev(8 * 6 * 4 * 4), dev(8 * 6 * 4 * 4)};
  expect(note(tp_shard_gather(dst.data(), 8, TP_F32, shape, 3, &sb.lay, out, 2, nullptr)) == TP_OK, "gather");
  expect(note(tp_shard_gather(dst.data(), 5, TP_F32, shape, 3, &sb.lay, out, 2, nullptr)) == TP_ERR_ARG, "num_src");
  expect(note(tp_shard_gather(dst.data(), 8, TP_F32, shape, 3, &sb.lay, out, 0, nullptr)) == TP_ERR_ARG, "num_out");
  const int64_t odd[3] = {7, 6, 4};
  expect(note(tp_shard_gather(dst.data(), 8, TP_F32, odd, 3, &sb.lay, out, 2, nullptr)) == TP_ERR_INDIVISIBLE, "odd");
}

void reduce_calls() {
  const int64_t rows = 64, cols = 48, ld = 56;
  std::vector<const float *> parts;
  for (int p = 0; p < 5; ++p) parts.push_back(static_cast<const float *>(dev(rows * ld * 4)));
  std::vector<float *> outs;
  for (int j = 0; j < 8; ++j) outs.push_back(static_cast<float *>(dev(rows / 8 * cols * 4)));
  float *full = static_cast<float *>(dev(rows * cols * 4));
  const float *bias = static_cast<const float *>(dev(cols * 4));
  for (int op = 0; op < 3; ++op) {
    expect(note(tp_partial_reduce_ex(parts.data(), 5, rows, cols, ld, TP_REDUCE_FULL, 1, &full, cols, op, bias, nullptr)) == TP_OK, "full");
    expect(note(tp_partial_reduce_ex(parts.data(), 5, rows, cols, ld, TP_REDUCE_SPLIT, 8, outs.data(), cols, op, nullptr, nullptr)) == TP_OK, "split");
  }
  float *in_place = const_cast<float *>(parts[0]);
  expect(note(tp_partial_reduce(parts.data(), 5, rows, cols, ld, TP_REDUCE_FULL, 1, &in_place, ld, nullptr)) == TP_OK, "in place");
  expect(note(tp_partial_reduce(parts.data(), 5, rows, cols, ld, TP_REDUCE_SPLIT, 6, outs.data(), cols, nullptr)) == TP_ERR_INDIVISIBLE, "S");
  expect(note(tp_partial_reduce(parts.data(), 0, rows, cols, ld, TP_REDUCE_FULL, 1, &full, cols, nullptr)) == TP_ERR_ARG, "P");
  expect(note(tp_partial_reduce(parts.data(), 65, rows, cols, ld, TP_REDUCE_FULL, 1, &full, cols, nullptr)) == TP_ERR_UNSUPPORTED, "P max");
  expect(note(tp_partial_reduce(parts.data(), 5, rows, cols, 8, TP_REDUCE_FULL, 1, &full, cols, nullptr)) == TP_ERR_ARG, "ld");
  expect(note(tp_partial_reduce(parts.data(), 5, rows, cols, ld, 7, 1, &full, cols, nullptr)) == TP_ERR_ARG, "mode");
  expect(note(tp_partial_reduce_ex(parts.data(), 5, rows, cols, ld, TP_REDUCE_FULL, 1, &full, cols, 4, nullptr, nullptr)) == TP_ERR_ARG, "op");
  float *clash = const_cast<float *>(parts[2]) + 8;
  expect(note(tp_partial_reduce(parts.data(), 5, rows, cols, ld, TP_REDUCE_FULL, 1, &clash, cols, nullptr)) == TP_ERR_ARG, "alias");
}

struct MlpBufs {
  int64_t M, H, F, es;
  void *X, *A, *B, *Y, *Hs, *Xn;
  float *Z, *Zo, *bias;
  std::vector<const float *> peers;
  std::vector<const void *> xs;
  std::vector<float *> zs;
};

MlpBufs mlp_bufs(int64_t M, int64_t H, int64_t F, int64_t P, int64_t S, int32_t dtype) {
  MlpBufs b{M, H, F, dtype == TP_BF16 ? 2 : 4};
  b.X = dev(M * H * b.es);
  b.A = dev(H * F * b.es);
  b.B = dev(F * H * b.es);
  b.Y = dev(M * F * b.es);
  b.Hs = dev(M * F * b.es);
  b.Xn = dev(M * H * b.es);
  b.Z = static_cast<float *>(dev(M * H * 4));
  b.Zo = static_cast<float *>(dev(M * H * 4));
  b.bias = static_cast<float *>(dev(H * 4));
  for (int64_t p = 1; p < P; ++p) b.peers.push_back(static_cast<const float *>(dev(M * H * 4)));
  for (int64_t j = 0; j < S; ++j) {
    b.xs.push_back(dev(M / S * H * b.es));
    b.zs.push_back(static_cast<float *>(dev(M / S * H * 4)));
  }
  return b;
}

tp_mlp_args mlp_args(const MlpBufs& b, int32_t dtype, int64_t R, int64_t C, int64_t P) {
  tp_mlp_args a{};
  a.dtype = dtype;
  a.act = TP_ACT_GELU_ERF;
  a.M = b.M;
  a.H = b.H;
  a.F = b.F;
  a.X = b.X;
  a.A_i = b.A;
  a.B_i = b.B;
  a.Y_ws = b.Y;
  a.Z_i = b.Z;
  a.row_chunks = R;
  a.col_chunks = C;
  a.P = P;
  a.peer_partials = P > 1 ? b.peers.data() : nullptr;
  a.Z_out = P > 1 ? b.Zo : nullptr;
  return a;
}

void mlp_calls() {
  long ok = 0;
  for (int32_t dtype : {TP_BF16, TP_F32})
    for (int64_t P : {1, 3, 5, 9})
      for (int64_t S : {0, 2, 4, 8}) {
        stub_reset();
        const int64_t M = 512, H = 256, F = 96;
        MlpBufs b = mlp_bufs(M, H, F, P, S, dtype);
        for (int64_t R : {1, 2, 4})
          for (int64_t C : {1, 2})
            for (int variant = 0; variant < 6; ++variant)
              for (int32_t fusion : {TP_REDUCE_FUSION_AUTO, TP_REDUCE_FUSION_OFF}) {
                tp_mlp_args a = mlp_args(b, dtype, R, C, P);
                a.reduce_fusion = fusion;
                if (variant == 1) a.Z_out = b.Z;                        // in place
                if (variant == 2) a.bias = b.bias, a.Z_out = b.Zo;
                if (variant == 3) a.X_next = b.Xn, a.Z_out = nullptr;
                if (variant == 4) a.H_out = b.Hs;
                if (variant == 5) a.X_next = b.Xn, a.bias = b.bias;
                if (S > 1) {
                  a.seq_splits = S;
                  a.X_shards = b.xs.data();
                  if (variant != 3 && variant != 5) {
                    a.Z_split = b.zs.data();
                    a.Z_out = nullptr;
                  }
                }
                const int rc = note(tp_colrow_mlp(&a, nullptr, nullptr));
                expect(rc == TP_OK || rc == TP_ERR_UNSUPPORTED || (rc == TP_ERR_ARG && P == 1 && variant == 2),
                       "valid forward");
                ok += rc == TP_OK;
              }
        // X read where its sequence blocks lie (X = NULL); with 256-row blocks
        // GEMM1 may cover several, or (one stream, the chunks' sums folded
        // but not the whole layer's) every block in one launch.
        if (S > 1 && dtype == TP_BF16) {
          const int64_t Mb = 256 * S;
          MlpBufs bb = mlp_bufs(Mb, H, F, P, S, dtype);
          for (int64_t R : {1, 2, 4, 8})
            for (int64_t C : {1, 2})
              for (int32_t layout : {TP_WEIGHTS_MATH, TP_WEIGHTS_LINEAR})
                for (int32_t fusion : {TP_REDUCE_FUSION_AUTO, TP_REDUCE_FUSION_OFF}) {
                  if (Mb % R) continue;
                  tp_mlp_args a = mlp_args(bb, dtype, R, C, P);
                  a.X = nullptr;
                  a.seq_splits = S;
                  a.X_shards = bb.xs.data();
                  a.Z_split = bb.zs.data();
                  a.Z_out = nullptr;
                  a.weight_layout = layout;
                  a.reduce_fusion = fusion;
                  const int rc = note(tp_colrow_mlp(&a, nullptr, nullptr));
                  expect(rc == TP_OK || rc == TP_ERR_UNSUPPORTED, "valid forward, X in place");
                  ok += rc == TP_OK;
                }
        }
        // each rejection
        tp_mlp_args a = mlp_args(b, dtype, 1, 1, P);
        a.row_chunks = 3;
        expect(note(tp_colrow_mlp(&a, nullptr, nullptr)) == TP_ERR_INDIVISIBLE, "R");
        a = mlp_args(b, dtype, 1, 1, P);
        a.col_chunks = 5;
        expect(note(tp_colrow_mlp(&a, nullptr, nullptr)) == TP_ERR_INDIVISIBLE, "C");
        a = mlp_args(b, dtype, 1, 1, P);
        a.Y_ws = static_cast<char *>(b.X) + 64;
        expect(note(tp_colrow_mlp(&a, nullptr, nullptr)) == TP_ERR_ARG, "Y overlaps X");
        a = mlp_args(b, dtype, 1, 1, P);
        a.act = 7;
        expect(note(tp_colrow_mlp(&a, nullptr, nullptr)) == TP_ERR_ARG, "act");
        a.act = TP_ACT_NONE;
        a.H_out = b.Hs;
        expect(note(tp_colrow_mlp(&a, nullptr, nullptr)) == TP_ERR_ARG, "H_out without act");
        expect(note(tp_colrow_mlp(nullptr, nullptr, nullptr)) == TP_ERR_ARG, "NULL args");
        // a stack of two layers linked through X_next
        if (S == 0) {
          MlpBufs b2 = mlp_bufs(M, H, F, P, 0, dtype);
          tp_mlp_args l[2] = {mlp_args(b, dtype, 2, 2, P), mlp_args(b2, dtype, 2, 2, P)};
          l[0].X_next = b2.X;
          expect(note(tp_colrow_mlp_stack(l, 2, nullptr, nullptr)) == TP_OK, "stack");
          l[0].X_next = b.Xn;
          expect(note(tp_colrow_mlp_stack(l, 2, nullptr, nullptr)) == TP_ERR_ARG, "broken link");
          expect(note(tp_colrow_mlp_stack(l, 0, nullptr, nullptr)) == TP_ERR_ARG, "no layers");
        }
      }
  expect(ok > 500, "enough valid forward calls");
}

void backward_calls() {
  for (int32_t dtype : {TP_BF16, TP_F32})
    for (int64_t P : {1, 3, 9})
      for (int64_t S : {0, 2, 4}) {
        stub_reset();
        const int64_t M = 384, H = 192, F = 128, es = dtype == TP_BF16 ? 2 : 4;
        void *X = dev(M * H * es), *A = dev(H * F * es), *B = dev(F * H * es), *Hs = dev(M * F * es),
             *Y = dev(M * F * es), *dZ = dev(M * H * es), *dH = dev(M * F * es);
        float *dX = static_cast<float *>(dev(M * H * 4)), *dXo = static_cast<float *>(dev(M * H * 4));
        float *dA = static_cast<float *>(dev(H * F * 4)), *dB = static_cast<float *>(dev(F * H * 4));
        std::vector<const float *> peers;
        for (int64_t p = 1; p < P; ++p) peers.push_back(static_cast<const float *>(dev(M * H * 4)));
        std::vector<const void *> gs;
        std::vector<float *> xs;
        for (int64_t j = 0; j < S; ++j) {
          gs.push_back(dev(M / S * H * es));
          xs.push_back(static_cast<float *>(dev(M / S * H * 4)));
        }
        for (int64_t R : {1, 2, 3, 4})
          for (int variant = 0; variant < 3; ++variant) {
            tp_mlp_bwd_args a{};
            a.dtype = dtype;
            a.act = variant == 2 ? TP_ACT_NONE : TP_ACT_GELU_ERF;
            a.M = M;
            a.H = H;
            a.F = F;
            a.X = X;
            a.A_i = A;
            a.B_i = B;
            a.H_i = Hs;
            a.Y_i = Y;
            a.dZ = dZ;
            a.dH_ws = dH;
            a.dX_i = dX;
            a.dA_i = dA;
            a.dB_i = dB;
            a.accumulate = variant == 1;
            a.row_chunks = R;
            a.P = P;
            a.peer_dX = P > 1 ? peers.data() : nullptr;
            a.dX_out = P > 1 ? (variant == 1 ? dX : dXo) : nullptr;
            if (S > 1) {
              a.seq_splits = S;
              a.dZ_shards = gs.data();
              a.dX_split = xs.data();
              a.dX_out = nullptr;
            }
            const int rc = note(tp_colrow_mlp_backward(&a, nullptr, nullptr));
            expect(rc == TP_OK || rc == TP_ERR_UNSUPPORTED || (rc == TP_ERR_INDIVISIBLE && M % R), "valid backward");
            if (rc != TP_OK) continue;
            a.H_i = nullptr;
            if (a.act == TP_ACT_GELU_ERF) expect(note(tp_colrow_mlp_backward(&a, nullptr, nullptr)) == TP_ERR_ARG, "H_i");
            a.H_i = Hs;
            a.dA_i = reinterpret_cast<float *>(static_cast<char *>(X) + 4);
            expect(note(tp_colrow_mlp_backward(&a, nullptr, nullptr)) == TP_ERR_ARG, "dA overlaps X");
          }
      }
}

}  // namespace

int main() {
  brute_force_specs();
  brute_force_meshes();
  checker();
  layout_calls();
  reduce_calls();
  mlp_calls();
  backward_calls();
  tp_kernel_stat st[16];
  expect(note(tp_timing_read(nullptr)) == TP_ERR_ARG, "timing NULL");
  expect(note(tp_timing_read(st)) == TP_OK, "timing read");
  for (int code : {TP_OK, TP_ERR_ARG, TP_ERR_SPEC, TP_ERR_INDIVISIBLE, TP_ERR_UNSUPPORTED})
    expect(g_codes[code] > 0, "every status but TP_ERR_HIP reached");
  std::printf("calls %ld ok %ld arg %ld spec %ld indivisible %ld unsupported %ld hip %ld launches %ld\n", g_calls,
              g_codes[TP_OK], g_codes[TP_ERR_ARG], g_codes[TP_ERR_SPEC], g_codes[TP_ERR_INDIVISIBLE],
              g_codes[TP_ERR_UNSUPPORTED], g_codes[TP_ERR_HIP], stub_launches());
  return 0;
}
