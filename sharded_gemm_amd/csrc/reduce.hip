// Partial reduction: out = op over p of partial_p (+ bias[col]), fp32,
// ascending p ([SBP] "SBP": partial-sum pieces add up to the tensor, and min
// and max apply to partial tensors the same way; [CAI] section 2.1: one
// all-reduce sums the row-parallel partials; section 5.2: the row-parallel
// layer's bias acts on the full output, so it is added once after the sum;
// sections 3 and 5.3: the reduce-scatter form leaves rank j with row block j).
//
// Pure HBM streaming, inputs read once and outputs written once, both
// bypassing cache retention (non-temporal), in one of two forms:
//  * alone on the chip (a one-shot grid) over whole rows: each lane owns four
//    output vectors, 256 lanes apart, and walks the partials in ascending p
//    one 16-byte load at a time, each waited for before the next is issued,
//    so a wave reads one partial's contiguous kilobyte at a time.  On MI355X,
//    cold, that is 2-12% faster than keeping every partial's load in flight
//    (78% of HBM on an 8-way sum of 67 MB partials, against 70%);
//  * beside a GEMM (a capped grid striding over the rows), or over a column
//    block of wider rows: each lane owns one vector and keeps eight partials'
//    loads in flight before adding; with the few workgroups the GEMM leaves
//    room for, one load at a time per wave would not keep the reduce's share
//    of HBM busy (6.7B step: 553 against 424 us).
// Rows may be strided (ld), which is how a column block of a wider matrix is
// reduced.  Besides (or instead of) the fp32 result the kernel can write a
// copy in the next layer's input precision (bf16, rounded to nearest even, or
// fp32), so a stack of layers needs no separate conversion pass.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <type_traits>

#include "common.h"
#include "shard.h"

namespace tpshard {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxP = 64;
constexpr int kMaxOut = 64;
constexpr int kGroup = 8;   // partials loaded together before adding (capped grids)

struct RedArgs {
  const float *in[kMaxP];
  float *out[kMaxOut];
  const float *bias;        // [cols], or null
  void *lo;                 // second output (bf16 or fp32), FULL mode only, or null
  int64_t ld_lo;            // elements
  int32_t P;
  uint32_t cols_v;          // vectors per row
  uint32_t total_v;         // rows * cols_v
  uint32_t rows_per_out;
  int64_t ld_in, ld_out;    // elements
};

typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int VW> struct FVec;
template <> struct FVec<4> { typedef f32x4_t T; };
template <> struct FVec<1> { typedef float T; };

// OP: 0 sum, 1 max, 2 min (fmaxf / fminf: a NaN partial loses to a number).
template <int OP, class V>
__device__ __forceinline__ V combine(V acc, V v) {
  if constexpr (OP == 0) {
    return acc + v;
  } else if constexpr (sizeof(V) == sizeof(float)) {
    return OP == 1 ? fmaxf(acc, v) : fminf(acc, v);
  } else {
    V r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = OP == 1 ? fmaxf(acc[e], v[e]) : fminf(acc[e], v[e]);
    return r;
  }
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 in one word (lo in the low half), round to nearest,
// ties to even, a NaN kept a NaN with its quiet bit set: gfx950's packed
// conversion (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t bf16_pack2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// LO: 0 no second output, 1 bf16 copy, 2 fp32 copy.  HI: write the fp32 result.
// The second output is the next layer's input, read by its GEMM right after,
// so it is stored through the caches (the fp32 result streams past them).
template <int LO, class V>
__device__ __forceinline__ void store_lo(void *base, int64_t off, V v) {
  if constexpr (LO == 2) {
    *reinterpret_cast<V *>(static_cast<float *>(base) + off) = v;
  } else if constexpr (LO == 1) {
    if constexpr (sizeof(V) == sizeof(float)) {
      static_cast<uint16_t *>(base)[off] = static_cast<uint16_t>(bf16_pack2(v, 0.f) & 0xffffu);
    } else {
      typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
      u32x2_t w;
      w[0] = bf16_pack2(v[0], v[1]);
      w[1] = bf16_pack2(v[2], v[3]);
      *reinterpret_cast<u32x2_t *>(static_cast<uint16_t *>(base) + off) = w;
    }
  }
}

// SER: the serialised form (UNROLL vectors per lane), else the grouped one.
template <int VW, int UNROLL, int OP, bool BIAS, bool HI, int LO, bool NT, bool SER>
__global__ void __launch_bounds__(kThreads) reduce_kernel(RedArgs a) {
  typedef typename FVec<VW>::T V;
  const uint32_t stride = gridDim.x * kThreads * UNROLL;
  for (uint32_t base = blockIdx.x * kThreads * UNROLL + threadIdx.x; base < a.total_v; base += stride) {
    int64_t in_off[UNROLL];
    bool ok[UNROLL];
    uint32_t row[UNROLL], col[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const uint32_t idx = base + u * kThreads;
      ok[u] = idx < a.total_v;
      row[u] = ok[u] ? idx / a.cols_v : 0;
      col[u] = ok[u] ? idx - row[u] * a.cols_v : 0;
      in_off[u] = static_cast<int64_t>(row[u]) * a.ld_in + static_cast<int64_t>(col[u]) * VW;
    }
    V acc[UNROLL];
    if constexpr (SER) {
      for (int p = 0; p < a.P; ++p) {
        const float *src = a.in[p];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          if (!ok[u]) continue;
          const V v = NT ? __builtin_nontemporal_load(reinterpret_cast<const V *>(src + in_off[u]))
                         : *reinterpret_cast<const V *>(src + in_off[u]);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          acc[u] = p == 0 ? v : combine<OP>(acc[u], v);
        }
      }
    } else {
      for (int p0 = 0; p0 < a.P; p0 += kGroup) {
        V v[kGroup][UNROLL];
#pragma unroll
        for (int g = 0; g < kGroup; ++g)
#pragma unroll
          for (int u = 0; u < UNROLL; ++u)
            if (p0 + g < a.P && ok[u])
              v[g][u] = NT ? __builtin_nontemporal_load(reinterpret_cast<const V *>(a.in[p0 + g] + in_off[u]))
                           : *reinterpret_cast<const V *>(a.in[p0 + g] + in_off[u]);
#pragma unroll
        for (int g = 0; g < kGroup; ++g)
#pragma unroll
          for (int u = 0; u < UNROLL; ++u)
            if (p0 + g < a.P) acc[u] = (p0 + g == 0) ? v[g][u] : combine<OP>(acc[u], v[g][u]);
      }
    }
    if constexpr (BIAS) {
#pragma unroll
      for (int u = 0; u < UNROLL; ++u)
        if (ok[u]) acc[u] = acc[u] + *reinterpret_cast<const V *>(a.bias + static_cast<int64_t>(col[u]) * VW);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      if (!ok[u]) continue;
      const uint32_t j = row[u] / a.rows_per_out;
      const int64_t r = row[u] - static_cast<int64_t>(j) * a.rows_per_out;
      if constexpr (HI) {
        float *dst = a.out[j] + r * a.ld_out + static_cast<int64_t>(col[u]) * VW;
        if constexpr (NT) __builtin_nontemporal_store(acc[u], reinterpret_cast<V *>(dst));
        else *reinterpret_cast<V *>(dst) = acc[u];
      }
      if constexpr (LO != 0) store_lo<LO>(a.lo, static_cast<int64_t>(row[u]) * a.ld_lo + static_cast<int64_t>(col[u]) * VW, acc[u]);
    }
  }
}

}  // namespace

int partial_reduce_launch(const float *const *partials, int P, int64_t rows, int64_t cols, int64_t ld_in,
                          float *const *out, int nout, int64_t rows_per_out, int64_t ld_out,
                          hipStream_t stream, int64_t max_wgs, int op, const float *bias, void *lo, int lo_dtype,
                          int64_t ld_lo) {
  if (rows == 0 || cols == 0) return TP_OK;
  RedArgs a{};
  auto al16 = [](const void *q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
  const bool hi = out[0] != nullptr;
  const int lo_kind = lo ? (lo_dtype == TP_BF16 ? 1 : 2) : 0;
  bool vec = (cols % 4 == 0) && (ld_in % 4 == 0) && (ld_out % 4 == 0) && (!bias || al16(bias));
  if (lo_kind) vec = vec && (ld_lo % 4 == 0) && (reinterpret_cast<uintptr_t>(lo) & (lo_kind == 1 ? 7u : 15u)) == 0;
  a.bias = bias;
  a.lo = lo;
  a.ld_lo = ld_lo;
  for (int p = 0; p < P; ++p) {
    a.in[p] = partials[p];
    vec = vec && al16(partials[p]);
  }
  for (int j = 0; j < nout; ++j) {
    a.out[j] = out[j];
    vec = vec && (!hi || al16(out[j]));
  }
  const int vw = vec ? 4 : 1;
  const int64_t cols_v = cols / vw;
  const int64_t total_v = rows * cols_v;
  if (total_v >= (int64_t(1) << 31) || rows_per_out >= (int64_t(1) << 31))
    return fail(TP_ERR_UNSUPPORTED, "reduce of %lld x %lld exceeds the 32-bit index range", (long long)rows, (long long)cols);
  a.P = P;
  a.cols_v = static_cast<uint32_t>(cols_v);
  a.total_v = static_cast<uint32_t>(total_v);
  a.rows_per_out = static_cast<uint32_t>(rows_per_out);
  a.ld_in = ld_in;
  a.ld_out = ld_out;
  // Alone over whole rows: four vectors per lane in a one-shot grid,
  // serialised loads (measured best on MI355X of 1, 2 and 4 vectors and of 1
  // to 8 workgroups per CU).  Capped, or a column block of wider rows: one
  // vector per lane, grouped loads (the GPT-3 175B step's last column-block
  // reduce ran 8% slower serialised, 81 against 75 us).
  const bool ser = max_wgs <= 0 && ld_in == cols;
  const int64_t per_wg = kThreads * (ser ? 4 : 1);
  const int64_t want = (total_v + per_wg - 1) / per_wg;
  const int64_t cap = max_wgs > 0 ? std::min<int64_t>(max_wgs, 1 << 20) : (1 << 20);
  const dim3 grid(static_cast<unsigned>(std::min<int64_t>(want, cap)));
  // Small reduces (inputs and outputs within kCachedBytes) use cached loads and
  // stores: their inputs were just written or are still in the caches.
  constexpr int64_t kCachedBytes = int64_t(128) << 20;
  const bool nt = 4.0 * (P + nout) * static_cast<double>(rows) * cols > static_cast<double>(kCachedBytes);
  auto go = [&](auto vw, auto o, auto b, auto h, auto l) {
    constexpr int VW = decltype(vw)::value, OP = decltype(o)::value, LO = decltype(l)::value;
    constexpr bool BI = decltype(b)::value, HI = decltype(h)::value;
    if (ser) {
      if (nt) hipLaunchKernelGGL((reduce_kernel<VW, 4, OP, BI, HI, LO, true, true>), grid, dim3(kThreads), 0, stream, a);
      else hipLaunchKernelGGL((reduce_kernel<VW, 4, OP, BI, HI, LO, false, true>), grid, dim3(kThreads), 0, stream, a);
    } else {
      if (nt) hipLaunchKernelGGL((reduce_kernel<VW, 1, OP, BI, HI, LO, true, false>), grid, dim3(kThreads), 0, stream, a);
      else hipLaunchKernelGGL((reduce_kernel<VW, 1, OP, BI, HI, LO, false, false>), grid, dim3(kThreads), 0, stream, a);
    }
  };
  using std::integral_constant;
  // The second output exists for sums only (a layer's output feeding the next layer).
  auto by_op = [&](auto vw, auto b) {
    if (op == 1) go(vw, integral_constant<int, 1>{}, b, std::true_type{}, integral_constant<int, 0>{});
    else if (op == 2) go(vw, integral_constant<int, 2>{}, b, std::true_type{}, integral_constant<int, 0>{});
    else if (lo_kind == 0) go(vw, integral_constant<int, 0>{}, b, std::true_type{}, integral_constant<int, 0>{});
    else if (lo_kind == 1 && hi) go(vw, integral_constant<int, 0>{}, b, std::true_type{}, integral_constant<int, 1>{});
    else if (lo_kind == 1) go(vw, integral_constant<int, 0>{}, b, std::false_type{}, integral_constant<int, 1>{});
    else if (hi) go(vw, integral_constant<int, 0>{}, b, std::true_type{}, integral_constant<int, 2>{});
    else go(vw, integral_constant<int, 0>{}, b, std::false_type{}, integral_constant<int, 2>{});
  };
  auto by_bias = [&](auto vw) {
    if (bias) by_op(vw, std::true_type{}); else by_op(vw, std::false_type{});
  };
  if (vec) by_bias(integral_constant<int, 4>{}); else by_bias(integral_constant<int, 1>{});
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TP_ERR_HIP, "reduce launch: %s", hipGetErrorString(e));
  return TP_OK;
}

}  // namespace tpshard
