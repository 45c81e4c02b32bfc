// Dense GEMMs of the column->row MLP on gfx950, forward and backward.
//
//   C[M,N] = epi(A[M,K] * W[K,N])
//
// Each operand is given either k-contiguous (A as [M][lda], or W as W^T
// [N][ldw]) or m/n-contiguous (A as A^T [K][lda], or W as [K][ldw]); the
// layout flags of GemmArgs say which.
//
// Forward: GEMM1 is X * A_i followed by GeLU, stored as bf16 ([CAI] section 2,
// column-parallel linear; [DOM] "GeMM GeLU GeMM"); GEMM2 is Y * B_i stored as
// the fp32 partial ([CAI] section 2.1, row-parallel linear).
// Backward ([CAI] section 2.2, [DOM] backward): dY = dZ * B_i^T with the GeLU
// derivative fused (W given transposed), dX_i = dH * A_i^T (W transposed),
// dA_i = X^T * dH and dB_i = Y^T * dZ (A transposed, accumulating over token
// chunks).
//
// Main path (bf16_gemm_dma): v_mfma_f32_16x16x32_bf16, fp32 accumulation.
//  * 8 waves per workgroup (2 per SIMD) in a 2 x 4 grid over the output tile,
//    so one wave's MFMAs cover the other wave's memory instructions.
//  * Both operand tiles go global -> LDS with the LDS-DMA load
//    (global_load_lds_dwordx4: each lane's 16 bytes land at M0 + 16 * lane),
//    into an S-slot ring; no VGPRs stage the data and nothing waits on a load
//    until its slot is needed.  These loads are issued from inline assembly:
//    the compiler, when it sees the builtin form, waits for every
//    outstanding DMA (vmcnt(0)) before each LDS read, which would empty the
//    ring; here the kernel counts vmcnt itself, per stage.
//  * A k-contiguous operand tile is read with ds_read_b128.  An m/n-contiguous
//    one stays that way in LDS and is read with the gfx950 transposing read
//    ds_read_b64_tr_b16, which hands each lane the 4 consecutive k of one
//    row / column (two reads make the 8 k an MFMA operand needs), so no
//    transpose pass exists anywhere.
//  * XOR swizzles on 16-byte chunks keep the DMA writes and both kinds of LDS
//    read free of bank conflicts.
//  * Fragments are double-buffered in registers across k steps: the LDS reads
//    of step u+1 are in flight while the MFMAs of step u run.
//  * The MFMA gets W as its first operand and A as its second, so each lane
//    owns one output row and four adjacent columns: 16-byte (fp32) or 8-byte
//    (bf16) stores.
// Ping-pong path (bf16_gemm_pps) for the 256-row tiles: the same tile, DMA
// and LDS layout, but the two waves sharing a SIMD run in opposite phases.
// The waves of tile rows 0..127 (group A) and of rows 128..255 (group B) sit
// one barrier apart: between two barriers one group runs its MFMAs while the
// other reads its next stage from LDS, so the MFMA pipe is fed while LDS reads
// and their waits happen; each group issues its operand's DMA between its own
// MFMAs.
// Ragged path (bf16_gemm_ragged): the same MFMA on a 128 x 128 tile with
// register-staged, bounds-checked loads, for shapes the DMA path cannot take
// (K not a multiple of 32, N not a multiple of 8, misaligned pointers).
//
// All paths accumulate every output element over k in the same order (32-wide
// k steps, ascending), so results are bit-identical whichever path or tile
// shape runs, do not depend on how the caller chunks M and N, and continuing
// from C (acc_init) equals one pass over the concatenated k range.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <type_traits>

#include "gemm.h"

namespace tpshard {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

#define TP_LDS __attribute__((address_space(3)))

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;

// fp32 output continuing from C's contents (GemmArgs::acc_init): its own
// instantiation, so the forward's kernels carry no code for it (it costs the
// largest tiles their last free registers).
constexpr int kEpiF32Acc = 100;

// ---- numerics ----------------------------------------------------------

// erf(z) for z >= 0 by Abramowitz & Stegun, Handbook of Mathematical
// Functions, formula 7.1.26: 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) e^{-z^2}
// with t = 1 / (1 + p z); absolute error at most 1.5e-7.  Odd extension for z < 0.
// Evaluated with the hardware reciprocal and exponential, it costs about a dozen
// instructions and few registers, which matters next to 256 live accumulators.
__device__ __forceinline__ float erf_as7126(float z) {
  const float a = fabsf(z);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, a, 1.0f));
  float poly = fmaf(t, 1.061405429f, -1.453152027f);
  poly = fmaf(t, poly, 1.421413741f);
  poly = fmaf(t, poly, -0.284496736f);
  poly = fmaf(t, poly, 0.254829592f);
  const float e = __expf(-a * a);
  const float r = 1.0f - t * poly * e;
  return copysignf(r, z);
}

// GeLU(x) = x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)) in fp32, with the same
// erf approximation folded: q = erfc(|x| / sqrt 2) / 2 = t p(t) e^{-x^2/2} / 2,
// and Phi(x) = 1 - q for x >= 0, q for x < 0.  The 1/sqrt 2 and the 1/2 live
// in the constants, which saves a third of the instructions of the epilogue
// that applies it to every output of GEMM1.
__device__ __forceinline__ float gelu_erf(float x) {
  const float a = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f * 0.70710678118654752440f, a, 1.0f));
  float poly = fmaf(t, 0.5f * 1.061405429f, 0.5f * -1.453152027f);
  poly = fmaf(t, poly, 0.5f * 1.421413741f);
  poly = fmaf(t, poly, 0.5f * -0.284496736f);
  poly = fmaf(t, poly, 0.5f * 0.254829592f);
  // e^{-x^2/2} = 2^{x (x (-log2(e) / 2))}
  const float q = t * poly * __builtin_amdgcn_exp2f(x * (x * -0.72134752044448170368f));
  return x * (x >= 0.0f ? 1.0f - q : q);
}

// GeLU'(x) = Phi(x) + x * phi(x), phi the standard normal density
// exp(-x^2/2) / sqrt(2 pi), in fp32.
__device__ __forceinline__ float gelu_erf_deriv(float x) {
  const float cdf = 0.5f * (1.0f + erf_as7126(x * 0.70710678118654752440f));
  return cdf + x * 0.39894228040143267794f * __expf(-0.5f * x * x);
}

// Two fp32 -> two bf16 in one word (lo in the low half), round to nearest,
// ties to even, a NaN kept a NaN with its quiet bit set: gfx950's packed
// conversion (v_cvt_pk_bf16_f32), one instruction where the same rounding in
// integer arithmetic takes a dozen and a branch per value for the NaN case.
// It equals that integer rounding bit for bit on every fp32 input.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

__device__ __forceinline__ float bf16_to_f32(uint32_t bits) { return __uint_as_float(bits << 16); }

// ---- epilogue ------------------------------------------------------------
// The 4 accumulator values of one lane are C[m][n .. n+3].  `full`: all four
// columns lie inside N and the rows are aligned for vector access.

__device__ __forceinline__ void store_bf16x4(uint16_t *dst, f32x4_t v, bool full, int64_t left) {
  if (full) {
    *reinterpret_cast<u32x2_t *>(dst) = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e < left) dst[e] = static_cast<uint16_t>(bf16_bits_rne(v[e]));
  }
}

__device__ __forceinline__ f32x4_t load_bf16x4(const uint16_t *src, bool full, int64_t left) {
  f32x4_t v{0.f, 0.f, 0.f, 0.f};
  if (full) {
    const u32x2_t w = *reinterpret_cast<const u32x2_t *>(src);
    v = f32x4_t{bf16_to_f32(w[0] & 0xffffu), bf16_to_f32(w[0] >> 16), bf16_to_f32(w[1] & 0xffffu),
                bf16_to_f32(w[1] >> 16)};
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e < left) v[e] = bf16_to_f32(src[e]);
  }
  return v;
}

// kEpiF32Red: store the partial v, then its sum with the peers' partials and
// the bias, added in the separate reduction's order.  This whole-vector form
// takes the peers' vectors already loaded.
// SPLIT: the sum reduce-scattered over red.out[] (kEpiF32RedSplit).
template <bool SPLIT>
__device__ __forceinline__ void epi_store_red_vec(const GemmArgs& p, int64_t ldc, int64_t m, int64_t n, f32x4_t v,
                                                  const f32x4_t (&pv)[kMaxFusedPeers]) {
  const EpiReduce& r = p.red;
  const int64_t off = m * ldc + n;
  if (r.out[0] != p.c) *reinterpret_cast<f32x4_t *>(static_cast<float *>(p.c) + off) = v;
  f32x4_t sum = v;
#pragma unroll
  for (int q = 0; q < kMaxFusedPeers; ++q)
    if (q < r.np) sum = sum + pv[q];
  if (r.bias) sum = sum + *reinterpret_cast<const f32x4_t *>(r.bias + n);
  // The fp32 sum streams past the caches; the next layer's copy, read by its
  // GEMM next, goes through them (as in the separate reduction).
  if constexpr (SPLIT) {
    const int64_t j = m / r.rows_per_out;
    __builtin_nontemporal_store(sum, reinterpret_cast<f32x4_t *>(r.out[j] + (m - j * r.rows_per_out) * ldc + n));
  } else if (r.out[0]) {
    __builtin_nontemporal_store(sum, reinterpret_cast<f32x4_t *>(r.out[0] + off));
  }
  if (r.lo) {
    if (r.lo_bf16)
      *reinterpret_cast<u32x2_t *>(static_cast<uint16_t *>(r.lo) + off) =
          u32x2_t{pack_bf16x2(sum[0], sum[1]), pack_bf16x2(sum[2], sum[3])};
    else
      *reinterpret_cast<f32x4_t *>(static_cast<float *>(r.lo) + off) = sum;
  }
}

// The same with the peers' vectors loaded here, all before the first add.
// kEpiF32Red runs on the DMA path only, where every lane stores whole vectors.
template <bool SPLIT>
__device__ __forceinline__ void epi_store_red(const GemmArgs& p, int64_t ldc, int64_t m, int64_t n, f32x4_t v) {
  f32x4_t pv[kMaxFusedPeers];
#pragma unroll
  for (int q = 0; q < kMaxFusedPeers; ++q)
    if (q < p.red.np) pv[q] = *reinterpret_cast<const f32x4_t *>(p.red.peer[q] + m * ldc + n);
  epi_store_red_vec<SPLIT>(p, ldc, m, n, v, pv);
}

template <int EPI>
__device__ __forceinline__ void epi_store(const GemmArgs& p, int64_t ldc, int64_t m, int64_t n, f32x4_t v, bool full) {
  const int64_t left = p.N - n;
  if constexpr (EPI == kEpiF32Red || EPI == kEpiF32RedSplit) {
    epi_store_red<EPI == kEpiF32RedSplit>(p, ldc, m, n, v);
  } else if constexpr (EPI == kEpiF32 || EPI == kEpiF32Acc) {
    float *C = static_cast<float *>(p.c) + m * ldc + n;
    if (full) {
      *reinterpret_cast<f32x4_t *>(C) = v;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (e < left) C[e] = v[e];
    }
  } else {
    if constexpr (EPI == kEpiGeluSaveBf16)
      store_bf16x4(static_cast<uint16_t *>(p.aux) + m * p.ldaux + n, v, full, left);
    if constexpr (EPI == kEpiDGeluBf16) {
      const f32x4_t h = load_bf16x4(static_cast<const uint16_t *>(p.aux) + m * p.ldaux + n, full, left);
      v = f32x4_t{v[0] * gelu_erf_deriv(h[0]), v[1] * gelu_erf_deriv(h[1]), v[2] * gelu_erf_deriv(h[2]),
                  v[3] * gelu_erf_deriv(h[3])};
    }
    if constexpr (EPI == kEpiGeluBf16 || EPI == kEpiGeluSaveBf16)
      v = f32x4_t{gelu_erf(v[0]), gelu_erf(v[1]), gelu_erf(v[2]), gelu_erf(v[3])};
    store_bf16x4(static_cast<uint16_t *>(p.c) + m * ldc + n, v, full, left);
  }
}

// Starting accumulator of an fp32-output tile when C += A W is asked for.
__device__ __forceinline__ f32x4_t acc_start(const GemmArgs& p, int64_t ldc, int64_t m, int64_t n, bool full) {
  const float *C = static_cast<const float *>(p.c) + m * ldc + n;
  if (full) return *reinterpret_cast<const f32x4_t *>(C);
  f32x4_t v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (n + e < p.N) v[e] = C[e];
  return v;
}

// ---- XCD-aware tile order ------------------------------------------------
// Workgroups are dealt round-robin to the 8 XCDs, each with its own L2.
// Hand XCD x a contiguous range of logical tiles, then walk tiles in groups
// of kGroupM tile rows so neighbours share operand panels in that L2.
constexpr int kXcds = 8;
constexpr int kGroupM = 4;

__device__ __forceinline__ void tile_coords(int bid, int ntiles, int tiles_m, int tiles_n, int *tm, int *tn) {
  const int per = ntiles / kXcds, rem = ntiles % kXcds;
  const int x = bid % kXcds, i = bid / kXcds;
  const int t = x * per + (x < rem ? x : rem) + i;
  const int in_group = kGroupM * tiles_n;
  const int g = t / in_group;
  const int first_m = g * kGroupM;
  const int gm = (tiles_m - first_m) < kGroupM ? (tiles_m - first_m) : kGroupM;
  const int local = t - g * in_group;
  *tm = first_m + local % gm;
  *tn = local / gm;
}

// The part of A that holds the tile whose first row is m0: its base, the
// tile's first row within it and the rows it has (A itself, unless A comes as
// row blocks, none of which a tile straddles).  Wave-uniform.
struct APart {
  const void *base;
  int64_t row0, rows;
};
__device__ __forceinline__ APart a_part(const GemmArgs& p, int64_t m0) {
  if (p.a_blk_rows == 0) return {p.a, m0, p.M};
  const int64_t j = m0 / p.a_blk_rows, first = j * p.a_blk_rows;
  const void *base = p.a_blk[0];
#pragma unroll
  for (int q = 1; q < kMaxABlocks; ++q)
    if (j == q) base = p.a_blk[q];
  return {base, m0 - first, p.M - first < p.a_blk_rows ? p.M - first : p.a_blk_rows};
}

// ---- ragged path: register-staged, bounds-checked ------------------------
// LDS holds, per stage, X rows [m][k] and W columns [n][k] (k contiguous, 64
// bf16 per row, chunk c of row r at chunk position c ^ swz(r)).

// X tile rows are written 8 lanes per row and read 16 rows per lane group:
// rows r..r+7 must land on distinct chunk positions.
__device__ __forceinline__ uint32_t lds_off_a(int r, int c) {
  return static_cast<uint32_t>(r * 128 + ((c ^ (r & 7)) << 4));
}

// W tile rows (one per output column n) are written by lanes whose n differ by
// 8 and read by lanes whose n differ by 1: mix both bit groups.
__device__ __forceinline__ uint32_t lds_off_b(int n, int c) {
  return static_cast<uint32_t>(n * 128 + ((c ^ ((n ^ (n >> 3)) & 7)) << 4));
}

// VEC: 16-byte loads along the contiguous dimension (both operands in the
// forward layout, aligned).  Otherwise every element is loaded on its own
// through the layout's strides, for any layout and alignment.
template <int BM, int BN, bool VEC, int EPI>
struct Bf16Gemm {
  static constexpr int WM = BM / 2, WN = BN / 2;       // wave tile
  static constexpr int TM = WM / 16, TN = WN / 16;     // MFMA tiles per wave
  static constexpr int A_CHUNKS = BM * kBK / 8 / kThreads;   // 16B chunks of X per thread
  static constexpr int KB = BN / 32;                  // W rows (k) per thread
  static constexpr int NBLK = BN / 8;                 // 8-column groups of the W tile
  static constexpr int LDS_A = BM * kBK * 2;
  static constexpr int LDS_B = BN * kBK * 2;
  static constexpr int LDS_STAGE = LDS_A + LDS_B;
  static_assert(BM % 32 == 0 && BN % 64 == 0 && KB >= 2 && KB <= 8, "tile shape");
  static_assert(A_CHUNKS >= 1, "tile shape");

  struct Regs {
    u32x4_t a[A_CHUNKS];
    u32x4_t w[KB];
  };

  // Global -> registers for the stage starting at k0.  Out-of-range elements
  // read as zero, so the MFMA sees a zero-padded tile.
  __device__ __forceinline__ static void load(const GemmArgs& p, int m0, int n0, int k0, Regs& g) {
    const int t = threadIdx.x;
    const uint16_t *A = static_cast<const uint16_t *>(p.a);
    const uint16_t *W = static_cast<const uint16_t *>(p.w);
    // Element strides: A(m, k) = A[m * sam + k * sak], W(k, n) = W[k * swk + n * swn].
    const int64_t sam = p.a_t ? 1 : p.lda, sak = p.a_t ? p.lda : 1;
    const int64_t swk = p.w_t ? 1 : p.ldw, swn = p.w_t ? p.ldw : 1;
#pragma unroll
    for (int q = 0; q < A_CHUNKS; ++q) {
      const int idx = t + kThreads * q;
      const int row = idx >> 3, c = idx & 7;
      const int64_t gm = m0 + row;
      const int64_t gk = k0 + c * 8;
      if constexpr (VEC) {
        g.a[q] = (gm < p.M && gk < p.K)
                     ? *reinterpret_cast<const u32x4_t *>(A + gm * p.lda + gk)
                     : u32x4_t{0, 0, 0, 0};
      } else {
        uint32_t v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t k = gk + 2 * e;
          const uint32_t lo = (gm < p.M && k < p.K) ? A[gm * sam + k * sak] : 0u;
          const uint32_t hi = (gm < p.M && k + 1 < p.K) ? A[gm * sam + (k + 1) * sak] : 0u;
          v[e] = lo | (hi << 16);
        }
        g.a[q] = u32x4_t{v[0], v[1], v[2], v[3]};
      }
    }
    const int nb = t % NBLK, kb = t / NBLK;
    const int64_t gn = n0 + nb * 8;
#pragma unroll
    for (int q = 0; q < KB; ++q) {
      const int64_t gk = k0 + kb * KB + q;
      if constexpr (VEC) {
        g.w[q] = (gk < p.K && gn < p.N)
                     ? *reinterpret_cast<const u32x4_t *>(W + gk * p.ldw + gn)
                     : u32x4_t{0, 0, 0, 0};
      } else {
        uint32_t v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t n = gn + 2 * e;
          const uint32_t lo = (gk < p.K && n < p.N) ? W[gk * swk + n * swn] : 0u;
          const uint32_t hi = (gk < p.K && n + 1 < p.N) ? W[gk * swk + (n + 1) * swn] : 0u;
          v[e] = lo | (hi << 16);
        }
        g.w[q] = u32x4_t{v[0], v[1], v[2], v[3]};
      }
    }
  }

  // Registers -> LDS stage.  The W block (KB k-rows x 8 n-columns) is
  // transposed so that LDS holds, per column n, KB consecutive k values.
  __device__ __forceinline__ static void store(char *stage, const Regs& g) {
    const int t = threadIdx.x;
    char *As = stage;
    char *Bs = stage + LDS_A;
#pragma unroll
    for (int q = 0; q < A_CHUNKS; ++q) {
      const int idx = t + kThreads * q;
      const int row = idx >> 3, c = idx & 7;
      *reinterpret_cast<u32x4_t *>(As + lds_off_a(row, c)) = g.a[q];
    }
    const int nb = t % NBLK, kb = t / NBLK;
    const int kfirst = kb * KB;
    const int c = kfirst >> 3;
    const int byte_in_chunk = (kfirst & 7) * 2;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int n = nb * 8 + j;
      uint32_t d[KB / 2];
#pragma unroll
      for (int e = 0; e < KB / 2; ++e) {
        const uint32_t lo_src = g.w[2 * e][j >> 1];
        const uint32_t hi_src = g.w[2 * e + 1][j >> 1];
        d[e] = (j & 1) ? ((lo_src >> 16) | (hi_src & 0xffff0000u))
                       : ((lo_src & 0xffffu) | (hi_src << 16));
      }
      char *dst = Bs + lds_off_b(n, c) + byte_in_chunk;
      if constexpr (KB == 8) {
        *reinterpret_cast<u32x4_t *>(dst) = u32x4_t{d[0], d[1], d[2], d[3]};
      } else if constexpr (KB == 4) {
        *reinterpret_cast<u32x2_t *>(dst) = u32x2_t{d[0], d[1]};
      } else {
        *reinterpret_cast<uint32_t *>(dst) = d[0];
      }
    }
  }

  __device__ __forceinline__ static void compute(const char *stage, f32x4_t (&acc)[TM][TN]) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const char *As = stage;
    const char *Bs = stage + LDS_A;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c = kk * 4 + (lane >> 4);
      bf16x8_t a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t *>(As + lds_off_a(wm * WM + i * 16 + (lane & 15), c));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        b[j] = *reinterpret_cast<const bf16x8_t *>(Bs + lds_off_b(wn * WN + j * 16 + (lane & 15), c));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
    }
  }

  // Row m and first column n of accumulator (i, j) of this lane.
  __device__ __forceinline__ static void coords(int m0, int n0, int i, int j, int64_t *m, int64_t *n) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    *m = m0 + wm * WM + i * 16 + (lane & 15);
    *n = n0 + wn * WN + j * 16 + 4 * (lane >> 4);
  }

  __device__ __forceinline__ static void epilogue(const GemmArgs& p, int m0, int n0, const f32x4_t (&acc)[TM][TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        int64_t m, n;
        coords(m0, n0, i, j, &m, &n);
        if (m < p.M && n < p.N) epi_store<EPI>(p, p.ldc, m, n, acc[i][j], VEC && n + 3 < p.N);
      }
  }
};

template <int BM, int BN, bool VEC, int EPI>
__global__ void __launch_bounds__(kThreads, 1) bf16_gemm_ragged(GemmArgs p) {
  static_assert(EPI != kEpiF32Red && EPI != kEpiF32RedSplit, "the fused reduction stores whole vectors: DMA path only");
  using G = Bf16Gemm<BM, BN, VEC, EPI>;
  __shared__ __attribute__((aligned(16))) char smem[2 * G::LDS_STAGE];

  const int tiles_m = static_cast<int>((p.M + BM - 1) / BM);
  const int tiles_n = static_cast<int>((p.N + BN - 1) / BN);
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;

  f32x4_t acc[G::TM][G::TN];
#pragma unroll
  for (int i = 0; i < G::TM; ++i)
#pragma unroll
    for (int j = 0; j < G::TN; ++j) {
      acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if constexpr (EPI == kEpiF32Acc) {
        int64_t m, n;
        G::coords(m0, n0, i, j, &m, &n);
        if (m < p.M && n < p.N) acc[i][j] = acc_start(p, p.ldc, m, n, VEC && n + 3 < p.N);
      }
    }

  const int nk = static_cast<int>((p.K + kBK - 1) / kBK);
  typename G::Regs g;
  G::load(p, m0, n0, 0, g);
  G::store(smem, g);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    char *cur = smem + (kt & 1) * G::LDS_STAGE;
    char *nxt = smem + ((kt + 1) & 1) * G::LDS_STAGE;
    const bool more = kt + 1 < nk;
    if (more) G::load(p, m0, n0, (kt + 1) * kBK, g);
    G::compute(cur, acc);
    if (more) G::store(nxt, g);
    __syncthreads();
  }
  G::epilogue(p, m0, n0, acc);
}

// ---- main path: LDS-DMA ring, 8 waves ------------------------------------

// One LDS-DMA load: this lane's 16 bytes at g land at LDS byte address
// lds + 16 * lane.  lds must be wave-uniform (it goes to M0).
__device__ __forceinline__ void lds_dma16(const void *g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left alone).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(0) (vmcnt and expcnt left alone).
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

// One operand's tile of a stage in LDS.  ROWS is the output extent it feeds
// (BM for A, BN for W).
//  * KC (k-contiguous in memory): ROWS LDS rows of BK k (2 * BK bytes each);
//    chunk c of row r sits at c ^ swz(r), so that the 8 rows a DMA instruction
//    or a 16-lane read group touches hit distinct banks; fragments are one
//    ds_read_b128 per lane (row = lane & 15, k chunk = lane >> 4).
//  * otherwise (row/column-contiguous): BK LDS rows (one per k) of ROWS
//    elements; chunk c of k-row r sits at c ^ 2 (r & 3), so the 4 k-rows a
//    transposing read touches hit distinct banks; a fragment is two
//    ds_read_b64_tr_b16 (lane 4 r + q of group g reads k-row 8 g + r (+4),
//    columns 4 q .. 4 q + 3; lane j of the group then holds column j, 4 k).
// DMA pieces are 1 KiB: lane l of piece p covers tile bytes 1024 p + 16 l.
template <int ROWS, int BK, bool KC>
struct OpTile {
  static constexpr int BYTES = ROWS * BK * 2;
  static constexpr int PIECES = BYTES / 1024;
  static constexpr int RB = KC ? BK * 2 : ROWS * 2;   // bytes per LDS row
  static_assert(BYTES % 1024 == 0 && RB % 16 == 0, "operand tile");
  static_assert(KC || (RB / 16) % 8 == 0, "row-contiguous tiles need 8-chunk rows for their swizzle");

  __device__ __forceinline__ static int swz(int r) {
    return KC ? (BK == 32 ? ((r >> 1) & 3) : (r & 7)) : 2 * (r & 3);
  }
  // Element offset, from the operand base at k = 0, of this lane's 16 bytes
  // of piece `piece` for the tile whose first row (m or n) is row0.  Rows (KC)
  // or 8-column groups (otherwise) past nrows are clamped onto valid memory:
  // they only feed outputs that are never stored.
  __device__ __forceinline__ static int64_t src(int piece, int lane, int64_t row0, int64_t nrows, int64_t ld) {
    const int byte = piece * 1024 + lane * 16;
    const int r = byte / RB, c = ((byte % RB) >> 4) ^ swz(r);
    if constexpr (KC) {
      const int64_t g = (row0 + r < nrows) ? row0 + r : nrows - 1;
      return g * ld + c * 8;
    } else {
      const int64_t g = (row0 + c * 8 < nrows) ? row0 + c * 8 : nrows - 8;
      return static_cast<int64_t>(r) * ld + g;
    }
  }
  // Element advance of the source per stage (k0 -> k0 + BK).
  __device__ __forceinline__ static int64_t step(int64_t ld) { return KC ? BK : BK * ld; }
  // MFMA operand fragment of the 16 rows starting at tile row `row`, k-step kk.
  __device__ __forceinline__ static bf16x8_t frag(const TP_LDS char *base, int row, int kk, int lane) {
    if constexpr (KC) {
      const int r = row + (lane & 15), c = kk * 4 + (lane >> 4);
      return *(const TP_LDS bf16x8_t *)(base + r * RB + ((c ^ swz(r)) << 4));
    } else {
      const int col = row + 4 * (lane & 3);
      const int k = kk * 32 + 8 * (lane >> 4) + ((lane & 15) >> 2);
      const int o = k * RB + (((col >> 3) ^ swz(k)) << 4) + (col & 7) * 2;   // k + 4: same swizzle
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TP_LDS i16x4_t *)(base + o));
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TP_LDS i16x4_t *)(base + o + 4 * RB));
      return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }
};

// AT: A given transposed (m-contiguous); WT: W given transposed (k-contiguous).
template <int BM, int BN, int BK, int S, bool AT, bool WT, int WAVES_M_ = 2, int WAVES_N_ = 4>
struct DmaCfg {
  using TA = OpTile<BM, BK, !AT>;
  using TW = OpTile<BN, BK, WT>;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, NW = WAVES_M * WAVES_N, THREADS = 64 * NW;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N, TM = WM / 16, TN = WN / 16;
  static constexpr int KK = BK / 32;                   // MFMA k-steps per stage
  static constexpr int STAGE = TA::BYTES + TW::BYTES;
  // The A pieces split evenly over the waves; the W pieces are dealt
  // round-robin, so when they do not divide evenly the first W_REM waves
  // issue one more than the rest.
  static constexpr int A_PW = TA::PIECES / NW;
  static constexpr int W_PW = (TW::PIECES + NW - 1) / NW, W_REM = TW::PIECES % NW;
  static constexpr int L_HI = A_PW + W_PW, L_LO = W_REM ? L_HI - 1 : L_HI;   // per-wave DMA count
  static_assert((BK == 32 || BK == 64) && WN % 16 == 0 && WM % 16 == 0, "tile shape");
  static_assert(A_PW >= 1 && TA::PIECES % NW == 0 && TW::PIECES >= NW, "DMA split");
  static_assert((S - 1) * L_HI < 64, "vmcnt range");
  static_assert(S * STAGE <= 160 * 1024, "LDS");
};

// One workgroup's tile `bid` of the problem p (the body of the single-group
// kernels below).
template <int BM, int BN, int BK, int S, int EPI, bool AT, bool WT, int WAVES_M, int WAVES_N>
__device__ __forceinline__ void dma_tile(const GemmArgs& p, int bid) {
  using C = DmaCfg<BM, BN, BK, S, AT, WT, WAVES_M, WAVES_N>;
  using TA = typename C::TA;
  using TW = typename C::TW;
  constexpr int KK = C::KK;
  __shared__ __attribute__((aligned(1024))) char smem[S * C::STAGE];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int tiles_m = static_cast<int>((p.M + BM - 1) / BM);
  const int tiles_n = static_cast<int>((p.N + BN - 1) / BN);
  int tm, tn;
  tile_coords(bid, tiles_m * tiles_n, tiles_m, tiles_n, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((TP_LDS char *)smem));
  const APart ap = a_part(p, m0);
  const uint16_t *A = static_cast<const uint16_t *>(ap.base);
  const uint16_t *W = static_cast<const uint16_t *>(p.w);
  // The output stride is only used after the main loop; left to the compiler
  // its scalar load would still be in flight when the loop starts, and since
  // scalar loads return out of order the first LDS wait of every iteration
  // would have to drain all reads (lgkmcnt(0)).  Make it arrive here.
  const int64_t ldc = p.ldc;
  asm volatile("" ::"s"(ldc));

  // Source of each of this lane's DMA pieces (elements, at k = 0).  Lane order
  // fixes the LDS position, so the swizzle is applied by choosing which chunk
  // a lane fetches.  A piece index past the W tile (the short waves' last
  // slot) is never issued.
  int64_t a_src[C::A_PW], w_src[C::W_PW];
#pragma unroll
  for (int q = 0; q < C::A_PW; ++q) a_src[q] = TA::src(wave * C::A_PW + q, lane, ap.row0, ap.rows, p.lda);
#pragma unroll
  for (int q = 0; q < C::W_PW; ++q)
    w_src[q] = TW::src(min(wave + q * C::NW, TW::PIECES - 1), lane, n0, p.N, p.ldw);
  const int64_t a_step = TA::step(p.lda), w_step = TW::step(p.ldw);
  auto issue = [&](int st, int slot) {
    const uint32_t base = lds0 + slot * C::STAGE;
#pragma unroll
    for (int q = 0; q < C::A_PW; ++q) lds_dma16(A + a_src[q] + st * a_step, base + (wave * C::A_PW + q) * 1024);
#pragma unroll
    for (int q = 0; q < C::W_PW; ++q)
      if (C::W_REM == 0 || q + 1 < C::W_PW || wave < C::W_REM)
        lds_dma16(W + w_src[q] + st * w_step, base + TA::BYTES + (wave + q * C::NW) * 1024);
  };
  // s_waitcnt vmcnt(n * this wave's DMA count per stage).
  const bool dma_hi = C::W_REM == 0 || wave < C::W_REM;
  auto wait_stages = [&](auto n) {
    constexpr int N = decltype(n)::value;
    if (dma_hi) wait_vmcnt<N * C::L_HI>(); else wait_vmcnt<N * C::L_LO>();
  };

  static_assert(C::THREADS == 64 * WAVES_M * WAVES_N, "launch shape");
  auto read = [&](int u, bf16x8_t (&fa)[C::TM], bf16x8_t (&fb)[C::TN]) {
    const int kk = KK == 1 ? 0 : (u & 1);
    const TP_LDS char *base = (const TP_LDS char *)smem + ((u / KK) % S) * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::TM; ++i) fa[i] = TA::frag(base, wm * C::WM + i * 16, kk, lane);
#pragma unroll
    for (int j = 0; j < C::TN; ++j) fb[j] = TW::frag(base + TA::BYTES, wn * C::WN + j * 16, kk, lane);
  };
  auto coords = [&](int i, int j, int64_t *m, int64_t *n) {
    *m = m0 + wm * C::WM + i * 16 + (lane & 15);
    *n = n0 + wn * C::WN + j * 16 + 4 * (lane >> 4);
  };
  f32x4_t acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if constexpr (EPI == kEpiF32Acc) {
        int64_t m, n;
        coords(i, j, &m, &n);
        if (m < p.M && n < p.N) acc[i][j] = acc_start(p, ldc, m, n, true);
      }
    }
  // Rows inner: consecutive MFMAs share the W operand (measured a few percent
  // faster than sharing the A operand on the 8 x 3 wave tile).
  auto mma = [&](const bf16x8_t (&fa)[C::TM], const bf16x8_t (&fb)[C::TN]) {
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
  };

  // Stage t lives in slot t % S.  The barrier that opens stage t (after this
  // wave's loads of stage t have landed: vmcnt) also proves every wave has
  // read stage t-1 into registers (lgkmcnt(0) before it: the DMA is invisible
  // to the compiler's own waits), so stage t+S-1 is issued into its slot.
  const int nst = static_cast<int>(p.K / BK), nu = nst * KK;

  // The partial sum of kEpiF32Red reads the peers' partials of this tile.
  // With two slots they stream in during the main loop rather than after it:
  // each stage opening issues one 16-byte load per lane (vector j = fragment
  // j / np, peer j % np) right after that stage's DMA, so the next opening,
  // which needs that DMA, may leave exactly this one younger load in flight
  // (loads complete in issue order).  The load is issued for every lane (rows
  // past M read row M - 1, never stored), so the wave always counts it.
  // Vectors the stage openings do not reach are loaded in the epilogue.
  constexpr bool PF = (EPI == kEpiF32Red || EPI == kEpiF32RedSplit) && S == 2;
  constexpr int NF = C::TM * C::TN;
  f32x4_t pv[PF ? NF : 1][kMaxFusedPeers];
  const int np = PF ? p.red.np : 0;
  int pf_issued = 0, pf_pending = 0;
  auto peer_vec = [&](int f, int q) {
    int64_t m, n;
    coords(f / C::TN, f % C::TN, &m, &n);
    m = m < p.M ? m : p.M - 1;
    n = n < p.N ? n : p.N - 4;   // N % 8 == 0 on this path
    return *reinterpret_cast<const f32x4_t *>(p.red.peer[q] + m * ldc + n);
  };
  auto prefetch = [&]() {
    pf_pending = 0;
    if (pf_issued >= NF * np) return;
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int q = 0; q < kMaxFusedPeers; ++q)
        if (q < np && f * np + q == pf_issued) pv[f][q] = peer_vec(f, q);
    ++pf_issued;
    pf_pending = 1;
  };

  auto open_stage = [&](int st) {
    if constexpr (PF) {
      if (pf_pending) wait_vmcnt<1>(); else wait_vmcnt<0>();
    } else {
      if (st + S - 2 < nst) wait_stages(std::integral_constant<int, S - 2>{}); else wait_vmcnt<0>();
    }
    wait_lgkmcnt0();
    __syncthreads();
    if (st + S - 1 < nst) issue(st + S - 1, (st + S - 1) % S);
    if constexpr (PF) prefetch();
  };
#pragma unroll
  for (int st = 0; st < S; ++st)
    if (st < nst) issue(st, st);
  if (nst >= S) wait_stages(std::integral_constant<int, S - 1>{}); else wait_vmcnt<0>();
  __syncthreads();
  bf16x8_t fa0[C::TM], fb0[C::TN], fa1[C::TM], fb1[C::TN];
  read(0, fa0, fb0);
  int u = 0;
  for (; u + 2 <= nu; u += 2) {
    if ((u + 1) % KK == 0) open_stage((u + 1) / KK);
    read(u + 1, fa1, fb1);
    mma(fa0, fb0);
    if (u + 2 < nu) {
      if ((u + 2) % KK == 0) open_stage((u + 2) / KK);
      read(u + 2, fa0, fb0);
    }
    mma(fa1, fb1);
  }
  if (u < nu) mma(fa0, fb0);

  if constexpr (PF) {
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int q = 0; q < kMaxFusedPeers; ++q)
        if (q < np && f * np + q >= pf_issued) pv[f][q] = peer_vec(f, q);
  }
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      int64_t m, n;
      coords(i, j, &m, &n);
      if (m < p.M && n < p.N) {   // N % 8 == 0 on this path
        if constexpr (PF) epi_store_red_vec<EPI == kEpiF32RedSplit>(p, ldc, m, n, acc[i][j], pv[i * C::TN + j]);
        else epi_store<EPI>(p, ldc, m, n, acc[i][j], true);
      }
    }
}

template <int BM, int BN, int BK, int S, int EPI, bool AT, bool WT, int WAVES_M = 2, int WAVES_N = 4>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N, 1) bf16_gemm_dma(GemmArgs p) {
  dma_tile<BM, BN, BK, S, EPI, AT, WT, WAVES_M, WAVES_N>(p, blockIdx.x);
}

// Independent problems of one shape class in one launch (a grouped GEMM):
// problem q takes workgroups [start[q], start[q+1]).  GEMMs that each leave CUs
// idle (a few hundred small tiles) then share the chip instead of running one
// after the other.
constexpr int kMaxGroup = 4;
struct GemmGroup {
  GemmArgs p[kMaxGroup];
  int32_t start[kMaxGroup + 1];
  int32_t n;
};

template <int BM, int BN, int BK, int S, int EPI, bool AT, bool WT, int WAVES_M = 2, int WAVES_N = 4>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N, 1) bf16_gemm_dma_group(GemmGroup g) {
  const int bid = blockIdx.x;
  int q = 0;
  while (q + 1 < g.n && bid >= g.start[q + 1]) ++q;   // uniform: one problem per workgroup
  const GemmArgs *p = g.p + q;                          // stays in the argument segment
  dma_tile<BM, BN, BK, S, EPI, AT, WT, WAVES_M, WAVES_N>(*p, bid - g.start[q]);
}

// ---- ping-pong path -------------------------------------------------------

// DMA of 16 bytes at sbase + voff (32-bit byte offset) into LDS M0 + 16 * lane.
__device__ __forceinline__ void lds_dma16_s(const void *sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}
// Barriers of the schedule, each with the wait it needs folded in, so no LDS
// read or DMA can be moved across it.
__device__ __forceinline__ void barrier_lgkm0() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void barrier_vm0() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void barrier_raw() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// s_waitcnt vmcnt(n * L) for a run-time n in [0, NMAX] (the count must be an
// immediate), folded with the barrier that follows it.
template <int L, int NMAX>
__device__ __forceinline__ void barrier_vm_n(int n) {
  if constexpr (NMAX == 0) {
    barrier_vm0();
  } else {
    if (n >= NMAX) {
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(NMAX * L) : "memory");
      __builtin_amdgcn_sched_barrier(0);
    } else {
      barrier_vm_n<L, NMAX - 1>(n);
    }
  }
}

// The ping-pong kernel (bf16_gemm_pps): 8 waves (WGM x 8/WGM) on a 256-row
// tile, K staged 64 at a time.  Waves 0-3 (group A, tile rows 0..127) and
// 4-7 (group B, rows 128..255) run one barrier apart; wave w sits on SIMD
// w % 4, so each SIMD holds one wave of each group and feeds its matrix pipe
// from one while the other reads LDS.  With a single two-slot ring every DMA
// of stage s would have to leave in the one phase that follows the barrier
// after which both groups are done with stage s-2 and precedes the one after
// which group A reads stage s-1, the phase in which group A reads LDS: the
// issue of a stage's 40-64 DMA instructions (about 15 cycles each through the
// CU's address unit) then held up group A's reads while group B waited at the
// barrier (MI355X phase stamps on the 175B GEMM1 shape: about 830 of 2950
// cycles per stage).  Here the A tile has a ring of three slots and W's tile a
// ring of two, and each group issues its tile between its own MFMAs:
//   A: a0 a1 | #0 | R_0 #1 M_0+a2 #2 | R_1 #3 M_1+a3 #4 | ...
//   B: w0    | #0 | w1 #1 R_0 #2 M_0+w2 #3 R_1 #4 M_1+w3 ...
// (aS, wS: the A / W tile of stage S; R reads, M multiplies).  Group A's
// A tile of stage t+2 overwrites stage t-1's slot after #2t+1, group B's W
// tile of stage t+1 stage t-1's slot after #2t; both groups finished reading
// stage t-1 by #2t.  Before #2t+2, after which group A reads stage t+1, group
// A waits for its A tile of stage t+1 (stage t+2's stays in flight) and group
// B for its W tile of stage t+1.  Every MFMA phase carries its DMA, so the
// loop has one body and one MFMA chain per group (duplicated chains made the
// compiler spill): where the stage it would fetch does not exist, it fetches
// the last stage again, into the slot of the nominal stage, which nothing
// reads any more.  Same accumulation order as every other kernel, so the
// results are the same bits.  Measured on MI355X against the single-ring
// form: 7-15% faster on every 256 x 192 and 256 x 128 shape here, forward and
// backward, 8% on 256 x 256 and 9-14% with the accumulating epilogue.
template <int BM, int BN, int EPI, bool AT, bool WT, int WGM = 2>
__global__ void __launch_bounds__(512, 1) bf16_gemm_pps(GemmArgs p) {
  constexpr int BK = 64;
  using C = DmaCfg<BM, BN, BK, 2, AT, WT, WGM, 8 / WGM>;
  using TA = typename C::TA;
  using TW = typename C::TW;
  constexpr int KK = C::KK;
  constexpr int NG = 4;
  constexpr int A_PW = TA::PIECES / NG, W_PW = TW::PIECES / NG;
  constexpr int SA = 3, SW = 2;
  constexpr int W_BASE = SA * TA::BYTES;
  static_assert(TA::PIECES % NG == 0 && TW::PIECES % NG == 0, "DMA split");
  static_assert(SA * TA::BYTES + SW * TW::BYTES <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) char smem[SA * TA::BYTES + SW * TW::BYTES];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const bool grpA = wave < 4;
  const int tiles_m = static_cast<int>((p.M + BM - 1) / BM);
  const int tiles_n = static_cast<int>((p.N + BN - 1) / BN);
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m * tiles_n, tiles_m, tiles_n, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((TP_LDS char *)smem));
  const int64_t ldc = p.ldc;
  asm volatile("" ::"s"(ldc));

  // Source offsets are recomputed at each issue: kept in registers they
  // spill the 256 x 256 tile's accumulators.
  const uint32_t step = static_cast<uint32_t>((grpA ? TA::step(p.lda) : TW::step(p.ldw)) * 2);
  // Piece q of the tile of stage `st` (source) into the slot of stage `slot_st`.
  const APart ap = a_part(p, m0);
  auto dma_a = [&](int q, int st, int slot_st) {
    const uint32_t src = static_cast<uint32_t>(TA::src((wave & 3) * A_PW + q, lane, ap.row0, ap.rows, p.lda) * 2);
    lds_dma16_s(ap.base, src + st * step, lds0 + (slot_st % SA) * TA::BYTES + ((wave & 3) * A_PW + q) * 1024);
  };
  auto dma_w = [&](int q, int st, int slot_st) {
    const uint32_t src = static_cast<uint32_t>(TW::src((wave & 3) * W_PW + q, lane, n0, p.N, p.ldw) * 2);
    lds_dma16_s(p.w, src + st * step, lds0 + W_BASE + (slot_st % SW) * TW::BYTES + ((wave & 3) * W_PW + q) * 1024);
  };

  bf16x8_t fa[KK][C::TM], fb[KK][C::TN];
  auto read_stage = [&](int st) {
    const TP_LDS char *a_base = (const TP_LDS char *)smem + (st % SA) * TA::BYTES;
    const TP_LDS char *w_base = (const TP_LDS char *)smem + W_BASE + (st % SW) * TW::BYTES;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int i = 0; i < C::TM; ++i) fa[kk][i] = TA::frag(a_base, wm * C::WM + i * 16, kk, lane);
#pragma unroll
      for (int j = 0; j < C::TN; ++j) fb[kk][j] = TW::frag(w_base, wn * C::WN + j * 16, kk, lane);
    }
  };
  auto coords = [&](int i, int j, int64_t *m, int64_t *n) {
    *m = m0 + wm * C::WM + i * 16 + (lane & 15);
    *n = n0 + wn * C::WN + j * 16 + 4 * (lane >> 4);
  };
  f32x4_t acc[C::TM][C::TN];
  // Zeros, or C's tile: set right before each group's first MFMA, so that a
  // loaded tile is not live across the DMA set-up (it spilled there).
  auto init_acc = [&]() {
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if constexpr (EPI == kEpiF32Acc) {
          int64_t m, n;
          coords(i, j, &m, &n);
          if (m < p.M && n < p.N) acc[i][j] = acc_start(p, ldc, m, n, true);
        }
      }
  };
  // The stage's MFMAs with ND DMA pieces of stage `dst` spread between them:
  // piece q after MFMA number (q + 1/2) * NF / ND (ND = 0: none; measured
  // 1.5-3% faster than starting at the first MFMA).  Everything is
  // compile-time, so the chain is one basic block; the scheduling barriers
  // keep each DMA where it is written.
  constexpr int NF = KK * C::TN * C::TM;
  auto mma_stage = [&](auto nd, auto is_a, int dst, int dslot) {
    constexpr int ND = decltype(nd)::value;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
#pragma unroll
        for (int i = 0; i < C::TM; ++i) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[kk][j], fa[kk][i], acc[i][j], 0, 0, 0);
          if constexpr (ND > 0) {
            const int f = (kk * C::TN + j) * C::TM + i;
#pragma unroll
            for (int q = 0; q < ND; ++q)
              if (f == q * NF / ND + NF / (2 * ND)) {
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (decltype(is_a)::value) dma_a(q, dst, dslot); else dma_w(q, dst, dslot);
                __builtin_amdgcn_sched_barrier(0);
              }
          }
        }
  };
  using I0 = std::integral_constant<int, 0>;
  using IA = std::integral_constant<int, A_PW>;
  using IW = std::integral_constant<int, W_PW>;
  using T = std::true_type;
  using F = std::false_type;

  // Every MFMA phase carries its DMA, so the loop has one body: in the last
  // iterations, where the stage it would fetch does not exist, it fetches the
  // last stage again into a slot that nothing reads any more (A: the slot of
  // stage t-1, W: that of stage t-1, both finished by #2t), and the waits
  // stay as in the steady state.
  const int nst = static_cast<int>(p.K / BK);
  const int last = nst - 1;
  if (nst > 0) {
    if (grpA) {
#pragma unroll
      for (int q = 0; q < A_PW; ++q) dma_a(q, 0, 0);
#pragma unroll
      for (int q = 0; q < A_PW; ++q) dma_a(q, min(1, last), 1);
      wait_vmcnt<A_PW>();
    } else {
#pragma unroll
      for (int q = 0; q < W_PW; ++q) dma_w(q, 0, 0);
      wait_vmcnt<0>();
    }
  }
  barrier_raw();                                     // #0
  if (grpA) {
    init_acc();
    for (int t = 0; t < nst; ++t) {
      read_stage(t);
      barrier_lgkm0();                               // #2t+1
      mma_stage(IA{}, T{}, min(t + 2, last), t + 2);   // stage t+2's A tile, slot (t+2) % 3
      barrier_vm_n<A_PW, 1>(1);                      // #2t+2: stage t+1's A tile landed
    }
  } else if (nst > 0) {
#pragma unroll
    for (int q = 0; q < W_PW; ++q) dma_w(q, min(1, last), 1);
    barrier_raw();                                   // #1
    read_stage(0);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");   // #2
    __builtin_amdgcn_sched_barrier(0);
    init_acc();
    for (int t = 1; t < nst; ++t) {
      mma_stage(IW{}, F{}, min(t + 1, last), t + 1);   // stage t+1's W tile, slot (t+1) % 2
      barrier_raw();                                 // #2t+1
      read_stage(t);
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");   // #2t+2
      __builtin_amdgcn_sched_barrier(0);
    }
    mma_stage(I0{}, F{}, 0, 0);
  } else {
    init_acc();
  }
  wait_vmcnt<0>();                                   // the repeated fetches of the last stage

  if constexpr (EPI == kEpiF32Red) {
    // The block's sum over the peers, in the separate reduction's order (the
    // tile's own partial, every peer in turn, then the bias), with the peers
    // read as whole rows: the accumulators' layout (16 rows of 64 bytes per
    // vector load) would read them at half the rate.  Each half tile (128
    // rows, one wave group's accumulators) is written to LDS, then all 512
    // lanes walk it row by row: own value from LDS, the peers' vectors from
    // HBM (up to eight in flight), the sum to out[0] and lo, the partial to C
    // unless the sum goes in place over it (or, reduce-scattered, each row to
    // its sequence block).  The sum and lo stream past the caches: on these
    // sizes the next layer's input (lo) outgrows them before its GEMM reads it
    // (two GPT-3 6.7B layers: 811-812 against 835 us with lo stored through
    // them).
    const EpiReduce& r = p.red;
    constexpr int PITCH = BN * 4 + 16;                 // LDS bytes per row (16 bytes of padding)
    constexpr int VPR = BN / 4;                        // 16-byte vectors per row
    static_assert(128 * PITCH <= SA * TA::BYTES + SW * TW::BYTES, "half tile in LDS");
    TP_LDS char *half = (TP_LDS char *)smem;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      __syncthreads();                                 // LDS free: fragments read, DMA landed, previous half done
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
        const int tr = wm * C::WM + i * 16 + (lane & 15);   // row in the tile (uniform half per wave)
        if (tr / 128 != h) continue;
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
          *(TP_LDS f32x4_t *)(half + (tr - h * 128) * PITCH + (wn * C::WN + j * 16 + 4 * (lane >> 4)) * 4) = acc[i][j];
      }
      __syncthreads();
      for (int u = threadIdx.x; u < 128 * VPR; u += 512) {
        const int row = u / VPR, cv = u - row * VPR;
        const int64_t m = m0 + h * 128 + row, n = n0 + cv * 4;
        if (m >= p.M || n >= p.N) continue;
        const int64_t off = m * ldc + n;
        f32x4_t sum = *(const TP_LDS f32x4_t *)(half + row * PITCH + cv * 16);
        if (r.out[0] != p.c) *reinterpret_cast<f32x4_t *>(static_cast<float *>(p.c) + off) = sum;
        for (int q0 = 0; q0 < r.np; q0 += 8) {
          f32x4_t v[8];
#pragma unroll
          for (int g = 0; g < 8; ++g)
            if (q0 + g < r.np) v[g] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(r.peer[q0 + g] + off));
#pragma unroll
          for (int g = 0; g < 8; ++g)
            if (q0 + g < r.np) sum = sum + v[g];
        }
        if (r.bias) sum = sum + *reinterpret_cast<const f32x4_t *>(r.bias + n);
        if (r.nout > 1) {
          // reduce-scattered: row m to out[m / rows_per_out]
          const int64_t jo = m / r.rows_per_out;
          __builtin_nontemporal_store(sum, reinterpret_cast<f32x4_t *>(r.out[jo] + (m - jo * r.rows_per_out) * ldc + n));
        } else if (r.out[0]) {
          __builtin_nontemporal_store(sum, reinterpret_cast<f32x4_t *>(r.out[0] + off));
        }
        if (r.lo) {
          if (r.lo_bf16)
            __builtin_nontemporal_store(u32x2_t{pack_bf16x2(sum[0], sum[1]), pack_bf16x2(sum[2], sum[3])},
                                        reinterpret_cast<u32x2_t *>(static_cast<uint16_t *>(r.lo) + off));
          else
            __builtin_nontemporal_store(sum, reinterpret_cast<f32x4_t *>(static_cast<float *>(r.lo) + off));
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        int64_t m, n;
        coords(i, j, &m, &n);
        if (m < p.M && n < p.N) epi_store<EPI>(p, ldc, m, n, acc[i][j], true);
      }
  }
}

// ---- plain fp32 kernel (tiny fp32 workload) ------------------------------
// 32 x 32 tile, 256 threads of 2 x 2 outputs, K staged 64 at a time through
// LDS with the next slab's loads in flight (registers) while the current one
// is consumed; any operand layout (element strides).  The small tile gives the
// fp32 problems here (a few hundred rows and columns) enough workgroups; every
// output still accumulates k in ascending order with one fma per k.

constexpr int kF32Tile = 32;
constexpr int kF32BK = 64;

template <int EPI>
__global__ void __launch_bounds__(kThreads) f32_gemm_kernel(GemmArgs p) {
  constexpr int PER = kF32BK * kF32Tile / kThreads;   // slab elements per thread, per operand
  __shared__ float As[kF32BK][kF32Tile + 1];
  __shared__ float Ws[kF32BK][kF32Tile + 1];
  const float *A = static_cast<const float *>(p.a);
  const float *W = static_cast<const float *>(p.w);
  const int64_t sam = p.a_t ? 1 : p.lda, sak = p.a_t ? p.lda : 1;
  const int64_t swk = p.w_t ? 1 : p.ldw, swn = p.w_t ? p.ldw : 1;
  const int tiles_n = static_cast<int>((p.N + kF32Tile - 1) / kF32Tile);
  const int64_t m0 = static_cast<int64_t>(blockIdx.x / tiles_n) * kF32Tile;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x % tiles_n) * kF32Tile;
  const int t = threadIdx.x;
  const int tr = t / 16, tc = t % 16;
  float *C = static_cast<float *>(p.c);
  float acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t m = m0 + tr * 2 + i, n = n0 + tc * 2 + j;
      acc[i][j] = (EPI == kEpiPlainF32 && p.acc_init && m < p.M && n < p.N) ? C[m * p.ldc + n] : 0.f;
    }
  // Slab element q of this thread: A at (row e / BK, k e % BK), W at (k e / TILE, col e % TILE), e = t + q * threads.
  float ra[PER], rw[PER];
  auto load = [&](int64_t k0) {
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = t + q * kThreads;
      const int r = e / kF32BK, k = e % kF32BK;
      ra[q] = (m0 + r < p.M && k0 + k < p.K) ? A[(m0 + r) * sam + (k0 + k) * sak] : 0.f;
      const int kk = e / kF32Tile, n = e % kF32Tile;
      rw[q] = (k0 + kk < p.K && n0 + n < p.N) ? W[(k0 + kk) * swk + (n0 + n) * swn] : 0.f;
    }
  };
  load(0);
  for (int64_t k0 = 0; k0 < p.K; k0 += kF32BK) {
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = t + q * kThreads;
      As[e % kF32BK][e / kF32BK] = ra[q];
      Ws[e / kF32Tile][e % kF32Tile] = rw[q];
    }
    __syncthreads();
    if (k0 + kF32BK < p.K) load(k0 + kF32BK);
#pragma unroll
    for (int k = 0; k < kF32BK; ++k) {
      const float a0 = As[k][tr * 2], a1 = As[k][tr * 2 + 1];
      const float w0 = Ws[k][tc * 2], w1 = Ws[k][tc * 2 + 1];
      acc[0][0] = fmaf(a0, w0, acc[0][0]);
      acc[0][1] = fmaf(a0, w1, acc[0][1]);
      acc[1][0] = fmaf(a1, w0, acc[1][0]);
      acc[1][1] = fmaf(a1, w1, acc[1][1]);
    }
    __syncthreads();
  }
  float *X = static_cast<float *>(p.aux);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t m = m0 + tr * 2 + i;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t n = n0 + tc * 2 + j;
      if (n >= p.N) continue;
      float v = acc[i][j];
      if constexpr (EPI == kEpiPlainF32Red) {
        // The partial, then its sum in the separate reduction's order.
        const EpiReduce& r = p.red;
        const int64_t off = m * p.ldc + n;
        if (r.out[0] != p.c) C[off] = v;
        float sum = v;
        for (int q = 0; q < r.np; ++q) sum = sum + r.peer[q][off];
        if (r.bias) sum = sum + r.bias[n];
        if (r.nout > 1) {
          const int64_t jo = m / r.rows_per_out;
          r.out[jo][(m - jo * r.rows_per_out) * p.ldc + n] = sum;
        } else if (r.out[0]) {
          r.out[0][off] = sum;
        }
        if (r.lo) static_cast<float *>(r.lo)[off] = sum;
        continue;
      }
      if constexpr (EPI == kEpiGeluSaveF32) X[m * p.ldaux + n] = v;
      if constexpr (EPI == kEpiDGeluF32) v *= gelu_erf_deriv(X[m * p.ldaux + n]);
      if constexpr (EPI == kEpiGeluF32 || EPI == kEpiGeluSaveF32) v = gelu_erf(v);
      C[m * p.ldc + n] = v;
    }
  }
}

// ---- launchers and tile choice ---------------------------------------------

template <int BM, int BN, int BK, int S, int EPI, bool AT, bool WT, int WAVES_M = 2, int WAVES_N = 4>
hipError_t launch_dma(const GemmArgs& p, hipStream_t s) {
  const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  hipLaunchKernelGGL((bf16_gemm_dma<BM, BN, BK, S, EPI, AT, WT, WAVES_M, WAVES_N>), dim3(static_cast<unsigned>(tiles)),
                     dim3(64 * WAVES_M * WAVES_N), 0, s, p);
  return hipGetLastError();
}

template <int BM, int BN, int BK, int S, int EPI, bool AT, bool WT, int WAVES_M = 2, int WAVES_N = 4>
hipError_t launch_dma_group(const GemmArgs *ps, int n, hipStream_t s) {
  GemmGroup g{};
  g.n = n;
  int64_t total = 0;
  for (int q = 0; q < n; ++q) {
    g.p[q] = ps[q];
    g.start[q] = static_cast<int32_t>(total);
    total += ((ps[q].M + BM - 1) / BM) * ((ps[q].N + BN - 1) / BN);
  }
  g.start[n] = static_cast<int32_t>(total);
  hipLaunchKernelGGL((bf16_gemm_dma_group<BM, BN, BK, S, EPI, AT, WT, WAVES_M, WAVES_N>),
                     dim3(static_cast<unsigned>(total)), dim3(64 * WAVES_M * WAVES_N), 0, s, g);
  return hipGetLastError();
}

template <int BM, int BN, int EPI, bool AT, bool WT, int WGM = 2>
hipError_t launch_pps(const GemmArgs& p, hipStream_t s) {
  const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  hipLaunchKernelGGL((bf16_gemm_pps<BM, BN, EPI, AT, WT, WGM>), dim3(static_cast<unsigned>(tiles)), dim3(512), 0, s, p);
  return hipGetLastError();
}

template <int EPI>
hipError_t launch_ragged(const GemmArgs& p, bool vec, hipStream_t s) {
  const int64_t tiles = ((p.M + 127) / 128) * ((p.N + 127) / 128);
  if (vec)
    hipLaunchKernelGGL((bf16_gemm_ragged<128, 128, true, EPI>), dim3(static_cast<unsigned>(tiles)), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((bf16_gemm_ragged<128, 128, false, EPI>), dim3(static_cast<unsigned>(tiles)), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

// Tile choice for the DMA path: estimated time = (waves of workgroups over the
// 256 CUs) x (work per tile) / (relative per-CU throughput of that tile, as
// measured on MI355X: the larger tile reuses each operand byte more).
constexpr int kCUs = 256;

template <int EPI, bool AT, bool WT>
hipError_t dispatch_bf16(const GemmArgs& p, bool dma_ok, bool vec, hipStream_t s) {
  if (!dma_ok) return launch_ragged<EPI>(p, vec, s);
  auto cost = [&](int bm, int bn, double eff) {
    const int64_t tiles = ((p.M + bm - 1) / bm) * ((p.N + bn - 1) / bn);
    return static_cast<double>((tiles + kCUs - 1) / kCUs) * bm * bn / eff;
  };
  // The tiles staging K 64 at a time need K % 64 == 0.
  const bool k64 = p.K % 64 == 0;
  // Problems too small to give every CU a 128 x 128 tile run 64 x 64 tiles
  // (4 waves, 32 KiB of LDS): several workgroups then share each CU and hide
  // one another's pipeline fill and write-out, which dominate at this size.
  if (((p.M + 127) / 128) * ((p.N + 127) / 128) < kCUs) {
    if (k64) return launch_dma<64, 64, 64, 2, EPI, AT, WT, 2, 2>(p, s);
    return launch_dma<64, 64, 32, 4, EPI, AT, WT, 2, 2>(p, s);
  }
  // The ping-pong kernel addresses operands with 32-bit byte offsets.
  const int64_t a_span = (AT ? p.K : p.M) * p.lda * 2, w_span = (WT ? p.N : p.K) * p.ldw * 2;
  const bool off32 = a_span < (int64_t{1} << 31) && w_span < (int64_t{1} << 31);
  // The 256 x 256 tile keeps its 128 accumulators in registers only without
  // the transposing reads of A and without the accumulator prologue.
  constexpr bool big_ok = !AT && EPI != kEpiF32Acc;
  const double c256 = big_ok && k64 && off32 ? cost(256, 256, 1.0) : 1e300;
  const double c192 = k64 && off32 ? cost(256, 192, 0.95) : 1e300;
  const double c128w = k64 ? cost(256, 128, 0.85) : 1e300, c128 = cost(128, 128, 0.7);
  const double best = std::min(std::min(c256, c192), std::min(c128w, c128));
  // Split rings: 8% faster than the single ring on 4096 x 4096 x 2048.
  if constexpr (big_ok)
    if (c256 == best) return launch_pps<256, 256, EPI, AT, WT>(p, s);
  if (c192 == best) {
    // A read transposed (weight gradients): 4 x 2 waves, 2-3% faster.
    if constexpr (AT) return launch_pps<256, 192, EPI, AT, WT, 4>(p, s);
    else return launch_pps<256, 192, EPI, AT, WT>(p, s);
  }
  // 256 x 128 tiles: the ping-pong kernel where its 32-bit offsets reach
  // (measured 10-12% faster than the single-group kernel on 4096 x 2048 x 4096).
  // With an operand read transposed (the backward's GEMMs) 4 x 2 waves, whose
  // 64 x 64 wave tiles read a fifth fewer LDS bytes, are 7-11% faster; the
  // forward keeps 2 x 4.
  if (c128w == best) {
    if (off32) {
      if constexpr (AT || WT) return launch_pps<256, 128, EPI, AT, WT, 4>(p, s);
      else return launch_pps<256, 128, EPI, AT, WT>(p, s);
    }
    return launch_dma<256, 128, 64, 3, EPI, AT, WT>(p, s);
  }
  return launch_dma<128, 128, 32, 8, EPI, AT, WT>(p, s);
}

bool aligned16(const void *q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; }

// GEMM2 with the block's sum in the epilogue on the 256-row tiles: the tile
// the cost model takes among the split-ring ones (the only kernels with that
// epilogue).
template <bool WT>
hipError_t dispatch_red_tiles(const GemmArgs& p, hipStream_t s) {
  auto cost = [&](int bm, int bn, double eff) {
    const int64_t tiles = ((p.M + bm - 1) / bm) * ((p.N + bn - 1) / bn);
    return static_cast<double>((tiles + kCUs - 1) / kCUs) * bm * bn / eff;
  };
  const double c256 = cost(256, 256, 1.0), c192 = cost(256, 192, 0.95), c128w = cost(256, 128, 0.85);
  if (c256 <= c192 && c256 <= c128w) return launch_pps<256, 256, kEpiF32Red, false, WT>(p, s);
  if (c192 <= c128w) return launch_pps<256, 192, kEpiF32Red, false, WT>(p, s);
  return launch_pps<256, 128, kEpiF32Red, false, WT>(p, s);
}

// Fewer 128 x 128 tiles than CUs: the small-tile path.
bool small_problem(const GemmArgs& p) { return ((p.M + 127) / 128) * ((p.N + 127) / 128) < kCUs; }

}  // namespace

// Conditions for 16-byte access along every operand's contiguous dimension
// and for whole-vector output (and aux) rows.
bool gemm_vec_ok(const GemmArgs& p, int64_t out_esize, bool uses_aux) {
  bool ok = aligned16(p.a) && aligned16(p.w) && aligned16(p.c) && (p.K % 8 == 0) && (p.N % 8 == 0) &&
            (p.lda % 8 == 0) && (p.ldw % 8 == 0) && (p.ldc % (16 / out_esize) == 0);
  if (p.a_t) ok = ok && p.M % 8 == 0;
  if (uses_aux) ok = ok && aligned16(p.aux) && p.ldaux % 8 == 0;
  return ok;
}

hipError_t gemm_launch(const GemmArgs& p, int epi_in, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  if (p.a_blk_rows && !gemm_blocks_ok(p, epi_in)) return hipErrorInvalidValue;
  int epi = epi_in;
  const bool fp32 = epi == kEpiGeluF32 || epi == kEpiPlainF32 || epi == kEpiGeluSaveF32 || epi == kEpiDGeluF32 ||
                    epi == kEpiPlainF32Red;
  if (epi == kEpiPlainF32Red && !gemm_red_ok_f32(p)) return hipErrorInvalidValue;
  if (fp32) {
    const int64_t tiles = ((p.M + kF32Tile - 1) / kF32Tile) * ((p.N + kF32Tile - 1) / kF32Tile);
    const dim3 grid(static_cast<unsigned>(tiles));
    switch (epi) {
      case kEpiGeluF32: hipLaunchKernelGGL((f32_gemm_kernel<kEpiGeluF32>), grid, dim3(kThreads), 0, s, p); break;
      case kEpiGeluSaveF32: hipLaunchKernelGGL((f32_gemm_kernel<kEpiGeluSaveF32>), grid, dim3(kThreads), 0, s, p); break;
      case kEpiDGeluF32: hipLaunchKernelGGL((f32_gemm_kernel<kEpiDGeluF32>), grid, dim3(kThreads), 0, s, p); break;
      case kEpiPlainF32Red: hipLaunchKernelGGL((f32_gemm_kernel<kEpiPlainF32Red>), grid, dim3(kThreads), 0, s, p); break;
      default: hipLaunchKernelGGL((f32_gemm_kernel<kEpiPlainF32>), grid, dim3(kThreads), 0, s, p); break;
    }
    return hipGetLastError();
  }
  if (epi == kEpiF32 && p.acc_init) epi = kEpiF32Acc;
  const bool uses_aux = epi == kEpiGeluSaveBf16 || epi == kEpiDGeluBf16;
  const bool vec = gemm_vec_ok(p, epi == kEpiF32 || epi == kEpiF32Acc || epi == kEpiF32Red ? 4 : 2, uses_aux);
  // The DMA path reads whole 32-deep k steps and 8-column groups unchecked.
  const bool dma_ok = vec && p.K % 32 == 0 && p.K > 0;
  // Forward layout: vector loads on the ragged path too.
  if (!p.a_t && !p.w_t) {
    switch (epi) {
      case kEpiGeluBf16: return dispatch_bf16<kEpiGeluBf16, false, false>(p, dma_ok, vec, s);
      case kEpiIdentBf16: return dispatch_bf16<kEpiIdentBf16, false, false>(p, dma_ok, vec, s);
      case kEpiF32: return dispatch_bf16<kEpiF32, false, false>(p, dma_ok, vec, s);
      case kEpiF32Acc: return dispatch_bf16<kEpiF32Acc, false, false>(p, dma_ok, vec, s);
      case kEpiGeluSaveBf16: return dispatch_bf16<kEpiGeluSaveBf16, false, false>(p, dma_ok, vec, s);
      case kEpiDGeluBf16: return dispatch_bf16<kEpiDGeluBf16, false, false>(p, dma_ok, vec, s);
      case kEpiF32Red:
        if (!gemm_red_ok(p)) return hipErrorInvalidValue;
        if (!small_problem(p)) return dispatch_red_tiles<false>(p, s);
        if (p.red.nout > 1) {
          if (p.K % 64 == 0) return launch_dma<64, 64, 64, 2, kEpiF32RedSplit, false, false, 2, 2>(p, s);
          return launch_dma<64, 64, 32, 4, kEpiF32RedSplit, false, false, 2, 2>(p, s);
        }
        if (p.K % 64 == 0) return launch_dma<64, 64, 64, 2, kEpiF32Red, false, false, 2, 2>(p, s);
        return launch_dma<64, 64, 32, 4, kEpiF32Red, false, false, 2, 2>(p, s);
      default: return hipErrorInvalidValue;
    }
  }
  // Backward layouts: input gradients (W given transposed) and weight
  // gradients (A given transposed).  Their ragged path loads element-wise.
  if (!p.a_t && p.w_t) {
    switch (epi) {
      case kEpiF32Red:
        if (!gemm_red_ok(p)) return hipErrorInvalidValue;
        if (!small_problem(p)) return dispatch_red_tiles<true>(p, s);
        if (p.K % 64 == 0) return launch_dma<64, 64, 64, 2, kEpiF32Red, false, true, 2, 2>(p, s);
        return launch_dma<64, 64, 32, 4, kEpiF32Red, false, true, 2, 2>(p, s);
      case kEpiGeluBf16: return dispatch_bf16<kEpiGeluBf16, false, true>(p, dma_ok, false, s);
      case kEpiGeluSaveBf16: return dispatch_bf16<kEpiGeluSaveBf16, false, true>(p, dma_ok, false, s);
      case kEpiDGeluBf16: return dispatch_bf16<kEpiDGeluBf16, false, true>(p, dma_ok, false, s);
      case kEpiIdentBf16: return dispatch_bf16<kEpiIdentBf16, false, true>(p, dma_ok, false, s);
      case kEpiF32: return dispatch_bf16<kEpiF32, false, true>(p, dma_ok, false, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (p.a_t && !p.w_t) {
    if (epi == kEpiF32) return dispatch_bf16<kEpiF32, true, false>(p, dma_ok, false, s);
    if (epi == kEpiF32Acc) return dispatch_bf16<kEpiF32Acc, true, false>(p, dma_ok, false, s);
  }
  return hipErrorInvalidValue;
}

bool gemm_red_ok(const GemmArgs& p) {
  const EpiReduce& r = p.red;
  if (p.a_t || p.acc_init || r.np < 0 || p.K <= 0 || p.K % 32 != 0 || !gemm_vec_ok(p, 4, false)) return false;
  if (!small_problem(p)) {
    // The split-ring tiles: 64-deep stages, 32-bit operand offsets.
    const bool off32 = p.M * p.lda * 2 < (int64_t{1} << 31) && (p.w_t ? p.N : p.K) * p.ldw * 2 < (int64_t{1} << 31);
    if (r.np > kMaxEpiPeers || p.K % 64 != 0 || !off32) return false;
  } else if (r.np > kMaxFusedPeers || (p.w_t && r.nout > 1)) {
    return false;
  }
  bool ok = !r.bias || aligned16(r.bias);
  for (int q = 0; q < r.np; ++q) ok = ok && r.peer[q] && aligned16(r.peer[q]);
  if (r.nout < 1 || r.nout > kMaxFusedOuts) return false;
  if (r.nout > 1) {
    // Reduce-scattered: whole blocks of rows per output, no second copy.
    if (r.lo || r.rows_per_out < 1 || static_cast<int64_t>(r.rows_per_out) * r.nout != p.M) return false;
    for (int j = 0; j < r.nout; ++j) ok = ok && r.out[j] && aligned16(r.out[j]);
  } else if (r.out[0]) {
    ok = ok && aligned16(r.out[0]);
  }
  if (r.lo) ok = ok && (reinterpret_cast<uintptr_t>(r.lo) & (r.lo_bf16 ? 7u : 15u)) == 0;
  return ok;
}

bool gemm_blocks_ok(const GemmArgs& p, int epi) {
  if (p.a_blk_rows <= 0 || p.a_blk_rows % 256 != 0 || p.a_t || p.M <= 0 || p.K <= 0 || p.K % 32 != 0) return false;
  if (epi != kEpiGeluBf16 && epi != kEpiIdentBf16 && epi != kEpiF32 && epi != kEpiGeluSaveBf16 && epi != kEpiF32Red)
    return false;
  const int64_t nblk = (p.M + p.a_blk_rows - 1) / p.a_blk_rows;
  if (nblk > kMaxABlocks) return false;
  for (int64_t j = 0; j < nblk; ++j)
    if (!p.a_blk[j] || !aligned16(p.a_blk[j])) return false;
  const int64_t out_esize = epi == kEpiF32 || epi == kEpiF32Red ? 4 : 2;
  return gemm_vec_ok(p, out_esize, epi == kEpiGeluSaveBf16);
}

bool gemm_red_ok_f32(const GemmArgs& p) {
  const EpiReduce& r = p.red;
  if (p.a_t || p.w_t || p.acc_init || r.np < 0 || r.np > kMaxFusedPeers || r.nout < 1 || r.nout > kMaxFusedOuts)
    return false;
  for (int q = 0; q < r.np; ++q)
    if (!r.peer[q]) return false;
  if (r.nout > 1) {
    if (r.lo || r.rows_per_out < 1 || static_cast<int64_t>(r.rows_per_out) * r.nout != p.M) return false;
    for (int j = 0; j < r.nout; ++j)
      if (!r.out[j]) return false;
  }
  return true;
}

// The grouped launch covers the weight gradients of a small layer: bf16
// operands, A given transposed, fp32 output (fresh or continued, the same for
// all), every problem on the small-tile path with the same k depth, so each
// would run the same kernel on its own.
bool gemm_group_ok(const GemmArgs *ps, int n, int epi) {
  if (n < 1 || n > kMaxGroup || epi != kEpiF32) return false;
  int64_t total = 0;
  for (int q = 0; q < n; ++q) {
    const GemmArgs& p = ps[q];
    const bool small = ((p.M + 127) / 128) * ((p.N + 127) / 128) < kCUs;
    if (!p.a_t || p.w_t || p.acc_init != ps[0].acc_init || p.K != ps[0].K || p.M <= 0 || p.N <= 0 || p.K <= 0 ||
        p.K % 32 != 0 || !small || !gemm_vec_ok(p, 4, false))
      return false;
    total += ((p.M + 63) / 64) * ((p.N + 63) / 64);
  }
  return total < (int64_t{1} << 31);
}

hipError_t gemm_launch_group(const GemmArgs *ps, int n, int epi, hipStream_t s) {
  if (!gemm_group_ok(ps, n, epi)) return hipErrorInvalidValue;
  const bool k64 = ps[0].K % 64 == 0;
  if (ps[0].acc_init)
    return k64 ? launch_dma_group<64, 64, 64, 2, kEpiF32Acc, true, false, 2, 2>(ps, n, s)
               : launch_dma_group<64, 64, 32, 4, kEpiF32Acc, true, false, 2, 2>(ps, n, s);
  return k64 ? launch_dma_group<64, 64, 64, 2, kEpiF32, true, false, 2, 2>(ps, n, s)
             : launch_dma_group<64, 64, 32, 4, kEpiF32, true, false, 2, 2>(ps, n, s);
}

}  // namespace tpshard
