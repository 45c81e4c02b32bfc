// Dense GEMMs of the column->row MLP on gfx950.
//
//   C[M,N] = act(A[M,K] * W[K,N])      A row-major (K contiguous, row stride lda)
//                                      W row-major (N contiguous, row stride ldw)
//
// GEMM1 of the MLP is X * A_i followed by GeLU, stored as bf16 ([CAI] section
// 2, column-parallel linear; [DOM] "GeMM GeLU GeMM"); GEMM2 is Y * B_i stored
// as the fp32 partial ([CAI] section 2.1, row-parallel linear).
//
// bf16 path: v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  A workgroup of
// 4 waves (2 x 2) owns a BM x BN output tile; K advances 64 at a time through
// a double-buffered LDS stage.  Both operands sit in LDS K-contiguous (the W
// tile is transposed in registers, 8x8 bf16 at a time, on its way from global
// memory), so each lane reads its MFMA operand with one 16-byte LDS load.  An
// XOR swizzle of the 16-byte chunks keeps those loads and the stores free of
// bank conflicts.  The MFMA gets W as its first operand and A as its second,
// which hands every lane one output row and four adjacent output columns, so
// the epilogue writes 16 bytes (fp32) or 8 bytes (bf16) per lane.
//
// Every output element is accumulated over k in the same order (64-wide
// stages, ascending) whatever the tile shape, so results do not depend on the
// tile configuration or on how the caller chunks M and N.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gemm.h"

namespace tpshard {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;

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

// GeLU(x) = x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)) in fp32.
__device__ __forceinline__ float gelu_erf(float x) {
  return 0.5f * x * (1.0f + erf_as7126(x * 0.70710678118654752440f));
}

// fp32 -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (u >> 16) | 0x0040u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return bf16_bits_rne(lo) | (bf16_bits_rne(hi) << 16);
}

// ---- LDS addressing ----------------------------------------------------
// Each operand tile row holds 64 bf16 = 128 bytes = 8 chunks of 16 bytes.
// Chunk c of row r lives at chunk position c ^ swz(r).

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

// ---- the bf16 MFMA kernel ----------------------------------------------

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
          const uint32_t lo = (gm < p.M && k < p.K) ? A[gm * p.lda + k] : 0u;
          const uint32_t hi = (gm < p.M && k + 1 < p.K) ? A[gm * p.lda + k + 1] : 0u;
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
          const uint32_t lo = (gk < p.K && n < p.N) ? W[gk * p.ldw + n] : 0u;
          const uint32_t hi = (gk < p.K && n + 1 < p.N) ? W[gk * p.ldw + n + 1] : 0u;
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

  __device__ __forceinline__ static void epilogue(const GemmArgs& p, int m0, int n0, const f32x4_t (&acc)[TM][TN]) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t m = m0 + wm * WM + i * 16 + (lane & 15);
      if (m >= p.M) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t n = n0 + wn * WN + j * 16 + 4 * (lane >> 4);
        f32x4_t v = acc[i][j];
        if constexpr (EPI == kEpiGeluBf16) {
          v = f32x4_t{gelu_erf(v[0]), gelu_erf(v[1]), gelu_erf(v[2]), gelu_erf(v[3])};
        }
        if constexpr (EPI == kEpiF32) {
          float *C = static_cast<float *>(p.c) + m * p.ldc + n;
          if (VEC && n + 3 < p.N) {
            *reinterpret_cast<f32x4_t *>(C) = v;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < p.N) C[e] = v[e];
          }
        } else {
          uint16_t *C = static_cast<uint16_t *>(p.c) + m * p.ldc + n;
          if (VEC && n + 3 < p.N) {
            *reinterpret_cast<u32x2_t *>(C) = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < p.N) C[e] = static_cast<uint16_t>(bf16_bits_rne(v[e]));
          }
        }
      }
    }
  }
};

template <int BM, int BN, bool VEC, int EPI>
__global__ void __launch_bounds__(kThreads, 1) bf16_gemm_kernel(GemmArgs p) {
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
    for (int j = 0; j < G::TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

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

// ---- plain fp32 kernel (tiny fp32 workload) ------------------------------
// 64 x 64 tile, 256 threads of 4 x 4 outputs, K staged 16 at a time.

constexpr int kF32Tile = 64;
constexpr int kF32BK = 16;

template <int EPI>
__global__ void __launch_bounds__(kThreads) f32_gemm_kernel(GemmArgs p) {
  __shared__ float As[kF32BK][kF32Tile + 4];
  __shared__ float Ws[kF32BK][kF32Tile + 4];
  const float *A = static_cast<const float *>(p.a);
  const float *W = static_cast<const float *>(p.w);
  const int tiles_n = static_cast<int>((p.N + kF32Tile - 1) / kF32Tile);
  const int64_t m0 = static_cast<int64_t>(blockIdx.x / tiles_n) * kF32Tile;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x % tiles_n) * kF32Tile;
  const int t = threadIdx.x;
  const int tr = t / 16, tc = t % 16;
  float acc[4][4] = {};
  for (int64_t k0 = 0; k0 < p.K; k0 += kF32BK) {
    for (int e = t; e < kF32BK * kF32Tile; e += kThreads) {
      const int r = e / kF32BK, k = e % kF32BK;      // A element (row r, k)
      As[k][r] = (m0 + r < p.M && k0 + k < p.K) ? A[(m0 + r) * p.lda + k0 + k] : 0.f;
      const int kk = e / kF32Tile, n = e % kF32Tile;  // W element (k, col n)
      Ws[kk][n] = (k0 + kk < p.K && n0 + n < p.N) ? W[(k0 + kk) * p.ldw + n0 + n] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kF32BK; ++k) {
      float a[4], w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[k][tr * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = Ws[k][tc * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], w[j], acc[i][j]);
    }
    __syncthreads();
  }
  float *C = static_cast<float *>(p.c);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + tr * 4 + i;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + tc * 4 + j;
      if (n < p.N) C[m * p.ldc + n] = (EPI == kEpiGeluF32) ? gelu_erf(acc[i][j]) : acc[i][j];
    }
  }
}

template <int BM, int BN, bool VEC, int EPI>
hipError_t launch_bf16(const GemmArgs& p, hipStream_t s) {
  const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  hipLaunchKernelGGL((bf16_gemm_kernel<BM, BN, VEC, EPI>), dim3(static_cast<unsigned>(tiles)), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <int EPI>
hipError_t dispatch_bf16(const GemmArgs& p, bool vec, hipStream_t s) {
  // Shapes that break 16-byte alignment take the element-wise loader, on the
  // small tile only (they are rare, and it keeps register pressure low).
  if (!vec) return launch_bf16<128, 128, false, EPI>(p, s);
  // Pick the largest tile that still gives at least one workgroup per CU;
  // fall back to the smallest tile for small problems.
  const int64_t t256x256 = ((p.M + 255) / 256) * ((p.N + 255) / 256);
  const int64_t t256x128 = ((p.M + 255) / 256) * ((p.N + 127) / 128);
  if (t256x256 >= 256) return launch_bf16<256, 256, true, EPI>(p, s);
  if (t256x128 >= 256) return launch_bf16<256, 128, true, EPI>(p, s);
  return launch_bf16<128, 128, true, EPI>(p, s);
}

}  // namespace

bool gemm_vec_ok(const GemmArgs& p, int64_t esize) {
  auto al = [](const void *q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
  const int64_t per16 = 16 / esize;
  return al(p.a) && al(p.w) && (p.K % 8 == 0) && (p.N % 8 == 0) && (p.lda % 8 == 0) && (p.ldw % 8 == 0) &&
         (p.ldc % per16 == 0) && al(p.c);
}

hipError_t gemm_launch(const GemmArgs& p, int epi, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  if (epi == kEpiF32 || epi == kEpiGeluBf16) {
    // the output store width of the vector path is 16 bytes (fp32) or 8 bytes (bf16)
    const bool vec = gemm_vec_ok(p, epi == kEpiF32 ? 4 : 2);
    if (epi == kEpiF32) return dispatch_bf16<kEpiF32>(p, vec, s);
    return dispatch_bf16<kEpiGeluBf16>(p, vec, s);
  }
  if (epi == kEpiIdentBf16) return dispatch_bf16<kEpiIdentBf16>(p, gemm_vec_ok(p, 2), s);
  const int64_t tiles = ((p.M + kF32Tile - 1) / kF32Tile) * ((p.N + kF32Tile - 1) / kF32Tile);
  const dim3 grid(static_cast<unsigned>(tiles));
  if (epi == kEpiGeluF32)
    hipLaunchKernelGGL((f32_gemm_kernel<kEpiGeluF32>), grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((f32_gemm_kernel<kEpiPlainF32>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace tpshard
