// bf16 GEMM on the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16, fp32
// accumulation) for the dense products of the layer: the frozen-weight product
// and the batched block-diagonal products ([PX] = page "POET-X: Memory-efficient
// LLM Training by Scaling Orthogonal Transformation", Résumé technique §2.A and
// §2.C).
//
// C(m,n) = sum_k A(m,k) B(n,k). Each operand is either K-contiguous (row-major
// [rows, K]) or row-contiguous (row-major [K, rows]). Row-contiguous tiles are
// transposed in registers on their way into LDS, so the MFMA loop always reads
// 16-byte K-contiguous fragments.
//
// Work split: 4 waves (256 threads) per workgroup, each wave owns a WM x WN
// sub-tile built from 32x32 MFMA tiles. LDS holds two BM x BK and BN x BK
// stages (rows padded by 8 elements so that the 16-byte fragment reads of a
// wave hit distinct banks); the next K tile is fetched into registers while the
// current one is multiplied.
#include "poetx_internal.h"

namespace poetx {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int BK = 64;
constexpr int PAD = 8;
constexpr int LDK = BK + PAD;   // LDS row pitch in elements

template <int R, bool KMAJ>
struct TileLoader;

// K-contiguous operand: R rows x BK, 16-byte chunks along K.
template <int R>
struct TileLoader<R, true> {
  static constexpr int N = R * (BK / 8) / kThreads;
  uint4 v[N];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ base, long long ld, int row0,
                                       int rows, int k0, int kend) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = i * kThreads + threadIdx.x;
      const int r = c >> 3, kc = c & 7;
      const int gr = row0 + r, gk = k0 + kc * 8;
      if (gr < rows && gk < kend)
        v[i] = *reinterpret_cast<const uint4*>(base + (long long)gr * ld + gk);
      else
        v[i] = make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(uint16_t (*lds)[LDK]) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = i * kThreads + threadIdx.x;
      const int r = c >> 3, kc = c & 7;
      *reinterpret_cast<uint4*>(&lds[r][kc * 8]) = v[i];
    }
  }
};

// Row-contiguous operand stored [K, rows]: each thread moves 4 K-rows x 8 rows and
// writes them transposed (8 rows x 4 K) into LDS.
template <int R>
struct TileLoader<R, false> {
  static constexpr int RC = R / 8;                    // 8-row chunks per K-row
  static constexpr int N = (BK / 4) * RC / kThreads;  // sub-blocks per thread
  uint4 v[N][4];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ base, long long ld, int row0,
                                       int rows, int k0, int kend) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = i * kThreads + threadIdx.x;
      const int rc = c % RC, kg = c / RC;
      const int gr = row0 + rc * 8;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int gk = k0 + kg * 4 + q;
        if (gr < rows && gk < kend)
          v[i][q] = *reinterpret_cast<const uint4*>(base + (long long)gk * ld + gr);
        else
          v[i][q] = make_uint4(0, 0, 0, 0);
      }
    }
  }
  __device__ __forceinline__ static uint32_t half(const uint4& x, int e) {
    const uint32_t w = (e >> 1) == 0 ? x.x : (e >> 1) == 1 ? x.y : (e >> 1) == 2 ? x.z : x.w;
    return (e & 1) ? (w >> 16) : (w & 0xffffu);
  }
  __device__ __forceinline__ void store(uint16_t (*lds)[LDK]) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = i * kThreads + threadIdx.x;
      const int rc = c % RC, kg = c / RC;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint2 t;
        t.x = half(v[i][0], e) | (half(v[i][1], e) << 16);
        t.y = half(v[i][2], e) | (half(v[i][3], e) << 16);
        *reinterpret_cast<uint2*>(&lds[rc * 8 + e][kg * 4]) = t;
      }
    }
  }
};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 a = static_cast<__bf16>(lo);
  const __bf16 b = static_cast<__bf16>(hi);
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

template <int BM, int BN, int WM, int WN, bool AK, bool BKM, bool OUTF32>
__device__ __forceinline__ void gemm_body(const GemmBf16& p) {
  static_assert((BM / WM) * (BN / WN) == 4, "four waves per workgroup");
  constexpr int TM = WM / 32, TN = WN / 32;
  __shared__ __align__(16) uint16_t As[2][BM][LDK];
  __shared__ __align__(16) uint16_t Bs[2][BN][LDK];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm0 = (wave / (BN / WN)) * WM;
  const int wn0 = (wave % (BN / WN)) * WN;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const int g = blockIdx.z / p.splits, sp = blockIdx.z - g * p.splits;
  const uint16_t* A = reinterpret_cast<const uint16_t*>(p.A) + g * p.a_gs;
  const uint16_t* B = reinterpret_cast<const uint16_t*>(p.B) + g * p.b_gs;

  int kchunk = (p.K + p.splits - 1) / p.splits;
  kchunk = (kchunk + BK - 1) / BK * BK;
  const int kbeg = sp * kchunk;
  const int kend = min(p.K, kbeg + kchunk);
  const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  TileLoader<BM, AK> la;
  TileLoader<BN, BKM> lb;
  if (nk > 0) {
    la.load(A, p.lda, m0, p.M, kbeg, kend);
    lb.load(B, p.ldb, n0, p.N, kbeg, kend);
    la.store(As[0]);
    lb.store(Bs[0]);
  }
  __syncthreads();

  const int frow = lane & 31;
  const int fk = (lane >> 5) * 8;
  for (int t = 0; t < nk; ++t) {
    const int cur = t & 1;
    if (t + 1 < nk) {
      la.load(A, p.lda, m0, p.M, kbeg + (t + 1) * BK, kend);
      lb.load(B, p.ldb, n0, p.N, kbeg + (t + 1) * BK, kend);
    }
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(&As[cur][wm0 + i * 32 + frow][kk + fk]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(&Bs[cur][wn0 + j * 32 + frow][kk + fk]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          // B first: the result tile is C^T, so each lane ends up holding four
          // consecutive output columns of one output row.
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
    if (t + 1 < nk) {
      la.store(As[cur ^ 1]);
      lb.store(Bs[cur ^ 1]);
    }
    __syncthreads();
  }

  // Lane l holds C[m = .. + (l & 31)][n = .. + 8*q + 4*(l >> 5) + 0..3] in acc[.][.][4q..4q+3].
  const int cm = lane & 31;
  const int cn = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = m0 + wm0 + i * 32 + cm;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn0 + j * 32 + q * 8 + cn;
        if (n >= p.N) continue;
        const long long o = g * p.c_gs + sp * p.c_ss + (long long)m * p.ldc + n;
        if (OUTF32) {
          float4 v = make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                 acc[i][j][4 * q + 3]);
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.C) + o) = v;
        } else {
          uint2 v;
          v.x = pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
          v.y = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.C) + o) = v;
        }
      }
    }
  }
}

// One kernel symbol per role so that profiles attribute time to the stage:
//   w0_gemm_nt:    Wa = V Wt^T                  (both operands K-contiguous)
//   w0_gemm_nn:    G_V = G_Wa Wt                (Wt row-contiguous along N)
//   block_gemm_nt: out[:, blk] = in[:, blk] Q^T
//   block_gemm_nn: out[:, blk] = in[:, blk] Q
//   dq_gemm_tn:    dQ partials = G[:, blk]^T A[:, blk], reduced over tokens
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(kThreads) void w0_gemm_nt(GemmBf16 p) {
  gemm_body<BM, BN, WM, WN, true, true, false>(p);
}
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(kThreads) void w0_gemm_nn(GemmBf16 p) {
  gemm_body<BM, BN, WM, WN, true, false, false>(p);
}
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(kThreads) void block_gemm_nt(GemmBf16 p) {
  gemm_body<BM, BN, WM, WN, true, true, false>(p);
}
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(kThreads) void block_gemm_nn(GemmBf16 p) {
  gemm_body<BM, BN, WM, WN, true, false, false>(p);
}
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(kThreads) void dq_gemm_tn(GemmBf16 p) {
  gemm_body<BM, BN, WM, WN, false, false, true>(p);
}

template <int BM, int BN, int WM, int WN>
hipError_t dispatch(const GemmBf16& p, hipStream_t s) {
  dim3 grid((p.N + BN - 1) / BN, (p.M + BM - 1) / BM, p.groups * p.splits);
  const int a = p.a_kmajor, b = p.b_kmajor, f = p.out_f32;
  if (p.role == GEMM_W0 && a && b && !f)
    hipLaunchKernelGGL((w0_gemm_nt<BM, BN, WM, WN>), grid, dim3(kThreads), 0, s, p);
  else if (p.role == GEMM_W0 && a && !b && !f)
    hipLaunchKernelGGL((w0_gemm_nn<BM, BN, WM, WN>), grid, dim3(kThreads), 0, s, p);
  else if (p.role == GEMM_BLOCK && a && b && !f)
    hipLaunchKernelGGL((block_gemm_nt<BM, BN, WM, WN>), grid, dim3(kThreads), 0, s, p);
  else if (p.role == GEMM_BLOCK && a && !b && !f)
    hipLaunchKernelGGL((block_gemm_nn<BM, BN, WM, WN>), grid, dim3(kThreads), 0, s, p);
  else if (p.role == GEMM_DQ && !a && !b && f)
    hipLaunchKernelGGL((dq_gemm_tn<BM, BN, WM, WN>), grid, dim3(kThreads), 0, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmBf16& p, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0 || p.groups <= 0) return hipSuccess;
  if (block_regb_supported(p)) return launch_block_regb(p, s);
  const long long big_tiles = (long long)((p.M + 255) / 256) * ((p.N + 255) / 256) * p.groups * p.splits;
  // the token reduction (dQ) takes its tile size from dq_big_tiles, which its
  // split count was sized for
  const bool big = p.role == GEMM_DQ
                       ? (p.M == p.N && dq_big_tiles(p.M, p.groups, p.K) && gemm_lds_supported(p, 256, 256))
                       : big_tiles >= 256;
  // whole-tile shapes take the pipelined direct-to-LDS kernels; the rest (K not a
  // multiple of 64, partial tiles of row-contiguous operands) the kernels here
  if (big && w0_pipe_supported(p)) return launch_w0_pipe(p, s);
  if (gemm_lds_supported(p, big ? 256 : 128, big ? 256 : 128)) return launch_gemm_lds(p, big, s);
  // a column scale is applied by a separate pass here (one more rounding of
  // the bf16 output)
  if (p.col_scale && (p.out_f32 || p.c_gs != p.N)) return hipErrorInvalidValue;
  const hipError_t e = big ? dispatch<256, 256, 128, 128>(p, s) : dispatch<128, 128, 64, 64>(p, s);
  if (e != hipSuccess || !p.col_scale) return e;
  return launch_scale_cols(p.C, p.col_scale, p.M, p.N * p.groups, p.ldc, s);
}

}  // namespace poetx
