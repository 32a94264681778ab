// fp32 batched GEMM with general element strides. It serves the fp32 layer
// mode end to end, the exact Cayley transform, the merge, and the b x b power
// chains of block sizes the fused chain kernel does not take, where every
// product must keep fp32 accuracy.
//
// C(m,n) = alpha * sum_k A(m,k) B(n,k) + beta * Cin(m,n) + gamma * [m == n]
// E(m,n) = sum_k A(m,k) B(n,k)                        (optional second output)
#include <algorithm>

#include "poetx_internal.h"

namespace poetx {
namespace {

constexpr int BM = 64, BN = 64, BK = 16, kThreads = 256;

__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(GemmF32 p) {
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const int g = blockIdx.z / p.splits, sp = blockIdx.z - g * p.splits;
  if (p.iters && p.iters[g] <= p.it) return;
  const float* A = p.A + g * p.a_gs;
  const float* B = p.B + g * p.b_gs;

  int kchunk = (p.K + p.splits - 1) / p.splits;
  kchunk = (kchunk + BK - 1) / BK * BK;
  const int kbeg = sp * kchunk;
  const int kend = min(p.K, kbeg + kchunk);

  float acc[4][4] = {};
  const bool a_kc = (p.a_cs == 1);
  const bool b_kc = (p.b_cs == 1);
  for (int k0 = kbeg; k0 < kend; k0 += BK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + i * kThreads;
      int mm, kk;
      if (a_kc) { mm = e / BK; kk = e % BK; } else { mm = e % BM; kk = e / BM; }
      const int gm = m0 + mm, gk = k0 + kk;
      As[kk][mm] = (gm < p.M && gk < kend) ? A[gm * p.a_rs + gk * p.a_cs] : 0.0f;
      int nn, kb;
      if (b_kc) { nn = e / BK; kb = e % BK; } else { nn = e % BN; kb = e / BN; }
      const int gn = n0 + nn, gkb = k0 + kb;
      Bs[kb][nn] = (gn < p.N && gkb < kend) ? B[gn * p.b_rs + gkb * p.b_cs] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }

  float* C = p.C + g * p.c_gs + sp * p.c_ss;
  const float* Cin = p.Cin ? p.Cin + g * p.c_gs : nullptr;
  float* E = p.E ? p.E + g * p.c_gs : nullptr;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty + 16 * i;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx + 16 * j;
      if (n >= p.N) continue;
      const long long o = (long long)m * p.c_rs + n;
      float v = p.alpha * acc[i][j];
      if (p.splits == 1) {
        if (Cin) v += p.beta * Cin[o];
        if (m == n) v += p.gamma;
        if (E) E[o] = acc[i][j];
      }
      C[o] = v;
    }
  }
}

// The same product on the fp32 matrix cores (v_mfma_f32_16x16x4_f32, fp32
// inputs and accumulation) for operands with a unit stride along K or along
// their rows: MB x MB tiles (64, or 32 when the grid would not fill the chip),
// 32-deep K steps staged in LDS, 4 waves each owning MB/32 x MB/32 tiles of
// 16 x 16. The loads run along the operand's contiguous dimension.
constexpr int MK = 32;

// gz: group and split of this workgroup (g * splits + split)
template <bool AKC, bool BKC, int MB>
__device__ __forceinline__ void gemm_f32_mfma_body(const GemmF32& p, int gz) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  constexpr int MPAD = MB + 4, TW = MB / 32;   // 16 x 16 tiles per wave and dimension
  __shared__ float As[MK][MPAD];
  __shared__ float Bs[MK][MPAD];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int n0 = blockIdx.x * MB, m0 = blockIdx.y * MB;
  if (n0 >= p.N || m0 >= p.M) return;
  const int g = gz / p.splits, sp = gz - g * p.splits;
  if (p.iters && p.iters[g] <= p.it) return;
  const float* A = p.A + g * p.a_gs;
  const float* B = p.B + g * p.b_gs;
  int kchunk = (p.K + p.splits - 1) / p.splits;
  kchunk = (kchunk + MK - 1) / MK * MK;
  const int kbeg = sp * kchunk;
  const int kend = min(p.K, kbeg + kchunk);

  f32x4 acc[TW][TW];
#pragma unroll
  for (int i = 0; i < TW; ++i)
#pragma unroll
    for (int j = 0; j < TW; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const int li = lane & 15, lq = lane >> 4;
  // MB x MK elements per operand and K step, PER per thread, consecutive threads
  // along the contiguous dimension; the next step's values are loaded into
  // registers while the current step is multiplied
  constexpr int PER = MB * MK / kThreads;
  float ra[PER], rb[PER];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + i * kThreads;
      int mm, kk;
      if (AKC) { kk = e % MK; mm = e / MK; } else { mm = e % MB; kk = e / MB; }
      const int gm = m0 + mm, gk = k0 + kk;
      ra[i] = (gm < p.M && gk < kend) ? A[gm * p.a_rs + gk * p.a_cs] : 0.0f;
      int nn, kb;
      if (BKC) { kb = e % MK; nn = e / MK; } else { nn = e % MB; kb = e / MB; }
      const int gn = n0 + nn, gkb = k0 + kb;
      rb[i] = (gn < p.N && gkb < kend) ? B[gn * p.b_rs + gkb * p.b_cs] : 0.0f;
    }
  };
  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + i * kThreads;
      int mm, kk;
      if (AKC) { kk = e % MK; mm = e / MK; } else { mm = e % MB; kk = e / MB; }
      As[kk][mm] = ra[i];
      int nn, kb;
      if (BKC) { kb = e % MK; nn = e / MK; } else { nn = e % MB; kb = e / MB; }
      Bs[kb][nn] = rb[i];
    }
  };
  if (kbeg < kend) load(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += MK) {
    store();
    __syncthreads();
    if (k0 + MK < kend) load(k0 + MK);
#pragma unroll
    for (int kq = 0; kq < MK / 4; ++kq) {
      const int k = 4 * kq + lq;
      float a[TW], b[TW];
#pragma unroll
      for (int t = 0; t < TW; ++t) {
        a[t] = As[k][16 * TW * wr + 16 * t + li];
        b[t] = Bs[k][16 * TW * wc + 16 * t + li];
      }
#pragma unroll
      for (int i = 0; i < TW; ++i)
#pragma unroll
        for (int j = 0; j < TW; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

  // lane l holds rows 4 (l / 16) + r (r = 0..3) of column l % 16 of each 16 x 16 tile
  float* C = p.C + g * p.c_gs + sp * p.c_ss;
  const float* Cin = p.Cin ? p.Cin + g * p.c_gs : nullptr;
  float* E = p.E ? p.E + g * p.c_gs : nullptr;
#pragma unroll
  for (int i = 0; i < TW; ++i)
#pragma unroll
    for (int j = 0; j < TW; ++j) {
      const int n = n0 + 16 * TW * wc + 16 * j + li;
      if (n >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 16 * TW * wr + 16 * i + 4 * lq + r;
        if (m >= p.M) continue;
        const long long o = (long long)m * p.c_rs + n;
        const float x = acc[i][j][r];
        float v = p.alpha * x;
        if (p.splits == 1) {
          if (Cin) v += p.beta * Cin[o];
          if (m == n) v += p.gamma;
          if (E) E[o] = x;
        }
        C[o] = v;
      }
    }
}

template <bool AKC, bool BKC, int MB>
__global__ __launch_bounds__(kThreads) void gemm_f32_mfma_kernel(GemmF32 p) {
  gemm_f32_mfma_body<AKC, BKC, MB>(p, blockIdx.z);
}

// Several runs of the same shape and strides in one launch: blockIdx.z walks
// the groups of run 0, then of run 1, ...
template <bool AKC, bool BKC, int MB>
__global__ __launch_bounds__(kThreads) void gemm_f32_mfma_runs_kernel(GemmF32Runs rr) {
  int r = 0;
#pragma unroll
  for (int i = 1; i < kF32MaxRuns; ++i)
    if (i < rr.n && (int)blockIdx.z >= rr.z0[i]) r = i;
  GemmF32 p = rr.p;
  p.A = rr.r[r].A; p.B = rr.r[r].B; p.C = rr.r[r].C; p.Cin = rr.r[r].Cin; p.E = nullptr;
  p.groups = rr.r[r].groups;
  p.iters = rr.r[r].iters;
  gemm_f32_mfma_body<AKC, BKC, MB>(p, blockIdx.z - rr.z0[r]);
}

template <int MB>
hipError_t launch_mfma(const GemmF32& p, bool akc, bool bkc, hipStream_t s) {
  dim3 grid((p.N + MB - 1) / MB, (p.M + MB - 1) / MB, p.groups * p.splits);
  if (akc && bkc) hipLaunchKernelGGL((gemm_f32_mfma_kernel<true, true, MB>), grid, dim3(kThreads), 0, s, p);
  else if (akc) hipLaunchKernelGGL((gemm_f32_mfma_kernel<true, false, MB>), grid, dim3(kThreads), 0, s, p);
  else if (bkc) hipLaunchKernelGGL((gemm_f32_mfma_kernel<false, true, MB>), grid, dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL((gemm_f32_mfma_kernel<false, false, MB>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_f32(const GemmF32& p, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0 || p.groups <= 0) return hipSuccess;
  const bool akc = p.a_cs == 1, arc = p.a_rs == 1;
  const bool bkc = p.b_cs == 1, brc = p.b_rs == 1;
  if ((akc || arc) && (bkc || brc)) {
    const long long g64 = (long long)((p.N + 63) / 64) * ((p.M + 63) / 64) * p.groups * p.splits;
    if (g64 >= 512) return launch_mfma<64>(p, akc, bkc, s);
    return launch_mfma<32>(p, akc, bkc, s);
  }
  dim3 grid((p.N + BN - 1) / BN, (p.M + BM - 1) / BM, p.groups * p.splits);
  hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gemm_f32_runs(const GemmF32& shape, const GemmF32Run* runs, int n, hipStream_t s) {
  const bool akc = shape.a_cs == 1, arc = shape.a_rs == 1;
  const bool bkc = shape.b_cs == 1, brc = shape.b_rs == 1;
  if (shape.M <= 0 || shape.N <= 0 || shape.splits != 1) return hipErrorInvalidValue;
  if (!((akc || arc) && (bkc || brc))) {   // one launch per run on the generic kernel
    for (int i = 0; i < n; ++i) {
      GemmF32 p = shape;
      p.A = runs[i].A; p.B = runs[i].B; p.C = runs[i].C; p.Cin = runs[i].Cin; p.E = nullptr;
      p.groups = runs[i].groups;
      p.iters = runs[i].iters;
      const hipError_t e = launch_gemm_f32(p, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  for (int i0 = 0; i0 < n; i0 += kF32MaxRuns) {
    GemmF32Runs rr{};
    rr.p = shape;
    rr.n = std::min(kF32MaxRuns, n - i0);
    int z = 0;
    for (int i = 0; i < rr.n; ++i) {
      rr.r[i] = runs[i0 + i];
      rr.z0[i] = z;
      z += runs[i0 + i].groups;
    }
    if (z == 0) continue;
    const long long g64 = (long long)((shape.N + 63) / 64) * ((shape.M + 63) / 64) * z;
    const bool big = g64 >= 512;
    const int mb = big ? 64 : 32;
    dim3 grid((shape.N + mb - 1) / mb, (shape.M + mb - 1) / mb, z);
#define POETX_F32_RUNS(MBV)                                                                              \
  if (akc && bkc) hipLaunchKernelGGL((gemm_f32_mfma_runs_kernel<true, true, MBV>), grid, dim3(kThreads), 0, s, rr); \
  else if (akc) hipLaunchKernelGGL((gemm_f32_mfma_runs_kernel<true, false, MBV>), grid, dim3(kThreads), 0, s, rr); \
  else if (bkc) hipLaunchKernelGGL((gemm_f32_mfma_runs_kernel<false, true, MBV>), grid, dim3(kThreads), 0, s, rr); \
  else hipLaunchKernelGGL((gemm_f32_mfma_runs_kernel<false, false, MBV>), grid, dim3(kThreads), 0, s, rr);
    if (big) { POETX_F32_RUNS(64) } else { POETX_F32_RUNS(32) }
#undef POETX_F32_RUNS
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace poetx
