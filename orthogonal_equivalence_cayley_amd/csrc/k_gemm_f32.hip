// fp32 batched GEMM with general element strides. It serves the fp32 layer
// mode end to end and the b x b power chains of the Cayley-Neumann build and its
// backward, where every product must keep fp32 accuracy.
//
// C(m,n) = alpha * sum_k A(m,k) B(n,k) + beta * Cin(m,n) + gamma * [m == n]
// E(m,n) = sum_k A(m,k) B(n,k)                        (optional second output)
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

}  // namespace

hipError_t launch_gemm_f32(const GemmF32& p, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0 || p.groups <= 0) return hipSuccess;
  dim3 grid((p.N + BN - 1) / BN, (p.M + BM - 1) / BM, p.groups * p.splits);
  hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace poetx
