// INT8 storage of the frozen weight (POET-XQ, [PX] = page "POET-X:
// Memory-efficient LLM Training by Scaling Orthogonal Transformation", Résumé
// technique §2.E "Quantification": the base weights are kept in INT8 and
// dequantised on the fly).
//
// One workgroup per row of the pre-merged weight: row i of Wt is row pi_R[i]
// of W0 with its columns gathered by pi_P, so the row is staged in LDS with
// coalesced loads and its maximum magnitude found there (a row's maximum does
// not depend on the column order). Then, in fp32 with round-to-nearest-even:
//   inv = 127 / amax,  q = clamp(rint(w * inv), -127, 127),  s = amax / 127,
// and amax = 0 gives q = 0, s = 0. Division is the correctly rounded one.
#include "poetx_internal.h"

namespace poetx {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

__global__ __launch_bounds__(kThreads) void quantize_rows_kernel(const uint16_t* __restrict__ W0,
                                                                 const int32_t* __restrict__ pi_R,
                                                                 const int32_t* __restrict__ pi_P,
                                                                 int8_t* __restrict__ q,
                                                                 float* __restrict__ scale, int n) {
  extern __shared__ __align__(16) uint16_t row[];
  __shared__ float red[kThreads / 64];
  const int i = blockIdx.x;
  const uint16_t* src = W0 + (long long)pi_R[i] * n;
  float amax = 0.0f;
  for (int c = threadIdx.x * 8; c < n; c += kThreads * 8) {   // n % 8 == 0
    const uint4 v = *reinterpret_cast<const uint4*>(src + c);
    *reinterpret_cast<uint4*>(row + c) = v;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      amax = fmaxf(amax, fabsf(bf16_to_f32(w[e] & 0xffffu)));
      amax = fmaxf(amax, fabsf(bf16_to_f32(w[e] >> 16)));
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) amax = fmaxf(amax, red[w]);
  const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
  if (threadIdx.x == 0) scale[i] = amax > 0.0f ? amax / 127.0f : 0.0f;
  int8_t* dst = q + (long long)i * n;
  for (int c = threadIdx.x * 4; c < n; c += kThreads * 4) {   // n % 4 == 0
    uint32_t packed = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = bf16_to_f32(row[pi_P[c + e]]) * inv;
      const float r = fminf(fmaxf(rintf(v), -127.0f), 127.0f);
      packed |= (static_cast<uint32_t>(static_cast<int32_t>(r)) & 0xffu) << (8 * e);
    }
    *reinterpret_cast<uint32_t*>(dst + c) = packed;
  }
}

// out[i][j] = s[i] * q[i][j] in fp32 (exact: an int8 times an fp32)
__global__ __launch_bounds__(kThreads) void dequantize_rows_kernel(const int8_t* __restrict__ q,
                                                                   const float* __restrict__ scale,
                                                                   float* __restrict__ out, int n) {
  const int i = blockIdx.x;
  const float s = scale[i];
  for (int c = threadIdx.x; c < n; c += kThreads)
    out[(long long)i * n + c] = s * static_cast<float>(q[(long long)i * n + c]);
}

// out[e] = bf16(q[e]) for n elements (exact: every int8 is a bf16), 16 per
// thread and step with 16-byte loads where n allows it
__global__ __launch_bounds__(kThreads) void widen_i8_kernel(const int8_t* __restrict__ q,
                                                            uint16_t* __restrict__ out, long long n) {
  const long long n16 = n / 16;
  for (long long v = (long long)blockIdx.x * kThreads + threadIdx.x; v < n16;
       v += (long long)gridDim.x * kThreads) {
    const uint4 x = reinterpret_cast<const uint4*>(q)[v];
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t word = w[i / 2] >> (16 * (i & 1));
      const __bf16 lo = static_cast<__bf16>(static_cast<float>(static_cast<int8_t>(word & 0xff)));
      const __bf16 hi = static_cast<__bf16>(static_cast<float>(static_cast<int8_t>((word >> 8) & 0xff)));
      o[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    uint4* dst = reinterpret_cast<uint4*>(out) + 2 * v;
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
  }
  for (long long e = n16 * 16 + (long long)blockIdx.x * kThreads + threadIdx.x; e < n;
       e += (long long)gridDim.x * kThreads)
    out[e] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(static_cast<float>(q[e])));
}

// C[t][c] = bf16(float(C[t][c]) * scale[c]) for t < rows, c < cols (row stride ld)
__global__ __launch_bounds__(kThreads) void scale_cols_kernel(uint16_t* __restrict__ C,
                                                              const float* __restrict__ scale,
                                                              long long rows, int cols, long long ld) {
  const long long total = rows * cols;
  for (long long e = (long long)blockIdx.x * kThreads + threadIdx.x; e < total;
       e += (long long)gridDim.x * kThreads) {
    const long long t = e / cols;
    const int c = (int)(e - t * cols);
    uint16_t* x = C + t * ld + c;
    const __bf16 v = static_cast<__bf16>(bf16_to_f32(*x) * scale[c]);
    *x = __builtin_bit_cast(uint16_t, v);
  }
}

}  // namespace

hipError_t launch_scale_cols(void* C, const float* scale, long long rows, int cols, long long ld,
                             hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  long long blocks = (rows * cols + kThreads - 1) / kThreads;
  if (blocks > 256LL * 64) blocks = 256LL * 64;
  hipLaunchKernelGGL(scale_cols_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                     static_cast<uint16_t*>(C), scale, rows, cols, ld);
  return hipGetLastError();
}

hipError_t launch_quantize_rows(const void* W0, const int32_t* pi_R, const int32_t* pi_P,
                                int8_t* q, float* scale, int m, int n, hipStream_t s) {
  if (m <= 0) return hipSuccess;
  if (n % 8 || (size_t)n * 2 > 64 * 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(quantize_rows_kernel, dim3(m), dim3(kThreads), (size_t)n * 2, s,
                     static_cast<const uint16_t*>(W0), pi_R, pi_P, q, scale, n);
  return hipGetLastError();
}

hipError_t launch_widen_i8(const void* q, void* out, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (((uintptr_t)q & 15) || ((uintptr_t)out & 15)) return hipErrorInvalidValue;
  long long blocks = (n / 16 + kThreads - 1) / kThreads;
  if (blocks < 1) blocks = 1;
  if (blocks > 256LL * 16) blocks = 256LL * 16;
  hipLaunchKernelGGL(widen_i8_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                     static_cast<const int8_t*>(q), static_cast<uint16_t*>(out), n);
  return hipGetLastError();
}

hipError_t launch_dequantize_rows(const int8_t* q, const float* scale, float* out, int m, int n,
                                  hipStream_t s) {
  if (m <= 0) return hipSuccess;
  hipLaunchKernelGGL(dequantize_rows_kernel, dim3(m), dim3(kThreads), 0, s, q, scale, out, n);
  return hipGetLastError();
}

}  // namespace poetx
