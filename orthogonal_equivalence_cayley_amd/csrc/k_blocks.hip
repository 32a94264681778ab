// Elementwise kernels on the per-block arrays of the Cayley-Neumann
// parameterisation ([PX] = page "POET-X: Memory-efficient LLM Training by
// Scaling Orthogonal Transformation", Résumé technique §2.D): unpack of the
// stored upper triangle into the skew generator, packing of the parameter
// gradient, dtype casts and the fixed-order split-K reduction.
#include "poetx_internal.h"

namespace poetx {
namespace {

constexpr int kThreads = 256;

inline int grid1d(long long n) {
  long long g = (n + kThreads - 1) / kThreads;
  const long long cap = 256LL * 32;
  return (int)(g < 1 ? 1 : (g > cap ? cap : g));
}

// Offset of (i, j), i < j, in the row-major strict upper triangle of a b x b block.
__device__ __forceinline__ long long tri_index(int i, int j, int b) {
  return (long long)i * b - ((long long)i * (i + 1)) / 2 + (j - i - 1);
}

__global__ __launch_bounds__(kThreads) void unpack_skew_kernel(
    const float* __restrict__ theta, int b, int count, long long q_off, long long p_off,
    float* __restrict__ S, float* __restrict__ Q, float c1) {
  const long long bb = (long long)b * b;
  const long long np = (long long)b * (b - 1) / 2;
  const long long total = bb * count;
  for (long long e = (long long)blockIdx.x * kThreads + threadIdx.x; e < total;
       e += (long long)gridDim.x * kThreads) {
    const long long g = e / bb;
    const int r = (int)((e - g * bb) / b);
    const int c = (int)(e - g * bb - (long long)r * b);
    const float* th = theta + p_off + g * np;
    float v = 0.0f;
    if (r < c) v = th[tri_index(r, c, b)];
    else if (r > c) v = -th[tri_index(c, r, b)];
    S[q_off + e] = v;
    if (Q) Q[q_off + e] = (r == c ? 1.0f : 0.0f) + c1 * v;
  }
}

// Newton-Schulz start for N = (I - S)^{-1}: with c an upper bound of ||S||_2,
// the smaller of max_i sum_j |S[i][j]| and, when S2 = S S is given, the square
// root of max_i sum_j |S2[i][j]| (S2 is symmetric and ||S2||_2 = ||S||_2^2, so
// its largest row sum bounds ||S||_2^2; for generators of many small entries it
// is the much tighter bound), X0 = a (I + S) = a (I - S)^T with a = 2 / (2 + c^2).
// The residual R = I - (I - S) X0 is symmetric with eigenvalues 1 - a (1 + s^2)
// for the singular values s <= c of S, so ||R||_2 <= r = c^2 / (2 + c^2) < 1,
// and after j steps X <- X (2I - (I - S) X) it is R^(2^j). iters[block] = the
// least j with r^(2^j) <= 2^-30 (0 when S = 0), at most jmax.
//
// kNsParts workgroups per block: each finds c for the whole block (one thread
// per row, each row summed in column order, 16-byte loads where the rows allow
// them; the block is read from L2 by all but the first), then writes its share
// of the rows of X0; the first also writes iters.
constexpr int kNsParts = 8;
// largest row sum of |M| over the b x b block M (every thread of the workgroup)
__device__ float max_abs_row_sum(const float* __restrict__ M, int b, float* red) {
  const bool vec = (b % 4) == 0;   // then every row starts on a 16-byte boundary
  float mx = 0.0f;
  for (int r = threadIdx.x; r < b; r += kThreads) {
    const float* row = M + (long long)r * b;
    float sum = 0.0f;
    if (vec) {
      for (int c = 0; c < b; c += 4) {
        const float4 v = *reinterpret_cast<const float4*>(row + c);
        sum += fabsf(v.x);
        sum += fabsf(v.y);
        sum += fabsf(v.z);
        sum += fabsf(v.w);
      }
    } else {
      for (int c = 0; c < b; ++c) sum += fabsf(row[c]);
    }
    mx = fmaxf(mx, sum);
  }
  red[threadIdx.x] = mx;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  const float m = red[0];
  __syncthreads();   // red is reused by the next call
  return m;
}
__global__ __launch_bounds__(kThreads) void ns_init_kernel(const float* __restrict__ S,
                                                           const float* __restrict__ S2, int b,
                                                           float* __restrict__ X0,
                                                           int32_t* __restrict__ iters, int jmax) {
  __shared__ float red[kThreads];
  const int blk = blockIdx.x / kNsParts, part = blockIdx.x - blk * kNsParts;
  const long long bb = (long long)b * b;
  const float* Sg = S + blk * bb;
  float* Xg = X0 + blk * bb;
  double c = max_abs_row_sum(Sg, b, red);
  if (S2) c = fmin(c, sqrt((double)max_abs_row_sum(S2 + blk * bb, b, red)));
  const float a = (float)(2.0 / (2.0 + c * c));
  const int r0 = (int)((long long)b * part / kNsParts), r1 = (int)((long long)b * (part + 1) / kNsParts);
  for (long long e = (long long)r0 * b + threadIdx.x; e < (long long)r1 * b; e += kThreads) {
    const int r = (int)(e / b), col = (int)(e - (long long)r * b);
    Xg[e] = a * ((r == col ? 1.0f : 0.0f) + Sg[e]);
  }
  if (part == 0 && threadIdx.x == 0) {
    int j = 0;
    if (c > 0.0) {
      const double rho = c * c / (2.0 + c * c);
      // rho^(2^j) <= 2^-30  <=>  2^j >= 30 ln 2 / (-ln rho)
      const double need = 30.0 * 0.6931471805599453 / -log(rho);
      while (j < jmax && ldexp(1.0, j) < need) ++j;
    }
    iters[blk] = j;
  }
}

// After the iterations, block g's N sits in X0 for an even iteration count and
// in X1 for an odd one: N_out = N and Q = (I + S)(I - S)^{-1} = 2 N - I.
// Elementwise over all blocks of the run.
__global__ __launch_bounds__(kThreads) void ns_final_kernel(const float* __restrict__ X0,
                                                            const float* __restrict__ X1,
                                                            const int32_t* __restrict__ iters,
                                                            int b, long long total,
                                                            float* __restrict__ N,
                                                            float* __restrict__ Q) {
  const long long bb = (long long)b * b;
  for (long long e = (long long)blockIdx.x * kThreads + threadIdx.x; e < total;
       e += (long long)gridDim.x * kThreads) {
    const long long g = e / bb;
    const long long w = e - g * bb;
    const int r = (int)(w / b), col = (int)(w - (long long)r * b);
    const float v = ((iters[g] & 1) ? X1 : X0)[e];
    N[e] = v;
    Q[e] = 2.0f * v - (r == col ? 1.0f : 0.0f);
  }
}

__global__ __launch_bounds__(kThreads) void lincomb_kernel(LinComb lc, float* out, int b,
                                                           long long total) {
  const long long bb = (long long)b * b;
  for (long long e = (long long)blockIdx.x * kThreads + threadIdx.x; e < total;
       e += (long long)gridDim.x * kThreads) {
    const long long w = e % bb;
    const int r = (int)(w / b), c = (int)(w - (long long)r * b);
    float v = r == c ? lc.diag : 0.0f;
#pragma unroll
    for (int i = 0; i < kLinCombMax; ++i)
      if (i < lc.n) v += lc.coef[i] * lc.mats[i][e];
    out[e] = v;
  }
}

__global__ __launch_bounds__(kThreads) void pack_antisym_kernel(
    const float* __restrict__ Sbar, int b, int count, long long q_off, long long p_off,
    float sign, float* __restrict__ g) {
  const long long bb = (long long)b * b;
  const long long np = (long long)b * (b - 1) / 2;
  const long long total = bb * count;
  for (long long e = (long long)blockIdx.x * kThreads + threadIdx.x; e < total;
       e += (long long)gridDim.x * kThreads) {
    const long long blk = e / bb;
    const int r = (int)((e - blk * bb) / b);
    const int c = (int)(e - blk * bb - (long long)r * b);
    if (r < c) {
      const float* M = Sbar + q_off + blk * bb;
      g[p_off + blk * np + tri_index(r, c, b)] =
          sign * (M[(long long)r * b + c] - M[(long long)c * b + r]);
    }
  }
}

__global__ __launch_bounds__(kThreads) void cast_bf16_kernel(const float* __restrict__ in,
                                                             __bf16* __restrict__ out, long long n) {
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (long long)gridDim.x * kThreads)
    out[i] = static_cast<__bf16>(in[i]);   // round to nearest even
}

__global__ __launch_bounds__(kThreads) void widen_bf16_kernel(const __bf16* __restrict__ in,
                                                              float* __restrict__ out, long long n) {
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (long long)gridDim.x * kThreads)
    out[i] = static_cast<float>(in[i]);   // exact
}

// inv[pi[i]] = i
__global__ __launch_bounds__(kThreads) void invert_perm_kernel(const int32_t* __restrict__ pi,
                                                               int32_t* __restrict__ inv, int n) {
  for (int i = blockIdx.x * kThreads + threadIdx.x; i < n; i += gridDim.x * kThreads)
    inv[pi[i]] = i;
}

__global__ __launch_bounds__(kThreads) void copy_f32_kernel(const float* __restrict__ in,
                                                            float* __restrict__ out, long long n) {
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (long long)gridDim.x * kThreads)
    out[i] = in[i];
}

__global__ __launch_bounds__(kThreads) void scale2_kernel(const float* __restrict__ in, float c,
                                                          float* __restrict__ o1,
                                                          float* __restrict__ o2, long long n) {
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (long long)gridDim.x * kThreads) {
    const float v = c * in[i];
    o1[i] = v;
    if (o2) o2[i] = v;
  }
}

// out[i] = part[i] + part[stride + i] + ..., added in order of the split from
// 0.0f. The loads of eight splits are issued together before their adds (one
// at a time, each add would wait for its load); VEC consecutive elements per
// thread (VEC = 4: n, stride and the pointers are multiples of 4 floats).
template <int VEC>
__global__ __launch_bounds__(kThreads) void sum_splits_kernel(const float* __restrict__ part,
                                                              int nsplit, long long stride,
                                                              long long n, float* __restrict__ out) {
  typedef float V __attribute__((ext_vector_type(VEC)));
  for (long long i = ((long long)blockIdx.x * kThreads + threadIdx.x) * VEC; i < n;
       i += (long long)gridDim.x * kThreads * VEC) {
    V acc = (V)(0.0f);
    for (int s0 = 0; s0 < nsplit; s0 += 8) {
      V v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = s0 + u < nsplit ? *reinterpret_cast<const V*>(part + (s0 + u) * stride + i) : (V)(0.0f);
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (s0 + u < nsplit) acc += v[u];
    }
    *reinterpret_cast<V*>(out + i) = acc;
  }
}

__global__ __launch_bounds__(kThreads) void zero_kernel(float* __restrict__ out, long long n) {
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (long long)gridDim.x * kThreads)
    out[i] = 0.0f;
}

}  // namespace

hipError_t launch_unpack_skew(const float* theta, const Seg& g, float* S, float* Q, float c1,
                              hipStream_t s) {
  const long long total = (long long)g.b * g.b * g.count;
  hipLaunchKernelGGL(unpack_skew_kernel, dim3(grid1d(total)), dim3(kThreads), 0, s, theta, g.b,
                     g.count, g.q_off, g.p_off, S, Q, c1);
  return hipGetLastError();
}

hipError_t launch_ns_init(const float* S, const float* S2, int b, int count, float* X0, int32_t* iters,
                          int jmax, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(ns_init_kernel, dim3(count * kNsParts), dim3(kThreads), 0, s, S, S2, b, X0, iters,
                     jmax);
  return hipGetLastError();
}

hipError_t launch_ns_final(const float* X0, const float* X1, const int32_t* iters, int b, int count,
                           float* N, float* Q, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  const long long total = (long long)b * b * count;
  hipLaunchKernelGGL(ns_final_kernel, dim3(grid1d(total)), dim3(kThreads), 0, s, X0, X1, iters, b, total, N,
                     Q);
  return hipGetLastError();
}

hipError_t launch_lincomb(const LinComb& lc, float* out, int b, int count, hipStream_t s) {
  if (count <= 0 || lc.n < 0 || lc.n > kLinCombMax) return count <= 0 ? hipSuccess : hipErrorInvalidValue;
  const long long total = (long long)b * b * count;
  hipLaunchKernelGGL(lincomb_kernel, dim3(grid1d(total)), dim3(kThreads), 0, s, lc, out, b, total);
  return hipGetLastError();
}

hipError_t launch_pack_antisym(const float* M, const Seg& g, float sign, float* gtheta,
                               hipStream_t s) {
  const long long total = (long long)g.b * g.b * g.count;
  hipLaunchKernelGGL(pack_antisym_kernel, dim3(grid1d(total)), dim3(kThreads), 0, s, M, g.b,
                     g.count, g.q_off, g.p_off, sign, gtheta);
  return hipGetLastError();
}

hipError_t launch_cast(const float* in, void* out, long long n, int to_bf16, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (to_bf16)
    hipLaunchKernelGGL(cast_bf16_kernel, dim3(grid1d(n)), dim3(kThreads), 0, s, in, (__bf16*)out, n);
  else
    hipLaunchKernelGGL(copy_f32_kernel, dim3(grid1d(n)), dim3(kThreads), 0, s, in, (float*)out, n);
  return hipGetLastError();
}

hipError_t launch_widen(const void* in, float* out, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(widen_bf16_kernel, dim3(grid1d(n)), dim3(kThreads), 0, s, (const __bf16*)in, out,
                     n);
  return hipGetLastError();
}

hipError_t launch_invert_perm(const int32_t* pi, int32_t* inv, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(invert_perm_kernel, dim3(grid1d(n)), dim3(kThreads), 0, s, pi, inv, n);
  return hipGetLastError();
}

hipError_t launch_scale2(const float* in, float c, float* o1, float* o2, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(scale2_kernel, dim3(grid1d(n)), dim3(kThreads), 0, s, in, c, o1, o2, n);
  return hipGetLastError();
}

hipError_t launch_sum_splits(const float* part, int nsplit, long long stride, long long n,
                             float* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const bool v4 = n % 4 == 0 && stride % 4 == 0 && ((uintptr_t)part & 15) == 0 && ((uintptr_t)out & 15) == 0;
  if (v4)
    hipLaunchKernelGGL(sum_splits_kernel<4>, dim3(grid1d(n / 4)), dim3(kThreads), 0, s, part, nsplit,
                       stride, n, out);
  else
    hipLaunchKernelGGL(sum_splits_kernel<1>, dim3(grid1d(n)), dim3(kThreads), 0, s, part, nsplit,
                       stride, n, out);
  return hipGetLastError();
}

hipError_t launch_zero(float* out, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3(grid1d(n)), dim3(kThreads), 0, s, out, n);
  return hipGetLastError();
}

}  // namespace poetx
