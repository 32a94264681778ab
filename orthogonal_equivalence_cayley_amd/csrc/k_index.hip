// Index-mapping kernels: column gather / scatter inside each activation row and
// the one-time weight pre-merge. Permutations stay index arrays and are never
// formed as matrices ([PX] = page "POET-X: Memory-efficient LLM Training by
// Scaling Orthogonal Transformation", Résumé technique §2.B).
//
// A permutation inside a row touches the whole row at random, so each workgroup
// stages R whole rows in LDS with coalesced 16-byte global accesses and does the
// random part of the access pattern in LDS. Every global read and write is then
// a full-line, coalesced transfer; the index array is read once per R rows.
#include "poetx_internal.h"

namespace poetx {
namespace {

constexpr int kThreads = 256;
constexpr int kLdsBudget = 64 * 1024;   // bytes of LDS for staged rows per workgroup
constexpr int kMaxRows = 4;             // rows per workgroup: small tiles keep the grid full
// Second-phase items of the interleaved gather: (R / G) (dim / VEC) =
// R dim sizeof(E)^2 / (16 sizeof(W)) <= kLdsBudget sizeof(E) / (16 sizeof(W))
// <= kLdsBudget / 32 (G = sizeof(W) / sizeof(E), VEC = 16 / sizeof(E),
// sizeof(E) <= 4 with 8-byte words, sizeof(E) = 2 with 4-byte words).
static_assert(kLdsBudget / 32 <= 8 * 256, "gather index prefetch covers every item");

template <typename E, int VEC>
struct Vec { E v[VEC]; };

template <typename E, bool VECTOR>
__global__ __launch_bounds__(kThreads) void gather_cols_kernel(
    const E* __restrict__ in, long long in_ld, const int32_t* __restrict__ rows,
    const int32_t* __restrict__ idx, E* __restrict__ out, long long T, int dim, int R) {
  extern __shared__ __align__(16) unsigned char smem[];
  E* lds = reinterpret_cast<E*>(smem);
  constexpr int VEC = 16 / sizeof(E);
  using V = Vec<E, VEC>;
  for (long long t0 = (long long)blockIdx.x * R; t0 < T; t0 += (long long)gridDim.x * R) {
    const int nr = (int)((T - t0) < R ? (T - t0) : R);
    if (VECTOR) {
      const int cpr = dim / VEC;   // chunks per row
      for (int c = threadIdx.x; c < nr * cpr; c += kThreads) {
        const int r = c / cpr, q = c - r * cpr;
        const long long src_row = rows ? (long long)rows[t0 + r] : (t0 + r);
        const V* src = reinterpret_cast<const V*>(in + src_row * in_ld);
        reinterpret_cast<V*>(lds + (long long)r * dim)[q] = src[q];
      }
      __syncthreads();
      for (int q = threadIdx.x; q < cpr; q += kThreads) {
        int ix[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) ix[e] = idx[q * VEC + e];
        for (int r = 0; r < nr; ++r) {
          V v;
#pragma unroll
          for (int e = 0; e < VEC; ++e) v.v[e] = lds[r * dim + ix[e]];
          reinterpret_cast<V*>(out + (t0 + r) * dim)[q] = v;
        }
      }
    } else {
      for (int c = threadIdx.x; c < nr * dim; c += kThreads) {
        const int r = c / dim, q = c - r * dim;
        const long long src_row = rows ? (long long)rows[t0 + r] : (t0 + r);
        lds[(long long)r * dim + q] = in[src_row * in_ld + q];
      }
      __syncthreads();
      for (int q = threadIdx.x; q < dim; q += kThreads) {
        const int ix = idx[q];
        for (int r = 0; r < nr; ++r) out[(t0 + r) * dim + q] = lds[r * dim + ix];
      }
    }
    __syncthreads();
  }
}

template <typename E, bool VECTOR>
__global__ __launch_bounds__(kThreads) void scatter_cols_kernel(
    const E* __restrict__ in, const int32_t* __restrict__ idx, E* __restrict__ out,
    long long T, int dim, int R) {
  extern __shared__ __align__(16) unsigned char smem[];
  E* lds = reinterpret_cast<E*>(smem);
  constexpr int VEC = 16 / sizeof(E);
  using V = Vec<E, VEC>;
  for (long long t0 = (long long)blockIdx.x * R; t0 < T; t0 += (long long)gridDim.x * R) {
    const int nr = (int)((T - t0) < R ? (T - t0) : R);
    if (VECTOR) {
      const int cpr = dim / VEC;
      for (int q = threadIdx.x; q < cpr; q += kThreads) {
        int ix[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) ix[e] = idx[q * VEC + e];
        for (int r = 0; r < nr; ++r) {
          const V v = reinterpret_cast<const V*>(in + (t0 + r) * dim)[q];
#pragma unroll
          for (int e = 0; e < VEC; ++e) lds[r * dim + ix[e]] = v.v[e];
        }
      }
      __syncthreads();
      for (int c = threadIdx.x; c < nr * cpr; c += kThreads) {
        const int r = c / cpr, q = c - r * cpr;
        reinterpret_cast<V*>(out + (t0 + r) * dim)[q] =
            reinterpret_cast<const V*>(lds + (long long)r * dim)[q];
      }
    } else {
      for (int q = threadIdx.x; q < dim; q += kThreads) {
        const int ix = idx[q];
        for (int r = 0; r < nr; ++r) lds[r * dim + ix] = in[(t0 + r) * dim + q];
      }
      __syncthreads();
      for (int c = threadIdx.x; c < nr * dim; c += kThreads) {
        const int r = c / dim, q = c - r * dim;
        out[(t0 + r) * dim + q] = lds[(long long)r * dim + q];
      }
    }
    __syncthreads();
  }
}

// Interleaved variants: G = sizeof(W) / sizeof(E) rows share one LDS word W per
// column (with 8-byte words, word c of row group g holds element c of rows
// 4g..4g+3 for bf16), so one random LDS access moves the element of G rows.
// Rows too wide for 4 staged rows take 4-byte words (2 bf16 rows per word).
// Rows are read and written with coalesced 16-byte accesses; the interleave
// happens in registers.
template <typename E, typename W = uint64_t>
struct Inter {
  static constexpr int G = sizeof(W) / sizeof(E);   // rows per word
  static constexpr int VEC = 16 / sizeof(E);        // elements per 16-byte chunk
  static constexpr int BITS = 8 * sizeof(E);
  static_assert(G >= 2, "at least two rows per word");
  __device__ __forceinline__ static W elem(const uint4& v, int e) {
    const uint32_t w = (e * BITS / 32) == 0 ? v.x : (e * BITS / 32) == 1 ? v.y : (e * BITS / 32) == 2 ? v.z : v.w;
    if (BITS == 32) return w;
    return (e & 1) ? (w >> 16) : (w & 0xffffu);
  }
};

// out[t][i] = in[row(t)][idx[i]] for R rows per iteration (R a multiple of G).
// A thread's items of the second phase are the same in every iteration, so
// their indices are loaded once, before the first rows: the random LDS reads
// after the barrier then wait on nothing but LDS (ngrp * cpr <= NI * kThreads).
template <typename E, typename W, int NI>
__global__ __launch_bounds__(kThreads) void gather_cols_inter(
    const E* __restrict__ in, long long in_ld, const int32_t* __restrict__ rows,
    const int32_t* __restrict__ idx, E* __restrict__ out, long long T, int dim, int R) {
  using I = Inter<E, W>;
  constexpr int G = I::G, VEC = I::VEC, BITS = I::BITS;
  extern __shared__ __align__(16) unsigned char smem[];
  W* lds = reinterpret_cast<W*>(smem);   // [R / G][dim]
  const int cpr = dim / VEC;
  const int ngrp = R / G;
  int ixs[NI][VEC];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int c = threadIdx.x + j * kThreads;
    const int q = c < ngrp * cpr ? c % cpr : 0;
#pragma unroll
    for (int e = 0; e < VEC; ++e) ixs[j][e] = idx[q * VEC + e];
  }
  for (long long t0 = (long long)blockIdx.x * R; t0 < T; t0 += (long long)gridDim.x * R) {
    const int nr = (int)((T - t0) < R ? (T - t0) : R);
    // load G rows x VEC elements per item, interleave, write VEC words
    for (int c = threadIdx.x; c < ngrp * cpr; c += kThreads) {
      const int g = c / cpr, q = c - g * cpr;
      uint4 v[G];
#pragma unroll
      for (int r = 0; r < G; ++r) {
        const int rr = min(g * G + r, nr - 1);
        const long long src_row = rows ? (long long)rows[t0 + rr] : (t0 + rr);
        v[r] = reinterpret_cast<const uint4*>(in + src_row * in_ld)[q];
      }
      W* dst = lds + (long long)g * dim + q * VEC;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        W wv = 0;
#pragma unroll
        for (int r = 0; r < G; ++r) wv |= I::elem(v[r], e) << (BITS * r);
        dst[e] = wv;
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int c = threadIdx.x + j * kThreads;
      if (c >= ngrp * cpr) break;
      const int g = c / cpr, q = c - g * cpr;
      const W* src = lds + (long long)g * dim;
      W wv[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) wv[e] = src[ixs[j][e]];
#pragma unroll
      for (int r = 0; r < G; ++r) {
        const int row = g * G + r;
        if (row >= nr) break;
        uint32_t o[4] = {0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const uint32_t x = (uint32_t)((wv[e] >> (BITS * r)) & (BITS == 32 ? 0xffffffffu : 0xffffu));
          if (BITS == 32) o[e] = x;
          else o[e >> 1] |= x << (16 * (e & 1));
        }
        reinterpret_cast<uint4*>(out + (t0 + row) * dim)[q] = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
    __syncthreads();
  }
}

// out[t][idx[i]] = in[t][i]: rows interleaved into LDS at their destination
// columns, then written out row by row.
template <typename E, typename W>
__global__ __launch_bounds__(kThreads) void scatter_cols_inter(
    const E* __restrict__ in, const int32_t* __restrict__ idx, E* __restrict__ out, long long T,
    int dim, int R) {
  using I = Inter<E, W>;
  constexpr int G = I::G, VEC = I::VEC, BITS = I::BITS;
  extern __shared__ __align__(16) unsigned char smem[];
  W* lds = reinterpret_cast<W*>(smem);
  const int cpr = dim / VEC;
  const int ngrp = R / G;
  for (long long t0 = (long long)blockIdx.x * R; t0 < T; t0 += (long long)gridDim.x * R) {
    const int nr = (int)((T - t0) < R ? (T - t0) : R);
    for (int c = threadIdx.x; c < ngrp * cpr; c += kThreads) {
      const int g = c / cpr, q = c - g * cpr;
      uint4 v[G];
#pragma unroll
      for (int r = 0; r < G; ++r) {
        const int rr = min(g * G + r, nr - 1);
        v[r] = reinterpret_cast<const uint4*>(in + (t0 + rr) * dim)[q];
      }
      W* dst = lds + (long long)g * dim;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        W wv = 0;
#pragma unroll
        for (int r = 0; r < G; ++r) wv |= I::elem(v[r], e) << (BITS * r);
        dst[idx[q * VEC + e]] = wv;
      }
    }
    __syncthreads();
    for (int c = threadIdx.x; c < ngrp * cpr; c += kThreads) {
      const int g = c / cpr, q = c - g * cpr;
      const W* src = lds + (long long)g * dim + q * VEC;
      W wv[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) wv[e] = src[e];
#pragma unroll
      for (int r = 0; r < G; ++r) {
        const int row = g * G + r;
        if (row >= nr) break;
        uint32_t o[4] = {0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const uint32_t x = (uint32_t)((wv[e] >> (BITS * r)) & (BITS == 32 ? 0xffffffffu : 0xffffu));
          if (BITS == 32) o[e] = x;
          else o[e >> 1] |= x << (16 * (e & 1));
        }
        reinterpret_cast<uint4*>(out + (t0 + row) * dim)[q] = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
    __syncthreads();
  }
}

// Rows of `dim` elements too wide for LDS: plain per-element global access.
template <typename E>
__global__ __launch_bounds__(kThreads) void gather_cols_direct(
    const E* __restrict__ in, long long in_ld, const int32_t* __restrict__ rows,
    const int32_t* __restrict__ idx, E* __restrict__ out, long long T, int dim) {
  for (long long t = blockIdx.x; t < T; t += gridDim.x) {
    const long long src_row = rows ? (long long)rows[t] : t;
    for (int q = threadIdx.x; q < dim; q += kThreads) out[t * dim + q] = in[src_row * in_ld + idx[q]];
  }
}

template <typename E>
__global__ __launch_bounds__(kThreads) void scatter_cols_direct(
    const E* __restrict__ in, const int32_t* __restrict__ idx, E* __restrict__ out, long long T,
    int dim) {
  for (long long t = blockIdx.x; t < T; t += gridDim.x)
    for (int q = threadIdx.x; q < dim; q += kThreads) out[t * dim + idx[q]] = in[t * dim + q];
}

// out[c][r] = in[r][c] for an R x C matrix (32 x 32 tiles through LDS; edges
// of sizes that are not multiples of 32 checked)
template <typename E>
__global__ __launch_bounds__(256) void transpose_kernel(const E* __restrict__ in, E* __restrict__ out,
                                                        int R, int C) {
  __shared__ E t[32][33];
  const int tc = (C + 31) / 32;
  const int r0 = (blockIdx.x / tc) * 32, c0 = (blockIdx.x % tc) * 32;
  const int x = threadIdx.x & 31, y = threadIdx.x >> 5;   // 8 rows per pass
#pragma unroll
  for (int i = 0; i < 32; i += 8)
    if (r0 + y + i < R && c0 + x < C) t[y + i][x] = in[(long long)(r0 + y + i) * C + c0 + x];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 32; i += 8)
    if (c0 + y + i < C && r0 + x < R) out[(long long)(c0 + y + i) * R + r0 + x] = t[x][y + i];
}

inline int grid_for(long long units) {
  const long long cap = 256LL * 16;   // 16 workgroups per CU on 256 CUs
  return (int)(units < cap ? (units < 1 ? 1 : units) : cap);
}

template <typename E, typename W>
hipError_t gather_inter(const void* in, long long in_ld, const int32_t* rows, const int32_t* idx,
                        void* out, long long T, int dim, int R, hipStream_t s) {
  using I = Inter<E, W>;
  const size_t lds = (size_t)R * dim * sizeof(E);
  const long long items = (long long)(R / I::G) * (dim / I::VEC);   // second-phase items per workgroup
  const dim3 grid(grid_for((T + R - 1) / R)), block(kThreads);
  if (items <= kThreads)
    hipLaunchKernelGGL((gather_cols_inter<E, W, 1>), grid, block, lds, s, (const E*)in, in_ld, rows, idx,
                       (E*)out, T, dim, R);
  else if (items <= 2 * kThreads)
    hipLaunchKernelGGL((gather_cols_inter<E, W, 2>), grid, block, lds, s, (const E*)in, in_ld, rows, idx,
                       (E*)out, T, dim, R);
  else if (items <= 4 * kThreads)
    hipLaunchKernelGGL((gather_cols_inter<E, W, 4>), grid, block, lds, s, (const E*)in, in_ld, rows, idx,
                       (E*)out, T, dim, R);
  else if (items <= 8 * kThreads)
    hipLaunchKernelGGL((gather_cols_inter<E, W, 8>), grid, block, lds, s, (const E*)in, in_ld, rows, idx,
                       (E*)out, T, dim, R);
  else
    return hipErrorInvalidValue;   // not reached: R dim sizeof(E) <= kLdsBudget bounds the items
  return hipGetLastError();
}

template <typename E, typename W>
hipError_t scatter_inter(const void* in, const int32_t* idx, void* out, long long T, int dim, int R,
                         hipStream_t s) {
  const size_t lds = (size_t)R * dim * sizeof(E);
  hipLaunchKernelGGL((scatter_cols_inter<E, W>), dim3(grid_for((T + R - 1) / R)), dim3(kThreads), lds, s,
                     (const E*)in, idx, (E*)out, T, dim, R);
  return hipGetLastError();
}

template <typename E>
hipError_t gather_typed(const void* in, long long in_ld, const int32_t* rows, const int32_t* idx,
                        void* out, long long T, int dim, hipStream_t s) {
  if (T <= 0 || dim <= 0) return hipSuccess;
  const long long row_bytes = (long long)dim * sizeof(E);
  constexpr int VEC = 16 / sizeof(E);
  if (row_bytes > kLdsBudget) {
    hipLaunchKernelGGL(gather_cols_direct<E>, dim3(grid_for(T)), dim3(kThreads), 0, s,
                       (const E*)in, in_ld, rows, idx, (E*)out, T, dim);
    return hipGetLastError();
  }
  int R = (int)(kLdsBudget / row_bytes);
  if (R > kMaxRows) R = kMaxRows;
  const bool vec = (dim % VEC == 0) && (in_ld % VEC == 0) &&
                   ((uintptr_t)in % 16 == 0) && ((uintptr_t)out % 16 == 0);
  constexpr int G = 8 / sizeof(E);
  if (vec && R >= G)
    return gather_inter<E, uint64_t>(in, in_ld, rows, idx, out, T, dim, R / G * G, s);
  if constexpr (sizeof(E) == 2)   // rows too wide for 4 staged rows: 2 rows per 4-byte word
    if (vec && R >= 2) return gather_inter<E, uint32_t>(in, in_ld, rows, idx, out, T, dim, R / 2 * 2, s);
  const size_t lds = (size_t)R * row_bytes;
  const int grid = grid_for((T + R - 1) / R);
  if (vec)
    hipLaunchKernelGGL((gather_cols_kernel<E, true>), dim3(grid), dim3(kThreads), lds, s,
                       (const E*)in, in_ld, rows, idx, (E*)out, T, dim, R);
  else
    hipLaunchKernelGGL((gather_cols_kernel<E, false>), dim3(grid), dim3(kThreads), lds, s,
                       (const E*)in, in_ld, rows, idx, (E*)out, T, dim, R);
  return hipGetLastError();
}

template <typename E>
hipError_t scatter_typed(const void* in, const int32_t* idx, void* out, long long T, int dim,
                         hipStream_t s) {
  if (T <= 0 || dim <= 0) return hipSuccess;
  const long long row_bytes = (long long)dim * sizeof(E);
  constexpr int VEC = 16 / sizeof(E);
  if (row_bytes > kLdsBudget) {
    hipLaunchKernelGGL(scatter_cols_direct<E>, dim3(grid_for(T)), dim3(kThreads), 0, s,
                       (const E*)in, idx, (E*)out, T, dim);
    return hipGetLastError();
  }
  int R = (int)(kLdsBudget / row_bytes);
  if (R > kMaxRows) R = kMaxRows;
  const bool vec = (dim % VEC == 0) && ((uintptr_t)in % 16 == 0) && ((uintptr_t)out % 16 == 0);
  constexpr int G = 8 / sizeof(E);
  if (vec && R >= G) return scatter_inter<E, uint64_t>(in, idx, out, T, dim, R / G * G, s);
  if constexpr (sizeof(E) == 2)   // rows too wide for 4 staged rows: 2 rows per 4-byte word
    if (vec && R >= 2) return scatter_inter<E, uint32_t>(in, idx, out, T, dim, R / 2 * 2, s);
  const size_t lds = (size_t)R * row_bytes;
  const int grid = grid_for((T + R - 1) / R);
  if (vec)
    hipLaunchKernelGGL((scatter_cols_kernel<E, true>), dim3(grid), dim3(kThreads), lds, s,
                       (const E*)in, idx, (E*)out, T, dim, R);
  else
    hipLaunchKernelGGL((scatter_cols_kernel<E, false>), dim3(grid), dim3(kThreads), lds, s,
                       (const E*)in, idx, (E*)out, T, dim, R);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gather_cols(const void* in, long long in_ld, const int32_t* rows,
                              const int32_t* idx, void* out, long long T, int dim, int elsize,
                              hipStream_t s) {
  if (elsize == 2) return gather_typed<uint16_t>(in, in_ld, rows, idx, out, T, dim, s);
  return gather_typed<uint32_t>(in, in_ld, rows, idx, out, T, dim, s);
}

hipError_t launch_transpose(const void* in, void* out, int R, int C, int elsize, hipStream_t s) {
  if (R <= 0 || C <= 0) return hipSuccess;
  const long long tiles = (long long)((R + 31) / 32) * ((C + 31) / 32);
  if (tiles > INT32_MAX) return hipErrorInvalidValue;
  if (elsize == 1)
    hipLaunchKernelGGL(transpose_kernel<uint8_t>, dim3((unsigned)tiles), dim3(256), 0, s,
                       static_cast<const uint8_t*>(in), static_cast<uint8_t*>(out), R, C);
  else if (elsize == 2)
    hipLaunchKernelGGL(transpose_kernel<uint16_t>, dim3((unsigned)tiles), dim3(256), 0, s,
                       static_cast<const uint16_t*>(in), static_cast<uint16_t*>(out), R, C);
  else
    hipLaunchKernelGGL(transpose_kernel<uint32_t>, dim3((unsigned)tiles), dim3(256), 0, s,
                       static_cast<const uint32_t*>(in), static_cast<uint32_t*>(out), R, C);
  return hipGetLastError();
}

hipError_t launch_scatter_cols(const void* in, const int32_t* idx, void* out, long long T,
                               int dim, int elsize, hipStream_t s) {
  if (elsize == 2) return scatter_typed<uint16_t>(in, idx, out, T, dim, s);
  return scatter_typed<uint32_t>(in, idx, out, T, dim, s);
}

}  // namespace poetx
