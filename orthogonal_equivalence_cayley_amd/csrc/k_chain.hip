// fp32 power chains of the Cayley-Neumann parameterisation on the gfx950
// matrix cores (v_mfma_f32_16x16x4_f32) ([PX] = page "POET-X: Memory-efficient
// LLM Training by Scaling Orthogonal Transformation", Résumé technique §2.D:
// the Neumann series is evaluated in one fused kernel with its operands kept
// on chip).
//
// A row panel of a product X S only needs the same row panel of X and all of S,
// so every chain that multiplies by S from the right is row-local: one
// workgroup owns rows [r0, r0 + 16) of one block, keeps its current panel in
// LDS and runs every step of the chain without synchronising with other
// workgroups. S (b x b, fp32) streams from L2 as the MFMA B operand.
//
// Modes
//   BUILD : P_1 = S; P_j = P_{j-1} S; Q = I + sum_j c_j P_j. Writes Q (fp32)
//           and its copy in the activation dtype.
//   ABAR  : backward, A_{k+1} = c_{k+1} G; A_j = c_j G - A_{j+1} S  (S^T = -S).
//           Stores every A_j (j = 1..k+1).
//   TCHAIN: backward, transposed second chain T_j^T = A_j^T + T_{j+1}^T S with
//           T_{k+1} = A_{k+1}; writes T_1^T = (dL/dS)^T.
// Each workgroup has 4 waves; wave w owns the 16-column tiles w, w+4, ...
#include "poetx_internal.h"

namespace poetx {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int RP = 16;   // rows per panel

__device__ __forceinline__ float coef(int j, int k) { return (j == 0 || j == k + 1) ? 1.0f : 2.0f; }

// LDS layout: the current 16-row panel (pitch b + 4 floats: the 16 rows of an
// A-operand read fall in distinct banks) and two staged chunks of CR rows of S
// (pitch b + 16: the 4 rows x 16 columns of a B-operand read fall in distinct
// banks). Chunks are fetched with coalesced 16-byte loads one chunk ahead.
template <int MODE, int NT, int CR>
__global__ __launch_bounds__(kThreads) void chain_kernel(ChainArgs p) {
  extern __shared__ __align__(16) float lds[];
  const int b = p.b;
  const int pitch = b + 4;
  const int spitch = b + 16;
  float* panel = lds;
  float* sbuf = lds + RP * pitch;                   // 2 x CR x spitch
  const int panels = b / RP;
  // all panels of one block on one XCD (workgroups are dealt to the 8 XCDs
  // round-robin), so that block's S is fetched into a single L2
  const int nwg = gridDim.x;
  const int lid = (nwg % 8 == 0) ? (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8 : blockIdx.x;
  const int blk = lid / panels;
  const int r0 = (lid - blk * panels) * RP;
  const long long bb = (long long)b * b;
  const long long moff = p.q_off + blk * bb;       // this block inside the side arrays
  const float* S = p.S + moff;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ntiles = b / 16;
  // B-operand column of each of this wave's tiles; tiles past the last one are
  // clamped onto it (the MFMA loop stays branch-free; their results are dropped)
  int bcol[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) bcol[t] = min(wave + 4 * t, ntiles - 1) * 16;
  const int li = lane & 15, lk = lane >> 4;        // operand lane coordinates
  const int k = p.k;
  const int q4 = b / 4;                             // float4 per row of S
  constexpr int kLoads = 8;                         // float4 per thread per chunk (max)
  const int nvec = CR * q4;                         // float4 per chunk, <= kLoads * kThreads

  // initial panel
  float keep[NT][4];   // G (ABAR) or the running Q (BUILD) in accumulator layout
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tile = wave + 4 * t;
#pragma unroll
    for (int v = 0; v < 4; ++v) keep[t][v] = 0.0f;
    if (tile >= ntiles) continue;
    const int col = tile * 16 + li;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = 4 * lk + v;
      const long long o = (long long)(r0 + row) * b + col;
      float x;
      if (MODE == 0) {
        x = S[o];
        keep[t][v] = (r0 + row == col ? 1.0f : 0.0f) + coef(1, k) * x;
      } else if (MODE == 1) {
        const float g = p.G[moff + o];
        keep[t][v] = g;
        x = coef(k + 1, k) * g;
        p.out_f32[(long long)k * p.ne + moff + o] = x;
      } else {
        // A_{k+1}^T panel: element (row, col) = A_{k+1}[col][r0 + row]
        x = p.G[(long long)k * p.ne + moff + (long long)col * b + r0 + row];
      }
      panel[row * pitch + col] = x;
    }
  }

  const int nchunks = b / CR;
  f32x4 pre[kLoads];    // the next chunk of S, in registers
// Loads are unconditional (an index past the chunk is clamped onto its last
// float4), so the prefetch registers never need a memory-backed default.
#define POETX_FETCH(c)                                                              \
  _Pragma("unroll") for (int i = 0; i < kLoads; ++i) {                              \
    const int e = min(i * kThreads + (int)threadIdx.x, nvec - 1);                   \
    const int r = e / q4, q = e - r * q4;                                           \
    pre[i] = reinterpret_cast<const f32x4*>(S + (long long)((c) * CR + r) * b)[q]; \
  }
#define POETX_STASH(buf)                                                            \
  _Pragma("unroll") for (int i = 0; i < kLoads; ++i) {                              \
    const int e = i * kThreads + threadIdx.x;                                       \
    if (e < nvec) {                                                                 \
      const int r = e / q4, q = e - r * q4;                                         \
      *reinterpret_cast<f32x4*>(sbuf + (buf) * CR * spitch + r * spitch + 4 * q) = pre[i]; \
    }                                                                               \
  }

  const int nsteps = k;   // BUILD: j = 2..k+1; ABAR, TCHAIN: j = k..1
  for (int st = 0; st < nsteps; ++st) {
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    POETX_FETCH(0)
    __syncthreads();          // panel written; previous step's chunk reads done
    POETX_STASH(0)
    if (nchunks > 1) { POETX_FETCH(1) }
    __syncthreads();
    for (int c = 0; c < nchunks; ++c) {
      const float* sc = sbuf + (c & 1) * CR * spitch;
#pragma unroll
      for (int kk = 0; kk < CR; kk += 4) {
        const float a = panel[li * pitch + c * CR + kk + lk];
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, sc[(kk + lk) * spitch + bcol[t] + li],
                                                        acc[t], 0, 0, 0);
      }
      if (c + 1 < nchunks) {
        POETX_STASH((c + 1) & 1)   // the other buffer was last read in chunk c - 1
        if (c + 2 < nchunks) { POETX_FETCH(c + 2) }
      }
      __syncthreads();
    }
    const int j = (MODE == 0) ? st + 2 : k - st;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int tile = wave + 4 * t;
      if (tile >= ntiles) continue;
      const int col = tile * 16 + li;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 4 * lk + v;
        float x = acc[t][v];
        if (MODE == 0) {
          keep[t][v] += coef(j, k) * x;
        } else if (MODE == 1) {
          x = coef(j, k) * keep[t][v] - x;
          p.out_f32[(long long)(j - 1) * p.ne + moff + (long long)(r0 + row) * b + col] = x;
        } else {
          x += p.G[(long long)(j - 1) * p.ne + moff + (long long)col * b + r0 + row];
        }
        panel[row * pitch + col] = x;
      }
    }
  }
  __syncthreads();

  if (MODE == 0 || MODE == 2) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int tile = wave + 4 * t;
      if (tile >= ntiles) continue;
      const int col = tile * 16 + li;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 4 * lk + v;
        const long long o = moff + (long long)(r0 + row) * b + col;
        const float x = (MODE == 0) ? keep[t][v] : panel[row * pitch + col];
        p.out_f32[o] = x;
        if (MODE == 0 && p.out_act) {
          if (p.act_bf16)
            reinterpret_cast<__bf16*>(p.out_act)[o] = static_cast<__bf16>(x);
          else
            reinterpret_cast<float*>(p.out_act)[o] = x;
        }
      }
    }
  }
}

#undef POETX_FETCH
#undef POETX_STASH

template <int MODE, int CR>
hipError_t launch_cr(const ChainArgs& p, hipStream_t s) {
  const int panels = p.b / RP;
  dim3 grid(panels * p.count);
  const size_t lds = ((size_t)RP * (p.b + 4) + 2 * (size_t)CR * (p.b + 16)) * sizeof(float);
  const int nt = (p.b / 16 + 3) / 4;
  if (nt <= 1) hipLaunchKernelGGL((chain_kernel<MODE, 1, CR>), grid, dim3(kThreads), lds, s, p);
  else if (nt <= 2) hipLaunchKernelGGL((chain_kernel<MODE, 2, CR>), grid, dim3(kThreads), lds, s, p);
  else if (nt <= 4) hipLaunchKernelGGL((chain_kernel<MODE, 4, CR>), grid, dim3(kThreads), lds, s, p);
  else if (nt <= 8) hipLaunchKernelGGL((chain_kernel<MODE, 8, CR>), grid, dim3(kThreads), lds, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(const ChainArgs& p, hipStream_t s) {
  // chunk rows: each thread moves at most 8 float4 per chunk (CR * b / 4 <= 2048)
  if (p.b % 32 == 0 && p.b <= 256) return launch_cr<MODE, 32>(p, s);
  return launch_cr<MODE, 16>(p, s);
}

}  // namespace

// b % 16 == 0 keeps every row of S a whole number of float4 and every 16-row
// chunk a whole number of per-thread loads (b = 16 .. 512).
bool chain_supported(int b) { return b % 16 == 0 && b >= 16 && b <= 512; }

hipError_t launch_chain(int mode, const ChainArgs& p, hipStream_t s) {
  if (!chain_supported(p.b) || p.count <= 0) return hipErrorInvalidValue;
  switch (mode) {
    case CHAIN_BUILD: return launch_mode<0>(p, s);
    case CHAIN_ABAR: return launch_mode<1>(p, s);
    case CHAIN_TCHAIN: return launch_mode<2>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace poetx
