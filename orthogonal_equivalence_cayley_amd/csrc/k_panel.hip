// Index mapping fused with the block-diagonal products on gfx950
// (v_mfma_f32_32x32x16_bf16, fp32 accumulate, blocks of 256).
//
// [PX] = page "POET-X: Memory-efficient LLM Training by Scaling Orthogonal
// Transformation", Résumé technique: §2.B applies the permutations as index
// mappings on the activations, §2.C the block-diagonal factors as batched
// block products. Each pass of the layer over one side is
//   gather:  U[t][i] = X[t][pi[i]], then C[:, blk] = U[:, blk] B_g^T, or
//   scatter: C[:, blk] = A[:, blk] B_g^T, then Y[t][pi[i]] = C[t][i],
// with B_g(n, k) one 256 x 256 block of Q (forward) or of Q^T (backward).
//
// A permutation inside a row reaches the whole row, so a workgroup owns a
// panel of 32 whole token rows: they come from HBM into LDS with coalesced
// direct-to-LDS loads, are permuted inside LDS (random 2-byte accesses that
// pass through registers), multiplied block by block in place, permuted again
// if the output is scattered, and leave with coalesced 16-byte stores. The
// gathered input and the output make one trip through HBM each; a separate
// gather (or scatter) kernel would add a write and a read of the whole
// activation. Every wave owns 32 of a block's 256 output columns and takes its
// slice of B_g from L2 into registers (16 operand fragments), one block ahead
// of the multiplies.
//
// Panel in LDS: row r holds dim bf16 as dim / 8 chunks of 16 bytes; chunk c sits
// at slot c ^ (r & 15) of its row, so the 16 rows one pass of a fragment read
// touches fall in distinct banks (the XOR stays inside aligned groups of 16
// chunks, i.e. inside a block).
#include <algorithm>

#include "poetx_internal.h"

namespace poetx {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kB = 256;                  // block size
constexpr int kRows = 32;                // token rows per panel
constexpr int kWaves = 8;                // each owns 32 output columns of a block
constexpr int kThreads = kWaves * 64;
constexpr int kNKK = kB / 16;            // 16-deep K steps per block
constexpr int kMaxDim = 2048;            // panel of 32 rows: 128 KiB of LDS

__device__ __forceinline__ void dma16(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                   (void __attribute__((address_space(3)))*)lds_dst, 16, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16_pair(float lo, float hi) {
  const __bf16 a = static_cast<__bf16>(lo);
  const __bf16 b = static_cast<__bf16>(hi);
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// byte offset of element col of panel row r (rowb = bytes per row)
__device__ __forceinline__ int elem_off(int r, int col, int rowb) {
  return r * rowb + (((col >> 3) ^ (r & 15)) << 4) + ((col & 7) << 1);
}
__device__ __forceinline__ int chunk_off(int r, int c, int rowb) {
  return r * rowb + ((c ^ (r & 15)) << 4);
}

// B_g(ncol, 16 kk + 8 h .. + 7) (K-contiguous rows of 256)
__device__ __forceinline__ bf16x8 load_b(const uint16_t* Bg, int ncol, int h, int kk) {
  return *reinterpret_cast<const bf16x8*>(Bg + (long long)ncol * kB + 8 * h + 16 * kk);
}

// Row-local permutations of the panel go a quarter of its rows at a time: a
// row's elements are all read into registers before any of them is written
// back, and the quarters touch disjoint rows.
constexpr int kQuarter = kRows / 4;
constexpr int kQChunks = kQuarter * (kMaxDim / 8) / kThreads;   // chunks per thread and quarter

// GATHER: the panel arrives in the order of `in` and is permuted to
// P[t][i] = in[t][idx[i]] before the products; with in_copy set, the permuted
// panel is also written there. SCATTER: the products' output C is written as
// out[t][idx[i]] = C[t][i]; otherwise out = C.
template <bool GATHER, bool SCATTER>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void panel_block_kernel(const uint16_t* __restrict__ in, const int32_t* __restrict__ idx,
                        const uint16_t* __restrict__ Bq, uint16_t* __restrict__ out,
                        uint16_t* __restrict__ in_copy, long long T, int dim) {
  extern __shared__ __align__(16) unsigned char lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nl = lane & 31, h = lane >> 5;
  const int cpr = dim >> 3;              // 16-byte chunks per row
  const int rowb = dim * 2;
  const int total = kRows * cpr;         // chunks per panel
  const int qtotal = kQuarter * cpr;     // chunks per quarter
  const int nb = dim / kB;
  const int ncol = wave * 32 + nl;       // B column of this lane's operand fragments
  const long long npanel = (T + kRows - 1) / kRows;

  for (long long pnl = blockIdx.x; pnl < npanel; pnl += gridDim.x) {
    const long long row0 = pnl * kRows;
    // 1. rows -> LDS; slot s holds chunk (s % cpr) ^ (r & 15) of row r = s / cpr.
    //    Rows past T are loaded from row T - 1 and never stored. total is a
    //    multiple of 1024, so every wave issues whole loads.
    for (int s0 = 0; s0 < total; s0 += kThreads) {
      const int s = s0 + tid;
      const int r = s / cpr;
      const int c = (s - r * cpr) ^ (r & 15);
      const long long row = min(row0 + r, T - 1);
      dma16(in + row * dim + c * 8, lds + (s0 + wave * 64) * 16);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // 2. gather inside LDS: each thread reads its chunks of the permuted rows
    //    (8 random elements each), then writes them back in place
    if constexpr (GATHER) {
#pragma unroll 1
      for (int qr = 0; qr < 4; ++qr) {
        uint4 g[kQChunks];
#pragma unroll
        for (int u = 0; u < kQChunks; ++u) {
          const int q = u * kThreads + tid;
          if (q < qtotal) {
            const int r = qr * kQuarter + q / cpr, c = q % cpr;
            const int4 i0 = *reinterpret_cast<const int4*>(idx + c * 8);
            const int4 i1 = *reinterpret_cast<const int4*>(idx + c * 8 + 4);
            const int ix[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t lo = *reinterpret_cast<const uint16_t*>(lds + elem_off(r, ix[2 * e], rowb));
              const uint32_t hi = *reinterpret_cast<const uint16_t*>(lds + elem_off(r, ix[2 * e + 1], rowb));
              w[e] = lo | (hi << 16);
            }
            g[u] = make_uint4(w[0], w[1], w[2], w[3]);
          }
        }
        __syncthreads();   // the quarter's rows are read before they are overwritten
#pragma unroll
        for (int u = 0; u < kQChunks; ++u) {
          const int q = u * kThreads + tid;
          if (q < qtotal) {
            const int r = qr * kQuarter + q / cpr, c = q % cpr;
            *reinterpret_cast<uint4*>(lds + chunk_off(r, c, rowb)) = g[u];
            if (in_copy && row0 + r < T)
              *reinterpret_cast<uint4*>(in_copy + (row0 + r) * dim + c * 8) = g[u];
          }
        }
      }
      __syncthreads();
    }

    // 3. block products in place. Each wave holds its slice of B_j as 16
    //    operand fragments; each fragment is reloaded with block j + 1's as soon
    //    as its multiply has issued (the last block reloads itself, unused).
    {
      bf16x8 bq[kNKK];
#pragma unroll
      for (int kk = 0; kk < kNKK; ++kk) bq[kk] = load_b(Bq, ncol, h, kk);
#pragma unroll 1
      for (int j = 0; j < nb; ++j) {
        const uint16_t* Bn = Bq + (long long)min(j + 1, nb - 1) * kB * kB;
        f32x16 acc;
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
#pragma unroll
        for (int kk = 0; kk < kNKK; ++kk) {
          const bf16x8 af = *reinterpret_cast<const bf16x8*>(lds + chunk_off(nl, j * 32 + 2 * kk + h, rowb));
          // B first: the result is C^T; lane (nl, h) holds output row nl,
          // columns 8 q + 4 h .. + 3 of the wave's 32
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bq[kk], af, acc, 0, 0, 0);
          bq[kk] = load_b(Bn, ncol, h, kk);
        }
        __syncthreads();   // every wave has read block j's columns
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint2 v;
          v.x = pack_bf16_pair(acc[4 * q], acc[4 * q + 1]);
          v.y = pack_bf16_pair(acc[4 * q + 2], acc[4 * q + 3]);
          const int c = j * 32 + wave * 4 + q;
          *reinterpret_cast<uint2*>(lds + chunk_off(nl, c, rowb) + 8 * h) = v;
        }
      }
    }
    __syncthreads();

    // 4. output: scattered inside LDS first, then whole rows to HBM
    if constexpr (SCATTER) {
#pragma unroll 1
      for (int qr = 0; qr < 4; ++qr) {
        uint4 g[kQChunks];
#pragma unroll
        for (int u = 0; u < kQChunks; ++u) {
          const int q = u * kThreads + tid;
          if (q < qtotal) {
            const int r = qr * kQuarter + q / cpr, c = q % cpr;
            g[u] = *reinterpret_cast<const uint4*>(lds + chunk_off(r, c, rowb));
          }
        }
        __syncthreads();   // the quarter's rows are read before they are overwritten
#pragma unroll
        for (int u = 0; u < kQChunks; ++u) {
          const int q = u * kThreads + tid;
          if (q < qtotal) {
            const int r = qr * kQuarter + q / cpr, c = q % cpr;
            const int4 i0 = *reinterpret_cast<const int4*>(idx + c * 8);
            const int4 i1 = *reinterpret_cast<const int4*>(idx + c * 8 + 4);
            const int ix[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
            const uint32_t w[4] = {g[u].x, g[u].y, g[u].z, g[u].w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
              *reinterpret_cast<uint16_t*>(lds + elem_off(r, ix[e], rowb)) =
                  (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
          }
        }
      }
      __syncthreads();
    }
    for (int q = tid; q < total; q += kThreads) {
      const int r = q / cpr, c = q - r * cpr;
      if (row0 + r < T)
        *reinterpret_cast<uint4*>(out + (row0 + r) * dim + c * 8) =
            *reinterpret_cast<const uint4*>(lds + chunk_off(r, c, rowb));
    }
    __syncthreads();   // the panel's LDS is read out before the next panel arrives
  }
}

// QT[g][n][k] = Q[g][k][n] for count blocks of 256 x 256 bf16 (32 x 32 tiles via LDS)
__global__ __launch_bounds__(256) void transpose_blocks_kernel(const uint16_t* __restrict__ Q,
                                                               uint16_t* __restrict__ QT, int count) {
  __shared__ uint16_t t[32][33];
  const int tiles = (kB / 32) * (kB / 32);
  const int g = blockIdx.x / tiles, tile = blockIdx.x % tiles;
  if (g >= count) return;
  const int r0 = (tile / (kB / 32)) * 32, c0 = (tile % (kB / 32)) * 32;
  const uint16_t* src = Q + (long long)g * kB * kB;
  uint16_t* dst = QT + (long long)g * kB * kB;
  const int x = threadIdx.x & 31, y = threadIdx.x >> 5;   // 8 rows per pass
#pragma unroll
  for (int i = 0; i < 32; i += 8) t[y + i][x] = src[(r0 + y + i) * kB + c0 + x];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 32; i += 8) dst[(c0 + y + i) * kB + r0 + x] = t[x][y + i];
}

}  // namespace

bool panel_supported(int dim, int b, int nblocks) {
  return b == kB && nblocks * kB == dim && dim <= kMaxDim && dim > 0;
}

hipError_t launch_panel_block(const void* in, const int32_t* idx, const void* Bq, void* out,
                              void* in_copy, long long T, int dim, bool gather, bool scatter,
                              hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (dim % kB || dim > kMaxDim || gather == scatter) return hipErrorInvalidValue;
  if (((uintptr_t)in | (uintptr_t)idx | (uintptr_t)Bq | (uintptr_t)out | (uintptr_t)in_copy) & 15)
    return hipErrorInvalidValue;
  const long long npanel = (T + kRows - 1) / kRows;
  const size_t lds = (size_t)kRows * dim * 2;
  const long long per_cu = lds <= 80 * 1024 ? 2 : 1;
  const unsigned grid = (unsigned)std::min<long long>(npanel, 256 * per_cu);
  const uint16_t* a = static_cast<const uint16_t*>(in);
  const uint16_t* b = static_cast<const uint16_t*>(Bq);
  uint16_t* c = static_cast<uint16_t*>(out);
  uint16_t* cp = static_cast<uint16_t*>(in_copy);
  if (gather)
    hipLaunchKernelGGL((panel_block_kernel<true, false>), dim3(grid), dim3(kThreads), lds, s, a, idx,
                       b, c, cp, T, dim);
  else
    hipLaunchKernelGGL((panel_block_kernel<false, true>), dim3(grid), dim3(kThreads), lds, s, a, idx,
                       b, c, nullptr, T, dim);
  return hipGetLastError();
}

hipError_t launch_transpose_blocks(const void* Q, void* QT, int count, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  const int tiles = (kB / 32) * (kB / 32);
  hipLaunchKernelGGL(transpose_blocks_kernel, dim3((unsigned)(count * tiles)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(Q), static_cast<uint16_t*>(QT), count);
  return hipGetLastError();
}

}  // namespace poetx
