// fp32 power chains of the Cayley-Neumann parameterisation on the gfx950
// matrix cores (v_mfma_f32_16x16x4_f32) ([PX] = page "POET-X: Memory-efficient
// LLM Training by Scaling Orthogonal Transformation", Résumé technique §2.D:
// the Neumann series is evaluated in one fused kernel with its operands kept
// on chip).
//
// A row panel of a product X S only needs the same row panel of X and all of S,
// so every chain that multiplies by S from the right is row-local: one
// workgroup owns rows [r0, r0 + RP) of one block, keeps its current panel in
// LDS and runs every step of the chain without synchronising with other
// workgroups. S (b x b, fp32) streams from L2 straight into registers as the
// MFMA B operand; each B value feeds the RP / 16 row tiles of the panel.
//
// Modes
//   BUILD : P_1 = S; P_j = P_{j-1} S; Q = I + sum_j c_j P_j. Writes Q (fp32)
//           and its copy in the activation dtype.
//   ABAR  : backward, A_{k+1} = c_{k+1} G; A_j = c_j G - A_{j+1} S  (S^T = -S).
//           Stores every A_j (j = 1..k+1).
//   TCHAIN: backward, transposed second chain T_j^T = A_j^T + T_{j+1}^T S with
//           T_{k+1} = A_{k+1}; writes T_1^T = (dL/dS)^T. A lane's 4 accumulator
//           rows of one column are 4 consecutive elements of one row of A_j,
//           read with one 16-byte load.
// Each workgroup has 4 waves; wave w owns the 16-column tiles w, w+4, ... of
// all RP rows.
#include "poetx_internal.h"

namespace poetx {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

__device__ __forceinline__ float coef(int j, int k) { return (j == 0 || j == k + 1) ? 1.0f : 2.0f; }

// 4 consecutive floats at a 16-byte aligned address (b % 16 == 0, panel rows in
// groups of 4 from a multiple of 16).
__device__ __forceinline__ float4 load_t4(const float* src) { return *reinterpret_cast<const float4*>(src); }
__device__ __forceinline__ float f4(const float4& a, int v) {
  return v == 0 ? a.x : v == 1 ? a.y : v == 2 ? a.z : a.w;
}

// The run this workgroup belongs to. Constant indices only (fully unrolled), so
// the table stays in kernel-argument memory and scalar registers.
__device__ __forceinline__ ChainEntry select_entry(const ChainBatch& cb) {
  ChainEntry e = cb.e[0];
#pragma unroll
  for (int i = 1; i < kChainMaxEntries; ++i)
    if (i < cb.n && (int)blockIdx.x >= cb.e[i].wg0) e = cb.e[i];
  return e;
}

// MT row tiles of 16 (RP = 16 MT rows per panel), NT column tiles per wave,
// B operand prefetched U K-steps (of 4) ahead. The panel sits in LDS with pitch
// b + 4 floats: the 16 rows of an A-operand read fall in distinct banks.
template <int MODE, int NT, int MT, int U>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void chain_kernel(ChainBatch cb) {
  constexpr int RP = 16 * MT;
  extern __shared__ __align__(16) float lds[];
  const ChainEntry p = select_entry(cb);
  const int b = p.b;
  const int pitch = b + 4;
  float* panel = lds;
  const int panels = b / RP;
  // all panels of one block on one XCD (workgroups are dealt to the 8 XCDs
  // round-robin), so that block's S is fetched into a single L2
  const int nwg = panels * p.count;
  const int loc = blockIdx.x - p.wg0;
  if (loc >= nwg) return;   // padding of the run to a multiple of 8 workgroups
  const int lid = (nwg % 8 == 0 && p.wg0 % 8 == 0) ? (loc % 8) * (nwg / 8) + loc / 8 : loc;
  const int blk = lid / panels;
  const int r0 = (lid - blk * panels) * RP;
  const long long bb = (long long)b * b;
  const long long moff = blk * bb;                 // this block inside the run
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
  const int k = cb.k;

  // initial panel
  float keep[MT][NT][4];   // G (ABAR) or the running Q (BUILD) in accumulator layout
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int tile = wave + 4 * t;
#pragma unroll
      for (int v = 0; v < 4; ++v) keep[mt][t][v] = 0.0f;
      if (tile >= ntiles) continue;
      const int col = tile * 16 + li;
      float4 at;   // TCHAIN: A_{k+1}^T panel rows 16 mt + 4 lk + 0..3 = A_{k+1}[col][r0 + ...]
      if (MODE == 2)
        at = load_t4(p.G + (long long)k * p.stride + moff + (long long)col * b + r0 + 16 * mt + 4 * lk);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 16 * mt + 4 * lk + v;
        const long long o = (long long)(r0 + row) * b + col;
        float x;
        if (MODE == 0) {
          x = S[o];
          keep[mt][t][v] = (r0 + row == col ? 1.0f : 0.0f) + coef(1, k) * x;
        } else if (MODE == 1) {
          const float g = p.G[moff + o];
          keep[mt][t][v] = g;
          x = coef(k + 1, k) * g;
          p.out[(long long)k * p.stride + moff + o] = x;
        } else {
          x = f4(at, v);
        }
        panel[row * pitch + col] = x;
      }
    }

  const int nsteps = k;   // BUILD: j = 2..k+1; ABAR, TCHAIN: j = k..1
  for (int st = 0; st < nsteps; ++st) {
    f32x4 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[mt][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    __syncthreads();          // panel of the previous step written
    {
      // B operand straight from L2 into registers, U K-steps ahead; several
      // workgroups per CU hide the latency. Raw buffer loads over this block's S:
      // a per-lane byte offset for each column tile plus the K-step's row offset
      // in a scalar register (no 64-bit address per load), range-checked by the
      // hardware against the block's b * b floats.
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(S), (short)0, (int)(bb * 4), 0x00020000);
      int voff[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) voff[t] = (lk * b + bcol[t] + li) * 4;
      auto ldb = [&](int t, int krow) {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, voff[t], krow * b * 4, 0));
      };
      float bn[U][NT];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int t = 0; t < NT; ++t) bn[u][t] = ldb(t, 4 * u);
      for (int kc = 0; kc < b; kc += 4 * U) {
        float bc[U][NT];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int t = 0; t < NT; ++t) bc[u][t] = bn[u][t];
        const int kn = min(kc + 4 * U, b - 4 * U);   // clamped: the last prefetch is unused
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int t = 0; t < NT; ++t) bn[u][t] = ldb(t, kn + 4 * u);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float a[MT];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) a[mt] = panel[(16 * mt + li) * pitch + kc + 4 * u + lk];
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[mt], bc[u][t], acc[mt][t], 0, 0, 0);
        }
      }
    }
    __syncthreads();          // every wave has finished reading the panel
    const int j = (MODE == 0) ? st + 2 : k - st;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int tile = wave + 4 * t;
        if (tile >= ntiles) continue;
        const int col = tile * 16 + li;
        float4 at;
        if (MODE == 2)
          at = load_t4(p.G + (long long)(j - 1) * p.stride + moff + (long long)col * b + r0 + 16 * mt + 4 * lk);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = 16 * mt + 4 * lk + v;
          float x = acc[mt][t][v];
          if (MODE == 0) {
            keep[mt][t][v] += coef(j, k) * x;
          } else if (MODE == 1) {
            x = coef(j, k) * keep[mt][t][v] - x;
            p.out[(long long)(j - 1) * p.stride + moff + (long long)(r0 + row) * b + col] = x;
          } else {
            x += f4(at, v);
          }
          panel[row * pitch + col] = x;
        }
      }
  }
  __syncthreads();

  if (MODE == 0 || MODE == 2) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int tile = wave + 4 * t;
        if (tile >= ntiles) continue;
        const int col = tile * 16 + li;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = 16 * mt + 4 * lk + v;
          const long long o = moff + (long long)(r0 + row) * b + col;
          const float x = (MODE == 0) ? keep[mt][t][v] : panel[row * pitch + col];
          p.out[o] = x;
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

template <int MODE, int NT, int MT>
hipError_t launch_class(ChainBatch cb, hipStream_t s) {
  constexpr int RP = 16 * MT;
  int wg = 0, bmax = 0;
  for (int i = 0; i < cb.n; ++i) {
    cb.e[i].wg0 = wg;
    // runs start on a multiple of 8 workgroups so the XCD-aware order applies
    wg += (cb.e[i].b / RP * cb.e[i].count + 7) / 8 * 8;
    bmax = max(bmax, cb.e[i].b);
  }
  if (wg == 0) return hipSuccess;
  // b % 16 == 0: the prefetch of U = 4 K-steps of 4 rows stays inside S; the
  // chains prefetch 8 K-steps when every b is a multiple of 32 (the loads from
  // L2 are what the waves wait on: 16 K-steps was slower again)
  bool deep = true;
  for (int i = 0; i < cb.n; ++i)
    if (cb.e[i].b % 32) deep = false;
  const size_t lds = (size_t)RP * (bmax + 4) * sizeof(float);
  if (deep)
    hipLaunchKernelGGL((chain_kernel<MODE, NT, MT, 8>), dim3(wg), dim3(kThreads), lds, s, cb);
  else
    hipLaunchKernelGGL((chain_kernel<MODE, NT, MT, 4>), dim3(wg), dim3(kThreads), lds, s, cb);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(const ChainBatch& all, hipStream_t s) {
  // one launch per size class (column tiles per wave, and panels of 32 rows
  // where b allows them: each B value then feeds two row tiles)
  for (int nt = 1; nt <= 8; nt *= 2)
    for (int mt = 1; mt <= 2; ++mt) {
      ChainBatch cb;
      cb.n = 0;
      cb.k = all.k;
      for (int i = 0; i < all.n; ++i) {
        const int need = (all.e[i].b / 16 + 3) / 4;
        const int cls = need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : 8;
        // 32-row panels wherever b allows them (with S read through buffer loads
        // the extra accumulators still leave 2-3 waves per SIMD)
        const int m = (all.e[i].b % 32 == 0 && cls <= 4) ? 2 : 1;
        if (cls == nt && m == mt) cb.e[cb.n++] = all.e[i];
      }
      if (cb.n == 0) continue;
      hipError_t e;
      if (mt == 1) {
        if (nt == 1) e = launch_class<MODE, 1, 1>(cb, s);
        else if (nt == 2) e = launch_class<MODE, 2, 1>(cb, s);
        else if (nt == 4) e = launch_class<MODE, 4, 1>(cb, s);
        else e = launch_class<MODE, 8, 1>(cb, s);
      } else {
        if (nt == 1) e = launch_class<MODE, 1, 2>(cb, s);
        else if (nt == 2) e = launch_class<MODE, 2, 2>(cb, s);
        else e = launch_class<MODE, 4, 2>(cb, s);
      }
      if (e != hipSuccess) return e;
    }
  return hipSuccess;
}

}  // namespace

// b % 16 == 0 keeps every row of S a whole number of float4 and every 16-row
// chunk a whole number of per-thread loads (b = 16 .. 512).
bool chain_supported(int b) { return b % 16 == 0 && b >= 16 && b <= 512; }

hipError_t launch_chain_batch(int mode, const ChainBatch& cb, hipStream_t s) {
  if (cb.n < 0 || cb.n > kChainMaxEntries) return hipErrorInvalidValue;
  for (int i = 0; i < cb.n; ++i)
    if (!chain_supported(cb.e[i].b) || cb.e[i].count <= 0) return hipErrorInvalidValue;
  switch (mode) {
    case CHAIN_BUILD: return launch_mode<0>(cb, s);
    case CHAIN_ABAR: return launch_mode<1>(cb, s);
    case CHAIN_TCHAIN: return launch_mode<2>(cb, s);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- batched unpack / pack

namespace {

// Workgroup w belongs to the last entry whose first workgroup is <= w.
__device__ __forceinline__ TriEntry select_tri(const TriBatch& tb, int w) {
  TriEntry r = tb.e[0];
#pragma unroll
  for (int i = 1; i < kChainMaxEntries; ++i)
    if (i < tb.n && w >= tb.e[i].e0) r = tb.e[i];
  return r;
}

__device__ __forceinline__ long long tri_off(int i, int j, int b) {
  return (long long)i * b - ((long long)i * (i + 1)) / 2 + (j - i - 1);
}

// Rows of one block handled by one workgroup of the unpack / pack kernels; the
// mirrored half of those rows is a strip of kTriRows columns, staged in LDS
// with a padded pitch so that the transposed reads are conflict-free.
constexpr int kTriRows = 16;
constexpr int kTriPitch = kTriRows + 1;

struct TriWork {
  TriEntry t;
  int g, r0;
};
__device__ __forceinline__ TriWork tri_work(const TriBatch& tb) {
  TriWork w;
  w.t = select_tri(tb, blockIdx.x);
  const int tiles = w.t.b / kTriRows;
  const int loc = blockIdx.x - (int)w.t.e0;
  w.g = loc / tiles;
  w.r0 = (loc - w.g * tiles) * kTriRows;
  return w;
}

// S[r][c] = theta(r, c) above the diagonal, -theta(c, r) below, 0 on it, for
// rows r0 .. r0 + 15 of one block. Above the diagonal each row is a contiguous
// run of packed parameters; below it the values come from the 16 packed columns
// r0 .. r0 + 15 (rows 0 .. r0 + 15), read row-wise into LDS and used transposed.
__global__ __launch_bounds__(kThreads) void unpack_batch_kernel(TriBatch tb) {
  extern __shared__ float strip[];   // [largest b of the batch][kTriPitch]
  const TriWork w = tri_work(tb);
  const int b = w.t.b, r0 = w.r0;
  const float* th = w.t.src + (long long)w.g * ((long long)b * (b - 1) / 2);
  float* S = w.t.dst + (long long)w.g * b * b;
  const int nrow = r0 + kTriRows;
  for (int idx = threadIdx.x; idx < nrow * kTriRows; idx += kThreads) {
    const int c = idx / kTriRows, j = idx % kTriRows;
    const int col = r0 + j;
    strip[c * kTriPitch + j] = c < col ? th[tri_off(c, col, b)] : 0.0f;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int j = wave; j < kTriRows; j += kThreads / 64) {
    const int r = r0 + j;
    float* row = S + (long long)r * b;
    const float* up = th + (tri_off(r, r + 1, b) - (r + 1));   // theta(r, c) = up[c], c > r
    for (int c = lane; c < b; c += 64) {
      float v = 0.0f;
      if (c > r) v = up[c];
      else if (c < r) v = -strip[c * kTriPitch + j];
      row[c] = v;
    }
  }
}

// g(r, c) = sign * (M[r][c] - M[c][r]) for r < c, packed rows r0 .. r0 + 15 of
// one block. M[c][r] (c > r) comes from columns r0 .. r0 + 15 of rows
// r0 .. b - 1, read row-wise into LDS and used transposed.
__global__ __launch_bounds__(kThreads) void pack_batch_kernel(TriBatch tb) {
  extern __shared__ float strip[];   // [largest b of the batch][kTriPitch]
  const TriWork w = tri_work(tb);
  const int b = w.t.b, r0 = w.r0;
  const float* M = w.t.src + (long long)w.g * b * b;
  float* out = w.t.dst + (long long)w.g * ((long long)b * (b - 1) / 2);
  const int nrow = b - r0;
  for (int idx = threadIdx.x; idx < nrow * kTriRows; idx += kThreads) {
    const int cl = idx / kTriRows, j = idx % kTriRows;
    strip[cl * kTriPitch + j] = M[(long long)(r0 + cl) * b + r0 + j];
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float sign = tb.sign;
  for (int j = wave; j < kTriRows; j += kThreads / 64) {
    const int r = r0 + j;
    const float* row = M + (long long)r * b;
    float* dst = out + (tri_off(r, r + 1, b) - (r + 1));   // g(r, c) = dst[c], c > r
    for (int c = r + 1 + lane; c < b; c += 64)
      dst[c] = sign * (row[c] - strip[(c - r0) * kTriPitch + j]);
  }
}

// First workgroup of every entry; returns the total (blocks x row strips).
long long fill_offsets(TriBatch& tb) {
  long long tot = 0;
  for (int i = 0; i < tb.n; ++i) {
    tb.e[i].e0 = tot;
    tot += (long long)tb.e[i].count * (tb.e[i].b / kTriRows);
  }
  return tot;
}

// LDS of one workgroup: a strip of kTriRows columns over at most b rows, sized
// for the batch (a fixed 512-row strip held b = 256 batches to half the
// workgroups per CU).
size_t strip_bytes(const TriBatch& tb) {
  int bmax = 0;
  for (int i = 0; i < tb.n; ++i) bmax = max(bmax, tb.e[i].b);
  return (size_t)bmax * kTriPitch * sizeof(float);
}

bool tri_batch_ok(const TriBatch& tb) {
  if (tb.n > kChainMaxEntries) return false;
  for (int i = 0; i < tb.n; ++i)
    if (!chain_supported(tb.e[i].b) || tb.e[i].count < 1) return false;
  return true;
}

}  // namespace

hipError_t launch_unpack_batch(const TriBatch& in, hipStream_t s) {
  if (in.n <= 0) return hipSuccess;
  if (!tri_batch_ok(in)) return hipErrorInvalidValue;
  TriBatch tb = in;
  const long long wgs = fill_offsets(tb);
  if (wgs > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(unpack_batch_kernel, dim3((unsigned)wgs), dim3(kThreads), strip_bytes(tb), s, tb);
  return hipGetLastError();
}

hipError_t launch_pack_batch(const TriBatch& in, hipStream_t s) {
  if (in.n <= 0) return hipSuccess;
  if (!tri_batch_ok(in)) return hipErrorInvalidValue;
  TriBatch tb = in;
  const long long wgs = fill_offsets(tb);
  if (wgs > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_batch_kernel, dim3((unsigned)wgs), dim3(kThreads), strip_bytes(tb), s, tb);
  return hipGetLastError();
}

}  // namespace poetx
