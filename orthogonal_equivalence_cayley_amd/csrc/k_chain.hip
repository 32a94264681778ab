// Power chains of the Cayley-Neumann parameterisation on the gfx950 matrix
// cores ([PX] = page "POET-X: Memory-efficient LLM Training by Scaling
// Orthogonal Transformation", Résumé technique §2.D: the Neumann series is
// evaluated in one fused kernel with its operands kept on chip): fp32 plans on
// v_mfma_f32_16x16x4_f32; bf16 plans on split bf16 products (three
// v_mfma_f32_32x32x16_bf16 per product, see chain_split_kernel).
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

  // initial panel: every load first (out may alias G, so no load moves above a
  // store; a load under a branch waits for its value there); tiles past the
  // last one read the clamped columns and are dropped
  float keep[MT][NT][4];   // G (ABAR) or the running Q (BUILD) in accumulator layout
  float x0[MT][NT][4];     // the panel's values
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int col = bcol[t] + li;
      if constexpr (MODE == 2) {
        // A_{k+1}^T panel rows 16 mt + 4 lk + 0..3 = A_{k+1}[col][r0 + ...]
        const float4 at =
            load_t4(p.G + (long long)k * p.stride + moff + (long long)col * b + r0 + 16 * mt + 4 * lk);
#pragma unroll
        for (int v = 0; v < 4; ++v) x0[mt][t][v] = f4(at, v);
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const long long o = (long long)(r0 + 16 * mt + 4 * lk + v) * b + col;
          x0[mt][t][v] = MODE == 0 ? S[o] : p.G[moff + o];
        }
      }
    }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const bool valid = wave + 4 * t < ntiles;
      const int col = bcol[t] + li;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 16 * mt + 4 * lk + v;
        const long long o = (long long)(r0 + row) * b + col;
        float x = x0[mt][t][v];
        if (MODE == 0) {
          keep[mt][t][v] = valid ? (r0 + row == col ? 1.0f : 0.0f) + coef(1, k) * x : 0.0f;
        } else if (MODE == 1) {
          keep[mt][t][v] = valid ? x : 0.0f;
          x = coef(k + 1, k) * x;
          if (valid) p.out[(long long)k * p.stride + moff + o] = x;
        } else {
          keep[mt][t][v] = 0.0f;
        }
        if (valid) panel[row * pitch + col] = x;
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

// ---- split bf16 products (bf16 plans). Every product X S of a chain runs as
// Xh Mh + Xh Ml + Xl Mh on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16,
// fp32 accumulation), where X = Xh + Xl and M = -S = S^T = Mh + Ml are split
// into a bf16 value and its bf16 residual (16 significant bits together); the
// dropped Xl Ml and the two residual roundings leave about 2^-15 relative error
// per product term, next to the bf16 rounding the activation path applies to Q.
// One workgroup owns 32 rows of one block; the panel sits in LDS as its two bf16
// halves (row pitch b + 8, so that the 16 rows read by one pass of a fragment
// read fall in distinct banks); S^T streams from L2 as the MFMA A operand,
// stored by the unpack in fragment order (one contiguous KiB per operand load).
// Each lane holds 4 consecutive columns of one panel row per 32 x 32 output tile.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ void split4(float4 x, uint2& h, uint2& l) {
  const __bf16 h0 = static_cast<__bf16>(x.x), h1 = static_cast<__bf16>(x.y);
  const __bf16 h2 = static_cast<__bf16>(x.z), h3 = static_cast<__bf16>(x.w);
  const __bf16 l0 = static_cast<__bf16>(x.x - static_cast<float>(h0));
  const __bf16 l1 = static_cast<__bf16>(x.y - static_cast<float>(h1));
  const __bf16 l2 = static_cast<__bf16>(x.z - static_cast<float>(h2));
  const __bf16 l3 = static_cast<__bf16>(x.w - static_cast<float>(h3));
  auto u = [](__bf16 v) { return (uint32_t)__builtin_bit_cast(uint16_t, v); };
  h = make_uint2(u(h0) | (u(h1) << 16), u(h2) | (u(h3) << 16));
  l = make_uint2(u(l0) | (u(l1) << 16), u(l2) | (u(l3) << 16));
}

// NT 32-column tiles per wave (NW waves: 4 up to b = 256, 8 for b = 512, so
// that a wave's registers do not grow with b), U K-steps of 16 prefetched.
// BF: the block size when every entry of the launch has it (0: read per entry);
// with it fixed the K loop unrolls completely and each operand load is waited
// for exactly (in a rolled loop the compiler waits for every load each pass).
template <int MODE, int NT, int U, int BF, int NW = 4>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void chain_split_kernel(ChainBatch cb) {
  constexpr int RP = 32;
  extern __shared__ __align__(16) float lds[];
  const ChainEntry p = select_entry(cb);
  const int b = BF ? BF : p.b;
  const int pitch = b + 8;                         // bf16 elements per panel row
  uint16_t* const ph = reinterpret_cast<uint16_t*>(lds);
  uint16_t* const pl = ph + RP * pitch;
  const int panels = b / RP;
  const int nwg = panels * p.count;
  const int loc = blockIdx.x - p.wg0;
  if (loc >= nwg) return;   // padding of the run to a multiple of 8 workgroups
  // all panels of one block on one XCD, so that block's S^T is fetched into one L2
  const int lid = (nwg % 8 == 0 && p.wg0 % 8 == 0) ? (loc % 8) * (nwg / 8) + loc / 8 : loc;
  const int blk = lid / panels;
  const int r0 = (lid - blk * panels) * RP;
  const long long bb = (long long)b * b;
  const long long moff = blk * bb;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ntiles = b / 32;
  const int l32 = lane & 31, hf = lane >> 5;
  const int k = cb.k;
  // first column of each of this wave's tiles; tiles past the last one are
  // clamped onto it (the MFMA loop stays branch-free; their results are dropped)
  int n0[NT];
  bool valid[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    valid[t] = wave + NW * t < ntiles;
    n0[t] = min(wave + NW * t, ntiles - 1) * 32;
  }
  // this lane's panel row and its 4-column groups: row l32, columns n0 + 8 q + 4 hf + 0..3
  const int row = l32;
  const long long rowg = (long long)(r0 + row) * b;   // element offset of the row in a block

  // M = -S = S^T split into bf16 value and residual, in fragment order
  const uint16_t* Mh = p.Mh + moff;
  const uint16_t* Ml = p.Mh + (long long)p.count * bb + moff;
  const __amdgpu_buffer_rsrc_t rh =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Mh), (short)0, (int)(bb * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rl =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Ml), (short)0, (int)(bb * 2), 0x00020000);
  // fragment order: the 1 KiB of (tile n0 / 32, K-step kc / 16) at
  // ((n0 / 32) (b / 16) + kc / 16) KiB, this lane's 16 bytes at 16 lane
  int tbase[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) tbase[t] = (n0[t] >> 5) * (b >> 4) * 1024;
  const int voff = lane * 16;
  auto ldm = [&](const __amdgpu_buffer_rsrc_t& r, int t, int kc) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, tbase[t] + kc * 64, 0));
  };

  // the first U K-steps of M for the first step; later steps get theirs from
  // the previous step's last pass (M is the same in every step)
  bf16x8 bnh[U][NT], bnl[U][NT];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      bnh[u][t] = ldm(rh, t, 16 * u);
      bnl[u][t] = ldm(rl, t, 16 * u);
    }

  float keep[NT][16];   // running Q (BUILD) or G (ABAR), accumulator layout
  float last[NT][16];   // TCHAIN: the latest panel in fp32
  auto put_panel = [&](int t, int q, float4 x) {
    uint2 h, l;
    split4(x, h, l);
    const int c = n0[t] + 8 * q + 4 * hf;
    *reinterpret_cast<uint2*>(ph + row * pitch + c) = h;
    *reinterpret_cast<uint2*>(pl + row * pitch + c) = l;
  };
  // initial panel
  if constexpr (MODE == 0) {
    // the panel is S: its rows r0 .. r0 + 31 are the negated rows of M, which
    // the 1 KiB fragment blocks of tile r0 / 32 hold (lane l: row l % 32, the 8
    // columns from 16 ks + 8 (l / 32) in K-step ks); negating bf16 is exact.
    // Each wave copies K-steps wave, wave + NW, ... (b <= 64 NW: at most 4); loads
    // past the block's last K-step are not stored (those past the block's end
    // read zeros: buffer loads are range-checked)
    const int nk = b >> 4;
    const int rb = (r0 >> 5) * nk * 1024;
    uint4 fh[4], fl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ks = wave + NW * i;
      fh[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rh, voff, rb + ks * 1024, 0));
      fl[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rl, voff, rb + ks * 1024, 0));
    }
    constexpr uint32_t kNeg = 0x80008000u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ks = wave + NW * i;
      if (ks < nk) {
        const int c = 16 * ks + 8 * hf;
        *reinterpret_cast<uint4*>(ph + row * pitch + c) =
            make_uint4(fh[i].x ^ kNeg, fh[i].y ^ kNeg, fh[i].z ^ kNeg, fh[i].w ^ kNeg);
        *reinterpret_cast<uint4*>(pl + row * pitch + c) =
            make_uint4(fl[i].x ^ kNeg, fl[i].y ^ kNeg, fl[i].z ^ kNeg, fl[i].w ^ kNeg);
      }
    }
    __syncthreads();
    // the running sum I + c_1 S, S = value + residual read back from the panel
    const float c1 = coef(1, k);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = n0[t] + 8 * q + 4 * hf;
        const uint2 h = *reinterpret_cast<const uint2*>(ph + row * pitch + c);
        const uint2 l = *reinterpret_cast<const uint2*>(pl + row * pitch + c);
        const uint32_t hv[4] = {h.x << 16, h.x & 0xffff0000u, h.y << 16, h.y & 0xffff0000u};
        const uint32_t lv[4] = {l.x << 16, l.x & 0xffff0000u, l.y << 16, l.y & 0xffff0000u};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          keep[t][4 * q + e] = (r0 + row == c + e ? 1.0f : 0.0f) +
                               c1 * (__uint_as_float(hv[e]) + __uint_as_float(lv[e]));
      }
  } else {
    // every load first: out may alias G, so no load moves above a store
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = n0[t] + 8 * q + 4 * hf;
        if constexpr (MODE == 1) {
          const float4 g = *reinterpret_cast<const float4*>(p.G + moff + rowg + c);
          keep[t][4 * q + 0] = g.x; keep[t][4 * q + 1] = g.y;
          keep[t][4 * q + 2] = g.z; keep[t][4 * q + 3] = g.w;
        } else {
          // A_{k+1}^T: element (row, c + e) = A_{k+1}[c + e][r0 + row]
          const float* A = p.G + (long long)k * p.stride + moff + r0 + row;
#pragma unroll
          for (int e = 0; e < 4; ++e) last[t][4 * q + e] = A[(long long)(c + e) * b];
        }
      }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = n0[t] + 8 * q + 4 * hf;
        float4 x;
        if constexpr (MODE == 1) {
          const float ck = coef(k + 1, k);
          x = make_float4(ck * keep[t][4 * q], ck * keep[t][4 * q + 1], ck * keep[t][4 * q + 2],
                          ck * keep[t][4 * q + 3]);
          if (valid[t]) *reinterpret_cast<float4*>(p.out + (long long)k * p.stride + moff + rowg + c) = x;
        } else {
          x = make_float4(last[t][4 * q], last[t][4 * q + 1], last[t][4 * q + 2], last[t][4 * q + 3]);
        }
        if (valid[t]) put_panel(t, q, x);
      }
    }
  }

  for (int st = 0; st < k; ++st) {
    f32x16 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[t][v] = 0.0f;
    const int j = (MODE == 0) ? st + 2 : k - st;
    // TCHAIN: this step's A_j^T values (element (row, c) = A_j[c][r0 + row]),
    // loaded before the multiplies so that their latency hides behind them
    float at[MODE == 2 ? NT : 1][MODE == 2 ? 16 : 1];
    if (MODE == 2) {
      const float* A = p.G + (long long)(j - 1) * p.stride + moff + r0 + row;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            at[t][4 * q + e] = A[(long long)(n0[t] + 8 * q + 4 * hf + e) * b];
    }
    __syncthreads();   // panel of the previous step written
    // (the launcher picks U so that 16 U divides b: no pass runs past the block)
    constexpr int kUnroll = BF > 0 ? BF / 16 : 1;
#pragma unroll kUnroll
    for (int kc = 0; kc < b; kc += 16 * U) {
      bf16x8 bch[U][NT], bcl[U][NT];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          bch[u][t] = bnh[u][t];
          bcl[u][t] = bnl[u][t];
        }
      // the last pass fetches the first K-steps again, for the next step
      const int kn = kc + 16 * U < b ? kc + 16 * U : 0;
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          bnh[u][t] = ldm(rh, t, kn + 16 * u);
          bnl[u][t] = ldm(rl, t, kn + 16 * u);
        }
      // keep the next loads ahead of these multiplies (the scheduler would sink
      // them to their uses)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kk = kc + 16 * u + 8 * hf;
        const bf16x8 ah = *reinterpret_cast<const bf16x8*>(ph + row * pitch + kk);
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(pl + row * pitch + kk);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bcl[u][t], ah, acc[t], 0, 0, 0);
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bch[u][t], al, acc[t], 0, 0, 0);
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bch[u][t], ah, acc[t], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();   // every wave has finished reading the panel
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = n0[t] + 8 * q + 4 * hf;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = acc[t][4 * q + e];
        if (MODE == 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e) keep[t][4 * q + e] += coef(j, k) * x[e];
        } else if (MODE == 1) {
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = coef(j, k) * keep[t][4 * q + e] - x[e];
          if (valid[t])
            *reinterpret_cast<float4*>(p.out + (long long)(j - 1) * p.stride + moff + rowg + c) =
                make_float4(x[0], x[1], x[2], x[3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[e] += at[MODE == 2 ? t : 0][MODE == 2 ? 4 * q + e : 0];
            last[t][4 * q + e] = x[e];
          }
        }
        if (valid[t] && st + 1 < k) put_panel(t, q, make_float4(x[0], x[1], x[2], x[3]));
      }
    }
  }

  if (MODE == 0 || MODE == 2) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (!valid[t]) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = n0[t] + 8 * q + 4 * hf;
        const float* src = MODE == 0 ? keep[t] : last[t];
        const float4 x = make_float4(src[4 * q], src[4 * q + 1], src[4 * q + 2], src[4 * q + 3]);
        *reinterpret_cast<float4*>(p.out + moff + rowg + c) = x;
        if (MODE == 0 && p.out_act) {
          if (p.act_bf16) {
            uint2 h, l;
            split4(x, h, l);
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out_act) + moff + rowg + c) = h;
          } else {
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.out_act) + moff + rowg + c) = x;
          }
        }
      }
    }
  }
}

template <int MODE, int NT, int NW = 4>
hipError_t launch_split_class(ChainBatch cb, hipStream_t s) {
  constexpr int RP = 32;
  int wg = 0, bmax = 0, bmin = 1 << 30;
  bool by64 = true;
  for (int i = 0; i < cb.n; ++i) {
    cb.e[i].wg0 = wg;
    wg += (cb.e[i].b / RP * cb.e[i].count + 7) / 8 * 8;
    bmax = max(bmax, cb.e[i].b);
    bmin = min(bmin, cb.e[i].b);
    by64 = by64 && cb.e[i].b % 64 == 0;
  }
  if (wg == 0) return hipSuccess;
  const size_t lds = (size_t)2 * RP * (bmax + 8) * sizeof(uint16_t);
  // each pass of the K loop takes U K-steps of 16, so 16 U must divide every b
  // (b % 32 == 0 always allows U = 2; mixed sizes: the transposed chain's extra
  // loads leave registers for two steps only)
  constexpr int UM = MODE == 2 ? 2 : 4;
  const dim3 blk(NW * 64);
  if (NW == 8 && bmin == 512 && bmax == 512)
    hipLaunchKernelGGL((chain_split_kernel<MODE, NT, 4, 512, NW>), dim3(wg), blk, lds, s, cb);
  else if (NW == 4 && bmin == 256 && bmax == 256)
    hipLaunchKernelGGL((chain_split_kernel<MODE, NT, 4, 256, NW>), dim3(wg), blk, lds, s, cb);
  else if (UM == 2 || by64)
    hipLaunchKernelGGL((chain_split_kernel<MODE, NT, UM, 0, NW>), dim3(wg), blk, lds, s, cb);
  else
    hipLaunchKernelGGL((chain_split_kernel<MODE, NT, 2, 0, NW>), dim3(wg), blk, lds, s, cb);
  return hipGetLastError();
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
  // (eight column tiles per wave leave no registers for the deeper prefetch)
  constexpr int UD = NT < 8 ? 8 : 4;
  if (deep)
    hipLaunchKernelGGL((chain_kernel<MODE, NT, MT, UD>), dim3(wg), dim3(kThreads), lds, s, cb);
  else
    hipLaunchKernelGGL((chain_kernel<MODE, NT, MT, 4>), dim3(wg), dim3(kThreads), lds, s, cb);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(const ChainBatch& all, hipStream_t s) {
  // split bf16 products: one launch per class of 32-column tiles per wave
  for (int nt = 1; nt <= 2; ++nt) {
    ChainBatch cb;
    cb.n = 0;
    cb.k = all.k;
    for (int i = 0; i < all.n; ++i) {
      const ChainEntry& e = all.e[i];
      if (!e.Mh || !chain_split_supported(e.b) || e.b > 256) continue;
      if ((e.b / 32 + 3) / 4 == nt) cb.e[cb.n++] = e;
    }
    if (cb.n == 0) continue;
    const hipError_t e = nt == 1 ? launch_split_class<MODE, 1>(cb, s) : launch_split_class<MODE, 2>(cb, s);
    if (e != hipSuccess) return e;
  }
  {
    // blocks of 288 .. 512: 8 waves of up to two 32-column tiles each
    ChainBatch cb;
    cb.n = 0;
    cb.k = all.k;
    for (int i = 0; i < all.n; ++i)
      if (all.e[i].Mh && chain_split_supported(all.e[i].b) && all.e[i].b > 256) cb.e[cb.n++] = all.e[i];
    if (cb.n > 0) {
      const hipError_t e = launch_split_class<MODE, 2, 8>(cb, s);
      if (e != hipSuccess) return e;
    }
  }
  // one launch per size class (column tiles per wave, and panels of 32 rows
  // where b allows them: each B value then feeds two row tiles)
  for (int nt = 1; nt <= 8; nt *= 2)
    for (int mt = 1; mt <= 2; ++mt) {
      ChainBatch cb;
      cb.n = 0;
      cb.k = all.k;
      for (int i = 0; i < all.n; ++i) {
        if (all.e[i].Mh && chain_split_supported(all.e[i].b)) continue;   // launched above
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
// 32-row panels and 32-column tiles; at most two tiles per wave (8 waves above 256)
bool chain_split_supported(int b) { return b % 32 == 0 && b >= 32 && b <= 512; }

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

// Split operand of the bf16 chains in MFMA fragment order: for 32-row tile nt of
// M and K-step kc (16 columns), 64 lanes x 8 bf16 = 1 KiB, lane r + 32 h holding
// M[32 nt + r][16 kc + 8 h .. + 7]; so each operand load is one contiguous read.
[[maybe_unused]] __device__ __forceinline__ long long split_frag_offset(int n, int k, int b) {
  const int nt = n >> 5, r = n & 31, kc = k >> 4, h = (k >> 3) & 1, e = k & 7;
  return ((((long long)nt * (b >> 4) + kc) * 64) + r + 32 * h) * 8 + e;
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
// Loads are unconditional range-checked buffer loads issued in batches (a load
// under a branch would wait for its value there); strip rows past the block go
// to a spare LDS row and stores past a row's end to an offset outside the
// buffer, which the hardware drops. NI: 64-column passes per row (b <= 64 NI).
template <int NI>
__global__ __launch_bounds__(kThreads) void unpack_batch_kernel(TriBatch tb) {
  extern __shared__ float strip[];   // [largest b of the batch + 1][kTriPitch]
  const TriWork w = tri_work(tb);
  const int b = w.t.b, r0 = w.r0;
  const float* th = w.t.src + (long long)w.g * ((long long)b * (b - 1) / 2);
  float* S = w.t.dst + (long long)w.g * b * b;
  const __amdgpu_buffer_rsrc_t rth =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(th), (short)0, b * (b - 1) / 2 * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(S, (short)0, b * b * 4, 0x00020000);
  auto ld = [&](int idx) {   // theta[idx] of the block, 0 outside it
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rth, max(idx, 0) * 4, 0, 0));
  };
  const int tid = threadIdx.x;
  const int nrow = r0 + kTriRows;
  for (int base = 0; base < nrow * kTriRows; base += 8 * kThreads) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = base + u * kThreads + tid;
      const int c = idx / kTriRows, col = r0 + idx % kTriRows;
      v[u] = ld((int)tri_off(min(c, b - 1), col, b));
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = base + u * kThreads + tid;
      const int c = idx / kTriRows, j = idx % kTriRows;
      strip[min(c, b) * kTriPitch + j] = c < r0 + j ? v[u] : 0.0f;   // row b: the spare row
    }
  }
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6;
  constexpr int kRowsPerWave = kTriRows / (kThreads / 64);
  float up[kRowsPerWave][NI];
#pragma unroll
  for (int jj = 0; jj < kRowsPerWave; ++jj) {
    const int r = r0 + wave + 4 * jj;
    const int rs0 = (int)tri_off(r, r + 1, b) - (r + 1);   // theta(r, c) at rs0 + c, c > r
#pragma unroll
    for (int i = 0; i < NI; ++i) up[jj][i] = ld(rs0 + lane + 64 * i);
  }
#pragma unroll
  for (int jj = 0; jj < kRowsPerWave; ++jj) {
    const int j = wave + 4 * jj, r = r0 + j;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int c = lane + 64 * i;
      const float lo = -strip[min(c, b) * kTriPitch + j];
      const float v = c > r ? up[jj][i] : (c < r ? lo : 0.0f);
      const int off = c < b ? (r * b + c) * 4 : 0x7ffffff0;   // past the row: dropped
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rs, off, 0, 0);
    }
  }
}

// The split operand of the bf16 chains: M = -S = S^T, rows 32 nt .. 32 nt + 31
// of one block, rounded to bf16 values and residuals in fragment order
// (split_frag_offset). The tile of M is staged in LDS in fp32: above the
// diagonal, M[r][c] = -theta(r, c), one contiguous run of packed parameters per
// row; below it, M[r][c] = theta(c, r), 32 consecutive packed parameters of each
// row c < r (a 128-byte run), stored transposed. Each wave then writes whole
// 1 KiB fragment blocks of both halves.
constexpr int kSplitRows = 32;
// NP: 64-column passes per row (b <= 64 NP)
template <int NP>
__global__ __launch_bounds__(kThreads) void unpack_split_kernel(TriBatch tb) {
  extern __shared__ __align__(16) float tile[];   // [kSplitRows][b + 4]
  const TriEntry t = select_tri(tb, blockIdx.x);
  const int b = t.b;
  const int tiles = b / kSplitRows;
  const int n = t.count * tiles;
  const int loc = blockIdx.x - (int)t.e0;
  if (loc >= n) return;   // padding of the entry to a multiple of 8 workgroups
  // the tiles of one block on one XCD: each packed parameter is read twice (once
  // per triangle), the second time from that XCD's L2
  const int lid = (n % 8 == 0) ? (loc % 8) * (n / 8) + loc / 8 : loc;
  const int g = lid / tiles, nt = lid - g * tiles, R0 = nt * kSplitRows;
  const float* th = t.src + (long long)g * ((long long)b * (b - 1) / 2);
  const int pitch = b + 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // every load of both triangles is issued before the first LDS write (at most
  // 16 NP per lane), so that a workgroup waits for memory once. The
  // loads are unconditional range-checked buffer loads of the block's packed
  // parameters (an offset past the end reads 0) and the triangle tests select
  // among the loaded values: a load under a branch waits for its value there.
  const int nth = b * (b - 1) / 2;
  const __amdgpu_buffer_rsrc_t rth =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(th), (short)0, nth * 4, 0x00020000);
  auto ld = [&](int idx) {   // theta[idx], 0 outside the block
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rth, max(idx, 0) * 4, 0, 0));
  };
  // diagonal and above: rows R0 + wave + 4 jj, columns r .. b - 1 in NP
  // passes of 64 lanes; theta(r, c) at tri_off(r, c) = rs + c for c > r
  float vu[8][NP];
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const int r = R0 + wave + 4 * jj;
    const int rs = (int)tri_off(r, r + 1, b) - (r + 1);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int c = r + lane + 64 * i;
      const float v = ld(rs + c);
      vu[jj][i] = c > r ? -v : 0.0f;
    }
  }
  // below the diagonal: packed rows c < R0 + 31, two per wave instruction (half
  // a wave each), columns R0 + j with c < R0 + j
  const int j = lane & 31, col = R0 + j;
  float vl[NP][8];
#pragma unroll
  for (int pass = 0; pass < NP; ++pass)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = 64 * pass + 8 * u + 2 * wave + (lane >> 5);
      const float v = ld((int)tri_off(min(c, b - 1), col, b));
      vl[pass][u] = c < col ? v : 0.0f;
    }
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    const int jr = wave + 4 * jj, r = R0 + jr;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int c = r + lane + 64 * i;
      if (c < b) tile[jr * pitch + c] = vu[jj][i];
    }
  }
#pragma unroll
  for (int pass = 0; pass < NP; ++pass)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = 64 * pass + 8 * u + 2 * wave + (lane >> 5);
      if (c < col) tile[j * pitch + c] = vl[pass][u];
    }
  __syncthreads();
  uint16_t* mh = t.split + (long long)g * b * b;
  uint16_t* ml = mh + (long long)t.count * b * b;
  const int nk = b / 16;
  for (int ks = wave; ks < nk; ks += kThreads / 64) {
    const float* src = tile + (lane & 31) * pitch + 16 * ks + 8 * (lane >> 5);
    uint2 h0, l0, h1, l1;
    split4(*reinterpret_cast<const float4*>(src), h0, l0);
    split4(*reinterpret_cast<const float4*>(src + 4), h1, l1);
    const long long o = ((long long)(nt * nk + ks) * 64 + lane) * 8;
    *reinterpret_cast<uint4*>(mh + o) = make_uint4(h0.x, h0.y, h1.x, h1.y);
    *reinterpret_cast<uint4*>(ml + o) = make_uint4(l0.x, l0.y, l1.x, l1.y);
  }
}

// g(r, c) = sign * (M[r][c] - M[c][r]) for r < c, packed rows r0 .. r0 + 15 of
// one block. M[c][r] (c > r) comes from columns r0 .. r0 + 15 of rows
// r0 .. b - 1, read row-wise into LDS and used transposed. Loads are
// unconditional range-checked buffer loads issued in batches (a load under a
// branch would wait for its value there); strip rows past the block go to a
// spare LDS row and stores past a row's end to an offset outside the buffer,
// which the hardware drops. NI: 64-column passes per row (b <= 64 NI).
template <int NI>
__global__ __launch_bounds__(kThreads) void pack_batch_kernel(TriBatch tb) {
  extern __shared__ float strip[];   // [largest b of the batch + 1][kTriPitch]
  const TriWork w = tri_work(tb);
  const int b = w.t.b, r0 = w.r0;
  const float* M = w.t.src + (long long)w.g * b * b;
  float* out = w.t.dst + (long long)w.g * ((long long)b * (b - 1) / 2);
  const __amdgpu_buffer_rsrc_t rm =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(M), (short)0, b * b * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t ro =
      __builtin_amdgcn_make_buffer_rsrc(out, (short)0, b * (b - 1) / 2 * 4, 0x00020000);
  auto ldm = [&](int idx) {   // M[idx] of the block, 0 past its end
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rm, idx * 4, 0, 0));
  };
  const int nrow = b - r0;
  const int tid = threadIdx.x;
  for (int base = 0; base < nrow * kTriRows; base += 8 * kThreads) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = base + u * kThreads + tid;
      const int cl = idx / kTriRows, j = idx % kTriRows;
      v[u] = ldm((r0 + cl) * b + r0 + j);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = base + u * kThreads + tid;
      const int cl = idx / kTriRows, j = idx % kTriRows;
      strip[min(cl, b) * kTriPitch + j] = v[u];   // row b: the spare row
    }
  }
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6;
  const float sign = tb.sign;
  constexpr int kRowsPerWave = kTriRows / (kThreads / 64);
  float a[kRowsPerWave][NI];
#pragma unroll
  for (int jj = 0; jj < kRowsPerWave; ++jj) {
    const int r = r0 + wave + 4 * jj;
#pragma unroll
    for (int i = 0; i < NI; ++i) a[jj][i] = ldm(r * b + r + 1 + lane + 64 * i);
  }
#pragma unroll
  for (int jj = 0; jj < kRowsPerWave; ++jj) {
    const int j = wave + 4 * jj, r = r0 + j;
    const int rs = (int)tri_off(r, r + 1, b) - (r + 1);   // g(r, c) at rs + c, c > r
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int c = r + 1 + lane + 64 * i;
      const float g = sign * (a[jj][i] - strip[(min(c, b) - r0) * kTriPitch + j]);
      const int off = c < b ? (rs + c) * 4 : 0x7ffffff0;   // past the end: dropped
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, g), ro, off, 0, 0);
    }
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
  return (size_t)(bmax + 1) * kTriPitch * sizeof(float);
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
  // entries with an fp32 S (the strip kernel) and entries with a split (the
  // tile kernel; an entry with both goes to both)
  TriBatch tb = in, ts = in;
  tb.n = ts.n = 0;
  for (int i = 0; i < in.n; ++i) {
    const TriEntry& e = in.e[i];
    if (!e.dst && !e.split) return hipErrorInvalidValue;
    if (e.split && !chain_split_supported(e.b)) return hipErrorInvalidValue;
    if (e.dst) { tb.e[tb.n] = e; tb.e[tb.n++].split = nullptr; }
    if (e.split) { ts.e[ts.n] = e; ts.e[ts.n++].dst = nullptr; }
  }
  if (tb.n > 0) {
    const long long wgs = fill_offsets(tb);
    if (wgs > INT32_MAX) return hipErrorInvalidValue;
    int bmax = 0;
    for (int i = 0; i < tb.n; ++i) bmax = max(bmax, tb.e[i].b);
    if (bmax <= 256)
      hipLaunchKernelGGL(unpack_batch_kernel<4>, dim3((unsigned)wgs), dim3(kThreads), strip_bytes(tb), s, tb);
    else
      hipLaunchKernelGGL(unpack_batch_kernel<8>, dim3((unsigned)wgs), dim3(kThreads), strip_bytes(tb), s, tb);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (ts.n > 0) {
    // entries start on a multiple of 8 workgroups so the XCD-aware order applies
    long long wgs = 0;
    int bmax = 0;
    for (int i = 0; i < ts.n; ++i) {
      ts.e[i].e0 = wgs;
      wgs += ((long long)ts.e[i].count * (ts.e[i].b / kSplitRows) + 7) / 8 * 8;
      bmax = max(bmax, ts.e[i].b);
    }
    if (wgs > INT32_MAX) return hipErrorInvalidValue;
    const size_t lds = (size_t)kSplitRows * (bmax + 4) * sizeof(float);
    if (bmax <= 256)
      hipLaunchKernelGGL(unpack_split_kernel<4>, dim3((unsigned)wgs), dim3(kThreads), lds, s, ts);
    else
      hipLaunchKernelGGL(unpack_split_kernel<8>, dim3((unsigned)wgs), dim3(kThreads), lds, s, ts);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_pack_batch(const TriBatch& in, hipStream_t s) {
  if (in.n <= 0) return hipSuccess;
  if (!tri_batch_ok(in)) return hipErrorInvalidValue;
  TriBatch tb = in;
  const long long wgs = fill_offsets(tb);
  if (wgs > INT32_MAX) return hipErrorInvalidValue;
  int bmax = 0;
  for (int i = 0; i < tb.n; ++i) bmax = max(bmax, tb.e[i].b);
  if (bmax <= 256)
    hipLaunchKernelGGL(pack_batch_kernel<4>, dim3((unsigned)wgs), dim3(kThreads), strip_bytes(tb), s, tb);
  else
    hipLaunchKernelGGL(pack_batch_kernel<8>, dim3((unsigned)wgs), dim3(kThreads), strip_bytes(tb), s, tb);
  return hipGetLastError();
}

}  // namespace poetx
