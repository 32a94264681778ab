// Pipelined bf16 GEMM for gfx950 (v_mfma_f32_32x32x16_bf16, fp32 accumulate)
// used for the frozen-weight products and the batched block-diagonal products
// when the shapes are whole tiles ([PX] = page "POET-X: Memory-efficient LLM
// Training by Scaling Orthogonal Transformation", Résumé technique §2.A, §2.C).
//
// C(m,n) = sum_k A(m,k) B(n,k); each operand is K-contiguous ([rows, K]) or
// row-contiguous ([K, rows]).
//
//  * Tiles move HBM -> LDS with direct-to-LDS loads (global_load_lds_dwordx4):
//    no staging registers, two LDS stages, the next K tile in flight while the
//    current one is multiplied.
//  * A K-contiguous tile is stored as rows of LBK elements; a row-contiguous tile
//    as LBK rows of R elements. Each is XOR-swizzled in 16-byte units (the lane ->
//    address mapping of the loads picks the destination) so that fragment reads
//    hit distinct banks.
//  * Fragments: K-contiguous tiles are read with ds_read_b128; row-contiguous
//    tiles with two ds_read_b64_tr_b16 (the gfx950 transposing LDS read: within
//    16 lanes, lane p receives column p of a 4 x 16 block) per 8-element operand.
//  * 8 waves (two per SIMD), each owning a 128 x 64 (or 64 x 64) piece of the
//    tile. Workgroups are dealt to the 8 XCDs round-robin; each XCD gets a
//    contiguous range of tiles walked in groups of 4 tile-rows, so its resident
//    workgroups share A and B slices in that XCD's L2.
//
// Requirements (checked by the dispatcher): K % 64 == 0; M % BM == 0 when A is
// row-contiguous and N % BN == 0 when B is; 16-byte aligned rows. Rows past M or
// N of a K-contiguous operand are clamped (their results are not stored).
#include <type_traits>

#include "poetx_internal.h"

namespace poetx {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int GM = 4;   // tile-rows per group in the XCD-aware order

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Barrier that waits for this wave's LDS traffic only: the direct-to-LDS loads
// of later stages stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ void dma16(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                   (void __attribute__((address_space(3)))*)lds_dst, 16, 0, 0);
}

// ---- K-contiguous operand: R rows x KB elements, KB / 8 chunks of 16 B per row.
// Chunk c of row r sits at 16-byte slot r * CPR + (c ^ ((r / RPB) % CPR)), RPB rows
// per 256-byte bank line: the 16 rows read by one quarter-wave then cover all 64
// banks.
template <int R, int NT, int KB>
struct KTile {
  static constexpr int CPR = KB / 8;
  static constexpr int RPB = 256 / (KB * 2);
  static constexpr int SLOTS = R * CPR;
  static constexpr int L = SLOTS / NT;   // loads per thread per stage
  const uint16_t* src[L];
  __device__ __forceinline__ void init(const uint16_t* base, long long ld, int row0, int rows) {
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int s = i * NT + threadIdx.x;
      const int r = s / CPR, pos = s % CPR;
      const int c = pos ^ ((r / RPB) % CPR);
      const int gr = min(row0 + r, rows - 1);
      src[i] = base + (long long)gr * ld + c * 8;
    }
  }
  __device__ __forceinline__ void issue(unsigned char* st, int k0, int wave) const {
#pragma unroll
    for (int i = 0; i < L; ++i) dma16(src[i] + k0, st + (i * NT + wave * 64) * 16);
  }
  // 8 K-consecutive elements of row r at k = 16 * kk + 8 * half
  __device__ __forceinline__ static bf16x8 frag(const unsigned char* st, int r, int kk, int half) {
    const int c = 2 * kk + half;
    return *reinterpret_cast<const bf16x8*>(st + (r * CPR + (c ^ ((r / RPB) % CPR))) * 16);
  }
};

// ---- row-contiguous operand: KB K-rows x R elements (R / 8 chunks per K-row).
// Chunk c of K-row k sits at slot k * (R / 8) + (c ^ (4 * (k & 3))): the 4 K-rows x
// 4 chunks touched by 32 lanes of a transposing read fall in distinct banks.
template <int R, int NT, int KB>
struct MTile {
  static constexpr int CPR = R / 8;
  // the swizzle moves a chunk by up to 12 positions inside its K-row
  static_assert(CPR >= 16, "row-contiguous tiles need R >= 128");
  static constexpr int SLOTS = KB * CPR;
  static constexpr int L = SLOTS / NT;
  const uint16_t* src[L];
  __device__ __forceinline__ void init(const uint16_t* base, long long ld, int col0) {
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int s = i * NT + threadIdx.x;
      const int k = s / CPR, pos = s % CPR;
      const int c = pos ^ (4 * (k & 3));
      src[i] = base + (long long)k * ld + col0 + c * 8;
    }
  }
  __device__ __forceinline__ void issue(unsigned char* st, int k0, long long ld, int wave) const {
#pragma unroll
    for (int i = 0; i < L; ++i) dma16(src[i] + (long long)k0 * ld, st + (i * NT + wave * 64) * 16);
  }
  // operand for MFMA rows r0 .. r0 + 31 (lane & 31), k = 16 * kk + 8 * (lane >> 5) + 0..7
  __device__ __forceinline__ static bf16x8 frag(const unsigned char* st, int r0, int kk, int lane) {
    const int g = lane >> 4;                // 16-lane group
    const int s = lane & 15;                // source lane inside the group
    const int col = r0 + (g & 1) * 16 + 4 * (s & 3);
    const int kb = 16 * kk + 8 * (g >> 1) + (s >> 2);
    i16x4 lo, hi;
    {
      const int k = kb;
      const int c = (col >> 3) ^ (4 * (k & 3));
      lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(st + (k * CPR + c) * 16 + (col & 7) * 2));
    }
    {
      const int k = kb + 4;
      const int c = (col >> 3) ^ (4 * (k & 3));
      hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(st + (k * CPR + c) * 16 + (col & 7) * 2));
    }
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
  }
};

template <int R, int NT, int KB, bool KMAJ>
struct Tile;
template <int R, int NT, int KB>
struct Tile<R, NT, KB, true> {
  KTile<R, NT, KB> t;
  static constexpr int BYTES = KTile<R, NT, KB>::SLOTS * 16;
  static constexpr int L = KTile<R, NT, KB>::L;
  __device__ __forceinline__ void init(const uint16_t* base, long long ld, int row0, int rows) {
    t.init(base, ld, row0, rows);
  }
  __device__ __forceinline__ void issue(unsigned char* st, int k0, long long, int wave) const {
    t.issue(st, k0, wave);
  }
  __device__ __forceinline__ static bf16x8 frag(const unsigned char* st, int r0, int kk, int lane) {
    return KTile<R, NT, KB>::frag(st, r0 + (lane & 31), kk, lane >> 5);
  }
};
template <int R, int NT, int KB>
struct Tile<R, NT, KB, false> {
  MTile<R, NT, KB> t;
  static constexpr int BYTES = MTile<R, NT, KB>::SLOTS * 16;
  static constexpr int L = MTile<R, NT, KB>::L;
  __device__ __forceinline__ void init(const uint16_t* base, long long ld, int row0, int) {
    t.init(base, ld, row0);
  }
  __device__ __forceinline__ void issue(unsigned char* st, int k0, long long ld, int wave) const {
    t.issue(st, k0, ld, wave);
  }
  __device__ __forceinline__ static bf16x8 frag(const unsigned char* st, int r0, int kk, int lane) {
    return MTile<R, NT, KB>::frag(st, r0, kk, lane);
  }
};

__device__ __forceinline__ uint32_t pack_bf16_pair(float lo, float hi) {
  const __bf16 a = static_cast<__bf16>(lo);
  const __bf16 b = static_cast<__bf16>(hi);
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Outstanding direct-to-LDS loads allowed while waiting for the oldest stage:
// the loads of the `pending` younger stages. Epilogue stores issued in between
// are not counted, so the wait also covers them (never too short).
template <int LOADS, int MAXP>
__device__ __forceinline__ void wait_stage(int pending) {
  if (MAXP >= 3 && pending >= 3) wait_vmcnt<LOADS * 3>();
  else if (MAXP >= 2 && pending >= 2) wait_vmcnt<LOADS * 2>();
  else if (MAXP >= 1 && pending >= 1) wait_vmcnt<LOADS>();
  else wait_vmcnt<0>();
}

template <int BM, int BN, int WM, int WN, int KB, int STAGES, bool AK, bool BKM, bool OUTF32>
__device__ __forceinline__ void gemm_lds_body(const GemmBf16& p) {
  static_assert(STAGES >= 2 && STAGES <= 5, "2 to 5 LDS stages");
  static_assert((STAGES - 2) * (KB / 8) * (BM + BN) / (BM / WM) / (BN / WN) / 64 <= 63,
                "direct-to-LDS loads of the pending stages exceed the vmcnt range");
  constexpr int NW = (BM / WM) * (BN / WN);
  constexpr int NT = NW * 64;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int LBK = KB;
  using TA = Tile<BM, NT, KB, AK>;
  using TB = Tile<BN, NT, KB, BKM>;
  constexpr int STAGE = TA::BYTES + TB::BYTES;
  constexpr int LOADS = TA::L + TB::L;   // direct-to-LDS loads per thread per stage
  extern __shared__ __align__(16) unsigned char lds[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm0 = (wave / (BN / WN)) * WM;
  const int wn0 = (wave % (BN / WN)) * WN;

  // Tiles of one group (blockIdx.z) in XCD-aware order: the 8 XCDs receive
  // workgroups round-robin, so each XCD gets a contiguous range of the tile
  // sequence, walked in groups of GM tile-rows (co-resident workgroups share A
  // and B slices in their XCD's L2). Each workgroup runs `tpw` consecutive tiles
  // of that sequence with one uninterrupted load pipeline.
  const int tn = (p.N + BN - 1) / BN, tm = (p.M + BM - 1) / BM, ntile = tn * tm;
  const int nwg = gridDim.x;
  int bx = blockIdx.x, bz = blockIdx.z;
  if (p.xcd_cluster) {
    // dispatch order w (x fastest) goes to XCD w % 8; give the gridDim.x tiles of
    // one (group, split) the same w % 8: w -> tile (w / 8) % X, slot w % 8 + 8 (w / 8X)
    const int X = gridDim.x;
    const int w = blockIdx.x + X * blockIdx.z;
    bx = (w / 8) % X;
    bz = (w % 8) + 8 * (w / (8 * X));
  }
  const int wlin = (!p.xcd_cluster && nwg % 8 == 0) ? (bx % 8) * (nwg / 8) + bx / 8 : bx;
  const int tpw = p.tpw;
  // this workgroup's tiles: t_first + i * t_step, i < t_count
  int t_first, t_step, t_count;
  if (p.xcd_stride) {
    const int x = bx % 8, sx = bx / 8;
    const int nx = nwg / 8 + (x < nwg % 8 ? 1 : 0);
    const int base = (int)((long long)ntile * x / 8), end = (int)((long long)ntile * (x + 1) / 8);
    t_first = base + sx;
    t_step = nx;
    t_count = t_first < end ? (end - t_first + nx - 1) / nx : 0;
  } else {
    t_first = wlin * tpw;
    t_step = 1;
    t_count = max(0, min(tpw, ntile - t_first));
  }
  auto tile_origin = [&](int lin, int& m0, int& n0) {
    const int grp = lin / (GM * tn);
    const int first = grp * GM;
    const int gsz = min(GM, tm - first);
    const int in = lin - grp * GM * tn;
    m0 = (first + in % gsz) * BM;
    n0 = (in / gsz) * BN;
  };

  const int g = bz / p.splits, sp = bz - g * p.splits;
  const uint16_t* A = reinterpret_cast<const uint16_t*>(p.A) + g * p.a_gs;
  const uint16_t* B = reinterpret_cast<const uint16_t*>(p.B) + g * p.b_gs;
  int kchunk = (p.K + p.splits - 1) / p.splits;
  kchunk = (kchunk + LBK - 1) / LBK * LBK;
  const int kbeg = sp * kchunk;
  const int kend = min(p.K, kbeg + kchunk);
  const int nk = kend > kbeg ? (kend - kbeg) / LBK : 0;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int cm = lane & 31;
  const int cn = (lane >> 5) * 4;
  // Epilogue. Lane l holds C[row l & 31][cols 8q + 4(l >> 5) .. +3] of each 32x32
  // tile (q = 0..3). bf16 output: lanes l and l ^ 32 swap half of their column
  // groups so that each lane owns 8 consecutive columns (16-byte stores: the
  // lower lane takes q = 0, 2, the upper q = 1, 3).
  const bool upper = (lane >> 5) != 0;
  auto store_tile = [&](int m0, int n0) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = m0 + wm0 + i * 32 + cm;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        if (OUTF32) {
          if (m >= p.M) continue;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int n = n0 + wn0 + j * 32 + q * 8 + cn;
            if (n >= p.N) continue;
            const long long o = g * p.c_gs + sp * p.c_ss + (long long)m * p.ldc + n;
            float4 v = make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                   acc[i][j][4 * q + 3]);
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(p.C) + o) = v;
          }
        } else {
          uint32_t w[4][2];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float4 sc = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
            const int nq = n0 + wn0 + j * 32 + q * 8 + cn;   // this lane's 4 columns (N % 8 == 0)
            if (p.col_scale && nq < p.N)
              sc = *reinterpret_cast<const float4*>(p.col_scale + g * p.c_gs + nq);
            w[q][0] = pack_bf16_pair(acc[i][j][4 * q] * sc.x, acc[i][j][4 * q + 1] * sc.y);
            w[q][1] = pack_bf16_pair(acc[i][j][4 * q + 2] * sc.z, acc[i][j][4 * q + 3] * sc.w);
          }
          // send the groups the partner lane completes: lower sends q = 1, 3
          uint32_t snd[2][2], rcv[2][2];
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int d = 0; d < 2; ++d) {
              snd[h][d] = upper ? w[2 * h][d] : w[2 * h + 1][d];
              rcv[h][d] = (uint32_t)__shfl_xor((int)snd[h][d], 32);
            }
          if (m >= p.M) continue;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int q = 2 * h + (upper ? 1 : 0);
            const int n = n0 + wn0 + j * 32 + q * 8;
            if (n >= p.N) continue;
            uint4 v;
            if (upper) {   // cols 8q .. 8q+3 come from the partner, 8q+4 .. from here
              v.x = rcv[h][0]; v.y = rcv[h][1]; v.z = w[q][0]; v.w = w[q][1];
            } else {
              v.x = w[q][0]; v.y = w[q][1]; v.z = rcv[h][0]; v.w = rcv[h][1];
            }
            const long long o = g * p.c_gs + sp * p.c_ss + (long long)m * p.ldc + n;
            *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p.C) + o) = v;
          }
        }
      }
    }
  };

  if (nk == 0) {   // empty K range of a split: its partial sums are zero
    for (int i = 0; i < t_count; ++i) {
      int m0, n0;
      tile_origin(t_first + i * t_step, m0, n0);
      store_tile(m0, n0);
    }
    return;
  }

  TA ta;
  TB tb;
  int cm0, cn0;   // origin of the tile being accumulated
  tile_origin(t_first, cm0, cn0);
  ta.init(A, p.lda, cm0, p.M);
  tb.init(B, p.ldb, cn0, p.N);
  const int total = t_count * nk;
  // loads run STAGES - 1 stages ahead of the multiplies
  int iss = 0, iss_kt = 0, iss_ti = 0;
  auto issue_next = [&]() {
    if (iss_kt == nk) {   // the next stage starts the next tile
      iss_kt = 0;
      ++iss_ti;
      int nm0, nn0;
      tile_origin(t_first + iss_ti * t_step, nm0, nn0);
      ta.init(A, p.lda, nm0, p.M);
      tb.init(B, p.ldb, nn0, p.N);
    }
    unsigned char* st = lds + (iss % STAGES) * STAGE;
    ta.issue(st, kbeg + iss_kt * LBK, p.lda, wave);
    tb.issue(st + TA::BYTES, kbeg + iss_kt * LBK, p.ldb, wave);
    ++iss;
    ++iss_kt;
  };
#pragma unroll
  for (int i = 0; i < STAGES - 1; ++i)
    if (iss < total) issue_next();
  int kt = 0, ti = 0;
  for (int it = 0; it < total; ++it) {
    wait_stage<LOADS, STAGES - 2>(iss - it - 1);
    lds_barrier();   // stage `it` visible to all waves; stage it-1 no longer read
    const unsigned char* sa = lds + (it % STAGES) * STAGE;
    const unsigned char* sb = sa + TA::BYTES;
    bf16x8 af[2][TM], bfr[2][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) af[0][i] = TA::frag(sa, wm0 + i * 32, 0, lane);
#pragma unroll
    for (int j = 0; j < TN; ++j) bfr[0][j] = TB::frag(sb, wn0 + j * 32, 0, lane);
    // the next stage's loads go out while the first fragments are in flight
    __builtin_amdgcn_sched_barrier(0);
    if (iss < total) issue_next();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < LBK / 16; ++kk) {
      const int cb = kk & 1, nb = cb ^ 1;
      if (kk + 1 < LBK / 16) {
#pragma unroll
        for (int i = 0; i < TM; ++i) af[nb][i] = TA::frag(sa, wm0 + i * 32, kk + 1, lane);
#pragma unroll
        for (int j = 0; j < TN; ++j) bfr[nb][j] = TB::frag(sb, wn0 + j * 32, kk + 1, lane);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          // B first: the result tile is C^T, so each lane holds four consecutive
          // output columns of one output row
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[cb][j], af[cb][i], acc[i][j], 0, 0, 0);
      if (kk + 1 < LBK / 16) {
        // the reads of step kk + 1 go out two at a time between the first
        // multiplies of step kk, so they have the rest of the step to land
        constexpr int NRD = TM * (AK ? 1 : 2) + TN * (BKM ? 1 : 2);   // ds_read per step
        constexpr int NG = (NRD + 1) / 2 < TM * TN ? (NRD + 1) / 2 : TM * TN;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // two LDS reads
        }
        if constexpr (TM * TN > NG) __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - NG, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (++kt == nk) {   // tile complete: write it out and start the next one
      store_tile(cm0, cn0);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
      kt = 0;
      ++ti;
      if (ti < t_count) tile_origin(t_first + ti * t_step, cm0, cn0);
    }
  }
  (void)LOADS;
}

// One symbol per role (as in the register-staged kernels) so profiles attribute
// time to the stage.
#define POETX_LDS_KERNEL(NAME, AK, BKM, OF)                                        \
  template <int BM, int BN, int WM, int WN, int KB, int ST>                       \
  __global__ __launch_bounds__((BM / WM) * (BN / WN) * 64)                        \
  __attribute__((amdgpu_waves_per_eu(2, 2))) void NAME(GemmBf16 p) {             \
    gemm_lds_body<BM, BN, WM, WN, KB, ST, AK, BKM, OF>(p);                        \
  }
POETX_LDS_KERNEL(w0_gemm_nt_lds, true, true, false)
POETX_LDS_KERNEL(w0_gemm_nn_lds, true, false, false)
POETX_LDS_KERNEL(block_gemm_nt_lds, true, true, false)
POETX_LDS_KERNEL(block_gemm_nn_lds, true, false, false)
POETX_LDS_KERNEL(dq_gemm_tn_lds, false, false, true)
POETX_LDS_KERNEL(block_gemm_tn_lds, false, true, false)
#undef POETX_LDS_KERNEL

template <int BM, int BN, int WM, int WN, int KB, int ST>
hipError_t dispatch_lds(const GemmBf16& p, hipStream_t s) {
  constexpr int NW = (BM / WM) * (BN / WN);
  const int ntile = ((p.N + BN - 1) / BN) * ((p.M + BM - 1) / BM);
  dim3 grid(p.xcd_stride ? std::min(ntile, 256) : (ntile + p.tpw - 1) / p.tpw, 1, p.groups * p.splits);
  // ST LDS stages of (BM + BN) x KB bf16
  const size_t lds = ST * (size_t)(BM + BN) * KB * 2;
  const int a = p.a_kmajor, b = p.b_kmajor, f = p.out_f32;
  if (p.role == GEMM_W0 && a && b && !f)
    hipLaunchKernelGGL((w0_gemm_nt_lds<BM, BN, WM, WN, KB, ST>), grid, dim3(NW * 64), lds, s, p);
  else if (p.role == GEMM_W0 && a && !b && !f)
    hipLaunchKernelGGL((w0_gemm_nn_lds<BM, BN, WM, WN, KB, ST>), grid, dim3(NW * 64), lds, s, p);
  else if (p.role == GEMM_BLOCK && a && b && !f)
    hipLaunchKernelGGL((block_gemm_nt_lds<BM, BN, WM, WN, KB, ST>), grid, dim3(NW * 64), lds, s, p);
  else if (p.role == GEMM_BLOCK && a && !b && !f)
    hipLaunchKernelGGL((block_gemm_nn_lds<BM, BN, WM, WN, KB, ST>), grid, dim3(NW * 64), lds, s, p);
  else if (p.role == GEMM_BLOCK && !a && b && !f)
    hipLaunchKernelGGL((block_gemm_tn_lds<BM, BN, WM, WN, KB, ST>), grid, dim3(NW * 64), lds, s, p);
  else if (p.role == GEMM_DQ && !a && !b && f)
    hipLaunchKernelGGL((dq_gemm_tn_lds<BM, BN, WM, WN, KB, ST>), grid, dim3(NW * 64), lds, s, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

bool gemm_lds_supported(const GemmBf16& p, int bm, int bn) {
  if (p.K % 64 != 0) return false;
  if (p.lda % 8 || p.ldb % 8 || p.ldc % 4) return false;
  if (!p.a_kmajor && p.M % bm) return false;
  if (!p.b_kmajor && p.N % bn) return false;
  if (!p.out_f32 && p.N % 8) return false;   // 16-byte epilogue stores
  if (((uintptr_t)p.A | (uintptr_t)p.B) & 15) return false;
  if (p.col_scale && (((uintptr_t)p.col_scale & 15) || p.c_gs % 4 || p.out_f32)) return false;
  return true;
}

hipError_t launch_gemm_lds(const GemmBf16& p_in, int big, hipStream_t s) {
  // tiles per workgroup: enough workgroups for one per CU (two for the small
  // tile), the rest of the work streamed through each workgroup's pipeline
  GemmBf16 p = p_in;
  const int bm = big ? 256 : 128, bn = bm;
  const long long ntile = (long long)((p.N + bn - 1) / bn) * ((p.M + bm - 1) / bm);
  const long long total = ntile * p.groups * p.splits;
  const long long slots = big ? 256 : 512;
  long long tpw = (total + slots - 1) / slots;
  tpw = tpw < 1 ? 1 : (tpw > 16 ? 16 : tpw);
  if (tpw > ntile) tpw = ntile;
  p.tpw = (int)tpw;
  p.xcd_cluster = (tpw == 1 && ntile <= 16 && (p.groups * p.splits) % 8 == 0 &&
                   p.role == GEMM_DQ) ? 1 : 0;
  p.xcd_stride = (big && p.role == GEMM_W0 && p.groups * p.splits == 1 && ntile >= 256) ? 1 : 0;
  if (big) return dispatch_lds<256, 256, 128, 64, 64, 2>(p, s);
  return dispatch_lds<128, 128, 64, 64, 64, 2>(p, s);
}

}  // namespace poetx
