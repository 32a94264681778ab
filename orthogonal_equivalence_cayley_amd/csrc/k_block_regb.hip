// Batched block-diagonal products with blocks of 256 or 512 on gfx950
// (v_mfma_f32_32x32x16_bf16, fp32 accumulate): C[:, blk g] = A[:, blk g] B_g,
// B_g(n, k) one b x b block of Q or of its transpose. These are the
// products of the orthogonal factors on the activations (Z = Wa D_R^T in the
// forward, G_U = G_V D_P in the backward) and the weight-side Wf = Wt D_P
// ([PX] = page "POET-X: Memory-efficient LLM Training by Scaling Orthogonal
// Transformation", Résumé technique §2.C: the block-diagonal factors applied as
// batched block products).
//
// K is only 256, so a tiled GEMM spends most of its time filling and draining
// its pipeline. Here the block of B stays in registers instead: each of the 8
// waves owns 32 output columns and keeps B_g(those columns, all 256 k) as its 16
// MFMA operand fragments (64 VGPRs), loaded once per workgroup (a workgroup
// stays on one block). A block of 512 takes two workgroups, each with 256 of
// its output columns and all 512 k (128 VGPRs of B per lane); its A tiles are
// 64 rows x 512 (64 KiB) in two stages. B is fetched before the first A tiles
// (natural-layout B through the still empty LDS ring: one part for a block of
// 256, two for a block of 512): behind them it would wait for all of them,
// which doubled the start-up of a workgroup that runs only 8 tiles. Row tiles
// of A (ROWS rows x the block's columns) stream from HBM into an LDS ring of ST
// stages with direct-to-LDS buffer loads, ST - 1 tiles in flight while one is
// multiplied; every wave reads the whole A tile from LDS, the fragments of the
// next 16-deep step before the MFMAs of the current one. An HBM stream needs on
// the order of 100 KiB in flight per CU, so the ring holds several small tiles
// rather than two large ones.
//
// A tile in LDS: row r of b bf16 is b / 8 chunks of 16 bytes; chunk c sits at
// slot r * b / 8 + (c ^ (r & 31)), so the 16 rows read by one pass of an
// operand read (one chunk each) fall in distinct banks.
#include "poetx_internal.h"

namespace poetx {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kB = 256;                         // output columns per workgroup
constexpr int kWaves = 8;                       // each owns 32 of the 256 columns
constexpr int kThreads = kWaves * 64;

__device__ __forceinline__ void dma16(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                   (void __attribute__((address_space(3)))*)lds_dst, 16, 0, 0);
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Waits for this wave's LDS reads, then for all waves: after a wait for the
// tile's loads, what they wrote is in LDS, and every earlier LDS read of the
// workgroup is done.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// Loads return in order among themselves, so allowing the loads of `younger`
// later tiles to stay outstanding covers this tile's; epilogue stores in between
// only make the count larger, i.e. the wait stricter, never shorter.
template <int LOADS, int MAXY>
__device__ __forceinline__ void wait_tile(int younger) {
  if (MAXY >= 3 && younger >= 3) wait_vmcnt<3 * LOADS>();
  else if (MAXY >= 2 && younger == 2) wait_vmcnt<2 * LOADS>();
  else if (MAXY >= 1 && younger == 1) wait_vmcnt<LOADS>();
  else wait_vmcnt<0>();
}

__device__ __forceinline__ uint32_t pack_bf16_pair(float lo, float hi) {
  const __bf16 a = static_cast<__bf16>(lo);
  const __bf16 b = static_cast<__bf16>(hi);
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// A row-contiguous A tile (A(m, k) = A[k lda + m]) sits in LDS as 256 K-rows of
// ROWS elements; chunk c of K-row k at slot k (ROWS / 8) + (c ^ 4 (k & 3)), so
// the 4 K-rows x 4 chunks touched by 32 lanes of a transposing read
// (ds_read_b64_tr_b16: within 16 lanes, lane p receives column p of a 4 x 16
// block) fall in distinct banks. Operand rows r0 .. r0 + 31 at k = 16 kk +
// 8 (lane / 32) .. + 7 take two such reads.
template <int ROWS>
__device__ __forceinline__ bf16x8 frag_t(const unsigned char* st, int r0, int kk, int lane) {
  constexpr int CPR = ROWS / 8;
  static_assert(CPR >= 16, "the swizzle moves a chunk by up to 12 positions");
  const int g = lane >> 4, s = lane & 15;
  const int col = r0 + (g & 1) * 16 + 4 * (s & 3);
  const int kb = 16 * kk + 8 * (g >> 1) + (s >> 2);
  i16x4 v[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int k = kb + 4 * i;
    const int c = (col >> 3) ^ (4 * (k & 3));
    v[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(st + (k * CPR + c) * 16 + (col & 7) * 2));
  }
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 w = __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, w);
}

// AKM: A(m, k) = A_g[m * lda + k] (K-contiguous); otherwise A_g[k * lda + m]
// (then M % ROWS == 0). BKM: B(n, k) = B_g[n * ldb + k] (K-contiguous, the
// transposed Q); otherwise B(n, k) = B_g[k * ldb + n]. KD: the block size, which
// is K; a block of 512 has its 512 output columns split over two workgroups of
// 256 each (NH = KD / 256 column slices). Workgroup w works on slice w / wpg
// (block g = slice / NH) and runs row tiles [(w % wpg) * per_wg, + per_wg) of
// it, so it loads its part of B_g only once.
template <bool AKM, bool BKM, int ROWS, int ST, bool SCALE, int KD = 256>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void block_regb_kernel(GemmBf16 p, int tiles_per_group, int wpg, int per_wg) {
  constexpr int NH = KD / kB;                      // column slices per block
  constexpr int kNKK = KD / 16;                    // 16-deep K steps
  constexpr int kCPR = KD / 8;                     // 16-byte chunks per row of A
  constexpr int STAGE = ROWS * KD * 2;             // bytes of one A tile in LDS
  constexpr int LOADS = ROWS * kCPR / kThreads;    // direct-to-LDS loads per thread per tile
  constexpr int MT = ROWS / 32;                    // 32-row MFMA tiles per wave and tile
  static_assert(ST >= 2 && ST <= 5 && LOADS * kThreads == ROWS * kCPR && ROWS % 32 == 0, "tile");
  static_assert(AKM || KD == 256, "row-contiguous A only for blocks of 256");
  extern __shared__ __align__(16) unsigned char lds[];   // ST A tiles
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gs = blockIdx.x / wpg;                 // column slice
  const int g = gs / NH, hs = gs - g * NH;
  const int t0 = (blockIdx.x - gs * wpg) * per_wg;
  const int t1 = min(tiles_per_group, t0 + per_wg);
  if (g >= p.groups || t0 >= t1) return;
  const uint16_t* Ag = static_cast<const uint16_t*>(p.A) + (long long)g * p.a_gs;
  const uint16_t* Bg = static_cast<const uint16_t*>(p.B) + (long long)g * p.b_gs +
                       (long long)hs * kB * (BKM ? p.ldb : 1);
  uint16_t* Cg = static_cast<uint16_t*>(p.C) + (long long)g * p.c_gs + hs * kB + wave * 32;
  const int nl = lane & 31, h = lane >> 5;
  const int ncol = wave * 32 + nl;   // B column of this lane's operand fragments
  auto stage = [&](int i) { return lds + i * STAGE; };

  // row tile t of A -> LDS stage st: lane `tid` of load i fills slot i * kThreads + tid.
  // Buffer loads (counted by vmcnt only, so the LDS reads of the K loop get
  // exact lgkmcnt waits while tiles are in flight) through a resource that
  // starts at the tile (its base and size in scalar registers, so offsets stay
  // small at any M); rows past M fall outside it and load zeros (their
  // results are not stored).
  auto issue = [&](int t, unsigned char* st) {
    const long long row0 = (long long)t * ROWS;
    const uint16_t* base = AKM ? Ag + row0 * p.lda : Ag + row0;
    const long long nrec = AKM ? (long long)min((long long)ROWS, p.M - row0) * p.lda * 2
                               : (long long)KD * p.lda * 2 - row0 * 2;
    const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(base), (short)0, (int)min(nrec, (long long)INT32_MAX), 0x00020000);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int s = i * kThreads + tid;
      uint32_t vo;
      if constexpr (AKM) {
        const int r = s / kCPR;
        const int c = (s % kCPR) ^ (r & 31);
        vo = (uint32_t)(((long long)r * p.lda + c * 8) * 2);
      } else {
        constexpr int CPR = ROWS / 8;   // chunks per K-row of the tile
        const int k = s / CPR;
        const int c = (s % CPR) ^ (4 * (k & 3));
        vo = (uint32_t)(((long long)k * p.lda + c * 8) * 2);
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsa, (__attribute__((address_space(3))) void*)(st + (i * kThreads + wave * 64) * 16), 16, vo, 0, 0, 0);
    }
  };

  // B_g(ncol, 16 kk + 8 h .. + 7) for kk = 0 .. 15. B goes out before the first
  // A tiles: loads return in order, so B queued behind ST - 1 tiles of A would
  // wait for all of them before the first multiply could start.
  bf16x8 bq[kNKK];
  // natural-layout B: the slice's K-rows (512 bytes each) go through the still
  // empty LDS ring in as few parts as fit (one for a block of 256, two of 256
  // K-rows for a block of 512), each part in one round trip
  constexpr int kRingParts = (KD * kB * 2 + ST * STAGE - 1) / (ST * STAGE);
  constexpr int kRingRows = KD / kRingParts;   // K-rows of B per part
  static_assert(BKM || (KD % kRingParts == 0 && kRingRows % 16 == 0 && kRingRows * kB * 2 <= ST * STAGE),
                "natural-layout B in whole 16-deep steps per part of the ring");
  if constexpr (BKM) {
#pragma unroll
    for (int kk = 0; kk < kNKK; ++kk)
      bq[kk] = *reinterpret_cast<const bf16x8*>(Bg + (long long)ncol * p.ldb + 16 * kk + 8 * h);
  } else {
    // K-row k of a part in the layout of a row-contiguous A tile (chunk c at
    // slot k (kB / 8) + (c ^ 4 (k & 3))), read back column-wise with the
    // transposing reads of frag_t
    constexpr int CPRB = kB / 8;
    constexpr int RLOADS = kRingRows * CPRB / kThreads;
    static_assert(RLOADS * kThreads == kRingRows * CPRB, "whole loads per part");
#pragma unroll
    for (int part = 0; part < kRingParts; ++part) {
#pragma unroll
      for (int i = 0; i < RLOADS; ++i) {
        const int s = i * kThreads + tid;
        const int k = s / CPRB;
        const int c = (s % CPRB) ^ (4 * (k & 3));
        dma16(Bg + (long long)(part * kRingRows + k) * p.ldb + c * 8, lds + (i * kThreads + wave * 64) * 16);
      }
      wait_vmcnt<0>();
      lds_barrier();
#pragma unroll
      for (int kk = 0; kk < kRingRows / 16; ++kk)
        bq[part * (kRingRows / 16) + kk] = frag_t<kB>(lds, wave * 32, kk, lane);
      lds_barrier();   // every wave has this part before the ring is reused
    }
  }
  // the first ST - 1 tiles of A
#pragma unroll
  for (int i = 0; i < ST - 1; ++i)
    if (t0 + i < t1) issue(t0 + i, stage(i));

  const bool upper = h != 0;
  for (int t = t0; t < t1; ++t) {
    const int it = t - t0;
    // tiles issued after this one: t + 1 .. min(t + ST - 2, t1 - 1)
    wait_tile<LOADS, ST - 2>(min(ST - 2, t1 - 1 - t));
    lds_barrier();   // tile t in LDS; the stage of tile t - 1 no longer read
    if (t + ST - 1 < t1) issue(t + ST - 1, stage((it + ST - 1) % ST));
    const unsigned char* st = stage(it % ST);
    f32x16 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mt][v] = 0.0f;
    // K-contiguous A: chunk 2 kk + h of row r = 32 mt + nl sits at byte
    // r kCPR 16 + (((2 kk + h) ^ nl) << 4) = (nl kCPR 16 + ((h ^ nl) << 4)) ^
    // (kk << 5) + mt 32 kCPR 16 (the XOR only permutes chunk bits below the
    // row's base): one XOR per step. The base passes through an empty asm so
    // that the per-step addresses are formed in the step, not hoisted out of
    // the tile loop and held live.
    uint32_t abase = (uint32_t)(nl * kCPR * 16 + ((h ^ nl) << 4));
    asm volatile("" : "+v"(abase));
    auto read_a = [&](bf16x8 (&af)[MT], int kk) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if constexpr (AKM) {
          af[mt] = *reinterpret_cast<const bf16x8*>(st + ((abase ^ (uint32_t)(kk << 5)) + mt * 32 * kCPR * 16));
        } else {
          af[mt] = frag_t<ROWS>(st, 32 * mt, kk, lane);
        }
      }
    };
    // the A fragments of step kk + 1 are read before the MFMAs of step kk (two
    // register sets), so a step's LDS latency hides behind the multiplies of
    // the step before instead of adding to them
    bf16x8 af[2][MT];
    read_a(af[0], 0);
#pragma unroll
    for (int kk = 0; kk < kNKK; ++kk) {
      const int cb = kk & 1;
      if (kk + 1 < kNKK) read_a(af[cb ^ 1], kk + 1);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        // B first: the result is C^T, each lane holds four consecutive output
        // columns (8 q + 4 h .. + 3 of the wave's 32) of output row nl
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bq[kk], af[cb][mt], acc[mt], 0, 0, 0);
      if (kk + 1 < kNKK) {
        // one scheduling region per step: the next step's reads and this
        // step's MFMAs (the reads are not hoisted further ahead, where their
        // registers would have to stay live)
        __builtin_amdgcn_sched_group_barrier(0x100, AKM ? MT : 2 * MT, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, MT, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // epilogue: lanes l and l ^ 32 swap half of their column groups so that each
    // lane stores 8 consecutive columns (the lower lane q = 0, 2, the upper 1, 3)
    const long long row0 = (long long)t * ROWS;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      uint32_t w[4][2];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float4 sc = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
        if (SCALE)   // column n scaled by col_scale[g * c_gs + n] before the rounding
          sc = *reinterpret_cast<const float4*>(p.col_scale + (long long)g * p.c_gs + hs * kB + wave * 32 +
                                                8 * q + 4 * h);
        w[q][0] = pack_bf16_pair(acc[mt][4 * q] * sc.x, acc[mt][4 * q + 1] * sc.y);
        w[q][1] = pack_bf16_pair(acc[mt][4 * q + 2] * sc.z, acc[mt][4 * q + 3] * sc.w);
      }
      const long long m = row0 + 32 * mt + nl;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        // own groups (q = 2 hh + upper) and the ones sent to the partner
        const uint32_t o0 = upper ? w[2 * hh + 1][0] : w[2 * hh][0];
        const uint32_t o1 = upper ? w[2 * hh + 1][1] : w[2 * hh][1];
        const uint32_t s0 = upper ? w[2 * hh][0] : w[2 * hh + 1][0];
        const uint32_t s1 = upper ? w[2 * hh][1] : w[2 * hh + 1][1];
        const uint32_t r0 = (uint32_t)__shfl_xor((int)s0, 32);
        const uint32_t r1 = (uint32_t)__shfl_xor((int)s1, 32);
        if (m >= p.M) continue;
        uint4 v;
        if (upper) {   // columns 8q .. 8q+3 come from the partner, 8q+4 .. from here
          v.x = r0; v.y = r1; v.z = o0; v.w = o1;
        } else {
          v.x = o0; v.y = o1; v.z = r0; v.w = r1;
        }
        *reinterpret_cast<uint4*>(Cg + m * p.ldc + 8 * (2 * hh + (upper ? 1 : 0))) = v;
      }
    }
  }
}

constexpr int kRows = 64;   // rows of A per tile
constexpr int kST = 4;      // LDS stages: three 32 KiB tiles in flight
constexpr int kST512 = 2;   // blocks of 512: 64 KiB tiles, two stages
constexpr int kRowsT = 128; // row-contiguous A: 128-row tiles (64 KiB, the swizzle needs 16 chunks)
constexpr int kSTT = 2;     // and two stages

}  // namespace

bool block_regb_supported(const GemmBf16& p) {
  if (p.role != GEMM_BLOCK || p.out_f32) return false;
  if (!((p.N == kB && p.K == kB) || (p.N == 2 * kB && p.K == 2 * kB && p.a_kmajor))) return false;
  // row-contiguous A (the transposed weight fold): whole tiles, K-contiguous Q,
  // no column scale
  if (!p.a_kmajor && (p.M % kRowsT || !p.b_kmajor || p.col_scale)) return false;
  if (p.splits != 1 || p.M <= 0 || p.groups <= 0) return false;
  if (p.col_scale && (((uintptr_t)p.col_scale & 15) || p.c_gs % 4)) return false;
  if (p.lda % 8 || p.a_gs % 8 || p.ldc % 8 || p.c_gs % 8) return false;   // 16-byte rows
  // a buffer resource per A tile: one tile's byte offsets below 2^31
  if ((long long)(p.a_kmajor ? kRows : p.K) * p.lda * 2 >= (1LL << 31)) return false;
  if (p.ldb % 8 || p.ldb < p.N) return false;   // 16-byte rows of B either way (N = K)
  if (((uintptr_t)p.A | (uintptr_t)p.C | (uintptr_t)p.B) & 15) return false;
  return true;
}

hipError_t launch_block_regb(const GemmBf16& p, hipStream_t s) {
  if (!block_regb_supported(p)) return hipErrorInvalidValue;
  const int rows = p.a_kmajor ? kRows : kRowsT;
  const long long tpg = (p.M + rows - 1) / rows;
  if (tpg > INT32_MAX) return hipErrorInvalidValue;
  // one workgroup per CU (the LDS ring): up to 256 / slices workgroups per
  // column slice (blocks of 512 have two), each on consecutive row tiles of it
  const long long slices = (long long)p.groups * (p.N / kB);
  const long long wmax = slices >= 256 ? 1 : 256 / slices;
  const long long per = (tpg + wmax - 1) / wmax;
  const long long wpg = (tpg + per - 1) / per;
  const long long wgs = wpg * slices;
  if (wgs > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)wgs), block(kThreads);
  const int a = (int)tpg, b = (int)wpg, c = (int)per;
  if (p.N == 2 * kB) {   // blocks of 512 (K-contiguous A)
    const size_t lds = (size_t)kST512 * kRows * 2 * kB * 2;
    if (p.b_kmajor && p.col_scale)
      hipLaunchKernelGGL((block_regb_kernel<true, true, kRows, kST512, true, 512>), grid, block, lds, s, p, a, b, c);
    else if (p.b_kmajor)
      hipLaunchKernelGGL((block_regb_kernel<true, true, kRows, kST512, false, 512>), grid, block, lds, s, p, a, b, c);
    else if (p.col_scale)
      hipLaunchKernelGGL((block_regb_kernel<true, false, kRows, kST512, true, 512>), grid, block, lds, s, p, a, b, c);
    else
      hipLaunchKernelGGL((block_regb_kernel<true, false, kRows, kST512, false, 512>), grid, block, lds, s, p, a, b, c);
    return hipGetLastError();
  }
  if (!p.a_kmajor) {   // the transposed weight fold: K-contiguous Q, no column scale
    if (!p.b_kmajor || p.col_scale) return hipErrorInvalidValue;
    const size_t lds = (size_t)kSTT * kRowsT * kB * 2;
    hipLaunchKernelGGL((block_regb_kernel<false, true, kRowsT, kSTT, false>), grid, block, lds, s, p, a, b, c);
    return hipGetLastError();
  }
  const size_t lds = (size_t)kST * kRows * kB * 2;
  if (p.b_kmajor && p.col_scale)
    hipLaunchKernelGGL((block_regb_kernel<true, true, kRows, kST, true>), grid, block, lds, s, p, a, b, c);
  else if (p.b_kmajor)
    hipLaunchKernelGGL((block_regb_kernel<true, true, kRows, kST, false>), grid, block, lds, s, p, a, b, c);
  else if (p.col_scale)
    hipLaunchKernelGGL((block_regb_kernel<true, false, kRows, kST, true>), grid, block, lds, s, p, a, b, c);
  else
    hipLaunchKernelGGL((block_regb_kernel<true, false, kRows, kST, false>), grid, block, lds, s, p, a, b, c);
  return hipGetLastError();
}

}  // namespace poetx
