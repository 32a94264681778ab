// Frozen-weight product C = A B^T with both operands K-contiguous, bf16 in,
// fp32 accumulate, bf16 out: the forward's Wa = V Wt^T and, with the weight
// kept beside its transpose, the backward's G_V = G_Wa Wt = G_Wa (WtT)^T ([PX] =
// page "POET-X: Memory-efficient LLM Training by Scaling Orthogonal
// Transformation", Résumé technique §2.A: the dense product with the frozen
// weight between the two block-diagonal factors).
//
// 256 x 256 output tiles, 8 waves (two per SIMD) of 128 x 64 each as 4 x 2
// tiles of v_mfma_f32_32x32x16_bf16, two LDS stages of 64-deep operand tiles
// (128 KiB), one workgroup per CU walking a contiguous, XCD-local range of
// tiles with one uninterrupted load pipeline. Against the general pipelined
// GEMM (k_gemm_lds.hip), which computes the same products in the same MFMA
// order (same bits), three things change:
//  * loads are buffer_load ... lds with one 32-bit row offset per lane and
//    operand and the wave-uniform part in soffset, so they hold no address
//    registers;
//  * a fragment address is base ^ (kk << 5) + 512 CPR i: the XOR swizzle only
//    permutes the chunk bits below a row's base, so each read is one XOR plus
//    an immediate offset;
//  * the schedule: each 16-deep step issues the next step's six fragment reads
//    one per MFMA, and only waves 0-3 load. A CU accepts the 64-lane
//    direct-to-LDS loads one every 10-16 cycles, so when all eight waves issue
//    theirs right after a barrier they stall together and the matrix cores
//    idle (in-kernel timestamps showed the last step of a stage taking about
//    three times its MFMA time). Here waves 0-3 issue the A tile of stage
//    s + 2 right after the barrier that frees its buffer (interleaved with
//    that step's MFMAs) and its B tile in halves during the first two steps of
//    stage s + 1; waves 4-7 only read fragments and multiply, and keep the
//    matrix cores busy while the loads queue: 5-12 % faster on the 16384 x
//    {2048, 5632} x {2048, 5632} shapes than all waves loading, same bits.
//
// Requirements (w0_pipe_supported): M, N multiples of 256, K of 64, 16-byte
// rows, 256 rows of each operand below 2 GiB (32-bit offsets within a tile's
// buffer resource), one group, no split.
#include <type_traits>

#include "poetx_internal.h"

namespace poetx {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTile = 256;       // output tile rows and columns
constexpr int kThr = 512;        // 8 waves
constexpr int kGroupRows = 4;    // tile-rows per group of the XCD-aware order

template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// One K-contiguous operand tile in LDS: 256 rows x KB, chunk c (16 bytes) of row
// r at slot r * CPR + (c ^ ((r / RPB) % CPR)), so the 16 rows one quarter-wave
// reads fall in distinct banks. Load i of a lane fills slot i * kThr + tid:
// row i * RPL + tid / CPR, and its chunk index does not depend on i.
template <int KB>
struct OpTile {
  static constexpr int CPR = KB / 8;
  static constexpr int RPB = 256 / (KB * 2);
  static constexpr int RPL = kThr / CPR;
  static constexpr int L = kTile / RPL;
  static constexpr int BYTES = kTile * KB * 2;
  static_assert(RPL % RPB == 0 && (RPL / RPB) % CPR == 0, "chunk index independent of the load");
  static __device__ __forceinline__ uint32_t lane_offset(int tid, long long ld) {
    const int r = tid / CPR, pos = tid % CPR;
    const int c = pos ^ ((r / RPB) % CPR);
    return (uint32_t)(((long long)r * ld + c * 8) * 2);
  }
  // Operand row r0 + 32 i + (lane & 31), k = 16 kk + 8 half: chunk
  // (2 kk + half) ^ sw with sw = (r / RPB) % CPR, the same for every i (r0 a
  // multiple of 32); base = the byte address at i = 0, kk = 0.
  static __device__ __forceinline__ uint32_t frag_base(int r, int half) {
    const int sw = (r / RPB) % CPR;
    return (uint32_t)(16 * (r * CPR + (half ^ (sw & 1)) + 2 * (sw >> 1)));
  }
  static __device__ __forceinline__ bf16x8 frag(const unsigned char* st, uint32_t base, int i, int kk) {
    return *reinterpret_cast<const bf16x8*>(st + ((base ^ (uint32_t)(kk << 5)) + i * 512 * CPR));
  }
};

// The same tile loaded by the 256 threads of waves 0-3: load i of thread g
// fills slot i * 256 + g (OpTile's slot -> row, chunk map), so one 32-bit row
// offset per lane serves every load of an operand.
template <int KB>
struct LoadTile {
  static constexpr int CPR = KB / 8;
  static constexpr int RPB = 256 / (KB * 2);
  static constexpr int RPL = 256 / CPR;     // rows per load
  static constexpr int L = kTile / RPL;     // loads per lane and operand
  static_assert(RPL % RPB == 0 && (RPL / RPB) % CPR == 0, "chunk index independent of the load");
  static __device__ __forceinline__ uint32_t lane_offset(int g, long long ld) {
    const int r = g / CPR, pos = g % CPR;
    const int c = pos ^ ((r / RPB) % CPR);
    return (uint32_t)(((long long)r * ld + c * 8) * 2);
  }
};

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const __bf16 a = static_cast<__bf16>(lo);
  const __bf16 b = static_cast<__bf16>(hi);
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// SCALE: output column n multiplied by col_scale[n] (fp32, before the rounding
// to bf16), for an INT8 weight's row scales when the weight comes in as its
// exact bf16 widening
template <int KB, bool SCALE>
__global__ __launch_bounds__(kThr) __attribute__((amdgpu_waves_per_eu(2, 2)))
void w0_gemm_nt_pipe(GemmBf16 p) {
  using Op = OpTile<KB>;
  using Ld = LoadTile<KB>;
  constexpr int ST = 2;                        // LDS stages
  constexpr int NK = KB / 16;                  // 16-deep steps per stage
  constexpr int STAGE = 2 * Op::BYTES;         // A tile, then B tile
  static_assert(NK >= 3 && NK % 2 == 0, "two B steps and a last step; fragment buffer parity across stages");
  static_assert(2 * Ld::L <= 63, "vmcnt range");
  extern __shared__ __align__(16) unsigned char lds[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave >> 2) * 128, wn0 = (wave & 3) * 64;

  // tiles of this workgroup: XCD x = blockIdx.x % 8 owns the contiguous range
  // [ntile x / 8, ntile (x + 1) / 8), walked by its workgroups with a stride of
  // their count; a tile index maps to (m0, n0) in groups of kGroupRows tile-rows
  const int tn = p.N / kTile, tm = p.M / kTile, ntile = tn * tm;
  const int nwg = gridDim.x, bx = blockIdx.x;
  const int x = bx % 8, sx = bx / 8;
  const int nx = nwg / 8 + (x < nwg % 8 ? 1 : 0);
  const int tbase = (int)((long long)ntile * x / 8), tend = (int)((long long)ntile * (x + 1) / 8);
  const int t_first = tbase + sx;
  const int t_count = t_first < tend ? (tend - t_first + nx - 1) / nx : 0;
  if (t_count == 0) return;
  auto origin = [&](int ti, int& m0, int& n0) {
    const int lin = t_first + ti * nx;
    const int grp = lin / (kGroupRows * tn);
    const int first = grp * kGroupRows;
    const int gsz = min(kGroupRows, tm - first);
    const int in = lin - grp * kGroupRows * tn;
    m0 = (first + in % gsz) * kTile;
    n0 = (in / gsz) * kTile;
  };

  // each load goes through a buffer resource that starts at its tile's first
  // row (base and size in scalar registers), so offsets stay below one tile's
  // 256 rows at any M and N
  const uint16_t* const pa = static_cast<const uint16_t*>(p.A);
  const uint16_t* const pb = static_cast<const uint16_t*>(p.B);
  const int tra = (int)(256LL * p.lda * 2), trb = (int)(256LL * p.ldb * 2);
  const int g = tid & 255;   // thread index within waves 0-3 (loaders)
  const uint32_t va = Ld::lane_offset(g, p.lda), vb = Ld::lane_offset(g, p.ldb);
  const int nk = p.K / KB;
  const int total = t_count * nk;

  // loads [i0, i1) of operand `op` (0: A, 1: B) of global stage s (past the
  // end: the last stage again, into a buffer nobody reads) into LDS buffer
  // s % ST, by waves 0-3; the wave-uniform part of each offset goes in soffset
  // (whole tiles: every access is inside the operand)
  auto issue = [&](int s, int op, int i0 = 0, int i1 = Ld::L) {
    const int buf = s % ST;
    s = min(s, total - 1);
    const int ti = s / nk, kt = s - ti * nk;
    int m0, n0;
    origin(ti, m0, n0);
    unsigned char* st = lds + buf * STAGE + op * Op::BYTES + (wave & 3) * 64 * 16;
    if (op == 0) {
      const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(pa + (long long)m0 * p.lda), (short)0, tra, 0x00020000);
      const uint32_t ka = (uint32_t)(kt * KB * 2);
#pragma unroll
      for (int i = i0; i < i1; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, (__attribute__((address_space(3))) void*)(st + i * 256 * 16), 16, va,
            (int)(ka + (uint32_t)(i * Ld::RPL * p.lda * 2)), 0, 0);
    } else {
      const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(pb + (long long)n0 * p.ldb), (short)0, trb, 0x00020000);
      const uint32_t kb = (uint32_t)(kt * KB * 2);
#pragma unroll
      for (int i = i0; i < i1; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb, (__attribute__((address_space(3))) void*)(st + i * 256 * 16), 16, vb,
            (int)(kb + (uint32_t)(i * Ld::RPL * p.ldb * 2)), 0, 0);
    }
  };

  const int cm = lane & 31, half = lane >> 5;
  const bool upper = half != 0;
  const uint32_t fa = Op::frag_base(wm0 + cm, half), fb = Op::frag_base(wn0 + cm, half) + Op::BYTES;
  // Lane l holds C[row l & 31][cols 8q + 4(l >> 5) .. +3] of each 32 x 32 tile;
  // lanes l and l ^ 32 swap half of their column groups so that each stores 8
  // consecutive columns (16 bytes).
  auto store_tile = [&](const f32x16 (&acc)[4][2], int m0, int n0) {
    // this lane's row of 32-row tile i starts at rowp + i * 32 ldc; its 8
    // columns of group (j, h) at + j * 32 + 16 h (immediate offsets)
    uint16_t* rowp = static_cast<uint16_t*>(p.C) + (long long)(m0 + wm0 + cm) * p.ldc + n0 + wn0 +
                     (upper ? 8 : 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        uint32_t w[4][2];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if constexpr (SCALE) {
            // this lane's columns n0 + wn0 + 32 j + 8 q + 4 (lane >> 5) .. + 3
            const float4 sc = *reinterpret_cast<const float4*>(p.col_scale + n0 + wn0 + j * 32 + 8 * q +
                                                               (upper ? 4 : 0));
            w[q][0] = pack2(acc[i][j][4 * q] * sc.x, acc[i][j][4 * q + 1] * sc.y);
            w[q][1] = pack2(acc[i][j][4 * q + 2] * sc.z, acc[i][j][4 * q + 3] * sc.w);
          } else {
            w[q][0] = pack2(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
            w[q][1] = pack2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
          }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          // own groups q = 2 h + upper, the partner's q = 2 h + 1 - upper
          const uint32_t o0 = upper ? w[2 * h + 1][0] : w[2 * h][0];
          const uint32_t o1 = upper ? w[2 * h + 1][1] : w[2 * h][1];
          const uint32_t r0 = (uint32_t)__shfl_xor((int)(upper ? w[2 * h][0] : w[2 * h + 1][0]), 32);
          const uint32_t r1 = (uint32_t)__shfl_xor((int)(upper ? w[2 * h][1] : w[2 * h + 1][1]), 32);
          uint4 v;
          v.x = upper ? r0 : o0;
          v.y = upper ? r1 : o1;
          v.z = upper ? o0 : r0;
          v.w = upper ? o1 : r1;
          *reinterpret_cast<uint4*>(rowp + (long long)i * 32 * p.ldc + j * 32 + 16 * h) = v;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // The two wave groups run separate copies of the loop (LD: waves 0-3), each
  // with its own instruction schedule. Stage s + 2 lands in the buffer stage s
  // leaves: its A tile is issued right after the barrier of stage s's last
  // step, its B tile in halves during the first two steps of stage s + 1, and
  // the loaders wait for both before the barrier of stage s + 1's last step.
  auto run = [&](auto ld_tag) {
    constexpr bool LD = decltype(ld_tag)::value;
    if constexpr (LD) {
      issue(0, 0);
      issue(0, 1);
      issue(1, 0);          // stage 1's A tile; its B tile goes out in stage 0's first steps
      vm_wait<Ld::L>();     // stage 0 landed
    }
    lds_sync();
    bf16x8 af[2][4], bf[2][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) af[0][i] = Op::frag(lds, fa, i, 0);
#pragma unroll
    for (int j = 0; j < 2; ++j) bf[0][j] = Op::frag(lds, fb, j, 0);

    for (int ti = 0; ti < t_count; ++ti) {
      int cm0, cn0;
      origin(ti, cm0, cn0);
      f32x16 acc[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
      for (int kt = 0; kt < nk; ++kt) {
        const int it = ti * nk + kt;
        const unsigned char* sa = lds + (it % ST) * STAGE;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          const int cb = kk & 1, nb = cb ^ 1;
          if (kk + 1 < NK) {
            if (LD && kk < 2) issue(it + 1, 1, kk * (Ld::L / 2), (kk + 1) * (Ld::L / 2));
#pragma unroll
            for (int i = 0; i < 4; ++i) af[nb][i] = Op::frag(sa, fa, i, kk + 1);
#pragma unroll
            for (int j = 0; j < 2; ++j) bf[nb][j] = Op::frag(sa, fb, j, kk + 1);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[cb][j], af[cb][i], acc[i][j], 0, 0, 0);
            // the next step's 6 reads (and the loaders' B tile) go out between
            // the first six MFMAs
#pragma unroll
            for (int q = 0; q < 6; ++q) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              if (LD && kk < 2) __builtin_amdgcn_sched_group_barrier(0x020, (Ld::L / 2 + 5) / 6, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_barrier(0);
          } else {
            // last step: stage it + 1 landed and stage it no longer read by
            // anyone once every wave is past this barrier
            if constexpr (LD) vm_wait<0>();
            lds_sync();
            if constexpr (LD) issue(it + ST, 0);
            const unsigned char* na = lds + ((it + 1) % ST) * STAGE;
#pragma unroll
            for (int i = 0; i < 4; ++i) af[nb][i] = Op::frag(na, fa, i, 0);
#pragma unroll
            for (int j = 0; j < 2; ++j) bf[nb][j] = Op::frag(na, fb, j, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[cb][j], af[cb][i], acc[i][j], 0, 0, 0);
            // the loaders' A tile and the next stage's first fragment reads go
            // out between the MFMAs
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              if (LD) __builtin_amdgcn_sched_group_barrier(0x020, (Ld::L + 7) / 8, 0);
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      store_tile(acc, cm0, cn0);
    }
  };
  if (wave < 4) run(std::true_type{});
  else run(std::false_type{});
  // the last iterations loaded the final stage again into buffers nobody reads:
  // let those direct-to-LDS writes land before the workgroup's LDS is released
  vm_wait<0>();
}

constexpr int kKB = 64;   // stage depth
constexpr int kST = 2;    // LDS stages (2 x 64 KiB), fixed in the kernel

}  // namespace

bool w0_pipe_supported(const GemmBf16& p) {
  if (p.role != GEMM_W0 || !p.a_kmajor || !p.b_kmajor || p.out_f32) return false;
  if (((uintptr_t)p.col_scale & 15) != 0) return false;   // 16-byte scale loads
  if (p.groups != 1 || p.splits != 1) return false;
  if (p.M <= 0 || p.N <= 0 || p.M % kTile || p.N % kTile || p.K <= 0 || p.K % kKB) return false;
  if (p.lda % 8 || p.ldb % 8 || p.ldc % 8 || p.lda < p.K || p.ldb < p.K || p.ldc < p.N) return false;
  // one tile's 256 rows of either operand within 32-bit buffer offsets
  if (256LL * p.lda * 2 >= (1LL << 31) || 256LL * p.ldb * 2 >= (1LL << 31)) return false;
  if (((uintptr_t)p.A | (uintptr_t)p.B | (uintptr_t)p.C) & 15) return false;
  return true;
}

hipError_t launch_w0_pipe(const GemmBf16& p, hipStream_t s) {
  if (!w0_pipe_supported(p)) return hipErrorInvalidValue;
  const long long ntile = (long long)(p.M / kTile) * (p.N / kTile);
  const size_t lds = (size_t)kST * 2 * kTile * kKB * 2;
  const dim3 grid((unsigned)std::min<long long>(ntile, 256));
  if (p.col_scale)
    hipLaunchKernelGGL((w0_gemm_nt_pipe<kKB, true>), grid, dim3(kThr), lds, s, p);
  else
    hipLaunchKernelGGL((w0_gemm_nt_pipe<kKB, false>), grid, dim3(kThr), lds, s, p);
  return hipGetLastError();
}

}  // namespace poetx
