// Internal interface between the host dispatcher (poetx_host.cpp) and the HIP
// kernels. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace poetx {

// A run of consecutive blocks of equal size on one side.
struct Seg {
  int b;              // block size
  int count;          // number of blocks in the run
  int dim_off;        // first feature index of the run (permuted index space)
  long long q_off;    // element offset of the run's first block in the b*b arrays
  long long p_off;    // offset of its first packed parameter
};

// ---------------------------------------------------------------- index ops
// out[t][i] = in[rows ? rows[t] : t][idx[i]]; in has row stride in_ld elements.
hipError_t launch_gather_cols(const void* in, long long in_ld, const int32_t* rows,
                              const int32_t* idx, void* out, long long T, int dim,
                              int elsize, hipStream_t s);
// out[c][r] = in[r][c] for an R x C row-major matrix of 2- or 4-byte elements
hipError_t launch_transpose(const void* in, void* out, int R, int C, int elsize, hipStream_t s);
// out[t][idx[i]] = in[t][i]
hipError_t launch_scatter_cols(const void* in, const int32_t* idx, void* out, long long T,
                               int dim, int elsize, hipStream_t s);

// Index mapping fused with the block products (k_panel.hip), bf16, blocks of 256,
// dim <= 2048: gather: out[:, blk] = P[:, blk] Bq_g^T with P[t][i] = in[t][idx[i]]
// (P also written to in_copy when non-null); scatter: C[:, blk] = in[:, blk]
// Bq_g^T and out[t][idx[i]] = C[t][i]. Bq holds the blocks K-contiguous
// (Bq_g(n, k) = Bq[g * 65536 + n * 256 + k]). All rows [T, dim] row-major.
bool panel_supported(int dim, int b, int nblocks);
hipError_t launch_panel_block(const void* in, const int32_t* idx, const void* Bq, void* out,
                              void* in_copy, long long T, int dim, bool gather, bool scatter,
                              hipStream_t s);
// QT[g][n][k] = Q[g][k][n] for count bf16 blocks of 256 x 256
hipError_t launch_transpose_blocks(const void* Q, void* QT, int count, hipStream_t s);

// ---------------------------------------------------------------- block helpers (fp32)
// S = skew(theta) for every block of the run; if Q != nullptr also Q = I + c1 * S.
hipError_t launch_unpack_skew(const float* theta, const Seg& g, float* S, float* Q, float c1,
                              hipStream_t s);
// Newton-Schulz inverse of I - S for count b x b blocks: X0 = a (I + S) with
// a = 2 / (2 + c^2), c = the smaller of the max row sum of |S| and the square
// root of the max row sum of |S2| (S2 = S S, or null: both bound ||S||_2);
// iters[g] = steps X <- X (2I - (I - S) X) block g needs for a residual below
// 2^-30 (<= jmax).
hipError_t launch_ns_init(const float* S, const float* S2, int b, int count, float* X0, int32_t* iters,
                          int jmax, hipStream_t s);
// N = the iterate of block g (X0 if iters[g] is even, else X1); Q = 2 N - I.
hipError_t launch_ns_final(const float* X0, const float* X1, const int32_t* iters, int b, int count,
                           float* N, float* Q, hipStream_t s);
// out = diag * I + sum_{i < n} coef[i] * mats[i] over count b x b blocks
// (elementwise; n <= kLinCombMax; out may be one of mats).
constexpr int kLinCombMax = 8;
struct LinComb {
  const float* mats[kLinCombMax];
  float coef[kLinCombMax];
  int n;
  float diag;
};
hipError_t launch_lincomb(const LinComb& lc, float* out, int b, int count, hipStream_t s);
// g[(i,j)] = sign * (M[i][j] - M[j][i]) for i < j, packed like theta.
hipError_t launch_pack_antisym(const float* M, const Seg& g, float sign, float* gtheta,
                               hipStream_t s);
// out = (to_bf16 ? bf16 : fp32) copy of n floats.
hipError_t launch_cast(const float* in, void* out, long long n, int to_bf16, hipStream_t s);
// out = float(in) for n bf16 values (exact)
hipError_t launch_widen(const void* in, float* out, long long n, hipStream_t s);
// INT8 rows of the pre-merged weight: q[i][j] = rint(W0[pi_R[i]][pi_P[j]] * 127 /
// amax_i) and scale[i] = amax_i / 127 (bf16 W0, n % 8 == 0, 2n <= 64 KiB)
hipError_t launch_quantize_rows(const void* W0, const int32_t* pi_R, const int32_t* pi_P,
                                int8_t* q, float* scale, int m, int n, hipStream_t s);
// bf16 C[t][c] *= scale[c] for t < rows, c < cols, row stride ld (one rounding)
hipError_t launch_scale_cols(void* C, const float* scale, long long rows, int cols, long long ld,
                             hipStream_t s);
// out[i][j] = scale[i] * q[i][j] (fp32)
// out = bf16(q) elementwise (exact), n int8 values; 16-byte aligned buffers
hipError_t launch_widen_i8(const void* q, void* out, long long n, hipStream_t s);
hipError_t launch_dequantize_rows(const int8_t* q, const float* scale, float* out, int m, int n,
                                  hipStream_t s);
// inv[pi[i]] = i for a permutation pi of 0..n-1
hipError_t launch_invert_perm(const int32_t* pi, int32_t* inv, int n, hipStream_t s);
// out1 = c * in; out2 = c * in (out2 may be null)
hipError_t launch_scale2(const float* in, float c, float* out1, float* out2, long long n,
                         hipStream_t s);
// out[i] = sum_{s < nsplit} part[s * stride + i], in order of s.
hipError_t launch_sum_splits(const float* part, int nsplit, long long stride, long long n,
                             float* out, hipStream_t s);
hipError_t launch_zero(float* out, long long n, hipStream_t s);

// ---------------------------------------------------------------- fp32 GEMM
// C(m,n) = alpha * sum_k A(m,k) B(n,k) + beta * Cin(m,n) + gamma * [m == n];
// optionally E(m,n) = sum_k A(m,k) B(n,k). General element strides, batched over
// `groups` (group strides) and split over K (`splits`, partial outputs c_ss apart;
// with splits > 1 only alpha applies).
struct GemmF32 {
  const float* A; const float* B; float* C; const float* Cin; float* E;
  int M, N, K;
  long long a_rs, a_cs, b_rs, b_cs, c_rs;
  long long a_gs, b_gs, c_gs;
  int groups, splits;
  long long c_ss;
  float alpha, beta, gamma;
  // when set, group g is skipped (C untouched) unless iters[g] > it
  const int32_t* iters = nullptr;
  int it = 0;
};
hipError_t launch_gemm_f32(const GemmF32& p, hipStream_t s);
// Runs of the same shape and strides (splits = 1, no E output) in one launch:
// run i has its own A, B, C, Cin and group count; group strides from `shape`.
struct GemmF32Run {
  const float* A; const float* B; float* C; const float* Cin;
  int groups;
  const int32_t* iters = nullptr;   // per-group skip (GemmF32::iters, with the shape's it)
};
constexpr int kF32MaxRuns = 16;
struct GemmF32Runs {
  GemmF32 p;
  int n;
  GemmF32Run r[kF32MaxRuns];
  int z0[kF32MaxRuns];
};
hipError_t launch_gemm_f32_runs(const GemmF32& shape, const GemmF32Run* runs, int n, hipStream_t s);

// ---------------------------------------------------------------- bf16 MFMA GEMM
// C(m,n) = sum_k A(m,k) B(n,k), bf16 inputs, fp32 accumulation.
// A(m,k) = A[m*lda + k] when a_kmajor, else A[k*lda + m]; same for B with ldb.
// Output bf16 (out_f32 = 0) or fp32; C(m,n) at C[m*ldc + n]. Batched over groups
// and split over K like GemmF32.
enum GemmRole { GEMM_BLOCK = 0, GEMM_W0 = 1, GEMM_DQ = 2 };
struct GemmBf16 {
  const void* A; const void* B; void* C;
  int role;   // GemmRole: selects the kernel symbol (layouts must match the role)
  int M, N, K;
  long long lda, ldb, ldc;
  int a_kmajor, b_kmajor, out_f32;
  long long a_gs, b_gs, c_gs;
  int groups, splits;
  long long c_ss;
  int tpw;    // output tiles per workgroup (set by the launcher)
  // bf16 output only: column n of group g is multiplied by col_scale[g * c_gs + n]
  // (fp32, before the rounding) when non-null
  const float* col_scale = nullptr;
  // the tiles of one (group, split) run on one XCD (they share A and B rows in
  // its L2): set by the launcher when tpw == 1 and groups * splits % 8 == 0
  int xcd_cluster = 0;
  // single-group launches with >= 256 tiles: 256 workgroups; the tiles of XCD x
  // are the contiguous range [ntile x / 8, ntile (x + 1) / 8), walked by its
  // workgroups with a stride of their count, so those resident together take
  // consecutive tiles (set by the launcher)
  int xcd_stride = 0;
};
hipError_t launch_gemm_bf16(const GemmBf16& p, hipStream_t s);
// The token reduction dQ = G^T A over `count` blocks of b (K = the tokens):
// 128 x 128 output tiles at two workgroups per CU, or, for blocks of 512 and up
// (whole-tile pipelined kernels only, so K a multiple of 64), 256 x 256 tiles at
// one per CU when a round of them fills the chip clearly better: 21 blocks of 512
// give 336 small tiles (a third of the chip idle at one split, two rounds at
// two) but 84 large ones (three splits, 252 workgroups). Where both fill it the
// small tiles win: same time per launch at half the partial sums. The host
// sizes the split count with the same rule.
inline double dq_round_fill(long long tiles, long long slots) {
  const long long s = tiles >= slots ? 1 : slots / tiles;
  const long long wgs = tiles * s;
  return (double)wgs / (double)(((wgs + slots - 1) / slots) * slots);
}
inline bool dq_big_tiles(int b, int count, long long K) {
  if (b < 512 || b % 256 || K % 64 || count <= 0) return false;
  const long long small = (long long)(b / 128) * (b / 128) * count;
  const long long big = (long long)(b / 256) * (b / 256) * count;
  return dq_round_fill(big, 256) > dq_round_fill(small, 512) + 0.1;
}
// Pipelined variant (direct-to-LDS loads, see k_gemm_lds.hip) for whole-tile shapes:
// big = 256 x 256 tiles, else 128 x 128.
bool gemm_lds_supported(const GemmBf16& p, int bm, int bn);
hipError_t launch_gemm_lds(const GemmBf16& p, int big, hipStream_t s);
// Frozen-weight NT product on whole 256 x 256 tiles (k_gemm_w0.hip).
bool w0_pipe_supported(const GemmBf16& p);
hipError_t launch_w0_pipe(const GemmBf16& p, hipStream_t s);
// Block products with b = 256 or 512 (N = K, GEMM_BLOCK, bf16 output, optional
// column scale): B in registers, A tiles streamed through LDS
// (k_block_regb.hip).
bool block_regb_supported(const GemmBf16& p);
hipError_t launch_block_regb(const GemmBf16& p, hipStream_t s);

// ---------------------------------------------------------------- fp32 MFMA chains
// Row-panel power chains (see k_chain.hip), batched over runs of equal blocks
// from any number of sides and layers so that one launch fills the chip.
enum ChainMode { CHAIN_BUILD = 0, CHAIN_ABAR = 1, CHAIN_TCHAIN = 2 };
constexpr int kChainMaxEntries = 32;
struct ChainEntry {
  const float* S;     // skew generators of the run's first block, fp32 (unused when Mh is set)
  const float* G;     // ABAR: dL/dQ of the run; TCHAIN: stored A_j of the run
  float* out;         // BUILD: Q; ABAR: A_j store; TCHAIN: T_1^T
  void* out_act;      // BUILD: copy of Q in the activation dtype, or null
  long long stride;   // elements between consecutive stored A_j (ABAR, TCHAIN)
  int b, count;       // block size and number of blocks of the run
  int wg0;            // first workgroup of the run (filled by the launcher)
  int act_bf16;
  // bf16 split of -S = S^T (the run's count blocks of b x b rounded to bf16,
  // then the count blocks of the residuals), written by the unpack; when set
  // (b % 32 == 0, b <= 256) the products run as three bf16 MFMAs each
  const uint16_t* Mh = nullptr;
};
struct ChainBatch {
  int n, k;
  ChainEntry e[kChainMaxEntries];
};
bool chain_supported(int b);
// Launches the entries of `cb` (all chain_supported), one kernel per size class.
hipError_t launch_chain_batch(int mode, const ChainBatch& cb, hipStream_t s);

// Batched unpack (theta -> S) and pack (sign * (M - M^T) -> packed gradient)
// over runs of chain_supported block sizes.
struct TriEntry {
  const float* src;   // unpack: packed theta of the run; pack: b x b matrices of the run
  float* dst;         // unpack: b x b matrices (or null: split only); pack: packed gradient of the run
  int b, count;
  long long e0;       // first workgroup of the run (set by the launcher)
  uint16_t* split = nullptr;   // unpack: also the bf16 split of -S (ChainEntry::Mh)
};
// Block sizes whose chains can run on the bf16 split products.
bool chain_split_supported(int b);
struct TriBatch {
  int n;
  float sign;
  TriEntry e[kChainMaxEntries];
};
hipError_t launch_unpack_batch(const TriBatch& tb, hipStream_t s);
hipError_t launch_pack_batch(const TriBatch& tb, hipStream_t s);

}  // namespace poetx
