/*
 * libpoetx: the POET-X orthogonal-equivalence linear layer y = R W0 P x on
 * AMD Instinct MI355X (gfx950), as hand-written HIP kernels behind a C ABI.
 *
 * Citations
 *   [PX]   page "POET-X: Memory-efficient LLM Training by Scaling Orthogonal
 *          Transformation" (gist.science, French), section "Résumé technique".
 *   [Pion] page "Pion：保持谱稳定的大语言模型训练优化器", section "数学原理".
 *
 * Mathematical conventions (shared with any independent checker)
 *   Activations are row-major [T, features]. One token maps as y = R W0 P x,
 *   i.e. Y = X P^T W0^T R^T for the whole batch.
 *   P = Pi_P^T D_P Pi_P and R = Pi_R^T D_R Pi_R, where (Pi v)_i = v[pi[i]] and
 *   D = blockdiag(Q_1, Q_2, ...) over contiguous blocks ([PX] §2.B, §2.C).
 *   Each block Q = (I + S) * sum_{j=0..k} S^j: the Cayley transform
 *   (I+S)(I-S)^{-1} with the inverse truncated to its Neumann series ([PX]
 *   §2.D). S is skew; only its strict upper triangle is stored, row-major,
 *   S[i][j] = theta, S[j][i] = -theta (b(b-1)/2 floats per block, [PX] §2.D),
 *   blocks concatenated in order.
 *   The weight is pre-merged with both permutations once per inner loop
 *   ([PX] §2.B): Wt[i][j] = W0[pi_R[i]][pi_P[j]].
 *
 * Memory and threading
 *   Every buffer is owned by the caller. Pointers marked "device" must be
 *   device memory (e.g. from hipMalloc / torch); "host" arrays are read during
 *   the call only. The library allocates no device memory: each call that needs
 *   scratch takes a caller-provided workspace of poetx_workspace_size() bytes.
 *   Calls are asynchronous on the given stream and never synchronise the host.
 *   A plan is immutable after creation and may be shared by threads as long as
 *   every concurrent call has its own workspace.
 *
 * Errors
 *   Every call returns a poetx_status and never aborts. Arguments are checked on
 *   the host before any launch; nothing is launched on error. Device pointers
 *   must be 16-byte aligned. Permutation arrays must hold permutations; this is
 *   the caller's guarantee and is not checked on the device.
 */
#ifndef POETX_H
#define POETX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  POETX_OK = 0,
  POETX_ERR_INVALID_ARG = 1,  /* NULL pointer, negative size, bad enum       */
  POETX_ERR_SHAPE = 2,        /* block sizes do not sum to m or n, k range    */
  POETX_ERR_DTYPE = 3,        /* unknown dtype                                */
  POETX_ERR_ALIGNMENT = 4,    /* a device pointer is not 16-byte aligned      */
  POETX_ERR_UNSUPPORTED = 5,  /* valid but not handled (see poetx_plan_create) */
  POETX_ERR_HIP = 6,          /* a kernel launch failed                       */
  POETX_ERR_WORKSPACE = 7     /* workspace NULL or smaller than required      */
} poetx_status;

typedef enum { POETX_FP32 = 0, POETX_BF16 = 1 } poetx_dtype;

/* Storage of the pre-merged frozen weight Wt that forward, backward and merge read.
 *   POETX_WEIGHT_DENSE:     [m, n] in the plan dtype (poetx_permute_weight).
 *   POETX_WEIGHT_INT8_ROWS: POET-XQ ([PX] §2.E "Quantification": base weights
 *     kept in INT8, dequantised on the fly); the pages give no scheme, this one
 *     is symmetric with one fp32 scale per row of Wt. Layout: int8 q [m, n]
 *     row-major, then at byte offset ceil(m n / 256) * 256 the fp32 scales [m];
 *     Wt[i][j] = s[i] * q[i][j]. Built by poetx_quantize_weight; needs bf16
 *     and m, n multiples of 256, n <= 32768.
 *   POETX_WEIGHT_DENSE_T:   POETX_WEIGHT_DENSE followed by the transpose of Wt,
 *     WtT [n, m] in the plan dtype at byte offset ceil(m n elsize / 256) * 256
 *     (poetx_permute_weight writes both). The frozen weight is kept twice so that
 *     the backward's product G_V = G_Wa Wt reads it K-contiguous, like the
 *     forward's V Wt^T; results are identical to POETX_WEIGHT_DENSE.
 *   POETX_WEIGHT_INT8_ROWS_T: POETX_WEIGHT_INT8_ROWS followed by the transpose
 *     of q, qT [n, m] int8, at byte offset ceil((ceil(m n / 256) * 256 + 4 m) /
 *     256) * 256 (poetx_quantize_weight writes all three), for the same reason;
 *     results are identical to POETX_WEIGHT_INT8_ROWS. */
typedef enum {
  POETX_WEIGHT_DENSE = 0,
  POETX_WEIGHT_INT8_ROWS = 1,
  POETX_WEIGHT_DENSE_T = 2,
  POETX_WEIGHT_INT8_ROWS_T = 3
} poetx_weight;

/* Orthogonal map of each block.
 *   POETX_CAYLEY_NEUMANN: Q = (I+S) sum_{j<=k} S^j, the truncated series of [PX]
 *     §2.D, and the gradient of that truncated Q (the default).
 *   POETX_CAYLEY_EXACT: the Cayley transform itself, Q = (I+S)(I-S)^{-1} =
 *     2 (I-S)^{-1} - I, as a reference build, and the exact gradient
 *     dL/dS = (I+Q)^T G (I-S)^{-T}. k is ignored. (I-S)^{-1} comes from the
 *     Newton-Schulz iteration X <- X (2I - (I-S) X) started at
 *     X0 = (I+S) 2 / (2 + c^2), c = max row sum of |S| >= ||S||_2, which
 *     converges for every skew S (the residual is symmetric with norm at most
 *     c^2 / (2 + c^2) and squares each step); each block runs the steps it needs
 *     for a residual below 2^-30 (6 at c = 2), at most 28 (c up to ~4000).
 *     fp32 products on the batched fp32 GEMM, one launch per step over every
 *     block of a size. */
typedef enum { POETX_CAYLEY_NEUMANN = 0, POETX_CAYLEY_EXACT = 1 } poetx_cayley;

/* Where the block-diagonal factors are applied.
 *   POETX_FOLD_NONE (the default): on the activations at every batch size, in
 *     the order of the input-centric method ([PX] §2.A): gather, blocks of P,
 *     Wt product, blocks of R, scatter (backward: the reverse). No weight-sized
 *     product with an orthogonal factor is ever formed.
 *   POETX_FOLD_WEIGHT: a variant that reassociates one product per pass when
 *     the batch is large: the forward forms Wt D_P (m x n, one side's blocks
 *     applied to the weight's columns) when T >= m and then Wa = U (Wt D_P)^T;
 *     the backward forms D_R Wt when T >= n and then G_V = G_Z (D_R Wt). Same
 *     results up to rounding (the bf16 rounding moves from the activation to the
 *     folded weight); not for INT8 weights. */
typedef enum { POETX_FOLD_NONE = 0, POETX_FOLD_WEIGHT = 1 } poetx_fold;

/* How the index mappings run ([PX] §2.B: permutations as index arrays).
 *   POETX_INDEX_SEPARATE (the default): each gather and scatter is its own
 *     pass over the rows (whole rows staged in LDS, coalesced 16-byte reads and
 *     writes), next to the block products, which keep each block of Q in
 *     registers while token tiles stream past.
 *   POETX_INDEX_FUSED: bf16 sides of 256-wide blocks up to 2048 features run
 *     the index mapping inside the block products: one pass stages 32 whole
 *     token rows in LDS, permutes them there and multiplies them block by block,
 *     so the permuted activation never goes through HBM. Each 32-row panel then
 *     streams every Q block of the side from L2 (4x the activation bytes it
 *     saves at 2048 features), which on MI355X makes these passes slower than
 *     the separate ones; same results. Other sides keep the separate kernels. */
typedef enum { POETX_INDEX_SEPARATE = 0, POETX_INDEX_FUSED = 1 } poetx_index;

/* How the build evaluates Q = sum_{j=0..k+1} c_j S^j (c_0 = c_{k+1} = 1,
 * c_j = 2 otherwise; [PX] §2.D) for POETX_CAYLEY_NEUMANN plans.
 *   POETX_SERIES_CHAIN (the default): the power chain P_j = P_{j-1} S, k
 *     products per block, fused in one kernel per block size (row panels of a
 *     block kept on chip).
 *   POETX_SERIES_PS: Paterson-Stockmeyer. With s = the step that minimises the
 *     product count, the powers S^2 .. S^s (s - 1 products), then
 *     Q = B_0 + S^s (B_1 + S^s (B_2 + ...)) with each B_i = sum_{l<s} c_{is+l}
 *     S^l formed from the stored powers without products (a last B_i that is a
 *     multiple of I is folded in the same way): 3 products at k = 4 and k = 5
 *     instead of 4 and 5, 2 sqrt(k) or so for large k. Batched fp32 products
 *     (fp32 accuracy in every plan). The backward is the same for both. */
typedef enum { POETX_SERIES_CHAIN = 0, POETX_SERIES_PS = 1 } poetx_series;
typedef enum { POETX_SIDE_R = 0, POETX_SIDE_P = 1 } poetx_side;
typedef enum {
  POETX_WS_BUILD = 0,       /* poetx_build_orth, one item of poetx_build_orth_batch */
  POETX_WS_FORWARD = 1,     /* poetx_forward                                        */
  POETX_WS_BACKWARD = 2,    /* poetx_backward and poetx_backward_dq                  */
  POETX_WS_PARAM_GRAD = 3,  /* one item of poetx_param_grad_batch (T is ignored)     */
  POETX_WS_MERGE = 4        /* poetx_merge_weight (T is ignored)                     */
} poetx_ws_kind;

typedef struct poetx_plan poetx_plan;   /* opaque, immutable after create */

typedef struct {
  int32_t m, n;             /* W0 is [m, n] row-major (out x in)                   */
  int32_t nb_R, nb_P;       /* number of blocks of R and of P                       */
  const int32_t* bsz_R;     /* host, nb_R block sizes, summing to m                  */
  const int32_t* bsz_P;     /* host, nb_P block sizes, summing to n                  */
  int32_t k;                /* Neumann order, 0 <= k <= 32: powers S^0..S^k          */
  int32_t dtype;            /* poetx_dtype of X, Y, W0, Wt, Q copies and gradients
                               of X/Y. Skew parameters and their gradients are
                               always fp32; accumulation is always fp32.            */
  int32_t weight;           /* poetx_weight: how Wt is stored                       */
  int32_t cayley;           /* poetx_cayley: truncated series or exact transform    */
  int32_t fold;             /* poetx_fold: activations only, or the weight-side fold */
  int32_t index;            /* poetx_index: separate index passes, or fused         */
  int32_t series;           /* poetx_series: power chain or Paterson-Stockmeyer     */
} poetx_desc;

/* Create a plan. Host only: no device call is made, so it works without a GPU.
 * POETX_ERR_SHAPE: m or n < 1, a block size < 1, sums differ from m / n, or
 *   k outside [0, 32].
 * POETX_ERR_UNSUPPORTED: dtype BF16 with m, n or a block size not a multiple of
 *   16 (fp32 plans take any sizes). */
poetx_status poetx_plan_create(const poetx_desc* desc, poetx_plan** out);
void poetx_plan_destroy(poetx_plan* plan);

/* Number of packed skew parameters of one side: sum_i b_i (b_i - 1) / 2. */
int64_t poetx_param_count(const poetx_plan* plan, int32_t side);
/* Number of elements of one side's block array: sum_i b_i^2. */
int64_t poetx_block_elems(const poetx_plan* plan, int32_t side);

/* Workspace bytes needed by a call of the given kind for T tokens (T is
 * ignored for POETX_WS_BUILD). Returns 0 for an invalid plan or kind. */
size_t poetx_workspace_size(const poetx_plan* plan, int64_t T, int32_t kind);

/* Short static description of a status code. */
const char* poetx_status_string(poetx_status status);

/* Description of the HIP error behind the calling thread's most recent
 * POETX_ERR_HIP (static string; "no HIP error" if there was none). */
const char* poetx_last_hip_error(void);

/* Pre-merge of the permutations into the frozen weight, once per inner loop
 * ([PX] §2.B "Réduction": permutations folded into W ahead of time, leaving
 * two index operations per step): Wt[i][j] = W0[pi_R[i]][pi_P[j]].
 *   W0   device [m, n] (dtype)        pi_R device int32 [m]
 *   pi_P device int32 [n]             Wt   device, poetx_weight_bytes(plan)
 *        bytes, not aliasing W0: [m, n] (dtype), for POETX_WEIGHT_DENSE_T plans
 *        followed by WtT[j][i] = Wt[i][j]
 * Bit-exact copy. POETX_ERR_UNSUPPORTED for INT8 plans (poetx_quantize_weight). */
poetx_status poetx_permute_weight(const poetx_plan* plan, const void* W0,
                                  const int32_t* pi_R, const int32_t* pi_P,
                                  void* Wt, void* stream);

/* Bytes of Wt for this plan (m n elsize dense; the int8 layout of
 * POETX_WEIGHT_INT8_ROWS otherwise). 0 for a NULL plan. */
size_t poetx_weight_bytes(const poetx_plan* plan);

/* POETX_WEIGHT_INT8_ROWS plans: pre-merge and quantise in one pass, the INT8
 * counterpart of poetx_permute_weight. Row i of Wt is row pi_R[i] of W0 with its
 * columns gathered by pi_P; in fp32, round to nearest even:
 *   amax = max_j |Wt[i][j]|, inv = 127 / amax, q[i][j] = clamp(rint(Wt[i][j] inv), -127, 127),
 *   s[i] = amax / 127 (amax = 0: q = 0, s = 0).
 *   W0 device [m, n] bf16     Wq device, poetx_weight_bytes(plan) bytes, not aliasing W0
 * POETX_ERR_UNSUPPORTED for dense plans. Bit-exact (integer decisions taken
 * in fp32 with correctly rounded division). */
poetx_status poetx_quantize_weight(const poetx_plan* plan, const void* W0, const int32_t* pi_R,
                                   const int32_t* pi_P, void* Wq, void* stream);

/* End of an inner loop: the orthogonal factors are folded into the weight,
 * W_out = R W0 P in the original coordinates (the two-sided orthogonal update
 * W_new = Q_left W Q_right of [Pion] "数学原理"; [PX] §2.B keeps W fixed for the
 * inner loop). The caller then starts the next inner loop from W_out with
 * theta = 0 and new permutations (poetx_permute_weight).
 *   Wt         device [m, n] (dtype): poetx_permute_weight(W0, pi_R, pi_P); for
 *              INT8 plans the poetx_quantize_weight layout (dequantised exactly
 *              to fp32 first), the result W_out is then dense bf16
 *   pi_R, pi_P device int32, the permutations Wt was built with
 *   Q_R, Q_P   device fp32 blocks (the Q_f32 output of poetx_build_orth)
 *   W_out      device [m, n] (dtype), not aliasing Wt
 *   ws         device, poetx_workspace_size(plan, 0, POETX_WS_MERGE) bytes.
 * The products run in fp32 from the fp32 blocks (Wt widened exactly); W_out is
 * rounded once to the dtype (bf16: round to nearest even). Deterministic. */
poetx_status poetx_merge_weight(const poetx_plan* plan, const void* Wt, const int32_t* pi_R,
                                const int32_t* pi_P, const float* Q_R, const float* Q_P,
                                void* W_out, void* ws, size_t ws_bytes, void* stream);

/* Cayley-Neumann blocks from packed skew parameters ([PX] §2.D).
 *   theta  device fp32 [poetx_param_count(side)]
 *   Q_f32  device fp32 [poetx_block_elems(side)]: block i row-major at offset
 *          sum_{j<i} b_j^2; Q = I + sum_{j=1..k+1} c_j S^j, c_j = 2 for j <= k
 *          and c_{k+1} = 1 (c_1 = 1 when k = 0)
 *   Q_act  device [poetx_block_elems(side)] in the plan dtype (round to nearest
 *          even for BF16), or NULL. FP32 plans may pass NULL and use Q_f32.
 *   ws     device, poetx_workspace_size(plan, 0, POETX_WS_BUILD) bytes. */
poetx_status poetx_build_orth(const poetx_plan* plan, int32_t side, const float* theta,
                              float* Q_f32, void* Q_act, void* ws, size_t ws_bytes,
                              void* stream);

/* Batched build: count independent (plan, side) items in as few launches as
 * possible (one per block-size class), e.g. every side of every layer of a
 * model once per optimizer step. The blocks of one side form a batch
 * computed block by block ([PX] §2.C); batching sides and layers only widens
 * the grid. Item i takes the arguments of poetx_build_orth: plans[i],
 * sides[i], thetas[i], Q_f32[i], Q_act ? Q_act[i] : NULL, ws[i] with
 * ws_bytes[i] >= poetx_workspace_size(plans[i], 0, POETX_WS_BUILD). Host arrays
 * of pointers; items must not share Q or workspace buffers. Every item is
 * checked before anything is launched; the first failing check is returned. */
poetx_status poetx_build_orth_batch(int32_t count, const poetx_plan* const* plans,
                                    const int32_t* sides, const float* const* thetas,
                                    float* const* Q_f32, void* const* Q_act, void* const* ws,
                                    const size_t* ws_bytes, void* stream);

/* Input-centric forward ([PX] §2.A): Y = R W0 P applied to the rows of X without
 * forming R W0 P. Stages: gather X by pi_P, blocks of P, product with Wt,
 * blocks of R, scatter by pi_R.
 *   X        device [T, n] (dtype)       Wt  device [m, n] from poetx_permute_weight,
 *            or for INT8 plans the poetx_quantize_weight layout: each call
 *            widens q exactly to bf16 in its workspace (m n 2 bytes of it) and
 *            the product applies s to the fp32 accumulators of each output
 *            column
 *   pi_R, pi_P device int32              Q_R, Q_P device block arrays in the plan dtype
 *   Y        device [T, m] (dtype)
 *   Wa_saved device [T, m] (dtype) or NULL: the output of the Wt product, the
 *            one extra activation kept for the backward (POET-Xfast, [PX] §2.E)
 *   U_saved  device [T, n] (dtype) or NULL: receives U = X Pi_P^T, the input in
 *            the permuted order the backward reads it in. A caller that keeps
 *            U_saved instead of X for the backward spares it a gather at no
 *            extra memory.
 *   X = NULL with U_saved set: U_saved already holds U (poetx_gather_cols of
 *            X by pi_P) and the forward skips its gather, so a caller can run
 *            the gather apart, e.g. on another stream ahead of the rest;
 *            X = NULL without U_saved is POETX_ERR_INVALID_ARG.
 *   ws       device, poetx_workspace_size(plan, T, POETX_WS_FORWARD) bytes.
 * T = 0 is a no-op. */
poetx_status poetx_forward(const poetx_plan* plan, int64_t T, const void* X, const void* Wt,
                           const int32_t* pi_R, const int32_t* pi_P,
                           const void* Q_R, const void* Q_P,
                           void* Y, void* Wa_saved, void* U_saved, void* ws, size_t ws_bytes,
                           void* stream);

/* poetx_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments without the workspace, which comes from a static device
 * array inside the library instead (poetx_forward_noalloc_max_bytes() bytes,
 * 64 MiB; each GPU holds its own copy from the library's first use on it until
 * the process ends). The call allocates nothing and runs the same kernels as
 * poetx_forward, with the same results.
 *   POETX_ERR_WORKSPACE when poetx_workspace_size(plan, T, POETX_WS_FORWARD)
 *   exceeds that size (checked before the device is touched); argument errors
 *   as for poetx_forward.
 * Every call on one GPU uses that GPU's one array: calls that overlap on one
 * GPU (concurrent streams or threads) race and must be serialised by the
 * caller. Nothing in the array needs to start at zero. */
poetx_status poetx_forward_noalloc(const poetx_plan* plan, int64_t T, const void* X, const void* Wt,
                                   const int32_t* pi_R, const int32_t* pi_P, const void* Q_R,
                                   const void* Q_P, void* Y, void* Wa_saved, void* U_saved,
                                   void* stream);
size_t poetx_forward_noalloc_max_bytes(void);

/* Backward of L = <G_Y, Y> w.r.t. X and both sides' skew parameters, for the
 * truncated Q the forward used. W0 is frozen and gets no gradient.
 *   X, Wt, pi_R, pi_P, Q_R, Q_P as in poetx_forward (INT8 plans: the scale
 *            of row i of Wt multiplies column i of G_Wa in the block product
 *            that produces it, so that G_V = (G_Wa diag(s)) q)
 *   theta_R, theta_P device fp32 packed parameters (rebuild S for the chain rule)
 *   Wa_saved device [T, m] from poetx_forward, or NULL: then the backward
 *            recomputes it from X (gather, blocks of P, Wt product: POET-Xmem,
 *            [PX] §2.E), trading one more forward's worth of the first three
 *            stages for T x m activations; results are identical either way
 *   U_saved  device [T, n] from poetx_forward's U_saved, or NULL: with it X is
 *            not read (may be NULL) and the backward skips its gather of X
 *   G_Y      device [T, m] (dtype)      G_X device [T, n] (dtype)
 *   g_theta_R, g_theta_P device fp32 [param_count] (overwritten)
 *   ws       device, poetx_workspace_size(plan, T, POETX_WS_BACKWARD) bytes.
 * Deterministic: all reductions run in a fixed order. T = 0 writes zero
 * parameter gradients. */
poetx_status poetx_backward(const poetx_plan* plan, int64_t T, const void* X, const void* Wt,
                            const int32_t* pi_R, const int32_t* pi_P,
                            const float* theta_R, const float* theta_P,
                            const void* Q_R, const void* Q_P, const void* Wa_saved,
                            const void* U_saved, const void* G_Y, void* G_X, float* g_theta_R,
                            float* g_theta_P, void* ws, size_t ws_bytes, void* stream);

/* The backward split in two, so that the chain rule through the parameterisation
 * of many layers can share launches:
 *   poetx_backward_dq: the activation path of poetx_backward. Writes G_X and
 *     dL/dQ of both sides (fp32, block layout of poetx_build_orth: dQ_R has
 *     poetx_block_elems(R) floats, dQ_P poetx_block_elems(P)), where Q is the
 *     block array the forward used. Same arguments and workspace as
 *     poetx_backward otherwise. T = 0 writes zero dQ.
 *   poetx_param_grad_batch: dL/dQ -> packed parameter gradient for count
 *     independent (plan, side) items: item i reads thetas[i] and dQs[i] (device
 *     fp32) and overwrites g_thetas[i] (device fp32, poetx_param_count floats),
 *     with its own workspace ws[i] of ws_bytes[i] >= poetx_workspace_size(
 *     plans[i], 0, POETX_WS_PARAM_GRAD). Host arrays of pointers. All items are
 *     checked before anything is launched.
 * poetx_backward(...) equals poetx_backward_dq(...) followed by
 * poetx_param_grad_batch over its two sides. */
poetx_status poetx_backward_dq(const poetx_plan* plan, int64_t T, const void* X, const void* Wt,
                               const int32_t* pi_R, const int32_t* pi_P,
                               const void* Q_R, const void* Q_P, const void* Wa_saved,
                               const void* U_saved, const void* G_Y, void* G_X, float* dQ_R,
                               float* dQ_P, void* ws, size_t ws_bytes, void* stream);
poetx_status poetx_param_grad_batch(int32_t count, const poetx_plan* const* plans,
                                    const int32_t* sides, const float* const* thetas,
                                    const float* const* dQs, float* const* g_thetas,
                                    void* const* ws, const size_t* ws_bytes, void* stream);

/* Single index operations, exposed for testing and for callers that apply the
 * permutations themselves ([PX] §2.B: index mapping, no permutation matrix).
 *   poetx_gather_cols:  out[t][i] = in[t][idx[i]]      (out = in Pi^T)
 *   poetx_scatter_cols: out[t][idx[i]] = in[t][i]      (out = in Pi)
 * in/out device [T, dim] row-major in the plan dtype, not aliasing; idx device
 * int32 [dim], a permutation of 0..dim-1. Bit-exact. */
poetx_status poetx_gather_cols(const poetx_plan* plan, int64_t T, int32_t dim, const void* in,
                               const int32_t* idx, void* out, void* stream);
poetx_status poetx_scatter_cols(const poetx_plan* plan, int64_t T, int32_t dim, const void* in,
                                const int32_t* idx, void* out, void* stream);

/* Optional stage timing for benchmarks. Stage i is timed when bit i of `mask`
 * is set: every later call records a pair of HIP events on its own stream
 * around that stage's kernels (event objects are created on demand; no device
 * memory is allocated). mask = 0 (the default) records nothing. */
typedef enum {
  POETX_STAGE_BUILD = 0,      /* poetx_build_orth, whole call                   */
  POETX_STAGE_GATHER = 1,     /* column gathers (forward and backward)          */
  POETX_STAGE_BLOCK_FWD = 2,  /* block-diagonal products in the forward         */
  POETX_STAGE_W0_FWD = 3,     /* Wa = V Wt^T                                    */
  POETX_STAGE_SCATTER = 4,    /* column scatters (forward and backward)         */
  POETX_STAGE_DQ = 5,         /* dL/dQ products and their fixed-order reduction  */
  POETX_STAGE_BLOCK_BWD = 6,  /* block-diagonal products in the backward        */
  POETX_STAGE_W0_BWD = 7,     /* G_V = G_Wa Wt                                  */
  POETX_STAGE_CNP_BWD = 8,    /* reverse mode through the Neumann series        */
  POETX_NUM_STAGES = 9
} poetx_stage;

poetx_status poetx_timing_enable(uint32_t mask);
/* Waits for the recorded events of one stage and returns their total time in
 * milliseconds and the number of recorded intervals since the last reset.
 * POETX_ERR_INVALID_ARG for a bad stage or NULL outputs; POETX_ERR_HIP if an
 * event query fails. */
poetx_status poetx_timing_read(int32_t stage, double* ms, int64_t* count);
/* Forget all recorded intervals (their events are kept for reuse). */
void poetx_timing_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* POETX_H */
