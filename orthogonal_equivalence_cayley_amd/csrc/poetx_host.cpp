// Host side of libpoetx: plan creation, argument checks, workspace layout and
// the launch sequence of each call. Everything here runs on the host; the
// arithmetic runs in the HIP kernels declared in poetx_internal.h.
//
// Citations
//   [PX] page "POET-X: Memory-efficient LLM Training by Scaling Orthogonal
//        Transformation" (gist.science, French), section "Résumé technique".
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/poetx.h"
#include "poetx_internal.h"

using poetx::Seg;

struct poetx_plan {
  int m = 0, n = 0, k = 0, dtype = 0;
  int weight = POETX_WEIGHT_DENSE;   // poetx_weight: how Wt is stored
  int cayley = POETX_CAYLEY_NEUMANN; // poetx_cayley: truncated series or exact transform
  int fold = POETX_FOLD_NONE;        // poetx_fold: activations only, or the weight-side fold
  int index = POETX_INDEX_SEPARATE;  // poetx_index: separate index passes, or fused
  int series = POETX_SERIES_CHAIN;   // poetx_series: power chain or Paterson-Stockmeyer
  std::vector<int> bsz[2];
  std::vector<Seg> segs[2];
  long long nparam[2] = {0, 0};
  long long nelem[2] = {0, 0};
  int dim[2] = {0, 0};   // m for R, n for P
};

namespace {

constexpr size_t kAlign = 256;

// INT8 weight: int8 [m, n] rows of Wt, then (256-byte aligned) the fp32 row
// scales, then for POETX_WEIGHT_INT8_ROWS_T (256-byte aligned) qT [n, m]
bool wq(const poetx_plan* pl) {
  return pl->weight == POETX_WEIGHT_INT8_ROWS || pl->weight == POETX_WEIGHT_INT8_ROWS_T;
}
bool wqpair(const poetx_plan* pl) { return pl->weight == POETX_WEIGHT_INT8_ROWS_T; }
// dense weight kept with its transpose: WtT [n, m] after Wt, 256-byte aligned
bool wpair(const poetx_plan* pl) { return pl->weight == POETX_WEIGHT_DENSE_T; }
size_t wtt_off(const poetx_plan* pl) {
  const size_t es = pl->dtype == POETX_BF16 ? 2 : 4;
  return ((size_t)pl->m * pl->n * es + kAlign - 1) / kAlign * kAlign;
}
const void* wtt(const poetx_plan* pl, const void* Wt) { return static_cast<const char*>(Wt) + wtt_off(pl); }
size_t qscale_off(const poetx_plan* pl) {
  return ((size_t)pl->m * pl->n + kAlign - 1) / kAlign * kAlign;
}
size_t qt_off(const poetx_plan* pl) {
  return (qscale_off(pl) + 4 * (size_t)pl->m + kAlign - 1) / kAlign * kAlign;
}
const void* qt(const poetx_plan* pl, const void* Wt) { return static_cast<const char*>(Wt) + qt_off(pl); }
const float* qscale(const poetx_plan* pl, const void* Wt) {
  return reinterpret_cast<const float*>(static_cast<const char*>(Wt) + qscale_off(pl));
}

// ------------------------------------------------------------------ stage timing
std::atomic<uint32_t> g_tmask{0};
std::mutex g_tmu;
struct TimingRec {
  int stage;
  hipEvent_t a, b;
};
std::vector<TimingRec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t pooled_event() {
  hipEvent_t e = nullptr;
  if (!g_pool.empty()) {
    e = g_pool.back();
    g_pool.pop_back();
  } else if (hipEventCreate(&e) != hipSuccess) {
    e = nullptr;
  }
  return e;
}

// Records HIP events around the kernels of one stage when its timing bit is set.
struct StageScope {
  int stage;
  hipStream_t s;
  hipEvent_t a = nullptr;
  StageScope(int st, hipStream_t str) : stage(st), s(str) {
    if (g_tmask.load(std::memory_order_relaxed) & (1u << st)) {
      std::lock_guard<std::mutex> lk(g_tmu);
      a = pooled_event();
      if (a && hipEventRecord(a, s) != hipSuccess) {
        g_pool.push_back(a);
        a = nullptr;
      }
    }
  }
  ~StageScope() {
    if (!a) return;
    std::lock_guard<std::mutex> lk(g_tmu);
    hipEvent_t b = pooled_event();
    if (b && hipEventRecord(b, s) == hipSuccess) {
      g_recs.push_back(TimingRec{stage, a, b});
    } else {
      g_pool.push_back(a);
      if (b) g_pool.push_back(b);
    }
  }
};

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool side_ok_fn(int32_t side) { return side == POETX_SIDE_R || side == POETX_SIDE_P; }
int elsize(const poetx_plan* pl) { return pl->dtype == POETX_BF16 ? 2 : 4; }

// Coefficients of Q = sum_{j=0..k+1} c_j S^j for Q = (I+S) sum_{j<=k} S^j.
float coef(int j, int k) {
  if (j == 0 || j == k + 1) return 1.0f;
  return 2.0f;
}

// Carves consecutive 256-byte-aligned regions out of a workspace.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  void* take(size_t bytes) {
    void* p = base ? base + off : nullptr;
    off += align_up(bytes);
    return p;
  }
};

// Split count over the tokens of dQ = G^T A for one run of equal blocks (each
// run is its own launch with its own partial sums): about one round of
// workgroups on the chip. bf16: 128 x 128 tiles at two workgroups per CU, or
// the 256 x 256 tiles of dq_big_tiles at one; fp32: 64 x 64 tiles of the
// generic kernel. A multiple of 8 (blocks x splits) where possible, so the
// tiles of one split share an XCD; at most one split per 256 tokens and 64.
int dq_splits(const poetx_plan* pl, const Seg& g, long long T) {
  long long s;
  if (pl->dtype == POETX_BF16) {
    const bool big = poetx::dq_big_tiles(g.b, g.count, T);
    const int tile = big ? 256 : 128;
    const long long slots = big ? 256 : 512;
    const long long per = (g.b + tile - 1) / tile;
    const long long tiles = std::max<long long>(1, per * per * g.count);
    s = std::max<long long>(1, slots / tiles);
    while (s > 1 && (g.count * s) % 8) --s;
    if ((g.count * s) % 8) s = std::max<long long>(1, slots / tiles);
  } else {
    const long long per = (g.b + 63) / 64;
    const long long tiles = std::max<long long>(1, per * per * g.count);
    s = (512 + tiles - 1) / tiles;
  }
  const long long maxs = std::max<long long>(1, (T + 255) / 256);
  s = std::min(s, maxs);
  s = std::max<long long>(1, std::min<long long>(s, 64));
  return (int)s;
}
// fp32 partial sums one side's dQ needs: splits x elements of each run
long long dq_part_elems(const poetx_plan* pl, int side, long long T) {
  long long n = 0;
  for (const Seg& g : pl->segs[side]) n += (long long)dq_splits(pl, g, T) * g.count * g.b * g.b;
  return n;
}

struct FwdWs { void *U, *V, *Wa, *Z, *Wf, *Wq; };
struct BwdWs {
  void *GZ, *GWa, *GV, *U, *GU, *Wf, *Wq;
  void* QT[2];   // bf16 Q^T of a side that runs the fused products (or null)
  float *dQ[2], *part;
};

// POETX_FOLD_WEIGHT plans only (the default keeps every block product on the
// activations): one side's blocks are folded into the frozen weight instead,
// Wa = (U D_P^T) Wt^T = U (Wt D_P)^T in the forward and G_V = (G_Z D_R) Wt =
// G_Z (D_R Wt) in the backward, whose G_Wa nothing else reads. The weight-side
// product costs 2 m n b flops against 2 T n b (2 T m b) on the activations plus
// a T x n (T x m) round trip through HBM, so it is taken when T >= m (T >= n).
// INT8 weights keep the activation-side products.
bool fold_fwd(const poetx_plan* pl, long long T) {
  return pl->fold == POETX_FOLD_WEIGHT && !wq(pl) && T > 0 && T >= pl->m;
}
bool fold_bwd(const poetx_plan* pl, long long T) {
  return pl->fold == POETX_FOLD_WEIGHT && !wq(pl) && T > 0 && T >= pl->n;
}

// POETX_INDEX_FUSED plans: one side's index mapping and block products in one
// pass over the rows (k_panel.hip), for bf16 sides made of 256-wide blocks, up
// to 2048 features.
bool panel_side(const poetx_plan* pl, int side) {
  if (pl->index != POETX_INDEX_FUSED) return false;
  if (pl->dtype != POETX_BF16 || pl->segs[side].size() != 1) return false;
  const Seg& g = pl->segs[side][0];
  return poetx::panel_supported(pl->dim[side], g.b, g.count);
}

// Buffers of the chain rule through the parameterisation, for one side.
struct ChainWs {
  float *S, *T, *A;            // fused chains: generators, T_1^T, stored A_j
  float *A0, *A1, *T0, *T1;    // generic path (block sizes the fused chain skips)
  int32_t* iters;              // exact transform: Newton-Schulz steps per block
};

size_t layout_chain(const poetx_plan* pl, int side, Carver& c, ChainWs* w) {
  const size_t start = c.off;
  const long long ne = pl->nelem[side];
  ChainWs x;
  x.S = (float*)c.take(4 * ne);
  x.T = (float*)c.take(4 * ne);
  x.A = (float*)c.take(4 * ne * (pl->k + 1));
  x.A0 = (float*)c.take(4 * ne);
  x.A1 = (float*)c.take(4 * ne);
  x.T0 = (float*)c.take(4 * ne);
  x.T1 = (float*)c.take(4 * ne);
  x.iters = pl->cayley == POETX_CAYLEY_EXACT ? (int32_t*)c.take(4 * pl->bsz[side].size()) : nullptr;
  if (w) *w = x;
  return c.off - start;
}

size_t layout_fwd(const poetx_plan* pl, long long T, void* base, FwdWs* w) {
  Carver c(base);
  const size_t es = elsize(pl);
  FwdWs x;
  const bool fold = fold_fwd(pl, T);
  x.U = c.take(es * T * pl->n);
  x.V = fold ? nullptr : c.take(es * T * pl->n);
  x.Wa = c.take(es * T * pl->m);
  x.Z = c.take(es * T * pl->m);
  x.Wf = fold ? c.take(es * (size_t)pl->m * pl->n) : nullptr;
  x.Wq = wq(pl) ? c.take(2 * (size_t)pl->m * pl->n) : nullptr;
  if (w) *w = x;
  return c.off;
}

// backward workspace: activation path, then (for poetx_backward) both sides' chains
size_t layout_bwd(const poetx_plan* pl, long long T, void* base, BwdWs* w, ChainWs* cw) {
  Carver c(base);
  const size_t es = elsize(pl);
  BwdWs x;
  x.GZ = c.take(es * T * pl->m);
  x.GWa = c.take(es * T * pl->m);
  x.GV = c.take(es * T * pl->n);
  x.U = c.take(es * T * pl->n);
  x.GU = c.take(es * T * pl->n);
  x.Wf = (fold_fwd(pl, T) || fold_bwd(pl, T)) ? c.take(es * (size_t)pl->m * pl->n) : nullptr;
  x.Wq = wq(pl) ? c.take(2 * (size_t)pl->m * pl->n) : nullptr;
  for (int side = 0; side < 2; ++side)
    x.QT[side] = panel_side(pl, side) ? c.take(2 * pl->nelem[side]) : nullptr;
  x.dQ[0] = (float*)c.take(4 * pl->nelem[0]);
  x.dQ[1] = (float*)c.take(4 * pl->nelem[1]);
  long long part = 0;
  for (int side = 0; side < 2; ++side) part = std::max(part, dq_part_elems(pl, side, T));
  x.part = (float*)c.take(4 * part);
  if (w) *w = x;
  for (int side = 0; side < 2; ++side) layout_chain(pl, side, c, cw ? &cw[side] : nullptr);
  return c.off;
}

size_t layout_param_grad(const poetx_plan* pl, int side, void* base, ChainWs* cw) {
  Carver c(base);
  layout_chain(pl, side, c, cw);
  return c.off;
}

// merge workspace: Wt in fp32 (bf16 plans), the two fp32 products, the bf16
// rounding of the result (bf16 plans), and both inverse permutations
struct MergeWs {
  float *F, *M1, *M2;
  void* C;
  int32_t *invR, *invP;
};
size_t layout_merge(const poetx_plan* pl, void* base, MergeWs* w) {
  Carver c(base);
  const long long mn = (long long)pl->m * pl->n;
  const bool bf16 = pl->dtype == POETX_BF16;
  MergeWs x;
  x.F = bf16 ? (float*)c.take(4 * mn) : nullptr;
  x.M1 = (float*)c.take(4 * mn);
  x.M2 = (float*)c.take(4 * mn);
  x.C = bf16 ? c.take(2 * mn) : nullptr;
  x.invR = (int32_t*)c.take(4 * (size_t)pl->m);
  x.invP = (int32_t*)c.take(4 * (size_t)pl->n);
  if (w) *w = x;
  return c.off;
}

// Paterson-Stockmeyer split of Q = sum_{j<=d} c_j S^j, d = k + 1: with step s,
// Q = sum_{i<=r} (S^s)^i B_i (r = d / s, B_i = sum_{l<s} c_{is+l} S^l), evaluated
// as H = B_r, H <- B_i + S^s H for i = r-1 .. 0. Products: s - 1 for S^2 .. S^s
// (d - 1 when r = 0) and r for the recurrence, one less when B_r = c_d I (then
// B_{r-1} + c_d S^s is formed without a product). Returns the s with the fewest
// products (the smallest on ties), s <= kLinCombMax.
int ps_step(int d, int* products = nullptr) {
  int best = 1, bestp = 1 << 30;
  for (int s = 1; s <= std::min(d, poetx::kLinCombMax); ++s) {
    const int r = d / s;
    const int pr = r == 0 ? std::max(0, d - 1) : (s - 1) + r - (d % s == 0 ? 1 : 0);
    if (pr < bestp) { bestp = pr; best = s; }
  }
  if (products) *products = bestp;
  return best;
}
bool build_ps(const poetx_plan* pl) {
  return pl->series == POETX_SERIES_PS && pl->cayley == POETX_CAYLEY_NEUMANN;
}

size_t layout_build(const poetx_plan* pl, void* base, float** S, float** P0, float** P1,
                    float** X0 = nullptr, float** X1 = nullptr, int32_t** iters = nullptr,
                    float** pw = nullptr) {
  Carver c(base);
  const long long ne = std::max(pl->nelem[0], pl->nelem[1]);
  float* s = (float*)c.take(4 * ne);
  float* p0 = (float*)c.take(4 * ne);
  float* p1 = (float*)c.take(4 * ne);
  if (S) { *S = s; *P0 = p0; *P1 = p1; }
  if (pl->cayley == POETX_CAYLEY_EXACT) {   // Newton-Schulz iterates and step counts
    float* x0 = (float*)c.take(4 * ne);
    float* x1 = (float*)c.take(4 * ne);
    int32_t* it = (int32_t*)c.take(4 * std::max(pl->bsz[0].size(), pl->bsz[1].size()));
    if (X0) { *X0 = x0; *X1 = x1; }
    if (iters) *iters = it;
  }
  if (build_ps(pl)) {   // S^2 .. S^s and the recurrence's B (P0 and P1 hold H)
    const int st = ps_step(pl->k + 1);
    float* w = (float*)c.take(4 * ne * st);
    if (pw) *pw = w;
  }
  return c.off;
}

// HIP error behind the calling thread's last POETX_ERR_HIP
thread_local hipError_t g_last_hip = hipSuccess;

#define HIP_TRY(expr)                                   \
  do {                                                  \
    const hipError_t e_ = (expr);                       \
    if (e_ != hipSuccess) {                             \
      g_last_hip = e_;                                  \
      return POETX_ERR_HIP;                             \
    }                                                   \
  } while (0)

// Operand view: element (row, k) at p[row * rs + k * cs].
struct Op {
  const void* p;
  long long rs, cs;
};

// C(m, n) = sum_k A(m, k) B(n, k) in the plan's dtype (fp32 output when out_f32).
poetx_status gemm(const poetx_plan* pl, int role, Op A, Op B, void* C, long long ldc, int M, int N,
                  int K, int groups, long long a_gs, long long b_gs, long long c_gs, int splits,
                  long long c_ss, bool out_f32, hipStream_t s, const float* col_scale = nullptr) {
  if (pl->dtype == POETX_BF16) {
    poetx::GemmBf16 g;
    g.A = A.p; g.B = B.p; g.C = C;
    g.role = role;
    g.M = M; g.N = N; g.K = K;
    g.a_kmajor = A.cs == 1;
    g.b_kmajor = B.cs == 1;
    g.lda = g.a_kmajor ? A.rs : A.cs;
    g.ldb = g.b_kmajor ? B.rs : B.cs;
    g.ldc = ldc;
    g.out_f32 = out_f32 ? 1 : 0;
    g.a_gs = a_gs; g.b_gs = b_gs; g.c_gs = c_gs;
    g.groups = groups; g.splits = splits; g.c_ss = c_ss;
    g.col_scale = col_scale;
    HIP_TRY(poetx::launch_gemm_bf16(g, s));
  } else {
    poetx::GemmF32 g;
    g.A = (const float*)A.p; g.B = (const float*)B.p; g.C = (float*)C; g.Cin = nullptr; g.E = nullptr;
    g.M = M; g.N = N; g.K = K;
    g.a_rs = A.rs; g.a_cs = A.cs; g.b_rs = B.rs; g.b_cs = B.cs; g.c_rs = ldc;
    g.a_gs = a_gs; g.b_gs = b_gs; g.c_gs = c_gs;
    g.groups = groups; g.splits = splits; g.c_ss = c_ss;
    g.alpha = 1.0f; g.beta = 0.0f; g.gamma = 0.0f;
    HIP_TRY(poetx::launch_gemm_f32(g, s));
  }
  return POETX_OK;
}

// fp32 batched b x b product over a run of blocks:
// C = alpha * X * Y + beta * Cin (+ E = X * Y), all row-major b x b.
poetx_status chain_gemm(const Seg& g, const float* X, const float* Y, float* C, const float* Cin,
                        float* E, float alpha, float beta, hipStream_t s) {
  poetx::GemmF32 p;
  p.A = X + g.q_off; p.B = Y + g.q_off; p.C = C + g.q_off;
  p.Cin = Cin ? Cin + g.q_off : nullptr;
  p.E = E ? E + g.q_off : nullptr;
  p.M = p.N = p.K = g.b;
  p.a_rs = g.b; p.a_cs = 1;        // X(m, k) = X[m * b + k]
  p.b_rs = 1; p.b_cs = g.b;        // Y(n, k) = Y[k * b + n]
  p.c_rs = g.b;
  p.a_gs = p.b_gs = p.c_gs = (long long)g.b * g.b;
  p.groups = g.count; p.splits = 1; p.c_ss = 0;
  p.alpha = alpha; p.beta = beta; p.gamma = 0.0f;
  HIP_TRY(poetx::launch_gemm_f32(p, s));
  return POETX_OK;
}

// Exact Cayley transform: N = (I - S)^{-1} by Newton-Schulz, X <- X (2I - (I -
// S) X) from X0 = a (I + S), which converges for every skew S (launch_ns_init),
// then Q = (I + S) N = 2 N - I. Each block stops after its own step count
// (iters, at most kNsMaxSteps: enough for max row sums of |S| up to ~4000; the
// GEMM launches skip finished blocks).
constexpr int kNsMaxSteps = 28;

// One run of the exact transform: one segment of one side; every pointer is at
// the segment's first block. N is written to P0.
struct ExactRun {
  Seg g;
  const float* theta;   // the side's packed parameters (segment offset applied by the unpack)
  float *S, *P0, *P1, *X0, *X1, *Q, *N;
  int32_t* iters;       // one step count per block of the run
};

// Batched product over runs of one block size b: C_r = alpha A_r B_r (+ beta
// Cin_r) (+ gamma I), all b x b row-major, A(m, k) = A_r[m * a_rs + k * a_cs],
// B(n, k) = B_r[n * b_rs + k * b_cs]; blocks whose iters <= it are skipped.
poetx_status f32_runs(int b, long long a_rs, long long a_cs, long long b_rs, long long b_cs,
                      const std::vector<poetx::GemmF32Run>& runs, float beta, hipStream_t s,
                      float alpha = 1.0f, float gamma = 0.0f, int it = 0) {
  poetx::GemmF32 p{};
  p.M = p.N = p.K = b;
  p.a_rs = a_rs; p.a_cs = a_cs; p.b_rs = b_rs; p.b_cs = b_cs; p.c_rs = b;
  p.a_gs = p.b_gs = p.c_gs = (long long)b * b;
  p.splits = 1;
  p.alpha = alpha; p.beta = beta; p.gamma = gamma;
  p.it = it;
  HIP_TRY(poetx::launch_gemm_f32_runs(p, runs.data(), (int)runs.size(), s));
  return POETX_OK;
}

// The exact transform of many runs at once: each Newton-Schulz product is one
// launch over all runs of a block size (a single side has too few blocks to
// fill the chip). Sets r.N (= r.P0) and writes r.Q.
poetx_status exact_cayley_runs(std::vector<ExactRun>& runs, hipStream_t s) {
  std::vector<int> sizes;
  for (const ExactRun& r : runs)
    if (std::find(sizes.begin(), sizes.end(), r.g.b) == sizes.end()) sizes.push_back(r.g.b);
  for (int b : sizes) {
    std::vector<ExactRun*> rs;
    for (ExactRun& r : runs)
      if (r.g.b == b) rs.push_back(&r);
    const size_t n = rs.size();
    for (size_t i = 0; i < n; ++i) {
      ExactRun& r = *rs[i];
      // the unpack takes base pointers and applies the segment offset
      HIP_TRY(poetx::launch_unpack_skew(r.theta, r.g, r.S - r.g.q_off, nullptr, 0.0f, s));
    }
    // S^2 (in P1, free until the iterations) for the tighter bound of ||S||_2:
    // at generators of many small entries it asks for fewer steps than the row
    // sums of S alone, for one product
    std::vector<poetx::GemmF32Run> v(n);
    for (size_t i = 0; i < n; ++i) v[i] = poetx::GemmF32Run{rs[i]->S, rs[i]->S, rs[i]->P1, nullptr, rs[i]->g.count};
    poetx_status st;
    if ((st = f32_runs(b, b, 1, 1, b, v, 0.0f, s)) != POETX_OK) return st;
    for (size_t i = 0; i < n; ++i) {
      ExactRun& r = *rs[i];
      HIP_TRY(poetx::launch_ns_init(r.S, r.P1, b, r.g.count, r.X0, r.iters, kNsMaxSteps, s));
    }
    for (int it = 0; it < kNsMaxSteps; ++it) {
      // Y = 2I - (I - S) X = S X - X + 2I (in P1), then X' = X Y
      for (size_t i = 0; i < n; ++i) {
        const float* X = (it & 1) ? rs[i]->X1 : rs[i]->X0;
        v[i] = poetx::GemmF32Run{rs[i]->S, X, rs[i]->P1, X, rs[i]->g.count, rs[i]->iters};
      }
      if ((st = f32_runs(b, b, 1, 1, b, v, -1.0f, s, 1.0f, 2.0f, it)) != POETX_OK) return st;
      for (size_t i = 0; i < n; ++i) {
        const float* X = (it & 1) ? rs[i]->X1 : rs[i]->X0;
        float* Xn = (it & 1) ? rs[i]->X0 : rs[i]->X1;
        v[i] = poetx::GemmF32Run{X, rs[i]->P1, Xn, nullptr, rs[i]->g.count, rs[i]->iters};
      }
      if ((st = f32_runs(b, b, 1, 1, b, v, 0.0f, s, 1.0f, 0.0f, it)) != POETX_OK) return st;
    }
    for (size_t i = 0; i < n; ++i) {
      ExactRun& r = *rs[i];
      HIP_TRY(poetx::launch_ns_final(r.X0, r.X1, r.iters, b, r.g.count, r.P0, r.Q, s));
      r.N = r.P0;
    }
  }
  return POETX_OK;
}

// Wa = A Wt^T for the forward form of the frozen-weight product. An INT8 weight
// (POET-XQ) is first widened exactly to bf16 into Wq (one pass over m n bytes),
// so the product runs on the bf16 kernels with the row scales of Wt applied to
// Wa's columns in its epilogue: Wa = (A q^T) diag(s), exact int8 values and an
// fp32 scale of each column's accumulator before the rounding to bf16.
poetx_status w0_forward_product(const poetx_plan* pl, Op A, const void* Wt, void* Wq, void* Wa,
                                long long T, hipStream_t s) {
  if (!wq(pl))
    return gemm(pl, poetx::GEMM_W0, A, Op{Wt, pl->n, 1}, Wa, pl->m, (int)T, pl->m, pl->n, 1, 0, 0, 0, 1, 0,
                false, s);
  HIP_TRY(poetx::launch_widen_i8(Wt, Wq, (long long)pl->m * pl->n, s));
  return gemm(pl, poetx::GEMM_W0, A, Op{Wq, pl->n, 1}, Wa, pl->m, (int)T, pl->m, pl->n, 1, 0, 0, 0, 1, 0,
              false, s, qscale(pl, Wt));
}

// Row-form product with one side's blocks: out[:, blk] = in[:, blk] Q^T
// (transpose_q = true) or in[:, blk] Q (false), for every block of the side.
poetx_status apply_blocks(const poetx_plan* pl, int side, long long T, const void* in,
                          const void* Q, void* out, bool transpose_q, hipStream_t s,
                          const float* col_scale = nullptr) {
  const size_t es = elsize(pl);
  const long long dim = pl->dim[side];
  for (const Seg& g : pl->segs[side]) {
    const char* a = static_cast<const char*>(in) + es * g.dim_off;
    const char* q = static_cast<const char*>(Q) + es * g.q_off;
    char* c = static_cast<char*>(out) + es * g.dim_off;
    // transpose_q: B(n, k) = Q[n][k]; otherwise B(n, k) = Q[k][n]
    Op B = transpose_q ? Op{q, g.b, 1} : Op{q, 1, g.b};
    poetx_status st = gemm(pl, poetx::GEMM_BLOCK, Op{a, dim, 1}, B, c, dim, (int)T, g.b, g.b, g.count, g.b,
                           (long long)g.b * g.b, g.b, 1, 0, false, s,
                           col_scale ? col_scale + g.dim_off : nullptr);
    if (st != POETX_OK) return st;
  }
  return POETX_OK;
}

// Wf = Wt D_P: every row of Wt times the P blocks, out[:, blk] = Wt[:, blk] Q.
poetx_status fold_p(const poetx_plan* pl, const void* Wt, const void* Q_P, void* Wf, hipStream_t s) {
  return apply_blocks(pl, POETX_SIDE_P, pl->m, Wt, Q_P, Wf, false, s);
}

// Wf = D_R Wt: the rows of each R block of Wt multiplied from the left by its Q,
// Wf[blk] = Q Wt[blk] (b x b times b x n per block).
poetx_status fold_r(const poetx_plan* pl, const void* Wt, const void* Q_R, void* Wf, hipStream_t s) {
  const size_t es = elsize(pl);
  const long long n = pl->n;
  for (const Seg& g : pl->segs[POETX_SIDE_R]) {
    const char* q = static_cast<const char*>(Q_R) + es * g.q_off;
    const char* w = static_cast<const char*>(Wt) + es * g.dim_off * n;
    char* c = static_cast<char*>(Wf) + es * g.dim_off * n;
    // A(m, k) = Q[m][k]; B(j, k) = Wt[off + k][j]
    poetx_status st = gemm(pl, poetx::GEMM_BLOCK, Op{q, g.b, 1}, Op{w, 1, n}, c, n, g.b, (int)n, g.b,
                           g.count, (long long)g.b * g.b, (long long)g.b * n, (long long)g.b * n, 1, 0,
                           false, s);
    if (st != POETX_OK) return st;
  }
  return POETX_OK;
}

// Transposed form of fold_r, WfT = (D_R Wt)^T [n, m]: the backward product then
// reads it K-contiguous (the faster NT form). Per block: WfT[:, blk] =
// Wt[blk]^T Q^T. bf16 plans need whole 256-row tiles of n and b % 64 == 0 (the
// pipelined kernel is the only one with this operand layout).
bool fold_rt_ok(const poetx_plan* pl) {
  if (pl->dtype != POETX_BF16) return true;
  if (pl->n % 256) return false;
  for (const Seg& g : pl->segs[POETX_SIDE_R])
    if (g.b % 64) return false;
  return true;
}
poetx_status fold_rt(const poetx_plan* pl, const void* Wt, const void* Q_R, void* WfT, hipStream_t s) {
  const size_t es = elsize(pl);
  const long long n = pl->n, m = pl->m;
  for (const Seg& g : pl->segs[POETX_SIDE_R]) {
    const char* q = static_cast<const char*>(Q_R) + es * g.q_off;
    const char* w = static_cast<const char*>(Wt) + es * g.dim_off * n;
    char* c = static_cast<char*>(WfT) + es * g.dim_off;
    // A(j, k) = Wt[off + k][j]; B(i, k) = Q[i][k]; C(j, i) at WfT[j][off + i]
    poetx_status st = gemm(pl, poetx::GEMM_BLOCK, Op{w, 1, n}, Op{q, g.b, 1}, c, m, (int)n, g.b, g.b,
                           g.count, (long long)g.b * n, (long long)g.b * g.b, g.b, 1, 0, false, s);
    if (st != POETX_OK) return st;
  }
  return POETX_OK;
}

// dQ[blk] = G[:, blk]^T A[:, blk] (reduction over tokens), fp32: each run of
// equal blocks splits the tokens its own way (dq_splits) into its own part of
// the partial sums, then sums them into its blocks of dQ.
poetx_status block_grads(const poetx_plan* pl, int side, long long T, const void* G, const void* A,
                         float* part, float* dQ, hipStream_t s) {
  const size_t es = elsize(pl);
  const long long dim = pl->dim[side];
  for (const Seg& g : pl->segs[side]) {
    const int splits = dq_splits(pl, g, T);
    const long long ne = (long long)g.count * g.b * g.b;
    const char* a = static_cast<const char*>(G) + es * g.dim_off;
    const char* b = static_cast<const char*>(A) + es * g.dim_off;
    // rows of the product index features, k indexes tokens
    poetx_status st = gemm(pl, poetx::GEMM_DQ, Op{a, 1, dim}, Op{b, 1, dim}, part, g.b, g.b, g.b,
                           (int)T, g.count, g.b, g.b, (long long)g.b * g.b, splits, ne, true, s);
    if (st != POETX_OK) return st;
    HIP_TRY(poetx::launch_sum_splits(part, splits, ne, ne, dQ + g.q_off, s));
    part += (long long)splits * ne;
  }
  return POETX_OK;
}

// bf16 plans: where the run's split of -S goes (its part of a b x b fp32
// buffer, 4 bytes per element for the two bf16 halves), or null for the fp32
// chains (fp32 plans, other block sizes, a part not on a 16-byte boundary).
uint16_t* split_buffer(const poetx_plan* pl, const Seg& g, float* buf) {
  if (pl->dtype != POETX_BF16 || !poetx::chain_split_supported(g.b)) return nullptr;
  float* p = buf + g.q_off;
  return ((uintptr_t)p & 15) ? nullptr : reinterpret_cast<uint16_t*>(p);
}

// One chain-rule item: dL/dQ of one side of one plan -> packed parameter gradient.
struct GradItem {
  const poetx_plan* pl;
  int side;
  const float* theta;
  const float* dQ;
  float* g;
  ChainWs w;
};

// Reverse mode through Q = sum_j c_j S^j for every block of every item:
//   A_{k+1} = c_{k+1} G,  A_j = c_j G + A_{j+1} S^T,
//   T_{k+1} = A_{k+1},    T_j = A_j + S^T T_{j+1},   dL/dS = T_1,
// then dL/dtheta(i,j) = dS[i][j] - dS[j][i]. Uses S^T = -S. Runs of supported
// block sizes of all items share one launch per chain (items with one Neumann
// order per launch); other sizes step through batched fp32 GEMMs.
poetx_status grad_items(const GradItem* items, int count, hipStream_t s) {
  poetx::TriBatch ub{}, pb{};
  poetx::ChainBatch ab{}, tb{};
  pb.sign = -1.0f;   // T_1^T is stored: g(i,j) = T^T[j][i] - T^T[i][j]
  int kk = -1;
  auto flush = [&]() -> poetx_status {
    HIP_TRY(poetx::launch_unpack_batch(ub, s));
    HIP_TRY(poetx::launch_chain_batch(poetx::CHAIN_ABAR, ab, s));
    HIP_TRY(poetx::launch_chain_batch(poetx::CHAIN_TCHAIN, tb, s));
    HIP_TRY(poetx::launch_pack_batch(pb, s));
    ub.n = pb.n = ab.n = tb.n = 0;
    return POETX_OK;
  };
  poetx_status st;
  for (int i = 0; i < count; ++i) {
    const GradItem& it = items[i];
    const poetx_plan* pl = it.pl;
    if (pl->cayley == POETX_CAYLEY_EXACT) continue;   // below
    if (kk != -1 && kk != pl->k && (st = flush()) != POETX_OK) return st;
    kk = pl->k;
    ab.k = tb.k = kk;
    for (const Seg& g : pl->segs[it.side]) {
      if (!poetx::chain_supported(g.b)) continue;
      if (ab.n == poetx::kChainMaxEntries && (st = flush()) != POETX_OK) return st;
      float* S = it.w.S + g.q_off;
      // bf16 plans: the chains run on split bf16 products; the split of -S goes
      // to this run's part of A0 (used only by the generic path of other sizes)
      uint16_t* split = split_buffer(pl, g, it.w.A0);
      // the split chains never read S itself
      ub.e[ub.n++] = poetx::TriEntry{it.theta + g.p_off, split ? nullptr : S, g.b, g.count, 0, split};
      poetx::ChainEntry e{};
      e.S = S; e.b = g.b; e.count = g.count; e.stride = pl->nelem[it.side];
      e.Mh = split;
      e.G = it.dQ + g.q_off;
      e.out = it.w.A + g.q_off;
      ab.e[ab.n++] = e;
      e.G = it.w.A + g.q_off;
      e.out = it.w.T + g.q_off;
      tb.e[tb.n++] = e;
      pb.e[pb.n++] = poetx::TriEntry{it.w.T + g.q_off, it.g + g.p_off, g.b, g.count, 0};
    }
  }
  if ((st = flush()) != POETX_OK) return st;
  std::vector<ExactRun> exact;
  std::vector<int> exact_items;
  for (int i = 0; i < count; ++i) {
    const GradItem& it = items[i];
    const poetx_plan* pl = it.pl;
    const int side = it.side, k = pl->k;
    if (pl->cayley == POETX_CAYLEY_EXACT) {
      // exact transform: rebuild N = (I - S)^{-1} and Q, then
      // dL/dS = (I + Q)^T G N^T and g(i, j) = dS[i][j] - dS[j][i] (batched below)
      const ChainWs& w = it.w;
      int blk = 0;
      for (const Seg& g : pl->segs[side]) {
        const long long o = g.q_off;
        exact.push_back(ExactRun{g, it.theta, w.S + o, w.A0 + o, w.A1 + o, w.T0 + o, w.T1 + o, w.T + o,
                                 nullptr, w.iters + blk});
        exact_items.push_back(i);
        blk += g.count;
      }
      continue;
    }
    bool any = false;
    for (const Seg& g : pl->segs[side]) any |= !poetx::chain_supported(g.b);
    if (!any) continue;
    const long long ne = pl->nelem[side];
    const ChainWs& w = it.w;
    const float* G = it.dQ;
    for (const Seg& g : pl->segs[side])
      if (!poetx::chain_supported(g.b))
        HIP_TRY(poetx::launch_unpack_skew(it.theta, g, w.S, nullptr, 0.0f, s));
    HIP_TRY(poetx::launch_scale2(G, coef(k + 1, k), w.A0, w.T1, ne, s));
    float *Acur = w.A0, *Anew = w.A1, *Tcur = w.T1, *Tnew = w.T0;
    for (int j = k; j >= 1; --j) {
      for (const Seg& g : pl->segs[side]) {
        if (poetx::chain_supported(g.b)) continue;
        // A_j = c_j G - A_{j+1} S
        if ((st = chain_gemm(g, Acur, w.S, Anew, G, nullptr, -1.0f, coef(j, k), s)) != POETX_OK)
          return st;
        // T_j = A_j - S T_{j+1}
        if ((st = chain_gemm(g, w.S, Tcur, Tnew, Anew, nullptr, -1.0f, 1.0f, s)) != POETX_OK)
          return st;
      }
      std::swap(Acur, Anew);
      std::swap(Tcur, Tnew);
    }
    for (const Seg& g : pl->segs[side])
      if (!poetx::chain_supported(g.b))
        HIP_TRY(poetx::launch_pack_antisym(Tcur, g, 1.0f, it.g, s));
  }
  if (exact.empty()) return POETX_OK;
  if ((st = exact_cayley_runs(exact, s)) != POETX_OK) return st;
  std::vector<int> sizes;
  for (const ExactRun& r : exact)
    if (std::find(sizes.begin(), sizes.end(), r.g.b) == sizes.end()) sizes.push_back(r.g.b);
  for (int b : sizes) {
    std::vector<poetx::GemmF32Run> v1, v2;
    for (size_t i = 0; i < exact.size(); ++i) {
      const ExactRun& r = exact[i];
      if (r.g.b != b) continue;
      const GradItem& it = items[exact_items[i]];
      const long long o = r.g.q_off;
      // A = Q^T G + G (A(m, k) = Q[k][m]), into the stored-A buffer
      v1.push_back(poetx::GemmF32Run{r.Q, it.dQ + o, it.w.A + o, it.dQ + o, r.g.count});
      // D = A N^T (B(n, k) = N[n][k]), into the Q buffer, free now
      v2.push_back(poetx::GemmF32Run{it.w.A + o, r.N, r.Q, nullptr, r.g.count});
    }
    if ((st = f32_runs(b, 1, b, 1, b, v1, 1.0f, s)) != POETX_OK) return st;
    if ((st = f32_runs(b, b, 1, b, 1, v2, 0.0f, s)) != POETX_OK) return st;
  }
  for (size_t i = 0; i < exact.size(); ++i) {
    const ExactRun& r = exact[i];
    HIP_TRY(poetx::launch_pack_antisym(r.Q - r.g.q_off, r.g, 1.0f, items[exact_items[i]].g, s));
  }
  return POETX_OK;
}

// Activation path of the backward (everything but the chain rule through the
// parameterisation): G_X and dL/dQ of both sides (fp32).
poetx_status backward_dq(const poetx_plan* pl, long long T, const void* X, const void* Wt,
                         const int32_t* pi_R, const int32_t* pi_P, const void* Q_R, const void* Q_P,
                         const void* Wa_saved, const void* U_saved, const void* G_Y, void* G_X,
                         float* const dQ[2], const BwdWs& w, hipStream_t s) {
  const int es = elsize(pl);
  poetx_status st;
  if (T == 0) {
    HIP_TRY(poetx::launch_zero(dQ[0], pl->nelem[0], s));
    HIP_TRY(poetx::launch_zero(dQ[1], pl->nelem[1], s));
    return POETX_OK;
  }
  // U = X Pi_P^T: kept by the caller, or gathered here (once)
  const void* U = U_saved ? U_saved : w.U;
  const bool foldb = fold_bwd(pl, T);
  const bool foldt = foldb && fold_rt_ok(pl);
  // fused R pass: gathers G_Y, keeps G_Z and applies the R blocks (B = Q_R^T)
  // in one pass; INT8 weights scale G_Wa's columns and keep the separate kernels
  const bool fused_r = !foldb && !wq(pl) && w.QT[0];

  // Without a saved Wa (POET-Xmem) the forward's first three stages run again,
  // with the forward's kernels and launch shapes, so Wa is bit-identical to the
  // one poetx_forward would have saved. V borrows the G_U buffer and Wa the G_Wa
  // buffer, both dead until their next writer. With the fused R pass (which
  // writes G_Wa and G_Z before dQ_R reads Wa) this runs after the Wt product has
  // consumed G_Wa; otherwise first.
  auto recompute_wa = [&]() -> poetx_status {
    const bool fold = fold_fwd(pl, T);
    // the fused pass gathers X and applies the P blocks at once, keeping U
    const bool fused = !fold && !U_saved && panel_side(pl, POETX_SIDE_P);
    if (!U_saved && !fused) {
      StageScope sc(POETX_STAGE_GATHER, s);
      HIP_TRY(poetx::launch_gather_cols(X, pl->n, nullptr, pi_P, w.U, T, pl->n, es, s));
    }
    {
      StageScope sc(POETX_STAGE_BLOCK_FWD, s);
      poetx_status r;
      if (fused) {
        HIP_TRY(poetx::launch_panel_block(X, pi_P, Q_P, w.GU, w.U, T, pl->n, true, false, s));
        r = POETX_OK;
      } else {
        r = fold ? fold_p(pl, Wt, Q_P, w.Wf, s) : apply_blocks(pl, POETX_SIDE_P, T, U, Q_P, w.GU, true, s);
      }
      if (r != POETX_OK) return r;
    }
    StageScope sc(POETX_STAGE_W0_FWD, s);
    const Op a = fold ? Op{U, pl->n, 1} : Op{w.GU, pl->n, 1};
    return w0_forward_product(pl, a, fold ? w.Wf : Wt, w.Wq, w.GWa, T, s);
  };
  const void* Wa = Wa_saved ? Wa_saved : w.GWa;
  if (!Wa_saved && !fused_r && (st = recompute_wa()) != POETX_OK) return st;

  // R side: G_Z = G_Y Pi_R^T; dQ_R = G_Z^T Wa per block; G_Wa = G_Z D_R
  if (fused_r) {
    StageScope sc(POETX_STAGE_BLOCK_BWD, s);
    HIP_TRY(poetx::launch_transpose_blocks(Q_R, w.QT[0], (int)pl->segs[0][0].count, s));
    HIP_TRY(poetx::launch_panel_block(G_Y, pi_R, w.QT[0], w.GWa, w.GZ, T, pl->m, true, false, s));
  } else {
    StageScope sc(POETX_STAGE_GATHER, s);
    HIP_TRY(poetx::launch_gather_cols(G_Y, pl->m, nullptr, pi_R, w.GZ, T, pl->m, es, s));
  }
  const bool dq_r_now = Wa_saved || !fused_r;
  if (dq_r_now) {
    StageScope sc(POETX_STAGE_DQ, s);
    if ((st = block_grads(pl, POETX_SIDE_R, T, w.GZ, Wa, w.part, dQ[0], s)) != POETX_OK) return st;
  }
  if (!fused_r) {
    StageScope sc(POETX_STAGE_BLOCK_BWD, s);
    // folded: Wf = D_R Wt (stored transposed where possible) replaces
    // G_Wa = G_Z D_R. INT8 weight: G_Wa leaves scaled by the row scales of Wt,
    // since G_Wa Wt = (G_Wa diag(s)) q
    st = foldt ? fold_rt(pl, Wt, Q_R, w.Wf, s)
         : foldb ? fold_r(pl, Wt, Q_R, w.Wf, s)
                 : apply_blocks(pl, POETX_SIDE_R, T, w.GZ, Q_R, w.GWa, false, s,
                                wq(pl) ? qscale(pl, Wt) : nullptr);
    if (st != POETX_OK) return st;
  }
  // frozen weight: G_V = G_Wa Wt (folded: G_V = G_Z (D_R Wt))
  {
    StageScope sc(POETX_STAGE_W0_BWD, s);
    const Op a = foldb ? Op{w.GZ, pl->m, 1} : Op{w.GWa, pl->m, 1};
    // B(j, i) = (D_R Wt)[i][j]: WfT[j][i] (K-contiguous) or Wf[i][j]; unfolded
    // B(j, i) = Wt[i][j], read K-contiguous from the kept transpose WtT[j][i]
    // (qT[j][i] for an INT8 weight, widened exactly to bf16 first; its row
    // scales are already in G_Wa)
    if (wq(pl))
      HIP_TRY(poetx::launch_widen_i8(wqpair(pl) ? qt(pl, Wt) : Wt, w.Wq, (long long)pl->m * pl->n, s));
    const Op b = foldt ? Op{w.Wf, pl->m, 1} : foldb ? Op{w.Wf, 1, pl->n}
                 : wpair(pl) ? Op{wtt(pl, Wt), pl->m, 1}
                 : wqpair(pl) ? Op{w.Wq, pl->m, 1} : wq(pl) ? Op{w.Wq, 1, pl->n} : Op{Wt, 1, pl->n};
    if ((st = gemm(pl, poetx::GEMM_W0, a, b, w.GV, pl->n, (int)T, pl->n, pl->m, 1, 0, 0, 0, 1, 0, false,
                   s)) != POETX_OK)
      return st;
  }
  if (!dq_r_now) {
    // POET-Xmem with the fused R pass: G_Wa is consumed, Wa goes into its buffer
    if ((st = recompute_wa()) != POETX_OK) return st;
    StageScope sc(POETX_STAGE_DQ, s);
    if ((st = block_grads(pl, POETX_SIDE_R, T, w.GZ, Wa, w.part, dQ[0], s)) != POETX_OK) return st;
  }
  // P side: U = X Pi_P^T; dQ_P = G_V^T U per block; G_U = G_V D_P; G_X = G_U Pi_P
  if (Wa_saved && !U_saved) {
    StageScope sc(POETX_STAGE_GATHER, s);
    HIP_TRY(poetx::launch_gather_cols(X, pl->n, nullptr, pi_P, w.U, T, pl->n, es, s));
  }
  {
    StageScope sc(POETX_STAGE_DQ, s);
    if ((st = block_grads(pl, POETX_SIDE_P, T, w.GV, U, w.part, dQ[1], s)) != POETX_OK) return st;
  }
  if (w.QT[1]) {
    // fused: G_U = G_V D_P (B = Q_P^T) scattered to G_X in the same pass
    StageScope sc(POETX_STAGE_BLOCK_BWD, s);
    HIP_TRY(poetx::launch_transpose_blocks(Q_P, w.QT[1], (int)pl->segs[1][0].count, s));
    HIP_TRY(poetx::launch_panel_block(w.GV, pi_P, w.QT[1], G_X, nullptr, T, pl->n, false, true, s));
    return POETX_OK;
  }
  {
    StageScope sc(POETX_STAGE_BLOCK_BWD, s);
    if ((st = apply_blocks(pl, POETX_SIDE_P, T, w.GV, Q_P, w.GU, false, s)) != POETX_OK) return st;
  }
  {
    StageScope sc(POETX_STAGE_SCATTER, s);
    HIP_TRY(poetx::launch_scatter_cols(w.GU, pi_P, G_X, T, pl->n, es, s));
  }
  return POETX_OK;
}

poetx_status check_backward_args(const poetx_plan* pl, long long T, const void* X, const void* Wt,
                                 const int32_t* pi_R, const int32_t* pi_P, const void* Q_R,
                                 const void* Q_P, const void* Wa_saved, const void* U_saved,
                                 const void* G_Y, const void* G_X, const void* ws, size_t ws_bytes) {
  if (!pl || T < 0) return POETX_ERR_INVALID_ARG;
  if (T > 0 && ((!X && !U_saved) || !Wt || !pi_R || !pi_P || !Q_R || !Q_P || !G_Y || !G_X))
    return POETX_ERR_INVALID_ARG;
  for (const void* p : {X, Wt, (const void*)pi_R, (const void*)pi_P, Q_R, Q_P, Wa_saved, U_saved, G_Y,
                        G_X, ws})
    if (!aligned16(p)) return POETX_ERR_ALIGNMENT;
  if (!ws || ws_bytes < poetx_workspace_size(pl, T, POETX_WS_BACKWARD)) return POETX_ERR_WORKSPACE;
  return POETX_OK;
}

// One build item: Q (and its activation-dtype copy) of one side of one plan.
struct BuildItem {
  const poetx_plan* pl;
  int side;
  const float* theta;
  float* Q;
  void* Qact;
  void* ws;
};

poetx_status check_build_item(const BuildItem& it, size_t ws_bytes) {
  if (!it.pl || !side_ok_fn(it.side) || !it.theta || !it.Q) return POETX_ERR_INVALID_ARG;
  if (!aligned16(it.theta) || !aligned16(it.Q) || !aligned16(it.Qact) || !aligned16(it.ws))
    return POETX_ERR_ALIGNMENT;
  if (!it.ws || ws_bytes < poetx_workspace_size(it.pl, 0, POETX_WS_BUILD)) return POETX_ERR_WORKSPACE;
  return POETX_OK;
}

// Q by Paterson-Stockmeyer (ps_step) for build items that share one Neumann
// order: S from the packed parameters, the powers S^2 .. S^s, then the
// recurrence H <- B_i + S^s H with each B_i a linear combination of I, S ..
// S^(s-1); fp32 throughout, Q cast to the activation dtype at the end. Every
// product is one launch over all runs of a block size across the items (one
// side of one layer has too few blocks to fill the chip); the unpacks, linear
// combinations and casts stay per run.
struct PsRun {
  const BuildItem* it;
  Seg g;
  std::vector<float*> P;   // P[j] = S^j, j = 1 .. s (at the run's first block)
  float *B, *H0, *H1, *Q;
};
poetx_status build_ps_group(const BuildItem* items, const std::vector<int>& idx, hipStream_t s) {
  if (idx.empty()) return POETX_OK;
  const poetx_plan* pl0 = items[idx[0]].pl;
  const int k = pl0->k, d = k + 1;
  const int st = ps_step(d);
  const int r = d / st;
  auto c = [&](int j) { return j <= d ? coef(j, k) : 0.0f; };
  std::vector<PsRun> runs;
  for (int i : idx) {
    const BuildItem& it = items[i];
    float *S, *H0, *H1, *pw;
    layout_build(it.pl, it.ws, &S, &H0, &H1, nullptr, nullptr, nullptr, &pw);
    const long long ne = std::max(it.pl->nelem[0], it.pl->nelem[1]);
    for (const Seg& g : it.pl->segs[it.side]) {
      const long long o = g.q_off;
      PsRun pr{&it, g, std::vector<float*>(st + 1, nullptr), pw + (st - 1) * ne + o, H0 + o, H1 + o,
               it.Q + o};
      pr.P[1] = S + o;
      for (int j = 2; j <= st; ++j) pr.P[j] = pw + (j - 2) * ne + o;
      runs.push_back(std::move(pr));
      // the unpack takes the side's base pointers and applies the run's offsets
      HIP_TRY(poetx::launch_unpack_skew(it.theta, g, S, nullptr, 0.0f, s));
    }
  }
  std::vector<int> sizes;
  for (const PsRun& pr : runs)
    if (std::find(sizes.begin(), sizes.end(), pr.g.b) == sizes.end()) sizes.push_back(pr.g.b);
  // C = A B (+ Cin) for every run of each block size: one launch per size
  auto products = [&](auto pick) -> poetx_status {
    for (int b : sizes) {
      std::vector<poetx::GemmF32Run> v;
      for (PsRun& pr : runs)
        if (pr.g.b == b) {
          const float *A, *Bm, *Cin;
          float* C;
          pick(pr, A, Bm, C, Cin);
          v.push_back(poetx::GemmF32Run{A, Bm, C, Cin, pr.g.count, nullptr});
        }
      const bool acc = v[0].Cin != nullptr;
      poetx_status e = f32_runs(b, b, 1, 1, b, v, acc ? 1.0f : 0.0f, s);
      if (e != POETX_OK) return e;
    }
    return POETX_OK;
  };
  // B_i = c_{is} I + sum_{0<l<s} c_{is+l} S^l; with fold, also + c_d S^s
  auto make_b = [&](const PsRun& pr, int i, float* out, bool fold_top) -> poetx_status {
    poetx::LinComb lc{};
    lc.diag = c(i * st);
    for (int l = 1; l < st; ++l) {
      lc.mats[lc.n] = pr.P[l];
      lc.coef[lc.n++] = c(i * st + l);
    }
    if (fold_top) {
      lc.mats[lc.n] = pr.P[st];
      lc.coef[lc.n++] = c(d);
    }
    HIP_TRY(poetx::launch_lincomb(lc, out, pr.g.b, pr.g.count, s));
    return POETX_OK;
  };
  poetx_status e;
  // powers up to S^s (up to S^d when r = 0, which needs d < s: never, s <= d)
  const int top = r == 0 ? d : st;
  for (int j = 2; j <= top; ++j)
    if ((e = products([&](PsRun& pr, const float*& A, const float*& Bm, float*& C, const float*& Cin) {
           A = pr.P[j - 1]; Bm = pr.P[1]; C = pr.P[j]; Cin = nullptr;
         })) != POETX_OK)
      return e;
  if (r == 0) {   // degree below s: Q = sum_j c_j S^j directly
    for (const PsRun& pr : runs) {
      poetx::LinComb lc{};
      lc.diag = c(0);
      for (int j = 1; j <= d; ++j) {
        lc.mats[lc.n] = pr.P[j];
        lc.coef[lc.n++] = c(j);
      }
      HIP_TRY(poetx::launch_lincomb(lc, pr.Q, pr.g.b, pr.g.count, s));
    }
  } else {
    // H = B_r, or H = B_{r-1} + c_d S^s when B_r = c_d I
    int i = r;
    bool h0 = true;   // H in H0 (else in H1)
    if (d % st == 0) --i;
    for (const PsRun& pr : runs)
      if ((e = make_b(pr, i, pr.H0, d % st == 0)) != POETX_OK) return e;
    for (--i; i >= 0; --i) {
      for (const PsRun& pr : runs)
        if ((e = make_b(pr, i, pr.B, false)) != POETX_OK) return e;
      const bool last = i == 0;
      if ((e = products([&](PsRun& pr, const float*& A, const float*& Bm, float*& C, const float*& Cin) {
             A = pr.P[st]; Bm = h0 ? pr.H0 : pr.H1; C = last ? pr.Q : (h0 ? pr.H1 : pr.H0); Cin = pr.B;
           })) != POETX_OK)
        return e;
      h0 = !h0;
    }
    if (d % st == 0 && r == 1)   // no product at all: H is Q
      for (const PsRun& pr : runs)
        HIP_TRY(poetx::launch_lincomb(poetx::LinComb{{h0 ? pr.H0 : pr.H1}, {1.0f}, 1, 0.0f}, pr.Q, pr.g.b,
                                      pr.g.count, s));
  }
  for (const PsRun& pr : runs)
    if (pr.it->Qact)
      HIP_TRY(poetx::launch_cast(pr.Q, static_cast<char*>(pr.it->Qact) + (size_t)elsize(pr.it->pl) * pr.g.q_off,
                                 (long long)pr.g.b * pr.g.b * pr.g.count, pr.it->pl->dtype == POETX_BF16, s));
  return POETX_OK;
}

// Builds every item: all runs of supported block sizes in one unpack launch and
// one fused chain launch per size class; other sizes through batched GEMMs.
poetx_status build_items(const BuildItem* items, int count, hipStream_t s) {
  poetx::TriBatch ub{};
  poetx::ChainBatch cb{};
  std::vector<ExactRun> exact;
  std::vector<int> exact_items, ps_items;
  int kk = -1;
  auto flush = [&]() -> poetx_status {
    HIP_TRY(poetx::launch_unpack_batch(ub, s));
    HIP_TRY(poetx::launch_chain_batch(poetx::CHAIN_BUILD, cb, s));
    ub.n = cb.n = 0;
    return POETX_OK;
  };
  for (int i = 0; i < count; ++i) {
    const BuildItem& it = items[i];
    const poetx_plan* pl = it.pl;
    if (pl->cayley == POETX_CAYLEY_EXACT) {   // batched after the loop
      float *S, *P0, *P1, *X0, *X1;
      int32_t* iters;
      layout_build(pl, it.ws, &S, &P0, &P1, &X0, &X1, &iters);
      int blk = 0;
      for (const Seg& g : pl->segs[it.side]) {
        const long long o = g.q_off;
        exact.push_back(ExactRun{g, it.theta, S + o, P0 + o, P1 + o, X0 + o, X1 + o, it.Q + o, nullptr,
                                 iters + blk});
        exact_items.push_back(i);
        blk += g.count;
      }
      continue;
    }
    if (build_ps(pl)) {   // Paterson-Stockmeyer: batched after the loop
      ps_items.push_back(i);
      continue;
    }
    if (kk != -1 && kk != pl->k) {   // one Neumann order per chain launch
      poetx_status st = flush();
      if (st != POETX_OK) return st;
    }
    kk = pl->k;
    cb.k = kk;
    float *S, *P0, *P1;
    layout_build(pl, it.ws, &S, &P0, &P1);
    const bool bf16 = pl->dtype == POETX_BF16;
    const int es = elsize(pl);
    for (const Seg& g : pl->segs[it.side]) {
      if (poetx::chain_supported(g.b)) {
        if (cb.n == poetx::kChainMaxEntries) {
          poetx_status st = flush();
          if (st != POETX_OK) return st;
        }
        // bf16 plans: split bf16 products, the split of -S in this run's part of
        // P0 (used only by the generic path of other sizes)
        uint16_t* split = split_buffer(pl, g, P0);
        // the split chains take their first panel from the split, not from S
        ub.e[ub.n++] = poetx::TriEntry{it.theta + g.p_off, split ? nullptr : S + g.q_off, g.b, g.count, 0, split};
        poetx::ChainEntry e{};
        e.S = S + g.q_off; e.G = nullptr; e.out = it.Q + g.q_off;
        e.Mh = split;
        e.out_act = it.Qact ? static_cast<char*>(it.Qact) + (size_t)es * g.q_off : nullptr;
        e.act_bf16 = bf16; e.b = g.b; e.count = g.count; e.stride = 0;
        cb.e[cb.n++] = e;
        continue;
      }
      HIP_TRY(poetx::launch_unpack_skew(it.theta, g, S, it.Q, coef(1, pl->k), s));
      // powers S^j = S^{j-1} S for j = 2..k+1, each added into Q with weight c_j
      const float* prev = S;
      float* bufs[2] = {P0, P1};
      for (int j = 2; j <= pl->k + 1; ++j) {
        float* next = (j < pl->k + 1) ? bufs[j & 1] : nullptr;
        poetx_status st = chain_gemm(g, prev, S, it.Q, it.Q, next, coef(j, pl->k), 1.0f, s);
        if (st != POETX_OK) return st;
        prev = next;
      }
      if (it.Qact)
        HIP_TRY(poetx::launch_cast(it.Q + g.q_off, static_cast<char*>(it.Qact) + es * g.q_off,
                                   (long long)g.b * g.b * g.count, bf16, s));
    }
  }
  poetx_status st = flush();
  if (st != POETX_OK) return st;
  // Paterson-Stockmeyer items, one batch per Neumann order
  while (!ps_items.empty()) {
    const int k = items[ps_items[0]].pl->k;
    std::vector<int> grp, rest;
    for (int i : ps_items) (items[i].pl->k == k ? grp : rest).push_back(i);
    if ((st = build_ps_group(items, grp, s)) != POETX_OK) return st;
    ps_items.swap(rest);
  }
  if (exact.empty()) return POETX_OK;
  if ((st = exact_cayley_runs(exact, s)) != POETX_OK) return st;
  for (size_t i = 0; i < exact.size(); ++i) {
    const BuildItem& it = items[exact_items[i]];
    if (!it.Qact) continue;
    const ExactRun& r = exact[i];
    const int es = elsize(it.pl);
    HIP_TRY(poetx::launch_cast(r.Q, static_cast<char*>(it.Qact) + (size_t)es * r.g.q_off,
                               (long long)r.g.b * r.g.b * r.g.count, it.pl->dtype == POETX_BF16, s));
  }
  return POETX_OK;
}

bool side_ok(int32_t side) { return side_ok_fn(side); }

// ------------------------------------------------------------------ allocation-free forward
// poetx_forward_noalloc takes its workspace from this array instead of the
// caller. Each GPU the library runs on holds its own copy until the process
// ends; every call on a GPU shares it, so calls that overlap on one GPU race.
// Host code never passes the array's name to a kernel (on the host it is a
// stand-in, not a device address): it uses the address hipGetSymbolAddress
// returns for the current device, looked up once per device.
constexpr size_t kScratchBytes = size_t(64) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

poetx_status scratch_for_current_device(void** out) {
  int dev = -1;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return POETX_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return POETX_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return POETX_OK;
}

}  // namespace

extern "C" {

const char* poetx_last_hip_error(void) {
  return g_last_hip == hipSuccess ? "no HIP error" : hipGetErrorString(g_last_hip);
}

const char* poetx_status_string(poetx_status st) {
  // callers may pass any integer: read it as one (a value outside the
  // enumerators is not a valid value of the enum type in C++)
  static_assert(sizeof(poetx_status) == sizeof(int), "status passed as an int");
  int v;
  std::memcpy(&v, &st, sizeof v);
  switch (v) {
    case POETX_OK: return "ok";
    case POETX_ERR_INVALID_ARG: return "invalid argument";
    case POETX_ERR_SHAPE: return "inconsistent shape";
    case POETX_ERR_DTYPE: return "unknown dtype";
    case POETX_ERR_ALIGNMENT: return "device pointer not 16-byte aligned";
    case POETX_ERR_UNSUPPORTED: return "unsupported configuration";
    case POETX_ERR_HIP: return "HIP launch failed";
    case POETX_ERR_WORKSPACE: return "workspace missing or too small";
  }
  return "unknown status";
}

poetx_status poetx_plan_create(const poetx_desc* d, poetx_plan** out) {
  if (!d || !out) return POETX_ERR_INVALID_ARG;
  *out = nullptr;
  if (d->dtype != POETX_FP32 && d->dtype != POETX_BF16) return POETX_ERR_DTYPE;
  if (d->m < 1 || d->n < 1 || d->nb_R < 1 || d->nb_P < 1) return POETX_ERR_SHAPE;
  if (!d->bsz_R || !d->bsz_P) return POETX_ERR_INVALID_ARG;
  if (d->k < 0 || d->k > 32) return POETX_ERR_SHAPE;
  if (d->weight != POETX_WEIGHT_DENSE && d->weight != POETX_WEIGHT_INT8_ROWS &&
      d->weight != POETX_WEIGHT_DENSE_T && d->weight != POETX_WEIGHT_INT8_ROWS_T)
    return POETX_ERR_INVALID_ARG;
  if (d->cayley != POETX_CAYLEY_NEUMANN && d->cayley != POETX_CAYLEY_EXACT)
    return POETX_ERR_INVALID_ARG;
  if (d->fold != POETX_FOLD_NONE && d->fold != POETX_FOLD_WEIGHT) return POETX_ERR_INVALID_ARG;
  if (d->index != POETX_INDEX_SEPARATE && d->index != POETX_INDEX_FUSED) return POETX_ERR_INVALID_ARG;
  if (d->series != POETX_SERIES_CHAIN && d->series != POETX_SERIES_PS) return POETX_ERR_INVALID_ARG;
  const int32_t* bs[2] = {d->bsz_R, d->bsz_P};
  const int nb[2] = {d->nb_R, d->nb_P};
  const int dims[2] = {d->m, d->n};
  for (int side = 0; side < 2; ++side) {
    long long sum = 0;
    for (int i = 0; i < nb[side]; ++i) {
      if (bs[side][i] < 1) return POETX_ERR_SHAPE;
      sum += bs[side][i];
    }
    if (sum != dims[side]) return POETX_ERR_SHAPE;
  }
  if (d->dtype == POETX_BF16) {
    if (d->m % 16 || d->n % 16) return POETX_ERR_UNSUPPORTED;
    for (int side = 0; side < 2; ++side)
      for (int i = 0; i < nb[side]; ++i)
        if (bs[side][i] % 16) return POETX_ERR_UNSUPPORTED;
  }
  // INT8 weight: bf16 activations and whole 256 x 256 tiles of the weight
  // (the quantiser also stages one bf16 row of W0 in 64 KiB of LDS)
  if ((d->weight == POETX_WEIGHT_INT8_ROWS || d->weight == POETX_WEIGHT_INT8_ROWS_T) &&
      (d->dtype != POETX_BF16 || d->m % 256 || d->n % 256 || d->n > 32768))
    return POETX_ERR_UNSUPPORTED;
  poetx_plan* pl = new (std::nothrow) poetx_plan;
  if (!pl) return POETX_ERR_INVALID_ARG;
  pl->m = d->m; pl->n = d->n; pl->k = d->k; pl->dtype = d->dtype;
  pl->weight = d->weight;
  pl->cayley = d->cayley;
  pl->fold = d->fold;
  pl->index = d->index;
  pl->series = d->series;
  for (int side = 0; side < 2; ++side) {
    pl->dim[side] = dims[side];
    long long q = 0, p = 0;
    int off = 0;
    for (int i = 0; i < nb[side]; ++i) {
      const int b = bs[side][i];
      pl->bsz[side].push_back(b);
      std::vector<Seg>& sg = pl->segs[side];
      if (!sg.empty() && sg.back().b == b) {
        sg.back().count += 1;
      } else {
        sg.push_back(Seg{b, 1, off, q, p});
      }
      off += b;
      q += (long long)b * b;
      p += (long long)b * (b - 1) / 2;
    }
    pl->nelem[side] = q;
    pl->nparam[side] = p;
  }
  *out = pl;
  return POETX_OK;
}

void poetx_plan_destroy(poetx_plan* pl) { delete pl; }

int64_t poetx_param_count(const poetx_plan* pl, int32_t side) {
  if (!pl || !side_ok(side)) return -1;
  return pl->nparam[side];
}

int64_t poetx_block_elems(const poetx_plan* pl, int32_t side) {
  if (!pl || !side_ok(side)) return -1;
  return pl->nelem[side];
}

size_t poetx_workspace_size(const poetx_plan* pl, int64_t T, int32_t kind) {
  if (!pl || T < 0) return 0;
  switch (kind) {
    case POETX_WS_BUILD: return layout_build(pl, nullptr, nullptr, nullptr, nullptr);
    case POETX_WS_FORWARD: return layout_fwd(pl, T, nullptr, nullptr);
    case POETX_WS_BACKWARD: return layout_bwd(pl, T, nullptr, nullptr, nullptr);
    case POETX_WS_MERGE: return layout_merge(pl, nullptr, nullptr);
    case POETX_WS_PARAM_GRAD: {
      size_t mx = 0;
      for (int side = 0; side < 2; ++side)
        mx = std::max(mx, layout_param_grad(pl, side, nullptr, nullptr));
      return mx;
    }
  }
  return 0;
}

poetx_status poetx_permute_weight(const poetx_plan* pl, const void* W0, const int32_t* pi_R,
                                  const int32_t* pi_P, void* Wt, void* stream) {
  if (!pl || !W0 || !pi_R || !pi_P || !Wt) return POETX_ERR_INVALID_ARG;
  if (!aligned16(W0) || !aligned16(Wt) || !aligned16(pi_R) || !aligned16(pi_P))
    return POETX_ERR_ALIGNMENT;
  if (W0 == Wt) return POETX_ERR_INVALID_ARG;
  if (wq(pl)) return POETX_ERR_UNSUPPORTED;   // poetx_quantize_weight builds that Wt
  HIP_TRY(poetx::launch_gather_cols(W0, pl->n, pi_R, pi_P, Wt, pl->m, pl->n, elsize(pl),
                                    (hipStream_t)stream));
  if (wpair(pl))
    HIP_TRY(poetx::launch_transpose(Wt, const_cast<void*>(wtt(pl, Wt)), pl->m, pl->n, elsize(pl),
                                    (hipStream_t)stream));
  return POETX_OK;
}

size_t poetx_weight_bytes(const poetx_plan* pl) {
  if (!pl) return 0;
  if (wqpair(pl)) return qt_off(pl) + (size_t)pl->m * pl->n;
  if (wq(pl)) return qscale_off(pl) + 4 * (size_t)pl->m;
  if (wpair(pl)) return wtt_off(pl) + (size_t)pl->m * pl->n * elsize(pl);
  return (size_t)pl->m * pl->n * elsize(pl);
}

poetx_status poetx_quantize_weight(const poetx_plan* pl, const void* W0, const int32_t* pi_R,
                                   const int32_t* pi_P, void* Wq, void* stream) {
  if (!pl || !W0 || !pi_R || !pi_P || !Wq) return POETX_ERR_INVALID_ARG;
  if (!wq(pl)) return POETX_ERR_UNSUPPORTED;
  if (!aligned16(W0) || !aligned16(Wq) || !aligned16(pi_R) || !aligned16(pi_P))
    return POETX_ERR_ALIGNMENT;
  if (W0 == Wq) return POETX_ERR_INVALID_ARG;
  HIP_TRY(poetx::launch_quantize_rows(W0, pi_R, pi_P, static_cast<int8_t*>(Wq),
                                      const_cast<float*>(qscale(pl, Wq)), pl->m, pl->n,
                                      (hipStream_t)stream));
  if (wqpair(pl))
    HIP_TRY(poetx::launch_transpose(Wq, const_cast<void*>(qt(pl, Wq)), pl->m, pl->n, 1,
                                    (hipStream_t)stream));
  return POETX_OK;
}

poetx_status poetx_merge_weight(const poetx_plan* pl, const void* Wt, const int32_t* pi_R,
                                const int32_t* pi_P, const float* Q_R, const float* Q_P,
                                void* W_out, void* ws, size_t ws_bytes, void* stream) {
  if (!pl || !Wt || !pi_R || !pi_P || !Q_R || !Q_P || !W_out) return POETX_ERR_INVALID_ARG;
  for (const void* p : {Wt, (const void*)pi_R, (const void*)pi_P, (const void*)Q_R,
                        (const void*)Q_P, (const void*)W_out, (const void*)ws})
    if (!aligned16(p)) return POETX_ERR_ALIGNMENT;
  if (Wt == W_out) return POETX_ERR_INVALID_ARG;
  if (!ws || ws_bytes < poetx_workspace_size(pl, 0, POETX_WS_MERGE)) return POETX_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  MergeWs w;
  layout_merge(pl, ws, &w);
  const long long m = pl->m, n = pl->n;
  const float* src = static_cast<const float*>(Wt);
  if (wq(pl)) {
    HIP_TRY(poetx::launch_dequantize_rows(static_cast<const int8_t*>(Wt), qscale(pl, Wt), w.F,
                                          (int)m, (int)n, s));
    src = w.F;
  } else if (pl->dtype == POETX_BF16) {
    HIP_TRY(poetx::launch_widen(Wt, w.F, m * n, s));
    src = w.F;
  }
  // M1 = D_R Wt: rows of each R block times its Q (M1[blk] = Q Wt[blk])
  for (const Seg& g : pl->segs[POETX_SIDE_R]) {
    poetx::GemmF32 p{};
    p.A = Q_R + g.q_off; p.a_rs = g.b; p.a_cs = 1; p.a_gs = (long long)g.b * g.b;
    p.B = src + g.dim_off * n; p.b_rs = 1; p.b_cs = n; p.b_gs = (long long)g.b * n;
    p.C = w.M1 + g.dim_off * n; p.c_rs = n; p.c_gs = (long long)g.b * n;
    p.M = g.b; p.N = (int)n; p.K = g.b; p.groups = g.count; p.splits = 1;
    p.alpha = 1.0f;
    HIP_TRY(poetx::launch_gemm_f32(p, s));
  }
  // M2 = M1 D_P: columns of each P block times its Q (M2[:, blk] = M1[:, blk] Q)
  for (const Seg& g : pl->segs[POETX_SIDE_P]) {
    poetx::GemmF32 p{};
    p.A = w.M1 + g.dim_off; p.a_rs = n; p.a_cs = 1; p.a_gs = g.b;
    p.B = Q_P + g.q_off; p.b_rs = 1; p.b_cs = g.b; p.b_gs = (long long)g.b * g.b;
    p.C = w.M2 + g.dim_off; p.c_rs = n; p.c_gs = g.b;
    p.M = (int)m; p.N = g.b; p.K = g.b; p.groups = g.count; p.splits = 1;
    p.alpha = 1.0f;
    HIP_TRY(poetx::launch_gemm_f32(p, s));
  }
  // back to the original coordinates: W_out = Pi_R^T M2 Pi_P, i.e.
  // W_out[a][c] = M2[invR[a]][invP[c]], one rounding to the dtype first
  HIP_TRY(poetx::launch_invert_perm(pi_R, w.invR, (int)m, s));
  HIP_TRY(poetx::launch_invert_perm(pi_P, w.invP, (int)n, s));
  const void* gsrc = w.M2;
  if (pl->dtype == POETX_BF16) {
    HIP_TRY(poetx::launch_cast(w.M2, w.C, m * n, 1, s));
    gsrc = w.C;
  }
  HIP_TRY(poetx::launch_gather_cols(gsrc, n, w.invR, w.invP, W_out, m, (int)n, elsize(pl), s));
  return POETX_OK;
}

poetx_status poetx_build_orth(const poetx_plan* pl, int32_t side, const float* theta, float* Q_f32,
                              void* Q_act, void* ws, size_t ws_bytes, void* stream) {
  BuildItem it{pl, side, theta, Q_f32, Q_act, ws};
  poetx_status st = check_build_item(it, ws_bytes);
  if (st != POETX_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  StageScope sc(POETX_STAGE_BUILD, s);
  return build_items(&it, 1, s);
}

poetx_status poetx_build_orth_batch(int32_t count, const poetx_plan* const* plans,
                                    const int32_t* sides, const float* const* thetas,
                                    float* const* Q_f32, void* const* Q_act, void* const* ws,
                                    const size_t* ws_bytes, void* stream) {
  if (count < 0) return POETX_ERR_INVALID_ARG;
  if (count == 0) return POETX_OK;
  if (!plans || !sides || !thetas || !Q_f32 || !ws || !ws_bytes) return POETX_ERR_INVALID_ARG;
  std::vector<BuildItem> items((size_t)count);
  for (int i = 0; i < count; ++i) {
    items[i] = BuildItem{plans[i], sides[i], thetas[i], Q_f32[i], Q_act ? Q_act[i] : nullptr, ws[i]};
    poetx_status st = check_build_item(items[i], ws_bytes[i]);
    if (st != POETX_OK) return st;
  }
  hipStream_t s = (hipStream_t)stream;
  StageScope sc(POETX_STAGE_BUILD, s);
  return build_items(items.data(), count, s);
}

poetx_status poetx_forward(const poetx_plan* pl, int64_t T, const void* X, const void* Wt,
                           const int32_t* pi_R, const int32_t* pi_P, const void* Q_R,
                           const void* Q_P, void* Y, void* Wa_saved, void* U_saved, void* ws,
                           size_t ws_bytes, void* stream) {
  if (!pl || T < 0) return POETX_ERR_INVALID_ARG;
  if (T == 0) return POETX_OK;
  // X may be NULL when U_saved already holds the gathered input
  if ((!X && !U_saved) || !Wt || !pi_R || !pi_P || !Q_R || !Q_P || !Y) return POETX_ERR_INVALID_ARG;
  for (const void* p : {X, Wt, (const void*)pi_R, (const void*)pi_P, Q_R, Q_P, (const void*)Y,
                        (const void*)Wa_saved, (const void*)U_saved, (const void*)ws})
    if (!aligned16(p)) return POETX_ERR_ALIGNMENT;
  if (!ws || ws_bytes < poetx_workspace_size(pl, T, POETX_WS_FORWARD)) return POETX_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  FwdWs w;
  layout_fwd(pl, T, ws, &w);
  void* Wa = Wa_saved ? Wa_saved : w.Wa;
  if (U_saved) w.U = U_saved;   // the gather writes the caller's buffer
  const int es = elsize(pl);
  poetx_status st;
  const bool fold = fold_fwd(pl, T);
  // 1 + 2 fused: one pass over X gathers it by pi_P and applies the P blocks
  // (U kept in U_saved when given)
  const bool fused_p = X && !fold && panel_side(pl, POETX_SIDE_P);
  // 1. gather: U = X Pi_P^T (none when the caller passes U instead of X)
  if (X && !fused_p) {
    StageScope sc(POETX_STAGE_GATHER, s);
    HIP_TRY(poetx::launch_gather_cols(X, pl->n, nullptr, pi_P, w.U, T, pl->n, es, s));
  }
  // 2. blocks of P: V = U D_P^T, or folded into the weight, Wf = Wt D_P
  {
    StageScope sc(POETX_STAGE_BLOCK_FWD, s);
    if (fused_p) {
      HIP_TRY(poetx::launch_panel_block(X, pi_P, Q_P, w.V, U_saved, T, pl->n, true, false, s));
      st = POETX_OK;
    } else {
      st = fold ? fold_p(pl, Wt, Q_P, w.Wf, s)
                : apply_blocks(pl, POETX_SIDE_P, T, w.U, Q_P, w.V, true, s);
    }
    if (st != POETX_OK) return st;
  }
  // 3. frozen weight: Wa = V Wt^T (folded: Wa = U Wf^T)
  {
    StageScope sc(POETX_STAGE_W0_FWD, s);
    const Op a = fold ? Op{w.U, pl->n, 1} : Op{w.V, pl->n, 1};
    if ((st = w0_forward_product(pl, a, fold ? w.Wf : Wt, w.Wq, Wa, T, s)) != POETX_OK) return st;
  }
  // 4 + 5 fused: Z = Wa D_R^T scattered to Y in one pass over the rows
  if (panel_side(pl, POETX_SIDE_R)) {
    StageScope sc(POETX_STAGE_BLOCK_FWD, s);
    HIP_TRY(poetx::launch_panel_block(Wa, pi_R, Q_R, Y, nullptr, T, pl->m, false, true, s));
    return POETX_OK;
  }
  // 4. blocks of R: Z = Wa D_R^T
  {
    StageScope sc(POETX_STAGE_BLOCK_FWD, s);
    if ((st = apply_blocks(pl, POETX_SIDE_R, T, Wa, Q_R, w.Z, true, s)) != POETX_OK) return st;
  }
  // 5. scatter: Y = Z Pi_R
  {
    StageScope sc(POETX_STAGE_SCATTER, s);
    HIP_TRY(poetx::launch_scatter_cols(w.Z, pi_R, Y, T, pl->m, es, s));
  }
  return POETX_OK;
}

size_t poetx_forward_noalloc_max_bytes(void) { return kScratchBytes; }

poetx_status poetx_forward_noalloc(const poetx_plan* pl, int64_t T, const void* X, const void* Wt,
                                   const int32_t* pi_R, const int32_t* pi_P, const void* Q_R,
                                   const void* Q_P, void* Y, void* Wa_saved, void* U_saved,
                                   void* stream) {
  // the argument checks of poetx_forward, before the device is touched
  if (!pl || T < 0) return POETX_ERR_INVALID_ARG;
  if (T == 0) return POETX_OK;
  if ((!X && !U_saved) || !Wt || !pi_R || !pi_P || !Q_R || !Q_P || !Y) return POETX_ERR_INVALID_ARG;
  for (const void* p : {X, Wt, (const void*)pi_R, (const void*)pi_P, Q_R, Q_P, (const void*)Y,
                        (const void*)Wa_saved, (const void*)U_saved})
    if (!aligned16(p)) return POETX_ERR_ALIGNMENT;
  if (poetx_workspace_size(pl, T, POETX_WS_FORWARD) > kScratchBytes) return POETX_ERR_WORKSPACE;
  void* ws = nullptr;
  poetx_status st = scratch_for_current_device(&ws);
  if (st != POETX_OK) return st;
  return poetx_forward(pl, T, X, Wt, pi_R, pi_P, Q_R, Q_P, Y, Wa_saved, U_saved, ws, kScratchBytes,
                       stream);
}

poetx_status poetx_backward(const poetx_plan* pl, int64_t T, const void* X, const void* Wt,
                            const int32_t* pi_R, const int32_t* pi_P, const float* theta_R,
                            const float* theta_P, const void* Q_R, const void* Q_P,
                            const void* Wa_saved, const void* U_saved, const void* G_Y, void* G_X,
                            float* g_theta_R, float* g_theta_P, void* ws, size_t ws_bytes,
                            void* stream) {
  poetx_status st = check_backward_args(pl, T, X, Wt, pi_R, pi_P, Q_R, Q_P, Wa_saved, U_saved, G_Y,
                                        G_X, ws, ws_bytes);
  if (st != POETX_OK) return st;
  if (!theta_R || !theta_P || !g_theta_R || !g_theta_P) return POETX_ERR_INVALID_ARG;
  for (const void* p : {(const void*)theta_R, (const void*)theta_P, (const void*)g_theta_R,
                        (const void*)g_theta_P})
    if (!aligned16(p)) return POETX_ERR_ALIGNMENT;
  hipStream_t s = (hipStream_t)stream;
  BwdWs w;
  ChainWs cw[2];
  layout_bwd(pl, T, ws, &w, cw);
  if ((st = backward_dq(pl, T, X, Wt, pi_R, pi_P, Q_R, Q_P, Wa_saved, U_saved, G_Y, G_X, w.dQ, w,
                        s)) != POETX_OK)
    return st;
  StageScope sc(POETX_STAGE_CNP_BWD, s);
  const GradItem items[2] = {{pl, POETX_SIDE_R, theta_R, w.dQ[0], g_theta_R, cw[0]},
                             {pl, POETX_SIDE_P, theta_P, w.dQ[1], g_theta_P, cw[1]}};
  return grad_items(items, 2, s);
}

poetx_status poetx_backward_dq(const poetx_plan* pl, int64_t T, const void* X, const void* Wt,
                               const int32_t* pi_R, const int32_t* pi_P, const void* Q_R,
                               const void* Q_P, const void* Wa_saved, const void* U_saved,
                               const void* G_Y, void* G_X, float* dQ_R, float* dQ_P, void* ws,
                               size_t ws_bytes, void* stream) {
  poetx_status st = check_backward_args(pl, T, X, Wt, pi_R, pi_P, Q_R, Q_P, Wa_saved, U_saved, G_Y,
                                        G_X, ws, ws_bytes);
  if (st != POETX_OK) return st;
  if (!dQ_R || !dQ_P) return POETX_ERR_INVALID_ARG;
  if (!aligned16(dQ_R) || !aligned16(dQ_P)) return POETX_ERR_ALIGNMENT;
  hipStream_t s = (hipStream_t)stream;
  BwdWs w;
  layout_bwd(pl, T, ws, &w, nullptr);
  float* const dQ[2] = {dQ_R, dQ_P};
  return backward_dq(pl, T, X, Wt, pi_R, pi_P, Q_R, Q_P, Wa_saved, U_saved, G_Y, G_X, dQ, w, s);
}

poetx_status poetx_param_grad_batch(int32_t count, const poetx_plan* const* plans,
                                    const int32_t* sides, const float* const* thetas,
                                    const float* const* dQs, float* const* g_thetas,
                                    void* const* ws, const size_t* ws_bytes, void* stream) {
  if (count < 0) return POETX_ERR_INVALID_ARG;
  if (count == 0) return POETX_OK;
  if (!plans || !sides || !thetas || !dQs || !g_thetas || !ws || !ws_bytes)
    return POETX_ERR_INVALID_ARG;
  std::vector<GradItem> items((size_t)count);
  for (int i = 0; i < count; ++i) {
    const poetx_plan* pl = plans[i];
    if (!pl || !side_ok_fn(sides[i]) || !thetas[i] || !dQs[i] || !g_thetas[i] || !ws[i])
      return POETX_ERR_INVALID_ARG;
    if (!aligned16(thetas[i]) || !aligned16(dQs[i]) || !aligned16(g_thetas[i]) || !aligned16(ws[i]))
      return POETX_ERR_ALIGNMENT;
    if (ws_bytes[i] < poetx_workspace_size(pl, 0, POETX_WS_PARAM_GRAD)) return POETX_ERR_WORKSPACE;
    items[i].pl = pl;
    items[i].side = sides[i];
    items[i].theta = thetas[i];
    items[i].dQ = dQs[i];
    items[i].g = g_thetas[i];
    layout_param_grad(pl, sides[i], ws[i], &items[i].w);
  }
  hipStream_t s = (hipStream_t)stream;
  StageScope sc(POETX_STAGE_CNP_BWD, s);
  return grad_items(items.data(), count, s);
}

poetx_status poetx_gather_cols(const poetx_plan* pl, int64_t T, int32_t dim, const void* in,
                               const int32_t* idx, void* out, void* stream) {
  if (!pl || T < 0 || dim < 0) return POETX_ERR_INVALID_ARG;
  if (T == 0 || dim == 0) return POETX_OK;
  if (!in || !idx || !out || in == out) return POETX_ERR_INVALID_ARG;
  if (!aligned16(in) || !aligned16(out) || !aligned16(idx)) return POETX_ERR_ALIGNMENT;
  HIP_TRY(poetx::launch_gather_cols(in, dim, nullptr, idx, out, T, dim, elsize(pl), (hipStream_t)stream));
  return POETX_OK;
}

poetx_status poetx_scatter_cols(const poetx_plan* pl, int64_t T, int32_t dim, const void* in,
                                const int32_t* idx, void* out, void* stream) {
  if (!pl || T < 0 || dim < 0) return POETX_ERR_INVALID_ARG;
  if (T == 0 || dim == 0) return POETX_OK;
  if (!in || !idx || !out || in == out) return POETX_ERR_INVALID_ARG;
  if (!aligned16(in) || !aligned16(out) || !aligned16(idx)) return POETX_ERR_ALIGNMENT;
  HIP_TRY(poetx::launch_scatter_cols(in, idx, out, T, dim, elsize(pl), (hipStream_t)stream));
  return POETX_OK;
}

poetx_status poetx_timing_enable(uint32_t mask) {
  g_tmask.store(mask & ((1u << POETX_NUM_STAGES) - 1u));
  return POETX_OK;
}

poetx_status poetx_timing_read(int32_t stage, double* ms, int64_t* count) {
  if (stage < 0 || stage >= POETX_NUM_STAGES || !ms || !count) return POETX_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(g_tmu);
  double tot = 0.0;
  int64_t n = 0;
  for (const TimingRec& r : g_recs) {
    if (r.stage != stage) continue;
    HIP_TRY(hipEventSynchronize(r.b));
    float t = 0.0f;
    HIP_TRY(hipEventElapsedTime(&t, r.a, r.b));
    tot += t;
    ++n;
  }
  *ms = tot;
  *count = n;
  return POETX_OK;
}

void poetx_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_tmu);
  for (const TimingRec& r : g_recs) {
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.clear();
}

}  // extern "C"
