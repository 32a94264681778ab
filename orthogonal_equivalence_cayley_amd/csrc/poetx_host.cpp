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
#include <mutex>
#include <new>
#include <vector>

#include "../../include/poetx.h"
#include "poetx_internal.h"

using poetx::Seg;

struct poetx_plan {
  int m = 0, n = 0, k = 0, dtype = 0;
  std::vector<int> bsz[2];
  std::vector<Seg> segs[2];
  long long nparam[2] = {0, 0};
  long long nelem[2] = {0, 0};
  int dim[2] = {0, 0};   // m for R, n for P
};

namespace {

constexpr size_t kAlign = 256;

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

// dQ products reduce over tokens; split the token range so that the grid fills
// the chip. Partial sums are reduced afterwards in a fixed order.
int dq_splits(const poetx_plan* pl, int side, long long T) {
  long long tiles = 0;
  const int tile = pl->dtype == POETX_BF16 ? 128 : 64;
  for (const Seg& g : pl->segs[side]) {
    const long long t = (g.b + tile - 1) / tile;
    tiles += t * t * g.count;
  }
  long long s = (512 + tiles - 1) / std::max<long long>(tiles, 1);
  const long long maxs = std::max<long long>(1, (T + 255) / 256);
  s = std::min(s, maxs);
  s = std::max<long long>(1, std::min<long long>(s, 64));
  return (int)s;
}

struct FwdWs { void *U, *V, *Wa, *Z; };
struct BwdWs {
  void *GZ, *GWa, *GV, *U, *GU;
  float *dQ[2], *part, *S, *A0, *A1, *T0, *T1, *Astore;
};

size_t layout_fwd(const poetx_plan* pl, long long T, void* base, FwdWs* w) {
  Carver c(base);
  const size_t es = elsize(pl);
  FwdWs x;
  x.U = c.take(es * T * pl->n);
  x.V = c.take(es * T * pl->n);
  x.Wa = c.take(es * T * pl->m);
  x.Z = c.take(es * T * pl->m);
  if (w) *w = x;
  return c.off;
}

size_t layout_bwd(const poetx_plan* pl, long long T, void* base, BwdWs* w) {
  Carver c(base);
  const size_t es = elsize(pl);
  BwdWs x;
  x.GZ = c.take(es * T * pl->m);
  x.GWa = c.take(es * T * pl->m);
  x.GV = c.take(es * T * pl->n);
  x.U = c.take(es * T * pl->n);
  x.GU = c.take(es * T * pl->n);
  x.dQ[0] = (float*)c.take(4 * pl->nelem[0]);
  x.dQ[1] = (float*)c.take(4 * pl->nelem[1]);
  long long part = 0;
  for (int side = 0; side < 2; ++side)
    part = std::max(part, (long long)dq_splits(pl, side, T) * pl->nelem[side]);
  x.part = (float*)c.take(4 * part);
  const long long ne = std::max(pl->nelem[0], pl->nelem[1]);
  x.S = (float*)c.take(4 * ne);
  x.A0 = (float*)c.take(4 * ne);
  x.A1 = (float*)c.take(4 * ne);
  x.T0 = (float*)c.take(4 * ne);
  x.T1 = (float*)c.take(4 * ne);
  x.Astore = (float*)c.take(4 * ne * (pl->k + 1));
  if (w) *w = x;
  return c.off;
}

size_t layout_build(const poetx_plan* pl, void* base, float** S, float** P0, float** P1) {
  Carver c(base);
  const long long ne = std::max(pl->nelem[0], pl->nelem[1]);
  float* s = (float*)c.take(4 * ne);
  float* p0 = (float*)c.take(4 * ne);
  float* p1 = (float*)c.take(4 * ne);
  if (S) { *S = s; *P0 = p0; *P1 = p1; }
  return c.off;
}

#define HIP_TRY(expr)                                   \
  do {                                                  \
    if ((expr) != hipSuccess) return POETX_ERR_HIP;     \
  } while (0)

// Operand view: element (row, k) at p[row * rs + k * cs].
struct Op {
  const void* p;
  long long rs, cs;
};

// C(m, n) = sum_k A(m, k) B(n, k) in the plan's dtype (fp32 output when out_f32).
poetx_status gemm(const poetx_plan* pl, int role, Op A, Op B, void* C, long long ldc, int M, int N,
                  int K, int groups, long long a_gs, long long b_gs, long long c_gs, int splits,
                  long long c_ss, bool out_f32, hipStream_t s) {
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

// Row-form product with one side's blocks: out[:, blk] = in[:, blk] Q^T
// (transpose_q = true) or in[:, blk] Q (false), for every block of the side.
poetx_status apply_blocks(const poetx_plan* pl, int side, long long T, const void* in,
                          const void* Q, void* out, bool transpose_q, hipStream_t s) {
  const size_t es = elsize(pl);
  const long long dim = pl->dim[side];
  for (const Seg& g : pl->segs[side]) {
    const char* a = static_cast<const char*>(in) + es * g.dim_off;
    const char* q = static_cast<const char*>(Q) + es * g.q_off;
    char* c = static_cast<char*>(out) + es * g.dim_off;
    // transpose_q: B(n, k) = Q[n][k]; otherwise B(n, k) = Q[k][n]
    Op B = transpose_q ? Op{q, g.b, 1} : Op{q, 1, g.b};
    poetx_status st = gemm(pl, poetx::GEMM_BLOCK, Op{a, dim, 1}, B, c, dim, (int)T, g.b, g.b, g.count, g.b,
                           (long long)g.b * g.b, g.b, 1, 0, false, s);
    if (st != POETX_OK) return st;
  }
  return POETX_OK;
}

// dQ[blk] = G[:, blk]^T A[:, blk] (reduction over tokens), fp32.
poetx_status block_grads(const poetx_plan* pl, int side, long long T, const void* G, const void* A,
                         float* part, float* dQ, hipStream_t s) {
  const size_t es = elsize(pl);
  const long long dim = pl->dim[side];
  const int splits = dq_splits(pl, side, T);
  const long long ne = pl->nelem[side];
  for (const Seg& g : pl->segs[side]) {
    const char* a = static_cast<const char*>(G) + es * g.dim_off;
    const char* b = static_cast<const char*>(A) + es * g.dim_off;
    // rows of the product index features, k indexes tokens
    poetx_status st = gemm(pl, poetx::GEMM_DQ, Op{a, 1, dim}, Op{b, 1, dim}, part + g.q_off, g.b, g.b, g.b,
                           (int)T, g.count, g.b, g.b, (long long)g.b * g.b, splits, ne, true, s);
    if (st != POETX_OK) return st;
  }
  HIP_TRY(poetx::launch_sum_splits(part, splits, ne, ne, dQ, s));
  return POETX_OK;
}

// Reverse mode through Q = sum_j c_j S^j for every block of one side:
//   A_{k+1} = c_{k+1} G,  A_j = c_j G + A_{j+1} S^T,
//   T_{k+1} = A_{k+1},    T_j = A_j + S^T T_{j+1},   dL/dS = T_1,
// then dL/dtheta(i,j) = dS[i][j] - dS[j][i]. Uses S^T = -S.
poetx_status cnp_backward(const poetx_plan* pl, int side, const float* theta, const float* G,
                          float* gtheta, float* S, float* A0, float* A1, float* T0, float* T1,
                          float* Astore, hipStream_t s) {
  const int k = pl->k;
  const long long ne = pl->nelem[side];
  for (const Seg& g : pl->segs[side]) HIP_TRY(poetx::launch_unpack_skew(theta, g, S, nullptr, 0.0f, s));
  bool any_generic = false;
  for (const Seg& g : pl->segs[side]) {
    if (!poetx::chain_supported(g.b)) {
      any_generic = true;
      continue;
    }
    // row-local first chain, then the transposed second chain, then pack
    poetx::ChainArgs c;
    c.S = S; c.G = G; c.out_f32 = Astore; c.out_act = nullptr; c.act_bf16 = 0;
    c.b = g.b; c.count = g.count; c.k = k; c.q_off = g.q_off; c.ne = ne;
    HIP_TRY(poetx::launch_chain(poetx::CHAIN_ABAR, c, s));
    c.G = Astore; c.out_f32 = T0;
    HIP_TRY(poetx::launch_chain(poetx::CHAIN_TCHAIN, c, s));
    HIP_TRY(poetx::launch_pack_antisym(T0, g, -1.0f, gtheta, s));
  }
  if (!any_generic) return POETX_OK;
  // blocks whose size the MFMA chain does not take: batched fp32 GEMM per step
  HIP_TRY(poetx::launch_scale2(G, coef(k + 1, k), A0, T1, ne, s));
  float *Acur = A0, *Anew = A1, *Tcur = T1, *Tnew = T0;
  for (int j = k; j >= 1; --j) {
    for (const Seg& g : pl->segs[side]) {
      if (poetx::chain_supported(g.b)) continue;
      // A_j = c_j G - A_{j+1} S
      poetx_status st = chain_gemm(g, Acur, S, Anew, G, nullptr, -1.0f, coef(j, k), s);
      if (st != POETX_OK) return st;
      // T_j = A_j - S T_{j+1}
      st = chain_gemm(g, S, Tcur, Tnew, Anew, nullptr, -1.0f, 1.0f, s);
      if (st != POETX_OK) return st;
    }
    std::swap(Acur, Anew);
    std::swap(Tcur, Tnew);
  }
  for (const Seg& g : pl->segs[side])
    if (!poetx::chain_supported(g.b)) HIP_TRY(poetx::launch_pack_antisym(Tcur, g, 1.0f, gtheta, s));
  return POETX_OK;
}

bool side_ok(int32_t side) { return side == POETX_SIDE_R || side == POETX_SIDE_P; }

}  // namespace

extern "C" {

const char* poetx_status_string(poetx_status st) {
  switch (st) {
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
  poetx_plan* pl = new (std::nothrow) poetx_plan;
  if (!pl) return POETX_ERR_INVALID_ARG;
  pl->m = d->m; pl->n = d->n; pl->k = d->k; pl->dtype = d->dtype;
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
    case POETX_WS_BACKWARD: return layout_bwd(pl, T, nullptr, nullptr);
  }
  return 0;
}

poetx_status poetx_permute_weight(const poetx_plan* pl, const void* W0, const int32_t* pi_R,
                                  const int32_t* pi_P, void* Wt, void* stream) {
  if (!pl || !W0 || !pi_R || !pi_P || !Wt) return POETX_ERR_INVALID_ARG;
  if (!aligned16(W0) || !aligned16(Wt) || !aligned16(pi_R) || !aligned16(pi_P))
    return POETX_ERR_ALIGNMENT;
  if (W0 == Wt) return POETX_ERR_INVALID_ARG;
  HIP_TRY(poetx::launch_gather_cols(W0, pl->n, pi_R, pi_P, Wt, pl->m, pl->n, elsize(pl),
                                    (hipStream_t)stream));
  return POETX_OK;
}

poetx_status poetx_build_orth(const poetx_plan* pl, int32_t side, const float* theta, float* Q_f32,
                              void* Q_act, void* ws, size_t ws_bytes, void* stream) {
  if (!pl || !side_ok(side) || !theta || !Q_f32) return POETX_ERR_INVALID_ARG;
  if (!aligned16(theta) || !aligned16(Q_f32) || !aligned16(Q_act) || !aligned16(ws))
    return POETX_ERR_ALIGNMENT;
  if (!ws || ws_bytes < poetx_workspace_size(pl, 0, POETX_WS_BUILD)) return POETX_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  StageScope sc(POETX_STAGE_BUILD, s);
  float *S, *P0, *P1;
  layout_build(pl, ws, &S, &P0, &P1);
  const int k = pl->k;
  const bool bf16 = pl->dtype == POETX_BF16;
  const int es = elsize(pl);
  for (const Seg& g : pl->segs[side]) {
    if (poetx::chain_supported(g.b)) {
      // one fused kernel per run of blocks: S -> powers -> Q (fp32 and act copy)
      HIP_TRY(poetx::launch_unpack_skew(theta, g, S, nullptr, 0.0f, s));
      poetx::ChainArgs c;
      c.S = S; c.G = nullptr; c.out_f32 = Q_f32; c.out_act = Q_act; c.act_bf16 = bf16;
      c.b = g.b; c.count = g.count; c.k = k; c.q_off = g.q_off; c.ne = pl->nelem[side];
      HIP_TRY(poetx::launch_chain(poetx::CHAIN_BUILD, c, s));
      continue;
    }
    HIP_TRY(poetx::launch_unpack_skew(theta, g, S, Q_f32, coef(1, k), s));
    // powers S^j = S^{j-1} S for j = 2..k+1, each added into Q with weight c_j
    const float* prev = S;
    float* bufs[2] = {P0, P1};
    for (int j = 2; j <= k + 1; ++j) {
      float* next = (j < k + 1) ? bufs[j & 1] : nullptr;
      poetx_status st = chain_gemm(g, prev, S, Q_f32, Q_f32, next, coef(j, k), 1.0f, s);
      if (st != POETX_OK) return st;
      prev = next;
    }
    if (Q_act)
      HIP_TRY(poetx::launch_cast(Q_f32 + g.q_off, static_cast<char*>(Q_act) + es * g.q_off,
                                 (long long)g.b * g.b * g.count, bf16, s));
  }
  return POETX_OK;
}

poetx_status poetx_forward(const poetx_plan* pl, int64_t T, const void* X, const void* Wt,
                           const int32_t* pi_R, const int32_t* pi_P, const void* Q_R,
                           const void* Q_P, void* Y, void* Wa_saved, void* ws, size_t ws_bytes,
                           void* stream) {
  if (!pl || T < 0) return POETX_ERR_INVALID_ARG;
  if (T == 0) return POETX_OK;
  if (!X || !Wt || !pi_R || !pi_P || !Q_R || !Q_P || !Y) return POETX_ERR_INVALID_ARG;
  for (const void* p : {X, Wt, (const void*)pi_R, (const void*)pi_P, Q_R, Q_P, (const void*)Y,
                        (const void*)Wa_saved, (const void*)ws})
    if (!aligned16(p)) return POETX_ERR_ALIGNMENT;
  if (!ws || ws_bytes < poetx_workspace_size(pl, T, POETX_WS_FORWARD)) return POETX_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  FwdWs w;
  layout_fwd(pl, T, ws, &w);
  void* Wa = Wa_saved ? Wa_saved : w.Wa;
  const int es = elsize(pl);
  poetx_status st;
  // 1. gather: U = X Pi_P^T
  {
    StageScope sc(POETX_STAGE_GATHER, s);
    HIP_TRY(poetx::launch_gather_cols(X, pl->n, nullptr, pi_P, w.U, T, pl->n, es, s));
  }
  // 2. blocks of P: V = U D_P^T
  {
    StageScope sc(POETX_STAGE_BLOCK_FWD, s);
    if ((st = apply_blocks(pl, POETX_SIDE_P, T, w.U, Q_P, w.V, true, s)) != POETX_OK) return st;
  }
  // 3. frozen weight: Wa = V Wt^T
  {
    StageScope sc(POETX_STAGE_W0_FWD, s);
    if ((st = gemm(pl, poetx::GEMM_W0, Op{w.V, pl->n, 1}, Op{Wt, pl->n, 1}, Wa, pl->m, (int)T, pl->m,
                   pl->n, 1, 0, 0, 0, 1, 0, false, s)) != POETX_OK)
      return st;
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

poetx_status poetx_backward(const poetx_plan* pl, int64_t T, const void* X, const void* Wt,
                            const int32_t* pi_R, const int32_t* pi_P, const float* theta_R,
                            const float* theta_P, const void* Q_R, const void* Q_P,
                            const void* Wa_saved, const void* G_Y, void* G_X, float* g_theta_R,
                            float* g_theta_P, void* ws, size_t ws_bytes, void* stream) {
  if (!pl || T < 0) return POETX_ERR_INVALID_ARG;
  if (!theta_R || !theta_P || !g_theta_R || !g_theta_P) return POETX_ERR_INVALID_ARG;
  if (T > 0 && (!X || !Wt || !pi_R || !pi_P || !Q_R || !Q_P || !Wa_saved || !G_Y || !G_X))
    return POETX_ERR_INVALID_ARG;
  for (const void* p : {X, Wt, (const void*)pi_R, (const void*)pi_P, (const void*)theta_R,
                        (const void*)theta_P, Q_R, Q_P, Wa_saved, G_Y, (const void*)G_X,
                        (const void*)g_theta_R, (const void*)g_theta_P, (const void*)ws})
    if (!aligned16(p)) return POETX_ERR_ALIGNMENT;
  if (!ws || ws_bytes < poetx_workspace_size(pl, T, POETX_WS_BACKWARD)) return POETX_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  BwdWs w;
  layout_bwd(pl, T, ws, &w);
  const int es = elsize(pl);
  poetx_status st;
  if (T > 0) {
    // R side: G_Z = G_Y Pi_R^T; dQ_R = G_Z^T Wa per block; G_Wa = G_Z D_R
    {
      StageScope sc(POETX_STAGE_GATHER, s);
      HIP_TRY(poetx::launch_gather_cols(G_Y, pl->m, nullptr, pi_R, w.GZ, T, pl->m, es, s));
    }
    {
      StageScope sc(POETX_STAGE_DQ, s);
      if ((st = block_grads(pl, POETX_SIDE_R, T, w.GZ, Wa_saved, w.part, w.dQ[0], s)) != POETX_OK)
        return st;
    }
    {
      StageScope sc(POETX_STAGE_BLOCK_BWD, s);
      if ((st = apply_blocks(pl, POETX_SIDE_R, T, w.GZ, Q_R, w.GWa, false, s)) != POETX_OK) return st;
    }
    // frozen weight: G_V = G_Wa Wt
    {
      StageScope sc(POETX_STAGE_W0_BWD, s);
      if ((st = gemm(pl, poetx::GEMM_W0, Op{w.GWa, pl->m, 1}, Op{Wt, 1, pl->n}, w.GV, pl->n, (int)T,
                     pl->n, pl->m, 1, 0, 0, 0, 1, 0, false, s)) != POETX_OK)
        return st;
    }
    // P side: U = X Pi_P^T; dQ_P = G_V^T U per block; G_U = G_V D_P; G_X = G_U Pi_P
    {
      StageScope sc(POETX_STAGE_GATHER, s);
      HIP_TRY(poetx::launch_gather_cols(X, pl->n, nullptr, pi_P, w.U, T, pl->n, es, s));
    }
    {
      StageScope sc(POETX_STAGE_DQ, s);
      if ((st = block_grads(pl, POETX_SIDE_P, T, w.GV, w.U, w.part, w.dQ[1], s)) != POETX_OK)
        return st;
    }
    {
      StageScope sc(POETX_STAGE_BLOCK_BWD, s);
      if ((st = apply_blocks(pl, POETX_SIDE_P, T, w.GV, Q_P, w.GU, false, s)) != POETX_OK) return st;
    }
    {
      StageScope sc(POETX_STAGE_SCATTER, s);
      HIP_TRY(poetx::launch_scatter_cols(w.GU, pi_P, G_X, T, pl->n, es, s));
    }
  } else {
    HIP_TRY(poetx::launch_zero(w.dQ[0], pl->nelem[0], s));
    HIP_TRY(poetx::launch_zero(w.dQ[1], pl->nelem[1], s));
  }
  StageScope sc(POETX_STAGE_CNP_BWD, s);
  if ((st = cnp_backward(pl, POETX_SIDE_R, theta_R, w.dQ[0], g_theta_R, w.S, w.A0, w.A1, w.T0,
                         w.T1, w.Astore, s)) != POETX_OK)
    return st;
  return cnp_backward(pl, POETX_SIDE_P, theta_P, w.dQ[1], g_theta_P, w.S, w.A0, w.A1, w.T0, w.T1,
                      w.Astore, s);
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
    if (hipEventSynchronize(r.b) != hipSuccess) return POETX_ERR_HIP;
    float t = 0.0f;
    if (hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) return POETX_ERR_HIP;
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
