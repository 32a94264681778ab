// Host-side checks of the C ABI (include/poetx.h) for a build of the library's
// host code under AddressSanitizer and UndefinedBehaviorSanitizer. Every call
// here either fails argument validation or is a no-op (T = 0), so nothing
// reaches a kernel launch and no device memory is touched: device pointers
// are fake addresses that the library only compares and checks for
// alignment. Exit status 0 when every returned status is the expected one.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include <hip/hip_runtime.h>

#include "poetx.h"

static int failures = 0;
#define EXPECT(cond)                                                            \
  do {                                                                          \
    if (!(cond)) {                                                              \
      std::printf("FAILED line %d: %s\n", __LINE__, #cond);                     \
      ++failures;                                                               \
    }                                                                           \
  } while (0)

namespace {

struct Desc {
  std::vector<int32_t> bR, bP;
  poetx_desc d{};
  Desc(int m, int n, std::vector<int32_t> r, std::vector<int32_t> p, int k, int dtype)
      : bR(std::move(r)), bP(std::move(p)) {
    d.m = m;
    d.n = n;
    d.nb_R = (int32_t)bR.size();
    d.nb_P = (int32_t)bP.size();
    d.bsz_R = bR.data();
    d.bsz_P = bP.data();
    d.k = k;
    d.dtype = dtype;
  }
};

// fake, 256-byte aligned device addresses: never dereferenced on the host
void* dev(uintptr_t i) { return reinterpret_cast<void*>(0x7f0000000000ull + 0x100000ull * i); }
void* mis(uintptr_t i) { return reinterpret_cast<void*>(0x7f0000000000ull + 0x100000ull * i + 4); }

void plan_options() {
  // every combination of options on a bf16 plan of 256-wide blocks, plus an
  // fp32 plan with ragged blocks
  for (int weight = 0; weight < 4; ++weight)
    for (int cayley = 0; cayley < 2; ++cayley)
      for (int fold = 0; fold < 2; ++fold)
        for (int index = 0; index < 2; ++index)
          for (int series = 0; series < 2; ++series) {
            Desc a(512, 768, {256, 256}, {256, 256, 256}, 4, POETX_BF16);
            a.d.weight = weight;
            a.d.cayley = cayley;
            a.d.fold = fold;
            a.d.index = index;
            a.d.series = series;
            poetx_plan* p = nullptr;
            const poetx_status s = poetx_plan_create(&a.d, &p);
            if (s == POETX_OK) {
              EXPECT(p != nullptr);
              EXPECT(poetx_param_count(p, POETX_SIDE_R) == 2 * 256 * 255 / 2);
              EXPECT(poetx_param_count(p, POETX_SIDE_P) == 3 * 256 * 255 / 2);
              EXPECT(poetx_param_count(p, 2) == -1);
              EXPECT(poetx_block_elems(p, POETX_SIDE_P) == 3 * 256 * 256);
              for (int kind = 0; kind <= 5; ++kind)
                for (int64_t T : {(int64_t)-1, (int64_t)0, (int64_t)1, (int64_t)16384, (int64_t)1 << 40}) {
                  const size_t w = poetx_workspace_size(p, T, kind);
                  if (kind > 4 || T < 0) EXPECT(w == 0);
                }
              EXPECT(poetx_weight_bytes(p) >= (size_t)512 * 768);
              poetx_plan_destroy(p);
            } else {
              EXPECT(p == nullptr);
              EXPECT(s == POETX_ERR_INVALID_ARG || s == POETX_ERR_UNSUPPORTED);
            }
          }
  Desc f(12, 9, {5, 7}, {4, 1, 4}, 0, POETX_FP32);
  poetx_plan* p = nullptr;
  EXPECT(poetx_plan_create(&f.d, &p) == POETX_OK);
  EXPECT(poetx_param_count(p, POETX_SIDE_R) == 5 * 4 / 2 + 7 * 6 / 2);
  poetx_plan_destroy(p);
  poetx_plan_destroy(nullptr);
}

void plan_rejects() {
  poetx_plan* p = nullptr;
  EXPECT(poetx_plan_create(nullptr, &p) == POETX_ERR_INVALID_ARG);
  Desc a(512, 256, {256, 256}, {256}, 4, POETX_BF16);
  EXPECT(poetx_plan_create(&a.d, nullptr) == POETX_ERR_INVALID_ARG);
  Desc sum(512, 256, {256, 255}, {256}, 4, POETX_BF16);
  EXPECT(poetx_plan_create(&sum.d, &p) == POETX_ERR_SHAPE && p == nullptr);
  Desc kbig(512, 256, {256, 256}, {256}, 33, POETX_BF16);
  EXPECT(poetx_plan_create(&kbig.d, &p) == POETX_ERR_SHAPE);
  Desc kneg(512, 256, {256, 256}, {256}, -1, POETX_BF16);
  EXPECT(poetx_plan_create(&kneg.d, &p) == POETX_ERR_SHAPE);
  Desc dt(512, 256, {256, 256}, {256}, 4, 7);
  EXPECT(poetx_plan_create(&dt.d, &p) == POETX_ERR_DTYPE);
  Desc zero(512, 256, {256, 0, 256}, {256}, 4, POETX_BF16);
  EXPECT(poetx_plan_create(&zero.d, &p) != POETX_OK);
  Desc nul(512, 256, {256, 256}, {256}, 4, POETX_BF16);
  nul.d.bsz_R = nullptr;
  EXPECT(poetx_plan_create(&nul.d, &p) == POETX_ERR_INVALID_ARG);
  Desc neg(-4, 256, {256, 256}, {256}, 4, POETX_BF16);
  EXPECT(poetx_plan_create(&neg.d, &p) != POETX_OK);
  for (int field = 0; field < 5; ++field) {
    Desc e(512, 256, {256, 256}, {256}, 4, POETX_BF16);
    int32_t* f[5] = {&e.d.weight, &e.d.cayley, &e.d.fold, &e.d.index, &e.d.series};
    *f[field] = 9;
    EXPECT(poetx_plan_create(&e.d, &p) == POETX_ERR_INVALID_ARG);
    *f[field] = -1;
    EXPECT(poetx_plan_create(&e.d, &p) == POETX_ERR_INVALID_ARG);
  }
}

void compute_calls() {
  Desc a(512, 256, {256, 256}, {128, 128}, 4, POETX_BF16);
  poetx_plan* p = nullptr;
  EXPECT(poetx_plan_create(&a.d, &p) == POETX_OK);
  const int64_t T = 300;
  const size_t wf = poetx_workspace_size(p, T, POETX_WS_FORWARD);
  const size_t wb = poetx_workspace_size(p, T, POETX_WS_BACKWARD);
  const size_t wbu = poetx_workspace_size(p, 0, POETX_WS_BUILD);
  const size_t wg = poetx_workspace_size(p, 0, POETX_WS_PARAM_GRAD);
  const size_t wm = poetx_workspace_size(p, 0, POETX_WS_MERGE);
  const int32_t* pi = static_cast<const int32_t*>(dev(9));
  const float* th = static_cast<const float*>(dev(10));

  // forward: T = 0 is a no-op; each other call has exactly one bad argument
  EXPECT(poetx_forward(p, 0, dev(1), dev(2), pi, pi, dev(3), dev(4), dev(5), nullptr, nullptr, dev(6),
                       wf, nullptr) == POETX_OK);
  EXPECT(poetx_forward(nullptr, T, dev(1), dev(2), pi, pi, dev(3), dev(4), dev(5), nullptr, nullptr,
                       dev(6), wf, nullptr) == POETX_ERR_INVALID_ARG);
  EXPECT(poetx_forward(p, -1, dev(1), dev(2), pi, pi, dev(3), dev(4), dev(5), nullptr, nullptr, dev(6),
                       wf, nullptr) == POETX_ERR_INVALID_ARG);
  EXPECT(poetx_forward(p, T, nullptr, dev(2), pi, pi, dev(3), dev(4), dev(5), nullptr, nullptr, dev(6),
                       wf, nullptr) == POETX_ERR_INVALID_ARG);
  EXPECT(poetx_forward(p, T, dev(1), dev(2), pi, pi, dev(3), dev(4), mis(5), nullptr, nullptr, dev(6),
                       wf, nullptr) == POETX_ERR_ALIGNMENT);
  EXPECT(poetx_forward(p, T, dev(1), dev(2), pi, pi, dev(3), dev(4), dev(5), nullptr, nullptr, dev(6),
                       wf - 1, nullptr) == POETX_ERR_WORKSPACE);
  EXPECT(poetx_forward(p, T, dev(1), dev(2), pi, pi, dev(3), dev(4), dev(5), nullptr, nullptr, nullptr,
                       wf, nullptr) == POETX_ERR_WORKSPACE);
  EXPECT(poetx_forward_noalloc(p, T, dev(1), dev(2), pi, pi, dev(3), dev(4), mis(5), nullptr, nullptr,
                               nullptr) == POETX_ERR_ALIGNMENT);
  EXPECT(poetx_forward_noalloc(p, (int64_t)1 << 30, dev(1), dev(2), pi, pi, dev(3), dev(4), dev(5),
                               nullptr, nullptr, nullptr) == POETX_ERR_WORKSPACE);
  EXPECT(poetx_forward_noalloc_max_bytes() == (size_t)64 << 20);

  // backward
  float* g = static_cast<float*>(dev(11));
  EXPECT(poetx_backward(p, T, dev(1), dev(2), pi, pi, th, th, dev(3), dev(4), dev(5), nullptr, dev(7),
                        dev(8), g, g, dev(6), wb - 1, nullptr) == POETX_ERR_WORKSPACE);
  EXPECT(poetx_backward(p, T, dev(1), dev(2), pi, pi, nullptr, th, dev(3), dev(4), dev(5), nullptr,
                        dev(7), dev(8), g, g, dev(6), wb, nullptr) == POETX_ERR_INVALID_ARG);
  EXPECT(poetx_backward(p, T, dev(1), dev(2), pi, pi, th, th, dev(3), dev(4), dev(5), nullptr, dev(7),
                        mis(8), g, g, dev(6), wb, nullptr) == POETX_ERR_ALIGNMENT);
  EXPECT(poetx_backward_dq(p, T, dev(1), dev(2), pi, pi, dev(3), dev(4), dev(5), nullptr, nullptr,
                           dev(8), g, g, dev(6), wb, nullptr) == POETX_ERR_INVALID_ARG);
  EXPECT(poetx_backward_dq(nullptr, T, dev(1), dev(2), pi, pi, dev(3), dev(4), dev(5), nullptr, dev(7),
                           dev(8), g, g, dev(6), wb, nullptr) == POETX_ERR_INVALID_ARG);

  // build and the batched calls
  EXPECT(poetx_build_orth(p, 3, th, g, dev(3), dev(6), wbu, nullptr) == POETX_ERR_INVALID_ARG);
  EXPECT(poetx_build_orth(p, 0, th, g, dev(3), dev(6), wbu - 1, nullptr) == POETX_ERR_WORKSPACE);
  EXPECT(poetx_build_orth(p, 0, reinterpret_cast<const float*>(mis(10)), g, dev(3), dev(6), wbu,
                          nullptr) == POETX_ERR_ALIGNMENT);
  const poetx_plan* plans[2] = {p, nullptr};
  const int32_t sides[2] = {0, 1};
  const float* ths[2] = {th, th};
  float* qs[2] = {g, g};
  void* qa[2] = {dev(3), dev(4)};
  void* ws[2] = {dev(6), dev(7)};
  const size_t wsb[2] = {wbu, wbu};
  EXPECT(poetx_build_orth_batch(0, plans, sides, ths, qs, qa, ws, wsb, nullptr) == POETX_OK);
  EXPECT(poetx_build_orth_batch(-1, plans, sides, ths, qs, qa, ws, wsb, nullptr) == POETX_ERR_INVALID_ARG);
  EXPECT(poetx_build_orth_batch(2, plans, sides, ths, qs, qa, ws, wsb, nullptr) == POETX_ERR_INVALID_ARG);
  EXPECT(poetx_build_orth_batch(1, nullptr, sides, ths, qs, qa, ws, wsb, nullptr) == POETX_ERR_INVALID_ARG);
  const float* dqs[2] = {g, g};
  float* gts[2] = {g, g};
  const size_t wgb[2] = {wg - 1, wg};
  const size_t wgok[2] = {wg, wg};
  EXPECT(poetx_param_grad_batch(1, plans, sides, ths, dqs, gts, ws, wgb, nullptr) == POETX_ERR_WORKSPACE);
  EXPECT(poetx_param_grad_batch(2, plans, sides, ths, dqs, gts, ws, wgok, nullptr) == POETX_ERR_INVALID_ARG);

  // weight set-up, merge, index helpers
  EXPECT(poetx_permute_weight(p, dev(1), pi, pi, mis(2), nullptr) == POETX_ERR_ALIGNMENT);
  EXPECT(poetx_permute_weight(nullptr, dev(1), pi, pi, dev(2), nullptr) == POETX_ERR_INVALID_ARG);
  EXPECT(poetx_quantize_weight(p, dev(1), pi, pi, dev(2), nullptr) == POETX_ERR_UNSUPPORTED);
  EXPECT(poetx_merge_weight(p, dev(1), pi, pi, g, g, dev(2), dev(6), wm - 1, nullptr) == POETX_ERR_WORKSPACE);
  EXPECT(poetx_merge_weight(p, nullptr, pi, pi, g, g, dev(2), dev(6), wm, nullptr) == POETX_ERR_INVALID_ARG);
  EXPECT(poetx_gather_cols(p, 0, 5, dev(1), pi, dev(2), nullptr) == POETX_OK);
  EXPECT(poetx_gather_cols(p, 3, 5, dev(1), pi, dev(1), nullptr) == POETX_ERR_INVALID_ARG);   // in place
  EXPECT(poetx_gather_cols(p, 3, 5, dev(1), pi, nullptr, nullptr) == POETX_ERR_INVALID_ARG);
  EXPECT(poetx_scatter_cols(p, 3, 256, dev(1), pi, mis(2), nullptr) == POETX_ERR_ALIGNMENT);
  EXPECT(poetx_scatter_cols(p, -3, 256, dev(1), pi, dev(2), nullptr) == POETX_ERR_INVALID_ARG);
  poetx_plan_destroy(p);
}

void status_and_timing() {
  for (int s = -2; s < 12; ++s) {
    const char* t = poetx_status_string(static_cast<poetx_status>(s));
    EXPECT(t != nullptr && std::strlen(t) > 0);
  }
  EXPECT(poetx_last_hip_error() != nullptr);
  double ms = 0.0;
  int64_t cnt = 0;
  EXPECT(poetx_timing_read(-1, &ms, &cnt) == POETX_ERR_INVALID_ARG);
  EXPECT(poetx_timing_read(POETX_NUM_STAGES, &ms, &cnt) == POETX_ERR_INVALID_ARG);
  EXPECT(poetx_timing_read(0, nullptr, &cnt) == POETX_ERR_INVALID_ARG);
  EXPECT(poetx_timing_enable(1u << POETX_NUM_STAGES) == POETX_OK);   // bits past the stages ignored
  EXPECT(poetx_timing_enable(0) == POETX_OK);
  poetx_timing_reset();
}

}  // namespace

int main() {
  // The fake device addresses must never reach a kernel: run only where no
  // GPU is visible (every call below is meant to stop in validation, and this
  // guard keeps a mistake in that from touching a device).
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0) {
    std::printf("skipped: a GPU is visible\n");
    return 77;
  }
  plan_options();
  plan_rejects();
  compute_calls();
  status_and_timing();
  std::printf("%s (%d failed checks)\n", failures ? "FAIL" : "OK", failures);
  return failures ? 1 : 0;
}
