// abi_example.cpp -- the C ABI used from C++ without Python: a warm-up with
// the variance norm, the freeze, then compression steps in the deferred
// layout with the implicit momentum, checked against the CPU oracle
// (teacher-forced per step: packed words bit for bit, floats within
// 1e-6 + 1e-5 |ref|).  Exit status 0 when everything matches.
//
// Build (test suite): hipcc abi_example.cpp -I include -I oracle -L <lib dirs> -loba -loracle
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "oba.h"
#include "oracle.h"

#define CHECK_OBA(call)                                                         \
  do {                                                                          \
    int rc_ = (call);                                                           \
    if (rc_ != OBA_OK) {                                                        \
      std::fprintf(stderr, "%s failed: %s\n", #call, oba_status_string(rc_));   \
      return 2;                                                                 \
    }                                                                           \
  } while (0)
#define CHECK_HIP(call)                                                         \
  do {                                                                          \
    hipError_t e_ = (call);                                                     \
    if (e_ != hipSuccess) {                                                     \
      std::fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));    \
      return 3;                                                                 \
    }                                                                           \
  } while (0)

template <class T>
static T* dev_alloc(size_t n) {
  void* p = nullptr;
  if (hipMalloc(&p, n * sizeof(T) + 16) != hipSuccess) return nullptr;
  return static_cast<T*>(p);
}

static int close_enough(const float* a, const float* b, size_t n, const char* what) {
  for (size_t k = 0; k < n; ++k) {
    const double r = b[k];
    if (!(std::fabs((double)a[k] - r) <= 1e-6 + 1e-5 * std::fabs(r))) {
      std::fprintf(stderr, "%s differs at %zu: %.9g vs %.9g\n", what, k, a[k], b[k]);
      return 0;
    }
  }
  return 1;
}

int main() {
  const int64_t d = 100003, ld = (d + 7) / 8 * 8, W = (d + 63) / 64;
  const int32_t n = 4;
  const double b1 = 0.9, b2 = 0.999, eta = 1e-8, lr = 1e-3;
  std::vector<int64_t> wseg = {0, d}, sseg(n + 1);
  for (int j = 0; j <= n; ++j) sseg[j] = j * d / n;

  oba_layout L = nullptr;
  CHECK_OBA(oba_layout_create(&L, d, n, ld, wseg.data(), 1, sseg.data(), n));
  const size_t ws_bytes = oba_workspace_bytes(L);

  float *g = dev_alloc<float>(n * ld), *x = dev_alloc<float>(d), *m = dev_alloc<float>(d);
  float *v = dev_alloc<float>(d), *den = dev_alloc<float>(d), *c = dev_alloc<float>(n * ld);
  float *a = dev_alloc<float>(d), *wsc = dev_alloc<float>(n), *ssc = dev_alloc<float>(n);
  uint64_t *wb = dev_alloc<uint64_t>(n * W), *sb = dev_alloc<uint64_t>(W);
  double* vn = dev_alloc<double>(1);
  void* ws = dev_alloc<char>(ws_bytes);
  if (!g || !x || !m || !v || !den || !c || !a || !wsc || !ssc || !wb || !sb || !vn || !ws) return 4;

  // host state and the oracle's copy
  std::mt19937_64 rng(5);
  std::normal_distribution<float> N01(0.0f, 1.0f);
  std::vector<float> hx(d), hm(d, 0.0f), hv(d, 0.0f), hg(n * ld, 0.0f);
  for (auto& e : hx) e = 0.02f * N01(rng);
  CHECK_HIP(hipMemcpy(x, hx.data(), d * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemset(m, 0, d * 4));
  CHECK_HIP(hipMemset(v, 0, d * 4));
  hipStream_t st = nullptr;

  // warm-up with the variance norm
  for (int t = 0; t < 3; ++t) {
    for (int32_t i = 0; i < n; ++i)
      for (int64_t k = 0; k < d; ++k) hg[i * ld + k] = 1e-2f * N01(rng);
    CHECK_HIP(hipMemcpy(g, hg.data(), n * ld * 4, hipMemcpyHostToDevice));
    CHECK_OBA(oba_adam_warmup_step_vnorm(L, g, OBA_F32, x, m, v, lr, b1, b2, eta, 1.0, 1.0, vn, ws,
                                         ws_bytes, st));
    oracle_adam_warmup_step(d, n, ld, hg.data(), 0, hx.data(), hm.data(), hv.data(), lr, b1, b2,
                            eta, 1.0, 1.0);
    double gvn = 0.0;
    CHECK_HIP(hipMemcpy(&gvn, vn, 8, hipMemcpyDeviceToHost));
    const double ovn = oracle_l2norm(d, hv.data());
    if (std::fabs(gvn - ovn) > 1e-5 * ovn) {
      std::fprintf(stderr, "variance norm %.17g vs %.17g\n", gvn, ovn);
      return 1;
    }
  }
  // freeze: denom from v; c, a and the scales start at zero
  CHECK_OBA(oba_freeze_variance(L, v, den, eta, 1.0, st));
  std::vector<float> hden(d), hdelta(n * ld, 0.0f), heps(d, 0.0f);
  oracle_freeze_variance(d, hv.data(), hden.data(), eta, 1.0);
  CHECK_HIP(hipMemset(c, 0, n * ld * 4));
  CHECK_HIP(hipMemset(a, 0, d * 4));
  CHECK_HIP(hipMemset(wsc, 0, n * 4));
  CHECK_HIP(hipMemset(ssc, 0, n * 4));

  std::vector<uint64_t> owb(n * W), osb(W), gwb(n * W), gsb(W);
  std::vector<float> owsc(n), ossc(n), gx(d);
  for (int t = 0; t < 4; ++t) {
    for (int32_t i = 0; i < n; ++i)
      for (int64_t k = 0; k < d; ++k) hg[i * ld + k] = 1e-2f * N01(rng);
    CHECK_HIP(hipMemcpy(g, hg.data(), n * ld * 4, hipMemcpyHostToDevice));
    if (t == 0)  // the first step reads the warm-up's m
      CHECK_OBA(oba_compress_deferred(L, g, OBA_F32, m, nullptr, nullptr, c, wb, wsc, b1, ws,
                                      ws_bytes, st));
    else  // later ones rebuild m from the last server message
      CHECK_OBA(oba_compress_deferred(L, g, OBA_F32, nullptr, sb, ssc, c, wb, wsc, b1, ws,
                                      ws_bytes, st));
    CHECK_OBA(oba_server_reduce_recompress_deferred(L, wb, wsc, a, sb, ssc, ws, ws_bytes, st));
    CHECK_OBA(oba_decompress_update(L, sb, ssc, den, nullptr, x, lr, st));
    // the oracle's step on its own state
    oracle_compress(d, n, ld, wseg.data(), 1, hg.data(), 0, hm.data(), hdelta.data(), owb.data(),
                    owsc.data(), b1);
    oracle_server_reduce_recompress(d, n, wseg.data(), 1, sseg.data(), n, owb.data(), owsc.data(),
                                    heps.data(), osb.data(), ossc.data());
    oracle_decompress_update(0, d, sseg.data(), n, osb.data(), ossc.data(), hden.data(),
                             hm.data(), hx.data(), lr);
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(gwb.data(), wb, n * W * 8, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(gsb.data(), sb, W * 8, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(gx.data(), x, d * 4, hipMemcpyDeviceToHost));
    std::vector<float> gwsc(n), gssc(n);
    CHECK_HIP(hipMemcpy(gwsc.data(), wsc, n * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(gssc.data(), ssc, n * 4, hipMemcpyDeviceToHost));
    if (std::memcmp(gwb.data(), owb.data(), n * W * 8) || std::memcmp(gsb.data(), osb.data(), W * 8)) {
      std::fprintf(stderr, "packed words differ at step %d\n", t);
      return 1;
    }
    if (!close_enough(gwsc.data(), owsc.data(), n, "worker scales") ||
        !close_enough(gssc.data(), ossc.data(), n, "server scales") ||
        !close_enough(gx.data(), hx.data(), d, "x"))
      return 1;
    // teacher forcing: continue both from the oracle's x
    CHECK_HIP(hipMemcpy(x, hx.data(), d * 4, hipMemcpyHostToDevice));
  }
  // the materialised momentum is the oracle's m
  CHECK_OBA(oba_server_momentum(L, sb, ssc, m, st));
  CHECK_HIP(hipDeviceSynchronize());
  std::vector<float> gm(d);
  CHECK_HIP(hipMemcpy(gm.data(), m, d * 4, hipMemcpyDeviceToHost));
  if (!close_enough(gm.data(), hm.data(), d, "momentum")) return 1;
  oba_layout_destroy(L);
  for (void* p : {(void*)g, (void*)x, (void*)m, (void*)v, (void*)den, (void*)c, (void*)a,
                  (void*)wsc, (void*)ssc, (void*)wb, (void*)sb, (void*)vn, ws})
    (void)hipFree(p);
  std::printf("abi_example: ok\n");
  return 0;
}
