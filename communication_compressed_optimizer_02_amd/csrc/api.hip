// api.hip -- the C ABI declared in include/oba.h: argument checks on the
// host, layout handles, kernel launches on the caller's stream, and the
// optional per-kernel event timing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <atomic>
#include <mutex>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "kernels.hpp"
#include "layout.hpp"
#include "oba.h"

// Grid of the 16-bit-state worker pass: 1 = the server grid (four spans or
// more per block), 0 = the compress grid (one span per block for n >= 4).  A
// span of 16-bit rows carries less data per block, so longer blocks amortise
// the block's set-up (bert_large: 3.53 -> 3.20 ms); a tuning knob.
#ifndef OBA_S16_GRID
#define OBA_S16_GRID 1
#endif
// Grid of the warm-up step: 1 = the update grid (one span per block), 0 = the
// server grid; a tuning knob.
#ifndef OBA_WARM_SPAN1
#define OBA_WARM_SPAN1 1
#endif
#ifndef OBA_WARM_SPAN1_TL
#define OBA_WARM_SPAN1_TL OBA_WARM_SPAN1
#endif

struct oba_layout_s {
  oba::Plan plan;
  int device = -1;
  uint64_t serial = 0;  // unique per handle made by this process (never reused)
  void* dev_tables = nullptr;
  oba::SegDev sig_c{};  // worker segments, compress grid
  oba::SegDev sig{};    // worker segments, server grid
  oba::SegDev tau{};    // server segments, server grid
  oba::SegDev tau_w{};  // server segments, update grid
  oba::SegDev tau_c{};  // server segments, compress grid (implicit momentum)
  oba::Geo geo_w{};     // update grid (one span per block)
  oba::Geo geo_c{};     // compress grid (deferred worker passes)
  oba::Geo geo_e{};     // explicit grid (explicit apply, per-worker momentum)
  oba::SegDev sig_e{};  // worker segments, explicit grid
  oba::Geo geo{};       // server grid
  size_t ws_worker = 0, ws_server = 0;
};

struct oba_tensors_s {
  int device = -1;
  int g_dtype = OBA_F32;
  int32_t T = 0;
  int32_t n = 0;
  // the layout the block tables were built for: its serial, d and grids
  uint64_t layout_serial = 0;
  int64_t d = 0;
  int32_t nblk_c = 0, nblk_w = 0, nblk = 0;
  void* dev = nullptr;  // one allocation holding every table below
  oba::TList tl_c{};    // block table of the compress grid
  oba::TList tl_w{};    // block table of the update grid
  oba::TList tl_s{};    // block table of the server grid
};

// The fixed device scratch of oba_compress_deferred_noalloc (see below).
static_assert(OBA_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) double scratch[OBA_NOALLOC_SCRATCH_BYTES / sizeof(double)];

namespace {

thread_local char g_hip_msg[256] = "HIP error";
std::atomic<uint64_t> g_layout_serial{0};

int hip_fail(hipError_t e, const char* what) {
  std::snprintf(g_hip_msg, sizeof(g_hip_msg), "HIP error in %s: %s", what, hipGetErrorString(e));
  return OBA_EHIP;
}

// ---- timing -------------------------------------------------------------
struct TimingRec {
  const char* name;
  hipEvent_t a, b;
};
std::mutex g_tmu;
bool g_timing = false;
std::vector<hipEvent_t> g_pool;  // free events
std::vector<TimingRec> g_recs;

void timing_drop_all() {
  for (auto& r : g_recs) {
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.clear();
}

// Launch `fn` on `st`, bracketed by timing events when enabled; check launch.
template <class F>
int launch(const char* name, hipStream_t st, F&& fn) {
  hipEvent_t a = nullptr, b = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_tmu);
    if (g_timing && g_pool.size() >= 2) {
      a = g_pool.back();
      g_pool.pop_back();
      b = g_pool.back();
      g_pool.pop_back();
    }
  }
  if (a && hipEventRecord(a, st) != hipSuccess) a = nullptr;
  fn();
  hipError_t e = hipGetLastError();
  if (a) {
    if (hipEventRecord(b, st) == hipSuccess) {
      std::lock_guard<std::mutex> lk(g_tmu);
      g_recs.push_back({name, a, b});
    } else {
      std::lock_guard<std::mutex> lk(g_tmu);
      g_pool.push_back(a);
      g_pool.push_back(b);
    }
  } else if (b) {
    std::lock_guard<std::mutex> lk(g_tmu);
    g_pool.push_back(b);
  }
  if (e != hipSuccess) return hip_fail(e, name);
  return OBA_OK;
}

// ---- fixed device scratch (oba_compress_deferred_noalloc) -----------------
// The binary64 partial sums of the worker pass, for callers that cannot
// allocate.  Each GPU holds its own copy of the array until the process ends.
// Host code never uses the array's name as an address: the device address of
// each GPU's copy is looked up once per device, when the first layout is
// created on it, and kept below.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (device `dev` must be current).
int scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return OBA_EINVAL;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress (scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return OBA_OK;
}

// ---- argument checks ------------------------------------------------------
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int check_layout(oba_layout L) {
  if (!L) return OBA_EINVAL;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != L->device) return OBA_EINVAL;
  return OBA_OK;
}

int check_buf(const void* p, uintptr_t align) {
  if (!p) return OBA_EINVAL;
  if (!aligned(p, align)) return OBA_EALIGN;
  return OBA_OK;
}

// A tensor-list handle is valid only with the layout it was built for: its
// per-block tables index that layout's grids.
int check_tensors(oba_layout L, oba_tensors H) {
  if (!H || H->device != L->device || H->layout_serial != L->serial || H->n != L->plan.n ||
      H->d != L->plan.d || H->nblk_c != L->plan.nblk_c || H->nblk_w != L->plan.nblk_w ||
      H->nblk != L->plan.nblk)
    return OBA_EINVAL;
  return OBA_OK;
}

bool is_finite(double x) { return std::isfinite(x); }
bool gdtype_ok(int t) { return t == OBA_F32 || t == OBA_F16 || t == OBA_BF16; }
bool beta_ok(double b) { return is_finite(b) && b >= 0.0 && b < 1.0; }

#define OBA_TRY(expr)          \
  do {                         \
    int rc_ = (expr);          \
    if (rc_ != OBA_OK) return rc_; \
  } while (0)

}  // namespace

extern "C" {

int oba_version(void) { return 100; }

const char* oba_status_string(int status) {
  switch (status) {
    case OBA_OK: return "ok";
    case OBA_EINVAL: return "invalid argument (null pointer, size, dtype, device or hyperparameter)";
    case OBA_EALIGN: return "buffer misaligned (16 B for float/half, 8 B for packed words and workspace, 4 B for scales)";
    case OBA_ESEG: return "segment table must rise strictly from 0 to d";
    case OBA_EWORKSPACE: return "workspace smaller than oba_workspace_bytes()";
    case OBA_EHIP: return g_hip_msg;
    case OBA_ENOMEM: return "allocation failed";
    case OBA_ESCRATCH:
      return "the layout needs more than the fixed device scratch of "
             "oba_compress_deferred_noalloc (OBA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int oba_layout_validate(int64_t d, int32_t n, int64_t ld, const int64_t* wseg, int32_t n_wseg,
                        const int64_t* sseg, int32_t n_sseg) {
  return oba::validate(d, n, ld, wseg, n_wseg, sseg, n_sseg);
}

int oba_layout_create(oba_layout* out, int64_t d, int32_t n, int64_t ld, const int64_t* wseg,
                      int32_t n_wseg, const int64_t* sseg, int32_t n_sseg) {
  if (!out) return OBA_EINVAL;
  oba_layout_s* L = new (std::nothrow) oba_layout_s();
  if (!L) return OBA_ENOMEM;
  int rc = oba::make_plan(d, n, ld, wseg, n_wseg, sseg, n_sseg, &L->plan);
  if (rc) {
    delete L;
    return rc;
  }
  const oba::Plan& P = L->plan;
  L->serial = ++g_layout_serial;
  hipError_t e = hipGetDevice(&L->device);
  if (e != hipSuccess) {
    delete L;
    return hip_fail(e, "hipGetDevice");
  }
  {  // set-up of this device's fixed scratch (once per device)
    void* sp = nullptr;
    rc = scratch_on(L->device, &sp);
    if (rc) {
      delete L;
      return rc;
    }
  }
  // one device allocation: int64 arrays first, then int32 arrays
  std::vector<int64_t> h64;
  std::vector<int32_t> h32;
  auto put = [&](const oba::Pieces& pc, const std::vector<int64_t>& off, size_t o64[2],
                 size_t o32[5]) {
    o64[0] = h64.size();
    h64.insert(h64.end(), off.begin(), off.end());
    o64[1] = h64.size();
    h64.insert(h64.end(), pc.hi.begin(), pc.hi.end());
    o32[0] = h32.size();
    h32.insert(h32.end(), pc.seg.begin(), pc.seg.end());
    o32[1] = h32.size();
    h32.insert(h32.end(), pc.blk_first.begin(), pc.blk_first.end());
    o32[2] = h32.size();
    h32.insert(h32.end(), pc.seg_first.begin(), pc.seg_first.end());
    o32[3] = h32.size();
    h32.insert(h32.end(), pc.item_q.begin(), pc.item_q.end());
    o32[4] = h32.size();
    h32.insert(h32.end(), pc.seg_item.begin(), pc.seg_item.end());
  };
  size_t w64[2], w32[5], v64[2], v32[5], s64[2], s32[5], t64[2], t32[5], c64[2], c32[5],
      e64[2], e32[5];
  try {
    put(P.wp, P.wseg, w64, w32);
    put(P.wp_s, P.wseg, v64, v32);
    put(P.sp, P.sseg, s64, s32);
    put(P.sp_w, P.sseg, t64, t32);
    put(P.sp_c, P.sseg, c64, c32);
    put(P.wp_e, P.wseg, e64, e32);
  } catch (...) {
    delete L;
    return OBA_ENOMEM;
  }
  const size_t bytes64 = h64.size() * sizeof(int64_t);
  const size_t bytes = bytes64 + h32.size() * sizeof(int32_t);
  if (bytes) {
    e = hipMalloc(&L->dev_tables, bytes);
    if (e != hipSuccess) {
      delete L;
      return OBA_ENOMEM;
    }
    e = hipMemcpy(L->dev_tables, h64.data(), bytes64, hipMemcpyHostToDevice);
    if (e == hipSuccess && !h32.empty())
      e = hipMemcpy(static_cast<char*>(L->dev_tables) + bytes64, h32.data(),
                    h32.size() * sizeof(int32_t), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      (void)hipFree(L->dev_tables);
      delete L;
      return hip_fail(e, "hipMemcpy (layout tables)");
    }
  }
  const int64_t* d64 = static_cast<const int64_t*>(L->dev_tables);
  const int32_t* d32 = reinterpret_cast<const int32_t*>(static_cast<const char*>(L->dev_tables) + bytes64);
  auto view = [&](const oba::Pieces& pc, size_t o64[2], size_t o32[5], int32_t n_seg) {
    oba::SegDev s;
    s.off = d64 + o64[0];
    s.phi = d64 + o64[1];
    s.pseg = d32 + o32[0];
    s.blk_first = d32 + o32[1];
    s.seg_first = d32 + o32[2];
    s.item_q = pc.item_q.empty() ? nullptr : d32 + o32[3];
    s.seg_item = pc.item_q.empty() ? nullptr : d32 + o32[4];
    s.n_seg = n_seg;
    s.n_pieces = (int32_t)pc.lo.size();
    s.n_items = pc.item_q.empty() ? 0 : (int32_t)pc.item_q.size() - 1;
    return s;
  };
  L->sig_c = view(P.wp, w64, w32, (int32_t)P.wseg.size() - 1);
  L->sig = view(P.wp_s, v64, v32, (int32_t)P.wseg.size() - 1);
  L->tau = view(P.sp, s64, s32, (int32_t)P.sseg.size() - 1);
  L->tau_w = view(P.sp_w, t64, t32, (int32_t)P.sseg.size() - 1);
  L->tau_c = view(P.sp_c, c64, c32, (int32_t)P.sseg.size() - 1);
  L->sig_e = view(P.wp_e, e64, e32, (int32_t)P.wseg.size() - 1);
  auto geo = [&](int32_t nblk) {  // an empty layout has no blocks
    return oba::Geo{P.d, P.ld, P.W, P.S, P.n, nblk, nblk ? P.S / nblk : 0,
                    nblk ? (int32_t)(P.S % nblk) : 0};
  };
  L->geo_w = geo(P.nblk_w);
  L->geo_c = geo(P.nblk_c);
  L->geo_e = geo(P.nblk_e);
  L->geo = geo(P.nblk);
  L->ws_worker = std::max({oba::partial_bytes(L->sig_c, P.n), oba::partial_bytes(L->sig, P.n),
                           oba::partial_bytes(L->sig_e, P.n),
                           ((size_t)std::max(P.nblk_w, P.nblk) * 8 + 255) / 256 * 256});
  L->ws_server = std::max(oba::partial_bytes(L->tau, 1), oba::partial_bytes(L->tau_c, 1));
  *out = L;
  return OBA_OK;
}

void oba_layout_destroy(oba_layout L) {
  if (!L) return;
  if (L->dev_tables) {
    (void)hipDeviceSynchronize();
    (void)hipFree(L->dev_tables);
  }
  delete L;
}

size_t oba_workspace_bytes(oba_layout L) {
  if (!L) return 0;
  return ((L->ws_worker + 255) / 256) * 256 + L->ws_server;
}

}  // extern "C"

namespace {

int warmup(oba_layout L, const void* g, int g_dtype, float* x, float* m, float* v, double lr,
           double beta1, double beta2, double eta, double bc1, double bc2, double* vnorm,
           void* ws, size_t ws_bytes, hipStream_t stream) {
  OBA_TRY(check_layout(L));
  if (!gdtype_ok(g_dtype)) return OBA_EINVAL;
  if (!is_finite(lr) || !beta_ok(beta1) || !beta_ok(beta2) || !is_finite(eta) || eta < 0.0 ||
      !is_finite(bc1) || bc1 <= 0.0 || !is_finite(bc2) || bc2 <= 0.0)
    return OBA_EINVAL;
  if (vnorm) OBA_TRY(check_buf(vnorm, 8));
  if (L->geo.d == 0) {  // the norm of an empty vector is 0
    if (!vnorm) return OBA_OK;
    return launch("adam_warmup", stream,
                  [&] { oba::launch_norm_finalize(nullptr, 0, vnorm, stream); });
  }
  if (vnorm) {
    OBA_TRY(check_buf(ws, 8));
    if (ws_bytes < oba_workspace_bytes(L)) return OBA_EWORKSPACE;
  }
  OBA_TRY(check_buf(g, 16));
  OBA_TRY(check_buf(x, 16));
  OBA_TRY(check_buf(m, 16));
  OBA_TRY(check_buf(v, 16));
  oba::AdamCoef C{(float)lr, (float)beta1, (float)(1.0 - beta1), (float)beta2,
                  (float)(1.0 - beta2), (float)eta, (float)bc1, (float)bc2};
  // one span per block (the update grid) with two resident blocks per CU:
  // 2.51 -> 2.31 ms at bert_large (same-box A/B; the server grid's four spans
  // per block with the same cap, 2.51 ms)
  const oba::Geo G = OBA_WARM_SPAN1 ? L->geo_w : L->geo;
  // one binary64 partial per block of G: the worker part of the workspace is
  // sized for them
  double* part = static_cast<double*>(ws);
  return launch("adam_warmup", stream, [&] {
    oba::launch_adam_warmup(G, g, g_dtype, x, m, v, C, part, vnorm, stream);
  });
}

}  // namespace

extern "C" {

int oba_adam_warmup_step(oba_layout L, const void* g, int g_dtype, float* x, float* m, float* v,
                         double lr, double beta1, double beta2, double eta, double bc1,
                         double bc2, hipStream_t stream) {
  return warmup(L, g, g_dtype, x, m, v, lr, beta1, beta2, eta, bc1, bc2, nullptr, nullptr, 0,
                stream);
}

int oba_adam_warmup_step_vnorm(oba_layout L, const void* g, int g_dtype, float* x, float* m,
                               float* v, double lr, double beta1, double beta2, double eta,
                               double bc1, double bc2, double* vnorm, void* ws, size_t ws_bytes,
                               hipStream_t stream) {
  if (!vnorm) return OBA_EINVAL;
  return warmup(L, g, g_dtype, x, m, v, lr, beta1, beta2, eta, bc1, bc2, vnorm, ws, ws_bytes,
                stream);
}

int oba_freeze_variance(oba_layout L, const float* v, float* denom, double eta, double bc2,
                        hipStream_t stream) {
  OBA_TRY(check_layout(L));
  if (!is_finite(eta) || eta < 0.0 || !is_finite(bc2) || bc2 <= 0.0) return OBA_EINVAL;
  if (L->geo.d == 0) return OBA_OK;
  OBA_TRY(check_buf(v, 16));
  OBA_TRY(check_buf(denom, 16));
  if ((const void*)v == (const void*)denom) return OBA_EINVAL;
  const oba::Geo G = L->geo;
  return launch("freeze_variance", stream,
                [&] { oba::launch_freeze(G, v, denom, (float)eta, (float)bc2, stream); });
}

int oba_compress(oba_layout L, const void* g, int g_dtype, const float* m, float* delta,
                 uint64_t* wbits, float* wscale, double beta1, void* ws, size_t ws_bytes,
                 hipStream_t stream) {
  OBA_TRY(check_layout(L));
  if (!gdtype_ok(g_dtype)) return OBA_EINVAL;
  if (!beta_ok(beta1)) return OBA_EINVAL;
  if (L->geo.d == 0) return OBA_OK;
  OBA_TRY(check_buf(g, 16));
  OBA_TRY(check_buf(m, 16));
  OBA_TRY(check_buf(delta, 16));
  OBA_TRY(check_buf(wbits, 8));
  OBA_TRY(check_buf(wscale, 4));
  OBA_TRY(check_buf(ws, 8));
  if (ws_bytes < oba_workspace_bytes(L)) return OBA_EWORKSPACE;
  const oba::Geo G = L->geo_e;
  double* part = static_cast<double*>(ws);
  const float b1 = (float)beta1, omb1 = (float)(1.0 - beta1);
  uint8_t* wbytes = reinterpret_cast<uint8_t*>(wbits);
  // the read-only norm pass runs on the server grid (a few spans per block:
  // its per-block reduction would dominate at one span per block)
  OBA_TRY(launch("compress_p1", stream, [&] {
    oba::launch_compress_norm(L->geo, g, g_dtype, m, delta, L->sig, part, b1, omb1,
                              stream);
  }));
  OBA_TRY(launch("finalize_scales", stream,
                 [&] { oba::launch_finalize(part, G.n, L->sig, wscale, stream); }));
  return launch("compress_p2", stream, [&] {
    oba::launch_compress_apply(G, g, g_dtype, m, delta, wbytes, L->sig_e, wscale, b1,
                               omb1, stream);
  });
}

int oba_server_reduce_recompress(oba_layout L, const uint64_t* wbits, const float* wscale,
                                 float* eps, uint64_t* sbits, float* sscale, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
  OBA_TRY(check_layout(L));
  if (L->geo.d == 0) return OBA_OK;
  OBA_TRY(check_buf(wbits, 8));
  OBA_TRY(check_buf(wscale, 4));
  OBA_TRY(check_buf(eps, 16));
  OBA_TRY(check_buf(sbits, 8));
  OBA_TRY(check_buf(sscale, 4));
  OBA_TRY(check_buf(ws, 8));
  if (ws_bytes < oba_workspace_bytes(L)) return OBA_EWORKSPACE;
  const oba::Geo G = L->geo;
  double* part = reinterpret_cast<double*>(static_cast<char*>(ws) +
                                           ((L->ws_worker + 255) / 256) * 256);
  const uint8_t* wbytes = reinterpret_cast<const uint8_t*>(wbits);
  uint8_t* sbytes = reinterpret_cast<uint8_t*>(sbits);
  OBA_TRY(launch("server_p1", stream, [&] {
    oba::launch_server_p1(G, wbytes, wscale, eps, sbytes, L->sig, L->tau, part, stream);
  }));
  OBA_TRY(launch("finalize_scales", stream,
                 [&] { oba::launch_finalize(part, 1, L->tau, sscale, stream); }));
  return launch("server_p2", stream,
                [&] { oba::launch_residual(G, eps, 0, eps, 0, 1, sscale, L->tau, stream); });
}

}  // extern "C"

namespace {

// oba_compress_deferred with its binary64 partials at `part` (workspace or
// the fixed scratch), after the checks common to both entry points.
int compress_deferred_checks(oba_layout L, const void* g, int g_dtype, const float* m,
                             const uint64_t* sbits_prev, const float* sscale_prev, float* c,
                             uint64_t* wbits, float* wscale, double beta1) {
  OBA_TRY(check_layout(L));
  if (!gdtype_ok(g_dtype)) return OBA_EINVAL;
  if (!beta_ok(beta1)) return OBA_EINVAL;
  const bool implicit_m = !m;
  if (implicit_m != (sbits_prev != nullptr) || implicit_m != (sscale_prev != nullptr))
    return OBA_EINVAL;
  if (L->geo.d == 0) return OBA_OK;
  OBA_TRY(check_buf(g, 16));
  if (implicit_m) {
    OBA_TRY(check_buf(sbits_prev, 8));
    OBA_TRY(check_buf(sscale_prev, 4));
  } else {
    OBA_TRY(check_buf(m, 16));
  }
  OBA_TRY(check_buf(c, 16));
  OBA_TRY(check_buf(wbits, 8));
  OBA_TRY(check_buf(wscale, 4));
  return OBA_OK;
}

int compress_deferred_run(oba_layout L, const void* g, int g_dtype, const float* m,
                          const uint64_t* sbits_prev, const float* sscale_prev, float* c,
                          uint64_t* wbits, float* wscale, double beta1, double* part,
                          hipStream_t stream) {
  const oba::Geo G = L->geo_c;
  const float b1 = (float)beta1, omb1 = (float)(1.0 - beta1);
  uint8_t* wbytes = reinterpret_cast<uint8_t*>(wbits);
  const oba::MomSrc ms{reinterpret_cast<const uint8_t*>(sbits_prev), sscale_prev, L->tau_c};
  OBA_TRY(launch("compress_deferred", stream, [&] {
    oba::launch_compress_deferred(G, g, g_dtype, m, c, wbytes, L->sig_c, part, wscale,
                                  b1, omb1, ms, stream);
  }));
  return launch("finalize_scales", stream,
                [&] { oba::launch_finalize(part, G.n, L->sig_c, wscale, stream); });
}

}  // namespace

extern "C" {

int oba_compress_deferred(oba_layout L, const void* g, int g_dtype, const float* m,
                          const uint64_t* sbits_prev, const float* sscale_prev, float* c,
                          uint64_t* wbits, float* wscale, double beta1, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  OBA_TRY(compress_deferred_checks(L, g, g_dtype, m, sbits_prev, sscale_prev, c, wbits, wscale,
                                   beta1));
  if (L->geo.d == 0) return OBA_OK;
  OBA_TRY(check_buf(ws, 8));
  if (ws_bytes < oba_workspace_bytes(L)) return OBA_EWORKSPACE;
  return compress_deferred_run(L, g, g_dtype, m, sbits_prev, sscale_prev, c, wbits, wscale,
                               beta1, static_cast<double*>(ws), stream);
}

int oba_compress_deferred_noalloc(oba_layout L, const void* g, int g_dtype, const float* m,
                                  const uint64_t* sbits_prev, const float* sscale_prev, float* c,
                                  uint64_t* wbits, float* wscale, double beta1,
                                  hipStream_t stream) {
  OBA_TRY(check_layout(L));
  // the partials of the compress grid, [n][pieces] (and [n][items]), must fit
  // the fixed scratch; refused before the buffers are looked at
  if (L->geo.d > 0 &&
      oba::partial_bytes(L->sig_c, L->plan.n) > (size_t)OBA_NOALLOC_SCRATCH_BYTES)
    return OBA_ESCRATCH;
  OBA_TRY(compress_deferred_checks(L, g, g_dtype, m, sbits_prev, sscale_prev, c, wbits, wscale,
                                   beta1));
  if (L->geo.d == 0) return OBA_OK;
  void* sp = nullptr;
  OBA_TRY(scratch_on(L->device, &sp));  // resolved when the layout was created
  return compress_deferred_run(L, g, g_dtype, m, sbits_prev, sscale_prev, c, wbits, wscale,
                               beta1, static_cast<double*>(sp), stream);
}

int oba_compress_deferred16(oba_layout L, const void* g, int g_dtype, const float* m,
                            const uint64_t* sbits_prev, const float* sscale_prev, void* c,
                            int c_dtype, uint64_t* wbits, float* wscale, double beta1, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  OBA_TRY(check_layout(L));
  if (!gdtype_ok(g_dtype)) return OBA_EINVAL;
  if (c_dtype != OBA_F16 && c_dtype != OBA_BF16) return OBA_EINVAL;
  if (!beta_ok(beta1)) return OBA_EINVAL;
  const bool implicit_m = !m;
  if (implicit_m != (sbits_prev != nullptr) || implicit_m != (sscale_prev != nullptr))
    return OBA_EINVAL;
  if (L->geo.d == 0) return OBA_OK;
  OBA_TRY(check_buf(g, 16));
  if (implicit_m) {
    OBA_TRY(check_buf(sbits_prev, 8));
    OBA_TRY(check_buf(sscale_prev, 4));
  } else {
    OBA_TRY(check_buf(m, 16));
  }
  OBA_TRY(check_buf(c, 8));
  OBA_TRY(check_buf(wbits, 8));
  OBA_TRY(check_buf(wscale, 4));
  OBA_TRY(check_buf(ws, 8));
  if (ws_bytes < oba_workspace_bytes(L)) return OBA_EWORKSPACE;
  // grid: the compress grid, or (OBA_S16_GRID = 1) the server grid's
  // blocks of several spans, whose tables also cover this pass
  const bool sg = OBA_S16_GRID != 0;
  const oba::Geo G = sg ? L->geo : L->geo_c;
  const oba::SegDev& sig = sg ? L->sig : L->sig_c;
  double* part = static_cast<double*>(ws);
  const float b1 = (float)beta1, omb1 = (float)(1.0 - beta1);
  uint8_t* wbytes = reinterpret_cast<uint8_t*>(wbits);
  const oba::MomSrc ms{reinterpret_cast<const uint8_t*>(sbits_prev), sscale_prev,
                       sg ? L->tau : L->tau_c};
  OBA_TRY(launch("compress_deferred16", stream, [&] {
    oba::launch_compress_deferred16(G, g, g_dtype, m, c, c_dtype, wbytes, sig, part, wscale, b1,
                                    omb1, ms, stream);
  }));
  return launch("finalize_scales", stream,
                [&] { oba::launch_finalize(part, G.n, sig, wscale, stream); });
}

int oba_compress_deferred_local(oba_layout L, const void* g, int g_dtype, float* m_local,
                                float* c, uint64_t* wbits, float* wscale, double beta1, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  OBA_TRY(check_layout(L));
  if (!gdtype_ok(g_dtype)) return OBA_EINVAL;
  if (!beta_ok(beta1)) return OBA_EINVAL;
  if (L->geo.d == 0) return OBA_OK;
  OBA_TRY(check_buf(g, 16));
  OBA_TRY(check_buf(m_local, 16));
  OBA_TRY(check_buf(c, 16));
  OBA_TRY(check_buf(wbits, 8));
  OBA_TRY(check_buf(wscale, 4));
  OBA_TRY(check_buf(ws, 8));
  if (ws_bytes < oba_workspace_bytes(L)) return OBA_EWORKSPACE;
  if ((const void*)m_local == (const void*)c) return OBA_EINVAL;
  const oba::Geo G = L->geo_e;
  double* part = static_cast<double*>(ws);
  const float b1 = (float)beta1, omb1 = (float)(1.0 - beta1);
  uint8_t* wbytes = reinterpret_cast<uint8_t*>(wbits);
  OBA_TRY(launch("compress_deferred_local", stream, [&] {
    oba::launch_compress_deferred_local(G, g, g_dtype, m_local, c, wbytes, L->sig_e,
                                        part, wscale, b1, omb1, stream);
  }));
  return launch("finalize_scales", stream,
                [&] { oba::launch_finalize(part, G.n, L->sig_e, wscale, stream); });
}

int oba_server_reduce_recompress_deferred(oba_layout L, const uint64_t* wbits,
                                          const float* wscale, float* a, uint64_t* sbits,
                                          float* sscale, void* ws, size_t ws_bytes,
                                          hipStream_t stream) {
  OBA_TRY(check_layout(L));
  if (L->geo.d == 0) return OBA_OK;
  OBA_TRY(check_buf(wbits, 8));
  OBA_TRY(check_buf(wscale, 4));
  OBA_TRY(check_buf(a, 16));
  OBA_TRY(check_buf(sbits, 8));
  OBA_TRY(check_buf(sscale, 4));
  OBA_TRY(check_buf(ws, 8));
  if (ws_bytes < oba_workspace_bytes(L)) return OBA_EWORKSPACE;
#ifndef OBA_SRV_GRID1
#define OBA_SRV_GRID1 0
#endif
  // grid: the server grid (several spans per block), or (OBA_SRV_GRID1) the
  // compress grid with its tables
  const bool g1 = OBA_SRV_GRID1 != 0;
  const oba::Geo G = g1 ? L->geo_c : L->geo;
  const oba::SegDev& sig = g1 ? L->sig_c : L->sig;
  const oba::SegDev& tau = g1 ? L->tau_c : L->tau;
  double* part = reinterpret_cast<double*>(static_cast<char*>(ws) +
                                           ((L->ws_worker + 255) / 256) * 256);
  const uint8_t* wbytes = reinterpret_cast<const uint8_t*>(wbits);
  uint8_t* sbytes = reinterpret_cast<uint8_t*>(sbits);
  OBA_TRY(launch("server_deferred", stream, [&] {
    oba::launch_server_deferred(G, wbytes, wscale, a, sbytes, sig, tau, part, sscale, stream);
  }));
  return launch("finalize_scales", stream,
                [&] { oba::launch_finalize(part, 1, tau, sscale, stream); });
}

int oba_deferred_errors(oba_layout L, const float* c, const float* wscale, const float* a,
                        const float* sscale, float* delta, float* eps, hipStream_t stream) {
  OBA_TRY(check_layout(L));
  if (L->geo.d == 0) return OBA_OK;
  if (!delta && !eps) return OBA_EINVAL;
  const oba::Geo G = L->geo;
  if (delta) {
    OBA_TRY(check_buf(c, 16));
    OBA_TRY(check_buf(wscale, 4));
    OBA_TRY(check_buf(delta, 16));
    if ((const void*)c == (const void*)delta) return OBA_EINVAL;
    OBA_TRY(launch("deferred_errors", stream, [&] {
      oba::launch_residual(G, c, G.ld, delta, G.ld, G.n, wscale, L->sig, stream);
    }));
  }
  if (eps) {
    OBA_TRY(check_buf(a, 16));
    OBA_TRY(check_buf(sscale, 4));
    OBA_TRY(check_buf(eps, 16));
    if ((const void*)a == (const void*)eps) return OBA_EINVAL;
    OBA_TRY(launch("deferred_errors", stream, [&] {
      oba::launch_residual(G, a, 0, eps, 0, 1, sscale, L->tau, stream);
    }));
  }
  return OBA_OK;
}

int oba_decompress_update(oba_layout L, const uint64_t* sbits, const float* sscale,
                          const float* denom, float* m, float* x, double lr, hipStream_t stream) {
  OBA_TRY(check_layout(L));
  if (!is_finite(lr)) return OBA_EINVAL;
  if (L->geo.d == 0) return OBA_OK;
  OBA_TRY(check_buf(sbits, 8));
  OBA_TRY(check_buf(sscale, 4));
  OBA_TRY(check_buf(denom, 16));
  if (m) OBA_TRY(check_buf(m, 16));
  OBA_TRY(check_buf(x, 16));
  // one span per block (the worker grid): the update streams best that way
  const oba::Geo G = L->geo_w;
  const uint8_t* sbytes = reinterpret_cast<const uint8_t*>(sbits);
  return launch("decompress_update", stream, [&] {
    oba::launch_decompress_update(G, sbytes, sscale, denom, m, x, L->tau_w, (float)lr, stream);
  });
}

int oba_server_momentum(oba_layout L, const uint64_t* sbits, const float* sscale, float* m,
                        hipStream_t stream) {
  OBA_TRY(check_layout(L));
  if (L->geo.d == 0) return OBA_OK;
  OBA_TRY(check_buf(sbits, 8));
  OBA_TRY(check_buf(sscale, 4));
  OBA_TRY(check_buf(m, 16));
  const oba::Geo G = L->geo_w;
  const uint8_t* sbytes = reinterpret_cast<const uint8_t*>(sbits);
  return launch("server_momentum", stream,
                [&] { oba::launch_server_momentum(G, sbytes, sscale, m, L->tau_w, stream); });
}

int oba_tensors_create(oba_tensors* out, oba_layout L, int32_t n_tensors,
                       const int64_t* lengths, float* const* x_ptrs, const void* const* g_ptrs,
                       int g_dtype) {
  if (!out || !x_ptrs || !g_ptrs) return OBA_EINVAL;
  OBA_TRY(check_layout(L));
  if (!gdtype_ok(g_dtype)) return OBA_EINVAL;
  const oba::Plan& P = L->plan;
  if (P.d == 0) return OBA_EINVAL;  // nothing to list
  std::vector<int64_t> off;
  int rc = oba::tensor_offsets(P, n_tensors, lengths, &off);
  if (rc) return rc;
  const int32_t T = n_tensors, n = P.n;
  const uintptr_t galign = g_dtype == OBA_F32 ? 16 : 8;  // a quad: 16 or 8 bytes
  for (int32_t t = 0; t < T; ++t) OBA_TRY(check_buf(x_ptrs[t], 16));
  for (int64_t r = 0; r < (int64_t)n * T; ++r) OBA_TRY(check_buf(g_ptrs[r], galign));
  // per-block tensor tables of the compress, update and server grids
  std::vector<oba::TBlk> tc, tw, ts;
  try {
    std::vector<int32_t> first;
    for (auto pr : {std::make_pair(P.nblk_c, &tc), std::make_pair(P.nblk_w, &tw),
                    std::make_pair(P.nblk, &ts)}) {
      oba::tensor_blocks(P, pr.first, off, &first);
      pr.second->resize(first.size());
      for (size_t b = 0; b < first.size(); ++b) {
        const int32_t t = first[b];
        (*pr.second)[b] = oba::TBlk{off[t], off[t + 1], t, 0};
      }
    }
  } catch (...) {
    return OBA_ENOMEM;
  }
  // layout of the allocation: block tables (compress, update, server grid) |
  // off | g pointers | x pointers
  const size_t b_bc = tc.size() * sizeof(oba::TBlk);
  const size_t b_bw = b_bc + tw.size() * sizeof(oba::TBlk);  // tables up to tw
  const size_t b_bs = ts.size() * sizeof(oba::TBlk);
  const size_t b_off = off.size() * sizeof(int64_t);
  const size_t b_g = (size_t)n * T * sizeof(void*);
  const size_t b_x = (size_t)T * sizeof(float*);
  const size_t bytes = b_off + b_g + b_x + b_bw + b_bs;
  oba_tensors_s* H = new (std::nothrow) oba_tensors_s();
  if (!H) return OBA_ENOMEM;
  H->device = L->device;
  H->g_dtype = g_dtype;
  H->T = T;
  H->n = n;
  H->layout_serial = L->serial;
  H->d = P.d;
  H->nblk_c = P.nblk_c;
  H->nblk_w = P.nblk_w;
  H->nblk = P.nblk;
  hipError_t e = hipMalloc(&H->dev, bytes);
  if (e != hipSuccess) {
    delete H;
    return OBA_ENOMEM;
  }
  char* base = static_cast<char*>(H->dev);
  const std::pair<const void*, size_t> parts[] = {
      {tc.data(), b_bc}, {tw.data(), b_bw - b_bc}, {ts.data(), b_bs}, {off.data(), b_off},
      {g_ptrs, b_g}, {x_ptrs, b_x}};
  size_t at = 0;
  for (const auto& pr : parts) {
    if (pr.second) e = hipMemcpy(base + at, pr.first, pr.second, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      (void)hipFree(H->dev);
      delete H;
      return hip_fail(e, "hipMemcpy (tensor tables)");
    }
    at += pr.second;
  }
  oba::TList tl{};
  tl.off = reinterpret_cast<const int64_t*>(base + b_bw + b_bs);
  tl.g = reinterpret_cast<const void* const*>(base + b_bw + b_bs + b_off);
  tl.x = reinterpret_cast<float* const*>(base + b_bw + b_bs + b_off + b_g);
  tl.T = T;
  H->tl_c = tl;
  H->tl_c.blk = reinterpret_cast<const oba::TBlk*>(base);
  H->tl_w = tl;
  H->tl_w.blk = reinterpret_cast<const oba::TBlk*>(base + b_bc);
  H->tl_s = tl;
  H->tl_s.blk = reinterpret_cast<const oba::TBlk*>(base + b_bw);
  *out = H;
  return OBA_OK;
}

void oba_tensors_destroy(oba_tensors H) {
  if (!H) return;
  if (H->dev) {
    (void)hipDeviceSynchronize();
    (void)hipFree(H->dev);
  }
  delete H;
}

int oba_adam_warmup_step_listed(oba_layout L, oba_tensors H, float* m, float* v, double lr,
                                double beta1, double beta2, double eta, double bc1, double bc2,
                                double* vnorm, void* ws, size_t ws_bytes, hipStream_t stream) {
  OBA_TRY(check_layout(L));
  OBA_TRY(check_tensors(L, H));
  if (!is_finite(lr) || !beta_ok(beta1) || !beta_ok(beta2) || !is_finite(eta) || eta < 0.0 ||
      !is_finite(bc1) || bc1 <= 0.0 || !is_finite(bc2) || bc2 <= 0.0)
    return OBA_EINVAL;
  OBA_TRY(check_buf(m, 16));
  OBA_TRY(check_buf(v, 16));
  if (vnorm) {
    OBA_TRY(check_buf(vnorm, 8));
    OBA_TRY(check_buf(ws, 8));
    if (ws_bytes < oba_workspace_bytes(L)) return OBA_EWORKSPACE;
  }
  oba::AdamCoef C{(float)lr, (float)beta1, (float)(1.0 - beta1), (float)beta2,
                  (float)(1.0 - beta2), (float)eta, (float)bc1, (float)bc2};
  // a grid of oba_adam_warmup_step, with its block table of the tensors
  const oba::Geo G = OBA_WARM_SPAN1_TL ? L->geo_w : L->geo;
  double* part = static_cast<double*>(ws);
  return launch("adam_warmup", stream, [&] {
    oba::launch_adam_warmup_listed(G, OBA_WARM_SPAN1_TL ? H->tl_w : H->tl_s, H->g_dtype, m, v, C,
                                   part, vnorm, stream);
  });
}

int oba_compress_deferred_listed(oba_layout L, oba_tensors H, const float* m,
                                 const uint64_t* sbits_prev, const float* sscale_prev, float* c,
                                 uint64_t* wbits, float* wscale, double beta1, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
  OBA_TRY(check_layout(L));
  OBA_TRY(check_tensors(L, H));
  if (!beta_ok(beta1)) return OBA_EINVAL;
  const bool implicit_m = !m;
  if (implicit_m != (sbits_prev != nullptr) || implicit_m != (sscale_prev != nullptr))
    return OBA_EINVAL;
  if (implicit_m) {
    OBA_TRY(check_buf(sbits_prev, 8));
    OBA_TRY(check_buf(sscale_prev, 4));
  } else {
    OBA_TRY(check_buf(m, 16));
  }
  OBA_TRY(check_buf(c, 16));
  OBA_TRY(check_buf(wbits, 8));
  OBA_TRY(check_buf(wscale, 4));
  OBA_TRY(check_buf(ws, 8));
  if (ws_bytes < oba_workspace_bytes(L)) return OBA_EWORKSPACE;
  const oba::Geo G = L->geo_c;
  double* part = static_cast<double*>(ws);
  const float b1 = (float)beta1, omb1 = (float)(1.0 - beta1);
  uint8_t* wbytes = reinterpret_cast<uint8_t*>(wbits);
  const oba::MomSrc ms{reinterpret_cast<const uint8_t*>(sbits_prev), sscale_prev, L->tau_c};
  OBA_TRY(launch("compress_deferred", stream, [&] {
    oba::launch_compress_deferred_listed(G, H->tl_c, H->g_dtype, m, c, wbytes,
                                         L->sig_c, part, wscale, b1, omb1, ms, stream);
  }));
  return launch("finalize_scales", stream,
                [&] { oba::launch_finalize(part, G.n, L->sig_c, wscale, stream); });
}

int oba_compress_deferred16_listed(oba_layout L, oba_tensors H, const float* m,
                                   const uint64_t* sbits_prev, const float* sscale_prev, void* c,
                                   int c_dtype, uint64_t* wbits, float* wscale, double beta1,
                                   void* ws, size_t ws_bytes, hipStream_t stream) {
  OBA_TRY(check_layout(L));
  OBA_TRY(check_tensors(L, H));
  if (c_dtype != OBA_F16 && c_dtype != OBA_BF16) return OBA_EINVAL;
  if (!beta_ok(beta1)) return OBA_EINVAL;
  const bool implicit_m = !m;
  if (implicit_m != (sbits_prev != nullptr) || implicit_m != (sscale_prev != nullptr))
    return OBA_EINVAL;
  if (implicit_m) {
    OBA_TRY(check_buf(sbits_prev, 8));
    OBA_TRY(check_buf(sscale_prev, 4));
  } else {
    OBA_TRY(check_buf(m, 16));
  }
  OBA_TRY(check_buf(c, 8));
  OBA_TRY(check_buf(wbits, 8));
  OBA_TRY(check_buf(wscale, 4));
  OBA_TRY(check_buf(ws, 8));
  if (ws_bytes < oba_workspace_bytes(L)) return OBA_EWORKSPACE;
  // the grid of oba_compress_deferred16, with its block table of the tensors
  const bool sg = OBA_S16_GRID != 0;
  const oba::Geo G = sg ? L->geo : L->geo_c;
  const oba::SegDev& sig = sg ? L->sig : L->sig_c;
  double* part = static_cast<double*>(ws);
  const float b1 = (float)beta1, omb1 = (float)(1.0 - beta1);
  uint8_t* wbytes = reinterpret_cast<uint8_t*>(wbits);
  const oba::MomSrc ms{reinterpret_cast<const uint8_t*>(sbits_prev), sscale_prev,
                       sg ? L->tau : L->tau_c};
  OBA_TRY(launch("compress_deferred16", stream, [&] {
    oba::launch_compress_deferred16_listed(G, sg ? H->tl_s : H->tl_c, H->g_dtype, m, c, c_dtype,
                                           wbytes, sig, part, wscale, b1, omb1, ms, stream);
  }));
  return launch("finalize_scales", stream,
                [&] { oba::launch_finalize(part, G.n, sig, wscale, stream); });
}

int oba_decompress_update_listed(oba_layout L, oba_tensors H, const uint64_t* sbits,
                                 const float* sscale, const float* denom, float* m, double lr,
                                 hipStream_t stream) {
  OBA_TRY(check_layout(L));
  OBA_TRY(check_tensors(L, H));
  if (!is_finite(lr)) return OBA_EINVAL;
  OBA_TRY(check_buf(sbits, 8));
  OBA_TRY(check_buf(sscale, 4));
  OBA_TRY(check_buf(denom, 16));
  if (m) OBA_TRY(check_buf(m, 16));
  const oba::Geo G = L->geo_w;
  const uint8_t* sbytes = reinterpret_cast<const uint8_t*>(sbits);
  return launch("decompress_update", stream, [&] {
    oba::launch_decompress_update_listed(G, H->tl_w, sbytes, sscale, denom, m, L->tau_w,
                                         (float)lr, stream);
  });
}

int oba_plateau_init(oba_plateau* p, int32_t window, double rtol, int32_t min_steps) {
  if (!p || window < 1 || window > OBA_PLATEAU_MAX_WINDOW || !is_finite(rtol) || rtol < 0.0 ||
      min_steps < 0)
    return OBA_EINVAL;
  std::memset(p, 0, sizeof(*p));
  p->window = window;
  p->min_steps = min_steps;
  p->rtol = rtol;
  return OBA_OK;
}

int oba_plateau_observe(oba_plateau* p, double value) {
  if (!p || p->window < 1 || p->window > OBA_PLATEAU_MAX_WINDOW || !is_finite(value))
    return OBA_EINVAL;
  if (p->steps == INT32_MAX) return p->fired;
  const int32_t t = ++p->steps;
  double& slot = p->ring[t % p->window];  // holds h_{t-window} once t > window
  if (!p->fired && t > p->window && t >= p->min_steps &&
      std::fabs(value - slot) <= p->rtol * std::fabs(value))
    p->fired = 1;
  slot = value;
  return p->fired;
}

int oba_step_small(oba_layout L, const void* g, int g_dtype, const float* m, float* c,
                   uint64_t* wbits, float* wscale, float* a, uint64_t* sbits, float* sscale,
                   const float* denom, float* m_out, float* x, double beta1, double lr,
                   hipStream_t stream) {
  OBA_TRY(check_layout(L));
  if (!gdtype_ok(g_dtype) || !beta_ok(beta1) || !is_finite(lr)) return OBA_EINVAL;
  const oba::Plan& P = L->plan;
  if (P.d > oba::kSmallMaxD || P.n > oba::kSmallMaxN ||
      (int64_t)P.wseg.size() - 1 > oba::kSmallMaxSeg ||
      (int64_t)P.sseg.size() - 1 > oba::kSmallMaxSeg)
    return OBA_EINVAL;
  if (P.d == 0) return OBA_OK;
  OBA_TRY(check_buf(g, 16));
  if (m) OBA_TRY(check_buf(m, 16));
  OBA_TRY(check_buf(c, 16));
  OBA_TRY(check_buf(wbits, 8));
  OBA_TRY(check_buf(wscale, 4));
  OBA_TRY(check_buf(a, 16));
  OBA_TRY(check_buf(sbits, 8));
  OBA_TRY(check_buf(sscale, 4));
  OBA_TRY(check_buf(denom, 16));
  if (m_out) OBA_TRY(check_buf(m_out, 16));
  OBA_TRY(check_buf(x, 16));
  oba::SmallArgs A{};
  A.d = P.d;
  A.ld = P.ld;
  A.W = P.W;
  A.n = P.n;
  A.n_wseg = (int32_t)P.wseg.size() - 1;
  A.n_sseg = (int32_t)P.sseg.size() - 1;
  A.wseg = L->sig.off;
  A.sseg = L->tau.off;
  A.g = g;
  A.m_in = m;
  A.c = c;
  A.wbits = wbits;
  A.wscale = wscale;
  A.a = a;
  A.sbits = sbits;
  A.sscale = sscale;
  A.denom = denom;
  A.m_out = m_out;
  A.x = x;
  A.b1 = (float)beta1;
  A.omb1 = (float)(1.0 - beta1);
  A.lr = (float)lr;
  return launch("step_small", stream, [&] { oba::launch_step_small(A, g_dtype, stream); });
}

int oba_timing_enable(int on, int32_t capacity) {
  std::lock_guard<std::mutex> lk(g_tmu);
  if (on) {
    if (capacity < 1 || capacity > (1 << 20)) return OBA_EINVAL;
    const size_t want = 2 * (size_t)capacity;
    size_t have = g_pool.size() + 2 * g_recs.size();
    while (have < want) {
      hipEvent_t ev;
      hipError_t e = hipEventCreate(&ev);
      if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
      g_pool.push_back(ev);
      ++have;
    }
  }
  g_timing = on != 0;
  return OBA_OK;
}

int oba_timing_read(const char* kernel, double* total_ms, int64_t* launches) {
  if (!kernel || !total_ms || !launches) return OBA_EINVAL;
  std::vector<TimingRec> recs;
  {
    std::lock_guard<std::mutex> lk(g_tmu);
    recs = g_recs;
  }
  double t = 0.0;
  int64_t c = 0;
  for (const auto& r : recs) {
    if (std::strcmp(r.name, kernel) != 0) continue;
    hipError_t e = hipEventSynchronize(r.b);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float ms = 0.0f;
    e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    t += ms;
    ++c;
  }
  *total_ms = t;
  *launches = c;
  return OBA_OK;
}

int oba_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_tmu);
  timing_drop_all();
  return OBA_OK;
}

}  // extern "C"
