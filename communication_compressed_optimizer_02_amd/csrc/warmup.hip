// warmup.hip -- the warm-up Adam step, the variance norm and the freeze (gfx950).
// Method passages are cited in include/oba.h beside each entry point.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device.hpp"
#include "occupancy.hpp"

namespace oba {

// ===========================================================================
// Warm-up Adam step on the mean gradient.  NORM: also the sum of squares of
// the new v, one binary64 partial per block (part[blockIdx.x]).  NB rows of g
// are loaded together (NB = n for n <= 8; larger n loops over groups of 8),
// after m, v and x, so that all of a span's loads are in flight at once.
// ===========================================================================

// A span's loads: m, v, x, then the gradient rows, summed in worker order.
// FULL (the span lies inside [0, d)) takes unchecked vector loads; the tail
// span checks every element.  The whole span is one branch: with a branch per
// row, each row's loads (16-bit rows are decoded as they arrive) would wait
// before the next row is requested, leaving one row in flight per wave.
template <bool FULL, typename GT, int NB, bool TL>
__device__ __forceinline__ void warm_span_loads(const Geo& G, const GT* __restrict__ g,
                                                const float* __restrict__ x,
                                                const float* __restrict__ m,
                                                const float* __restrict__ v, const TList& tl,
                                                const LaneT& lt, const Quads& q, int64_t lo,
                                                float (&mv)[8], float (&vv)[8], float (&xv)[8],
                                                float (&sum)[8]) {
  constexpr bool BUF = OBA_BUF_MISC != 0;
  if constexpr (FULL) {
    if constexpr (BUF) {
      load_full_buf(m, lo, mv);
      load_full_buf(v, lo, vv);
    } else {
      load_full(m, q, mv);
      load_full(v, q, vv);
    }
    if constexpr (TL)
      load_listed_x_q<false>(tl, lt, xv);
    else if constexpr (BUF)
      load_full_buf(x, lo, xv);
    else
      load_full(x, q, xv);
  } else {
    load_tail(m, q, G.d, mv);
    load_tail(v, q, G.d, vv);
    if constexpr (TL)
      load_listed_x_q<true>(tl, lt, xv);
    else
      load_tail(x, q, G.d, xv);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) sum[j] = 0.0f;
  // rows past n are clamped to a valid row and their terms skipped
  auto group = [&](int32_t i0) {
    float gv[NB][8];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int64_t row = min(i0 + u, G.n - 1);
      if constexpr (TL)
        load_listed_q<!FULL, GT>(tl, row, lt, gv[u]);
      else if constexpr (FULL)
        load_full(g + row * G.ld, q, gv[u]);
      else
        load_tail(g + row * G.ld, q, G.d, gv[u]);
    }
#pragma unroll
    for (int u = 0; u < NB; ++u)
      if (i0 + u < G.n) {
#pragma unroll
        for (int j = 0; j < 8; ++j) sum[j] = sum[j] + gv[u][j];
      }
  };
  if (G.n <= NB) {
    group(0);  // straight-line: a loop here would wait for every load at its head
  } else {
    for (int32_t i0 = 0; i0 < G.n; i0 += NB) group(i0);
  }
}

template <typename GT, int NB, bool NORM, bool TL>
__global__ __launch_bounds__(kBlock) void k_adam_warmup(Geo G, const GT* __restrict__ g,
                                                        float* __restrict__ x,
                                                        float* __restrict__ m,
                                                        float* __restrict__ v, AdamCoef C,
                                                        double* __restrict__ part, TList tl) {
  __shared__ double lds[kWaves];
  double acc[1] = {0.0};
  const int64_t s_lo = dspan(G, (int32_t)blockIdx.x);
  const int64_t s_hi = dspan(G, (int32_t)blockIdx.x + 1);
  TCur tcur{};  // tensor cursor (tensor lists: x and g listed)
  if constexpr (TL) tcur = tcur_start(tl, blockIdx.x);
  const float nf = (float)G.n;
  const bool pow2 = (G.n & (G.n - 1)) == 0;
  const float inv_n = 1.0f / nf;
  for (int64_t s = s_lo; s < s_hi; ++s) {
    const int64_t lo = s * kSpan;
    const Quads q = quads(lo);
    const bool full = lo + kSpan <= G.d;
    float sum[8], mv[8], vv[8], xv[8];
    LaneT lt{};
    if constexpr (TL) {
      tcur_advance(tl, tcur, lo);
      lt = lane_tensors(tl, tcur, q, min(lo + kSpan, G.d), G.d);
    }
    if (full)
      warm_span_loads<true, GT, NB, TL>(G, g, x, m, v, tl, lt, q, lo, mv, vv, xv, sum);
    else
      warm_span_loads<false, GT, NB, TL>(G, g, x, m, v, tl, lt, q, lo, mv, vv, xv, sum);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float gb = pow2 ? sum[j] * inv_n : sum[j] / nf;  // identical for n = 2^k
      const float mk = C.b1 * mv[j] + C.omb1 * gb;
      const float vk = C.b2 * vv[j] + C.omb2 * (gb * gb);
      mv[j] = mk;
      vv[j] = vk;
      xv[j] = xv[j] - (C.lr * (mk / C.bc1)) / (__builtin_sqrtf(vk / C.bc2) + C.eta);
    }
    constexpr bool BUF = OBA_BUF_MISC != 0;
    store8b<BUF>(m, q, lo, G.d, full, mv);
    store8b<BUF>(v, q, lo, G.d, full, vv);
    if constexpr (TL)
      store_listed_x(tl, lt, full, xv);
    else
      store8b<BUF>(x, q, lo, G.d, full, xv);
    if (NORM) acc[0] += sumsq8(vv);  // coordinates past d read 0 and give v = 0
  }
  if (NORM) flush_rows<1>(acc, 1, part + blockIdx.x, 0, lds);
}

// sqrt of the sum of n binary64 partials, in a fixed order.  One block.
constexpr int kNormBlock = 1024;

__global__ __launch_bounds__(kNormBlock) void k_norm_finalize(const double* __restrict__ part,
                                                              int32_t n,
                                                              double* __restrict__ out) {
  __shared__ double lds[kNormBlock / 64];
  double t = 0.0;
  for (int32_t q = threadIdx.x; q < n; q += kNormBlock) t += part[q];
  t = wave_sum(t);
  if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = t;
  __syncthreads();
  if (threadIdx.x == 0) {
    double S = 0.0;
    for (int w = 0; w < kNormBlock / 64; ++w) S += lds[w];  // fixed order
    out[0] = __builtin_sqrt(S);
  }
}

// ===========================================================================
// Variance freeze: denom = sqrt(v / bc2) + eta.
// ===========================================================================
__global__ __launch_bounds__(kBlock) void k_freeze(Geo G, const float* __restrict__ v,
                                                   float* __restrict__ denom, float eta,
                                                   float bc2) {
  const int64_t s_lo = dspan(G, (int32_t)blockIdx.x);
  const int64_t s_hi = dspan(G, (int32_t)blockIdx.x + 1);
  for (int64_t s = s_lo; s < s_hi; ++s) {
    const int64_t lo = s * kSpan;
    const Quads q = quads(lo);
    const bool full = lo + kSpan <= G.d;
    float vv[8];
    load8(v, q, G.d, full, vv);
#pragma unroll
    for (int j = 0; j < 8; ++j) vv[j] = __builtin_sqrtf(vv[j] / bc2) + eta;
    store8(denom, q, G.d, full, vv);
  }
}

// ---- launchers ----------------------------------------------------------------

void launch_norm_finalize(const double* part, int32_t n, double* out, hipStream_t st);

// Occupancy cap of the warm-up step (blocks per CU, 0: none), a tuning knob:
// with one span per block, 2 blocks per CU took the step from 2.42 to 2.31 ms
// at bert_large (3: 2.37 ms; same-box A/B); loading the gradient rows before
// m, v, x was slower (2.63 vs 2.49 ms on the server grid).
#ifndef OBA_WARM_BPC
#define OBA_WARM_BPC 2
#endif
// The tensor-list warm-up runs uncapped: the cap of 2 took it from 10.43 to
// 12.6-12.9 ms at gpt2_xl (388 tensors, n = 4, binary32 gradients; 3 blocks
// per CU: 10.50 ms; the server grid, uncapped: 10.73 ms; same-box A/B).
#ifndef OBA_WARM_BPC_TL
#define OBA_WARM_BPC_TL 0
#endif
template <typename GT, bool NORM, bool TL>
static void launch_warmup_nb(const Geo& G, const void* g, float* x, float* m, float* v,
                             const AdamCoef& C, double* part, const TList& tl, hipStream_t st) {
  const size_t lds = occupancy_lds(TL ? OBA_WARM_BPC_TL : OBA_WARM_BPC);
#define OBA_WARMUP_LAUNCH(NB)                                                                   \
  do {                                                                                          \
    allow_lds(reinterpret_cast<const void*>(&k_adam_warmup<GT, NB, NORM, TL>), lds);           \
    hipLaunchKernelGGL((k_adam_warmup<GT, NB, NORM, TL>), dim3(G.nblk), dim3(kBlock), lds, st, \
                       G, static_cast<const GT*>(g), x, m, v, C, part, tl);                     \
  } while (0)
  switch (G.n) {
    case 1: OBA_WARMUP_LAUNCH(1); break;
    case 2: OBA_WARMUP_LAUNCH(2); break;
    case 3: OBA_WARMUP_LAUNCH(3); break;
    case 4: OBA_WARMUP_LAUNCH(4); break;
    case 5: OBA_WARMUP_LAUNCH(5); break;
    case 6: OBA_WARMUP_LAUNCH(6); break;
    case 7: OBA_WARMUP_LAUNCH(7); break;
    default: OBA_WARMUP_LAUNCH(8); break;
  }
#undef OBA_WARMUP_LAUNCH
}

template <typename GT, bool TL>
static void launch_warmup(const Geo& G, const void* g, float* x, float* m, float* v,
                          const AdamCoef& C, double* part, double* vnorm, const TList& tl,
                          hipStream_t st) {
  if (!vnorm) {
    launch_warmup_nb<GT, false, TL>(G, g, x, m, v, C, nullptr, tl, st);
    return;
  }
  launch_warmup_nb<GT, true, TL>(G, g, x, m, v, C, part, tl, st);
  launch_norm_finalize(part, G.nblk, vnorm, st);
}

void launch_norm_finalize(const double* part, int32_t n, double* out, hipStream_t st) {
  hipLaunchKernelGGL(k_norm_finalize, dim3(1), dim3(kNormBlock), 0, st, part, n, out);
}

void launch_adam_warmup(const Geo& G, const void* g, int gdt, float* x, float* m, float* v,
                        const AdamCoef& C, double* part, double* vnorm, hipStream_t st) {
  if (gdt == kGradF16)
    launch_warmup<uint16_t, false>(G, g, x, m, v, C, part, vnorm, TList{}, st);
  else if (gdt == kGradBF16)
    launch_warmup<bf16_bits, false>(G, g, x, m, v, C, part, vnorm, TList{}, st);
  else
    launch_warmup<float, false>(G, g, x, m, v, C, part, vnorm, TList{}, st);
}

void launch_adam_warmup_listed(const Geo& G, const TList& tl, int gdt, float* m, float* v,
                               const AdamCoef& C, double* part, double* vnorm, hipStream_t st) {
  if (gdt == kGradF16)
    launch_warmup<uint16_t, true>(G, nullptr, nullptr, m, v, C, part, vnorm, tl, st);
  else if (gdt == kGradBF16)
    launch_warmup<bf16_bits, true>(G, nullptr, nullptr, m, v, C, part, vnorm, tl, st);
  else
    launch_warmup<float, true>(G, nullptr, nullptr, m, v, C, part, vnorm, tl, st);
}

void launch_freeze(const Geo& G, const float* v, float* denom, float eta, float bc2,
                   hipStream_t st) {
  hipLaunchKernelGGL(k_freeze, dim3(G.nblk), dim3(kBlock), 0, st, G, v, denom, eta, bc2);
}

}  // namespace oba
