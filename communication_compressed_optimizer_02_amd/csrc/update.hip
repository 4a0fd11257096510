// update.hip -- decompress, precondition and update; the momentum accessor (gfx950).
// Method passages are cited in include/oba.h beside each entry point.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device.hpp"
#include "occupancy.hpp"

namespace oba {

// ===========================================================================
// Decompress + precondition + update: m_hat = sbar*sign; m = m_hat (when
// WRITE_M); x = x - (lr*m_hat)/denom (when UPDATE_X).  Grid: the worker grid.
// ===========================================================================
template <bool WRITE_M, bool UPDATE_X, bool TL>
__global__ __launch_bounds__(kBlock) void k_decompress_update(Geo G,
                                                              const uint8_t* __restrict__ sbytes,
                                                              const float* __restrict__ sscale,
                                                              const float* __restrict__ denom,
                                                              float* __restrict__ m,
                                                              float* __restrict__ x, SegDev tau,
                                                              float lr, TList tl) {
  const int32_t b = blockIdx.x;
  TCur tcur{};  // tensor cursor (tensor lists: x listed)
  if constexpr (TL) tcur = tcur_start(tl, b);
  const int64_t s_lo = dspan(G, b), s_hi = dspan(G, b + 1);
  const int32_t p_end = tau.blk_first[b + 1];
  int32_t p = tau.blk_first[b];
  int64_t p_hi = tau.phi[p];
  for (int64_t s = s_lo; s < s_hi; ++s) {
    const int64_t lo = s * kSpan;
    const int64_t hi = min(lo + kSpan, G.d);
    const Quads q = quads(lo);
    const bool full = lo + kSpan <= G.d;
    float sv[8], dv[8], xv[8], mh[8];
    const uint32_t bits = full ? load_sign_bits<true, OBA_PAIRS_UPD>(sbytes, q, G.d)
                               : load_sign_bits<false, OBA_PAIRS_UPD>(sbytes, q, G.d);
    LaneT lt{};
    if constexpr (TL) {
      tcur_advance(tl, tcur, lo);
      lt = lane_tensors(tl, tcur, q, min(lo + kSpan, G.d), G.d);
    }
    if (UPDATE_X) {
      load8b<OBA_BUF_MISC != 0>(denom, q, lo, G.d, full, dv);
      if constexpr (TL)
        load_listed_x(tl, lt, full, xv);
      else
        load8b<OBA_BUF_MISC != 0>(x, q, lo, G.d, full, xv);
    }
    if (hi <= p_hi) {
      const float s_ = sscale[tau.pseg[p]];
#pragma unroll
      for (int j = 0; j < 8; ++j) sv[j] = s_;
    } else {
      int32_t js[8];
      lane_segs(tau.off, tau.pseg[p], q, G.d, js);
#pragma unroll
      for (int j = 0; j < 8; ++j) sv[j] = sscale[js[j]];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      mh[j] = ((bits >> j) & 1u) ? -sv[j] : sv[j];
      if (UPDATE_X) xv[j] = xv[j] - (lr * mh[j]) / dv[j];
    }
    if (WRITE_M) store8b<OBA_BUF_MISC != 0>(m, q, lo, G.d, full, mh);
    if (UPDATE_X) {
      if constexpr (TL)
        store_listed_x(tl, lt, full, xv);
      else
        store8b<OBA_BUF_MISC != 0>(x, q, lo, G.d, full, xv);
    }
    while (p < p_end && p_hi <= hi) {
      if (++p < p_end) p_hi = tau.phi[p];
    }
  }
}

// ---- launchers ----------------------------------------------------------------

// Occupancy cap of the update (blocks per CU, 0: none), a tuning knob: 3
// blocks per CU instead of the 8 its registers allow took it from 0.67 to
// 0.61 ms at bert_large (2: 0.72 ms, 4: 0.62 ms; same-box A/B).
#ifndef OBA_UPD_BPC
#define OBA_UPD_BPC 3
#endif
// The tensor-list update (x read and written in place through the tensor
// table) runs uncapped: the cap of 3 took it from 3.09 to 4.59 ms at gpt2_xl
// (388 tensors; 6 blocks per CU: 3.03 ms; same-box A/B).
#ifndef OBA_UPD_BPC_TL
#define OBA_UPD_BPC_TL 0
#endif

template <bool WRITE_M, bool TL>
static void launch_update_t(const Geo& G, const uint8_t* sbytes, const float* sscale,
                            const float* denom, float* m, float* x, const SegDev& tau, float lr,
                            const TList& tl, hipStream_t st) {
  const size_t lds = occupancy_lds(TL ? OBA_UPD_BPC_TL : OBA_UPD_BPC);
  allow_lds(reinterpret_cast<const void*>(&k_decompress_update<WRITE_M, true, TL>), lds);
  hipLaunchKernelGGL((k_decompress_update<WRITE_M, true, TL>), dim3(G.nblk), dim3(kBlock), lds,
                     st, G, sbytes, sscale, denom, m, x, tau, lr, tl);
}

void launch_decompress_update(const Geo& G, const uint8_t* sbytes, const float* sscale,
                              const float* denom, float* m, float* x, const SegDev& tau, float lr,
                              hipStream_t st) {
  if (m)
    launch_update_t<true, false>(G, sbytes, sscale, denom, m, x, tau, lr, TList{}, st);
  else
    launch_update_t<false, false>(G, sbytes, sscale, denom, m, x, tau, lr, TList{}, st);
}

void launch_decompress_update_listed(const Geo& G, const TList& tl, const uint8_t* sbytes,
                                     const float* sscale, const float* denom, float* m,
                                     const SegDev& tau, float lr, hipStream_t st) {
  if (m)
    launch_update_t<true, true>(G, sbytes, sscale, denom, m, nullptr, tau, lr, tl, st);
  else
    launch_update_t<false, true>(G, sbytes, sscale, denom, m, nullptr, tau, lr, tl, st);
}

void launch_server_momentum(const Geo& G, const uint8_t* sbytes, const float* sscale, float* m,
                            const SegDev& tau, hipStream_t st) {
  hipLaunchKernelGGL((k_decompress_update<true, false, false>), dim3(G.nblk), dim3(kBlock), 0, st,
                     G, sbytes, sscale, nullptr, m, nullptr, tau, 0.0f, TList{});
}

}  // namespace oba
