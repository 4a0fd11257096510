// server.hip -- the server pass and the residual pass (gfx950).
// Method passages are cited in include/oba.h beside each entry point.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device.hpp"
#include "occupancy.hpp"

namespace oba {

// ===========================================================================
// Residual pass: dst = c - s*sign(c) over one row of src, s = the row's scale
// of the segment holding each coordinate (dst may be src: in place).
// Grid: (nblk, rows); row r at src + r*src_ld and dst + r*dst_ld.
// ===========================================================================
__global__ __launch_bounds__(kBlock) void k_residual(Geo G, const float* src, int64_t src_ld,
                                                     float* dst, int64_t dst_ld,
                                                     const float* __restrict__ scale, SegDev T) {
  const int32_t b = blockIdx.x;
  const float* srow = src + (int64_t)blockIdx.y * src_ld;
  float* drow = dst + (int64_t)blockIdx.y * dst_ld;
  const float* sc = scale + (int64_t)blockIdx.y * T.n_seg;
  const int64_t s_lo = dspan(G, b), s_hi = dspan(G, b + 1);
  const int32_t p_end = T.blk_first[b + 1];
  int32_t p = T.blk_first[b];
  int64_t p_hi = T.phi[p];
  for (int64_t s = s_lo; s < s_hi; ++s) {
    const int64_t lo = s * kSpan;
    const int64_t hi = min(lo + kSpan, G.d);
    const Quads q = quads(lo);
    const bool full = lo + kSpan <= G.d;
    float c[8], sv[8];
    load8(srow, q, G.d, full, c);
    if (hi <= p_hi) {
      const float s_ = sc[T.pseg[p]];
#pragma unroll
      for (int j = 0; j < 8; ++j) sv[j] = s_;
    } else {
      int32_t js[8];
      lane_segs(T.off, T.pseg[p], q, G.d, js);
#pragma unroll
      for (int j = 0; j < 8; ++j) sv[j] = sc[js[j]];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = residual(c[j], sv[j]);
    store8(drow, q, G.d, full, c);
    while (p < p_end && p_hi <= hi) {
      if (++p < p_end) p_hi = T.phi[p];
    }
  }
}

// ===========================================================================
// Server pass: a = (sum_i s_i*sign_i)/n + eps per coordinate (workers in
// order), a stored over eps, server sign bits stored, binary64 sum of a^2
// reduced per server piece.  The sign bits and scales of NB workers are
// loaded before any is used, so their loads overlap (NB = n for n <= 8, else
// groups of 8).  DEFERRED: the buffer holds the last step's a' and
// sscale_prev its server scales; the server error is formed where it is
// consumed, eps = a' - s'*sign(a'), and a is stored over a'.  Grid: nblk.
// ===========================================================================
// Optional occupancy target of the server pass (waves per SIMD), a tuning knob.
#ifdef OBA_SRV_WAVES
#define OBA_SRV_ATTR __attribute__((amdgpu_waves_per_eu(OBA_SRV_WAVES, OBA_SRV_WAVES)))
#else
#define OBA_SRV_ATTR
#endif

template <int NB, bool DEFERRED>
__global__ __launch_bounds__(kBlock) OBA_SRV_ATTR void k_server_p1(Geo G, const uint8_t* __restrict__ wbytes,
                                                      const float* __restrict__ wscale,
                                                      float* __restrict__ eps,
                                                      uint8_t* __restrict__ sbytes, SegDev sig,
                                                      SegDev tau, double* __restrict__ part,
                                                      const float* __restrict__ sscale_prev) {
  __shared__ double lds[kWaves];
#ifndef OBA_SRV_LDS
#define OBA_SRV_LDS 1
#endif
  // OBA_SRV_LDS: a span's NB packed rows (256 bytes each) are staged in LDS
  // with 8-byte loads, then each lane reads its two bytes per row there
  // (measured 6 % faster than a byte load per lane and row plus a swap)
  // OBA_SRV_PAIR: two full spans inside one worker and one server piece are
  // taken together (n <= NB): both spans' packed rows and a' are requested
  // before either is used, twice the bytes in flight per wave (0.533 -> 0.504
  // ms at bert_large, same-box A/B; with eight spans per block, 0.59 ms)
#ifndef OBA_SRV_PAIR
#define OBA_SRV_PAIR 1
#endif
  __shared__ uint2 rows2_lds[2][OBA_SRV_LDS ? NB * 32 : 1];
  uint2* rows_lds = rows2_lds[0];
  const int32_t b = blockIdx.x;
  const int64_t s_lo = dspan(G, b), s_hi = dspan(G, b + 1);
  const int32_t ps_end = sig.blk_first[b + 1], pt_end = tau.blk_first[b + 1];
  int32_t ps = sig.blk_first[b], pt = tau.blk_first[b];
  int64_t ps_hi = sig.phi[ps], pt_hi = tau.phi[pt];
  // segments of the current pieces, read when a cursor moves (not per span,
  // so that no wait for them sits between a span's loads)
  int32_t js_cur = sig.pseg[ps], jt_cur = tau.pseg[pt];
  const int64_t rowbytes = G.W * 8;
  const float nf = (float)G.n;
  const bool pow2 = (G.n & (G.n - 1)) == 0;
  const float inv_n = 1.0f / nf;
  const bool stager = OBA_SRV_LDS != 0 && (int)threadIdx.x < NB * 32;
  double acc[1] = {0.0};
  for (int64_t s = s_lo; s < s_hi; ++s) {
    const int64_t lo = s * kSpan;
    if (OBA_SRV_PAIR != 0 && OBA_SRV_LDS != 0 && G.n <= NB && s + 1 < s_hi &&
        lo + 2 * kSpan <= G.d && lo + 2 * kSpan <= ps_hi && lo + 2 * kSpan <= pt_hi) {
      const int64_t lo1 = lo + kSpan, hi1 = lo1 + kSpan;
      const Quads q0 = quads(lo), q1 = quads(lo1);
      const int32_t js0 = js_cur;
      uint2 rv0 = make_uint2(0u, 0u), rv1 = make_uint2(0u, 0u);
      if (stager) {
        const int64_t r = min((int)(threadIdx.x >> 5), G.n - 1);
        const uint8_t* rb = wbytes + r * rowbytes + 8 * (threadIdx.x & 31);
        rv0 = *reinterpret_cast<const uint2*>(rb + (lo >> 3));
        rv1 = *reinterpret_cast<const uint2*>(rb + (lo1 >> 3));
      }
      float a0[8], a1[8];
      load_full(eps, q0, a0);
      load_full(eps, q1, a1);
      __syncthreads();  // the previous reads of the staged rows are done
      if (stager) {
        rows2_lds[0][threadIdx.x] = rv0;
        rows2_lds[1][threadIdx.x] = rv1;
      }
      __syncthreads();
      float sw[NB];
#pragma unroll
      for (int u = 0; u < NB; ++u) sw[u] = wscale[(int64_t)min(u, G.n - 1) * sig.n_seg + js0];
      const float sp = DEFERRED ? sscale_prev[jt_cur] : 0.0f;
      const uint32_t sh = (threadIdx.x & 1) ? 4u : 0u;
      // the single span's operations, in its order, for each of the two
      auto one = [&](const uint2* rows, float (&av)[8]) {
        const uint8_t* lb = reinterpret_cast<const uint8_t*>(rows);
        float t[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) t[j] = 0.0f;
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          const uint32_t ba = lb[u * 256 + (threadIdx.x >> 1)];
          const uint32_t bb = lb[u * 256 + 128 + (threadIdx.x >> 1)];
          const uint32_t bits = ((ba >> sh) & 0xFu) | (((bb >> sh) & 0xFu) << 4);
          if (u < G.n) {
#pragma unroll
            for (int j = 0; j < 8; ++j) t[j] = t[j] + (((bits >> j) & 1u) ? -sw[u] : sw[u]);
          }
        }
        if (DEFERRED) {
#pragma unroll
          for (int j = 0; j < 8; ++j) av[j] = residual(av[j], sp);
        }
        if (pow2) {
#pragma unroll
          for (int j = 0; j < 8; ++j) av[j] = t[j] * inv_n + av[j];
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) av[j] = t[j] / nf + av[j];
        }
      };
      one(rows2_lds[0], a0);
      one(rows2_lds[1], a1);
      store8(eps, q0, G.d, true, a0);
      store8(eps, q1, G.d, true, a1);
      store_sign_bits(sbytes, q0, sign_bits(a0), rowbytes);
      store_sign_bits(sbytes, q1, sign_bits(a1), rowbytes);
      acc[0] += sumsq8(a0);
      acc[0] += sumsq8(a1);
      // no piece ends inside the pair; one may end at its end
      while (ps < ps_end && ps_hi <= hi1) {
        if (++ps < ps_end) {
          ps_hi = sig.phi[ps];
          js_cur = sig.pseg[ps];
        }
      }
      if (hi1 == pt_hi) {
        flush_rows<1>(acc, 1, part + pt, 0, lds);
        if (++pt < pt_end) {
          pt_hi = tau.phi[pt];
          jt_cur = tau.pseg[pt];
        }
      }
      ++s;  // the loop's increment passes the second span
      continue;
    }
    const int64_t hi = min(lo + kSpan, G.d);
    const Quads q = quads(lo);
    float a[8];
    if (hi <= ps_hi && hi <= pt_hi && lo + kSpan <= G.d) {
      // fast path: full span, one worker and one server segment.  The first
      // group's packed rows are requested before a', so one wait covers both.
      const int32_t js0 = js_cur;
      uint2 rowv = make_uint2(0u, 0u);
      if constexpr (OBA_SRV_LDS != 0) {
        if (stager) {
          const int64_t r = min((int)(threadIdx.x >> 5), G.n - 1);
          rowv = *reinterpret_cast<const uint2*>(wbytes + r * rowbytes + (lo >> 3) +
                                                 8 * (threadIdx.x & 31));
        }
      }
      float t[8];
      load_full(eps, q, a);
#pragma unroll
      for (int j = 0; j < 8; ++j) t[j] = 0.0f;
      for (int32_t i0 = 0; i0 < G.n; i0 += NB) {  // one pass when n <= NB
        // rows past n are clamped to a valid row and their terms skipped
        uint32_t bits[NB];
        float sw[NB];
        if constexpr (OBA_SRV_LDS != 0) {
          if (i0 > 0 && stager) {
            const int64_t r = min(i0 + (int)(threadIdx.x >> 5), G.n - 1);
            rowv = *reinterpret_cast<const uint2*>(wbytes + r * rowbytes + (lo >> 3) +
                                                   8 * (threadIdx.x & 31));
          }
          __syncthreads();  // the previous reads of rows_lds are done
          if (stager) rows_lds[threadIdx.x] = rowv;
          __syncthreads();
          const uint8_t* lb = reinterpret_cast<const uint8_t*>(rows_lds);
          const uint32_t sh = (threadIdx.x & 1) ? 4u : 0u;
#pragma unroll
          for (int u = 0; u < NB; ++u) {
            const uint32_t ba = lb[u * 256 + (threadIdx.x >> 1)];
            const uint32_t bb = lb[u * 256 + 128 + (threadIdx.x >> 1)];
            bits[u] = ((ba >> sh) & 0xFu) | (((bb >> sh) & 0xFu) << 4);
            sw[u] = wscale[(int64_t)min(i0 + u, G.n - 1) * sig.n_seg + js0];
          }
        } else {
#pragma unroll
          for (int u = 0; u < NB; ++u) {
            const int64_t r = min(i0 + u, G.n - 1);
            bits[u] = load_sign_bits<true, false>(wbytes + r * rowbytes, q, G.d);
            sw[u] = wscale[r * sig.n_seg + js0];
          }
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          if (i0 + u < G.n) {
#pragma unroll
            for (int j = 0; j < 8; ++j) t[j] = t[j] + (((bits[u] >> j) & 1u) ? -sw[u] : sw[u]);
          }
        }
      }
      if (DEFERRED) {
        const float sp = sscale_prev[jt_cur];
#pragma unroll
        for (int j = 0; j < 8; ++j) a[j] = residual(a[j], sp);
      }
      if (pow2) {  // t * (1/n) is t / n exactly when n is a power of two
#pragma unroll
        for (int j = 0; j < 8; ++j) a[j] = t[j] * inv_n + a[j];
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) a[j] = t[j] / nf + a[j];
      }
      store8(eps, q, G.d, true, a);
    } else {
      // general path (a segment boundary in the span, or the tail): one
      // coordinate at a time, same operations in the same order
      int32_t js = js_cur;
      int32_t jt = jt_cur;
#pragma unroll 1
      for (int j = 0; j < 8; ++j) {
        const int64_t k = coord(q, j);
        a[j] = 0.0f;
        if (k < G.d) {
          js = seg_walk(sig.off, js, k);
          float e = eps[k];
          if (DEFERRED) {
            jt = seg_walk(tau.off, jt, k);
            e = residual(e, sscale_prev[jt]);
          }
          const uint32_t sh = (uint32_t)(k & 7);  // bit of k in its byte
          float t = 0.0f;
          for (int32_t i = 0; i < G.n; ++i) {
            const uint32_t byte = wbytes[(int64_t)i * rowbytes + (k >> 3)];
            const float s_ = wscale[(int64_t)i * sig.n_seg + js];
            t = t + (((byte >> sh) & 1u) ? -s_ : s_);
          }
          a[j] = t / nf + e;
          eps[k] = a[j];
        }
      }
    }
    store_sign_bits(sbytes, q, sign_bits(a), rowbytes);
    const double fs = sumsq8(a);  // coordinates past d hold 0
    // advance the worker-segment cursor to the piece holding hi
    while (ps < ps_end && ps_hi <= hi) {
      if (++ps < ps_end) {
        ps_hi = sig.phi[ps];
        js_cur = sig.pseg[ps];
      }
    }
    // server-segment reduction
    if (hi <= pt_hi) {
      acc[0] += fs;
      if (hi == pt_hi) {
        flush_rows<1>(acc, 1, part + pt, 0, lds);
        if (++pt < pt_end) {
          pt_hi = tau.phi[pt];
          jt_cur = tau.pseg[pt];
        }
      }
    } else {
      int64_t cur = lo;
      while (cur < hi) {
        const int64_t e = min(pt_hi, hi);
        acc[0] += sumsq_range(eps, q, cur, e);
        if (pt_hi <= hi) {
          flush_rows<1>(acc, 1, part + pt, 0, lds);
          if (++pt < pt_end) {
            pt_hi = tau.phi[pt];
            jt_cur = tau.pseg[pt];
          }
        }
        cur = e;
      }
    }
  }
}

// ---- launchers ----------------------------------------------------------------

void launch_residual(const Geo& G, const float* src, int64_t src_ld, float* dst, int64_t dst_ld,
                     int32_t rows, const float* scale, const SegDev& T, hipStream_t st) {
  hipLaunchKernelGGL(k_residual, dim3(G.nblk, rows), dim3(kBlock), 0, st, G, src, src_ld, dst,
                     dst_ld, scale, T);
}

// Occupancy cap of the deferred server pass (blocks per CU, 0: none), a
// tuning knob (3 blocks: 0.53 -> 0.71 ms, 4: 0.60 ms at bert_large; none
// kept).
#ifndef OBA_SRV_BPC
#define OBA_SRV_BPC 0
#endif

template <bool DEFERRED>
static void launch_server_t(const Geo& G, const uint8_t* wbytes, const float* wscale, float* eps,
                            uint8_t* sbytes, const SegDev& sig, const SegDev& tau, double* part,
                            const float* sscale_prev, hipStream_t st) {
  const size_t lds = DEFERRED ? occupancy_lds(OBA_SRV_BPC) : 0;
#define OBA_SERVER_LAUNCH(NB)                                                                   \
  do {                                                                                          \
    allow_lds(reinterpret_cast<const void*>(&k_server_p1<NB, DEFERRED>), lds);                 \
    hipLaunchKernelGGL((k_server_p1<NB, DEFERRED>), dim3(G.nblk), dim3(kBlock), lds, st, G,    \
                       wbytes, wscale, eps, sbytes, sig, tau, part, sscale_prev);               \
  } while (0)
  switch (G.n) {
    case 1: OBA_SERVER_LAUNCH(1); break;
    case 2: OBA_SERVER_LAUNCH(2); break;
    case 3: OBA_SERVER_LAUNCH(3); break;
    case 4: OBA_SERVER_LAUNCH(4); break;
    case 5: OBA_SERVER_LAUNCH(5); break;
    case 6: OBA_SERVER_LAUNCH(6); break;
    case 7: OBA_SERVER_LAUNCH(7); break;
    default: OBA_SERVER_LAUNCH(8); break;
  }
#undef OBA_SERVER_LAUNCH
}

void launch_server_p1(const Geo& G, const uint8_t* wbytes, const float* wscale, float* eps,
                      uint8_t* sbytes, const SegDev& sig, const SegDev& tau, double* part,
                      hipStream_t st) {
  launch_server_t<false>(G, wbytes, wscale, eps, sbytes, sig, tau, part, nullptr, st);
}

void launch_server_deferred(const Geo& G, const uint8_t* wbytes, const float* wscale, float* a,
                            uint8_t* sbytes, const SegDev& sig, const SegDev& tau, double* part,
                            const float* sscale_prev, hipStream_t st) {
  launch_server_t<true>(G, wbytes, wscale, a, sbytes, sig, tau, part, sscale_prev, st);
}

}  // namespace oba
