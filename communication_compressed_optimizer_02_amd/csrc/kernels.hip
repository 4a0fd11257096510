// kernels.hip -- HIP kernels of the 1-bit Adam compression-stage step, gfx950.
//
// All kernels are HBM-streaming: a few flops per byte, no contraction, so
// no matrix cores.  Every lane owns 8 consecutive coordinates, loaded as
// 16-byte vectors (two for binary32, one for binary16); the 8 sign bits of a
// lane form exactly one byte of the packed little-endian word array, so each
// lane writes its byte with one store and no cross-lane exchange.  A block
// walks a contiguous range of 2048-coordinate spans.  Sums of squares are
// binary64 per lane (the square of a binary32 value is exact there), reduced
// across the wave by a butterfly and across the 4 waves through LDS into one
// partial per (piece, row); a second tiny kernel sums a segment's partials in
// piece order.  No atomics: results are bitwise reproducible.
//
// Method passages are cited in include/oba.h beside each entry point.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace oba {

namespace {

// -------------------------------------------------------------------------
// 8-wide loads and stores with a guarded tail (coordinates >= d read as 0
// and are never written).  Row bases are 32-byte aligned for binary32 and
// 16-byte aligned for binary16 (16-byte-aligned base, ld % 8 == 0, k0 % 8 == 0).
// -------------------------------------------------------------------------
__device__ __forceinline__ void load8(const float* __restrict__ p, int64_t k0, int64_t d,
                                      float (&v)[8]) {
  if (k0 + 8 <= d) {
    const float4 a = *reinterpret_cast<const float4*>(p + k0);
    const float4 b = *reinterpret_cast<const float4*>(p + k0 + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (k0 + j < d) ? p[k0 + j] : 0.0f;
  }
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

__device__ __forceinline__ void load8(const uint16_t* __restrict__ p, int64_t k0, int64_t d,
                                      float (&v)[8]) {
  if (k0 + 8 <= d) {
    const uint4 a = *reinterpret_cast<const uint4*>(p + k0);
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = half_bits_to_float(w[j] & 0xFFFFu);
      v[2 * j + 1] = half_bits_to_float(w[j] >> 16);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (k0 + j < d) ? half_bits_to_float(p[k0 + j]) : 0.0f;
  }
}

__device__ __forceinline__ void store8(float* __restrict__ p, int64_t k0, int64_t d,
                                       const float (&v)[8]) {
  if (k0 + 8 <= d) {
    *reinterpret_cast<float4*>(p + k0) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + k0 + 4) = make_float4(v[4], v[5], v[6], v[7]);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (k0 + j < d) p[k0 + j] = v[j];
  }
}

__device__ __forceinline__ uint32_t sign_byte(const float (&c)[8]) {
  uint32_t b = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) b |= (c[j] < 0.0f ? 1u : 0u) << j;  // -0.0 gives 0 (+1)
  return b;
}

__device__ __forceinline__ double sumsq8(const float (&c)[8]) {
  double s = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const double x = (double)c[j];
    s = __builtin_fma(x, x, s);  // x*x is exact in binary64, so fma == mul+add
  }
  return s;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;  // every lane holds the same value (commutative butterfly)
}

// Block-reduce acc[0..nw) and write dst[0..nw); resets acc.  Uniform call.
template <int NB>
__device__ __forceinline__ void flush_rows(double (&acc)[NB], int nw, double* __restrict__ dst,
                                           double* lds) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    if (i < nw) {
      const double s = wave_sum(acc[i]);
      if (lane == 0) lds[wv * NB + i] = s;
    }
    acc[i] = 0.0;
  }
  __syncthreads();
  if ((int)threadIdx.x < nw) {
    const int i = threadIdx.x;
    dst[i] = ((lds[i] + lds[NB + i]) + lds[2 * NB + i]) + lds[3 * NB + i];
  }
  __syncthreads();
}

// First span of block b (same split as the host planner's span_begin).
__device__ __forceinline__ int64_t dspan(int64_t S, int32_t nblk, int32_t b) {
  return (int64_t)b * S / nblk;
}

// Segment of coordinate k, walking forward from segment j0 (k >= off[j0]).
__device__ __forceinline__ int32_t seg_walk(const int64_t* __restrict__ off, int32_t j0,
                                            int64_t k) {
  int32_t j = j0;
  while (off[j + 1] <= k) ++j;
  return j;
}

// Sum of squares of row[k] for the lane's coordinates k in [a, e).
__device__ __forceinline__ double sumsq_range(const float* row, int64_t k0, int64_t a,
                                              int64_t e) {
  double s = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t k = k0 + j;
    if (k >= a && k < e) {
      const double x = (double)row[k];
      s = __builtin_fma(x, x, s);
    }
  }
  return s;
}

}  // namespace

// ===========================================================================
// Warm-up Adam step on the mean gradient.
// ===========================================================================
template <typename GT>
__global__ __launch_bounds__(kBlock) void k_adam_warmup(Geo G, const GT* __restrict__ g,
                                                        float* __restrict__ x,
                                                        float* __restrict__ m,
                                                        float* __restrict__ v, AdamCoef C) {
  const int64_t s_lo = dspan(G.S, G.nblk, blockIdx.x);
  const int64_t s_hi = dspan(G.S, G.nblk, blockIdx.x + 1);
  const float nf = (float)G.n;
  for (int64_t s = s_lo; s < s_hi; ++s) {
    const int64_t k0 = s * kSpan + (int64_t)threadIdx.x * kVec;
    if (k0 >= G.d) continue;
    float sum[8], gv[8], mv[8], vv[8], xv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) sum[j] = 0.0f;
    for (int32_t i = 0; i < G.n; ++i) {
      load8(g + (int64_t)i * G.ld, k0, G.d, gv);
#pragma unroll
      for (int j = 0; j < 8; ++j) sum[j] = sum[j] + gv[j];
    }
    load8(m, k0, G.d, mv);
    load8(v, k0, G.d, vv);
    load8(x, k0, G.d, xv);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float gb = sum[j] / nf;
      const float mk = C.b1 * mv[j] + C.omb1 * gb;
      const float vk = C.b2 * vv[j] + C.omb2 * (gb * gb);
      mv[j] = mk;
      vv[j] = vk;
      xv[j] = xv[j] - (C.lr * (mk / C.bc1)) / (__builtin_sqrtf(vk / C.bc2) + C.eta);
    }
    store8(m, k0, G.d, mv);
    store8(v, k0, G.d, vv);
    store8(x, k0, G.d, xv);
  }
}

// ===========================================================================
// Variance freeze: denom = sqrt(v / bc2) + eta.
// ===========================================================================
__global__ __launch_bounds__(kBlock) void k_freeze(Geo G, const float* __restrict__ v,
                                                   float* __restrict__ denom, float eta,
                                                   float bc2) {
  const int64_t s_lo = dspan(G.S, G.nblk, blockIdx.x);
  const int64_t s_hi = dspan(G.S, G.nblk, blockIdx.x + 1);
  for (int64_t s = s_lo; s < s_hi; ++s) {
    const int64_t k0 = s * kSpan + (int64_t)threadIdx.x * kVec;
    if (k0 >= G.d) continue;
    float vv[8];
    load8(v, k0, G.d, vv);
#pragma unroll
    for (int j = 0; j < 8; ++j) vv[j] = __builtin_sqrtf(vv[j] / bc2) + eta;
    store8(denom, k0, G.d, vv);
  }
}

// ===========================================================================
// Worker pass 1: c = (b1*m + (1-b1)*g_i) + delta_i for NB workers at once
// (m is read once per coordinate), c stored over delta_i, sign byte stored,
// binary64 sum of c^2 reduced per (piece, worker).
// Grid: (nblk, ceil(n/NB)); block y handles workers [y*NB, y*NB+nw).
// ===========================================================================
template <typename GT, int NB>
__global__ __launch_bounds__(kBlock) void k_compress_p1(Geo G, const GT* __restrict__ g,
                                                        const float* __restrict__ m,
                                                        float* __restrict__ delta,
                                                        uint8_t* __restrict__ wbytes, SegDev sig,
                                                        double* __restrict__ part, float b1,
                                                        float omb1) {
  __shared__ double lds[4 * NB];
  const int32_t b = blockIdx.x;
  const int32_t i0 = blockIdx.y * NB;
  const int nw = min(NB, G.n - i0);
  const int64_t s_lo = dspan(G.S, G.nblk, b), s_hi = dspan(G.S, G.nblk, b + 1);
  const int32_t p_end = sig.blk_first[b + 1];
  int32_t p = sig.blk_first[b];
  int64_t p_hi = sig.phi[p];
  const int64_t rowbytes = G.W * 8;
  double acc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) acc[i] = 0.0;

  for (int64_t s = s_lo; s < s_hi; ++s) {
    const int64_t lo = s * kSpan;
    const int64_t hi = min(lo + kSpan, G.d);
    const int64_t k0 = lo + (int64_t)threadIdx.x * kVec;
    float mv[8];
    load8(m, k0, G.d, mv);
    double fs[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      fs[i] = 0.0;
      if (i < nw) {
        const int64_t row = (int64_t)(i0 + i) * G.ld;
        float gv[8], c[8];
        load8(g + row, k0, G.d, gv);
        load8(delta + row, k0, G.d, c);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float pj = b1 * mv[j] + omb1 * gv[j];
          c[j] = pj + c[j];
        }
        store8(delta + row, k0, G.d, c);
        if (k0 < 64 * G.W) wbytes[(int64_t)(i0 + i) * rowbytes + (k0 >> 3)] = (uint8_t)sign_byte(c);
        fs[i] = sumsq8(c);
      }
    }
    if (hi <= p_hi) {  // span inside the current piece
#pragma unroll
      for (int i = 0; i < NB; ++i) acc[i] += fs[i];
      if (hi == p_hi) {
        flush_rows<NB>(acc, nw, part + (int64_t)p * G.n + i0, lds);
        if (++p < p_end) p_hi = sig.phi[p];
      }
    } else {  // span crosses piece boundaries: re-read this lane's c from delta
      int64_t cur = lo;
      while (cur < hi) {
        const int64_t e = min(p_hi, hi);
#pragma unroll
        for (int i = 0; i < NB; ++i)
          if (i < nw) acc[i] += sumsq_range(delta + (int64_t)(i0 + i) * G.ld, k0, cur, e);
        if (p_hi <= hi) {
          flush_rows<NB>(acc, nw, part + (int64_t)p * G.n + i0, lds);
          if (++p < p_end) p_hi = sig.phi[p];
        }
        cur = e;
      }
    }
  }
}

// ===========================================================================
// Per-segment scale from the piece partials: s = sqrt(S / len) in binary64,
// rounded once to binary32.  Grid: (n_seg, rows).  part: [n_pieces][rows].
// ===========================================================================
__global__ __launch_bounds__(kBlock) void k_finalize_scales(const double* __restrict__ part,
                                                            int32_t rows, SegDev T,
                                                            float* __restrict__ scale) {
  __shared__ double lds[4];
  const int32_t j = blockIdx.x, r = blockIdx.y;
  const int32_t q0 = T.seg_first[j], q1 = T.seg_first[j + 1];
  double t = 0.0;
  for (int32_t q = q0 + threadIdx.x; q < q1; q += kBlock) t += part[(int64_t)q * rows + r];
  t = wave_sum(t);
  if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = t;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double S = ((lds[0] + lds[1]) + lds[2]) + lds[3];
    const double len = (double)(T.off[j + 1] - T.off[j]);
    scale[(int64_t)r * T.n_seg + j] = (float)__builtin_sqrt(S / len);
  }
}

// ===========================================================================
// Residual pass: err = c - s*sign(c) over one row, s = the row's scale of the
// segment holding each coordinate.  Grid: (nblk, rows); row r at base + r*ld.
// ===========================================================================
__global__ __launch_bounds__(kBlock) void k_residual(Geo G, float* __restrict__ buf, int64_t ld,
                                                     const float* __restrict__ scale, SegDev T) {
  const int32_t b = blockIdx.x;
  float* row = buf + (int64_t)blockIdx.y * ld;
  const float* sc = scale + (int64_t)blockIdx.y * T.n_seg;
  const int64_t s_lo = dspan(G.S, G.nblk, b), s_hi = dspan(G.S, G.nblk, b + 1);
  const int32_t p_end = T.blk_first[b + 1];
  int32_t p = T.blk_first[b];
  int64_t p_hi = T.phi[p];
  for (int64_t s = s_lo; s < s_hi; ++s) {
    const int64_t lo = s * kSpan;
    const int64_t hi = min(lo + kSpan, G.d);
    const int64_t k0 = lo + (int64_t)threadIdx.x * kVec;
    if (k0 < G.d) {
      float c[8], sv[8];
      load8(row, k0, G.d, c);
      if (hi <= p_hi) {
        const float s_ = sc[T.pseg[p]];
#pragma unroll
        for (int j = 0; j < 8; ++j) sv[j] = s_;
      } else {
        int32_t js = T.pseg[p];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (k0 + j < G.d) js = seg_walk(T.off, js, k0 + j);
          sv[j] = sc[js];
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = (c[j] < 0.0f) ? c[j] + sv[j] : c[j] - sv[j];
      store8(row, k0, G.d, c);
    }
    while (p < p_end && p_hi <= hi) {
      if (++p < p_end) p_hi = T.phi[p];
    }
  }
}

// ===========================================================================
// Server pass 1: a = (sum_i s_i*sign_i)/n + eps per coordinate (workers in
// order), a stored over eps, server sign byte stored, binary64 sum of a^2
// reduced per server piece.  Grid: nblk.
// ===========================================================================
__global__ __launch_bounds__(kBlock) void k_server_p1(Geo G, const uint8_t* __restrict__ wbytes,
                                                      const float* __restrict__ wscale,
                                                      float* __restrict__ eps,
                                                      uint8_t* __restrict__ sbytes, SegDev sig,
                                                      SegDev tau, double* __restrict__ part) {
  __shared__ double lds[4];
  const int32_t b = blockIdx.x;
  const int64_t s_lo = dspan(G.S, G.nblk, b), s_hi = dspan(G.S, G.nblk, b + 1);
  const int32_t ps_end = sig.blk_first[b + 1], pt_end = tau.blk_first[b + 1];
  int32_t ps = sig.blk_first[b], pt = tau.blk_first[b];
  int64_t ps_hi = sig.phi[ps], pt_hi = tau.phi[pt];
  const int64_t rowbytes = G.W * 8;
  const float nf = (float)G.n;
  double acc[1] = {0.0};
  for (int64_t s = s_lo; s < s_hi; ++s) {
    const int64_t lo = s * kSpan;
    const int64_t hi = min(lo + kSpan, G.d);
    const int64_t k0 = lo + (int64_t)threadIdx.x * kVec;
    double fs = 0.0;
    if (k0 < G.d) {
      float ev[8], t[8];
      load8(eps, k0, G.d, ev);
#pragma unroll
      for (int j = 0; j < 8; ++j) t[j] = 0.0f;
      const int64_t q = k0 >> 3;
      if (hi <= ps_hi) {  // one worker segment for the whole span
        const int32_t js = sig.pseg[ps];
        for (int32_t i = 0; i < G.n; ++i) {
          const uint32_t byte = wbytes[(int64_t)i * rowbytes + q];
          const float s_ = wscale[(int64_t)i * sig.n_seg + js];
#pragma unroll
          for (int j = 0; j < 8; ++j) t[j] = t[j] + (((byte >> j) & 1u) ? -s_ : s_);
        }
      } else {
        int32_t jseg[8];
        int32_t js = sig.pseg[ps];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (k0 + j < G.d) js = seg_walk(sig.off, js, k0 + j);
          jseg[j] = js;
        }
        for (int32_t i = 0; i < G.n; ++i) {
          const uint32_t byte = wbytes[(int64_t)i * rowbytes + q];
          const float* sc = wscale + (int64_t)i * sig.n_seg;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float s_ = sc[jseg[j]];
            t[j] = t[j] + (((byte >> j) & 1u) ? -s_ : s_);
          }
        }
      }
      float a[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) a[j] = (k0 + j < G.d) ? t[j] / nf + ev[j] : 0.0f;
      store8(eps, k0, G.d, a);
      sbytes[q] = (uint8_t)sign_byte(a);
      fs = sumsq8(a);
    } else if (k0 < 64 * G.W) {
      sbytes[k0 >> 3] = 0;
    }
    // advance the worker-segment cursor to the piece holding hi
    while (ps < ps_end && ps_hi <= hi) {
      if (++ps < ps_end) ps_hi = sig.phi[ps];
    }
    // server-segment reduction
    if (hi <= pt_hi) {
      acc[0] += fs;
      if (hi == pt_hi) {
        flush_rows<1>(acc, 1, part + pt, lds);
        if (++pt < pt_end) pt_hi = tau.phi[pt];
      }
    } else {
      int64_t cur = lo;
      while (cur < hi) {
        const int64_t e = min(pt_hi, hi);
        acc[0] += sumsq_range(eps, k0, cur, e);
        if (pt_hi <= hi) {
          flush_rows<1>(acc, 1, part + pt, lds);
          if (++pt < pt_end) pt_hi = tau.phi[pt];
        }
        cur = e;
      }
    }
  }
}

// ===========================================================================
// Decompress + precondition + update: m_hat = sbar*sign; m = m_hat;
// x = x - (lr*m_hat)/denom.  Grid: nblk.
// ===========================================================================
__global__ __launch_bounds__(kBlock) void k_decompress_update(Geo G,
                                                              const uint8_t* __restrict__ sbytes,
                                                              const float* __restrict__ sscale,
                                                              const float* __restrict__ denom,
                                                              float* __restrict__ m,
                                                              float* __restrict__ x, SegDev tau,
                                                              float lr) {
  const int32_t b = blockIdx.x;
  const int64_t s_lo = dspan(G.S, G.nblk, b), s_hi = dspan(G.S, G.nblk, b + 1);
  const int32_t p_end = tau.blk_first[b + 1];
  int32_t p = tau.blk_first[b];
  int64_t p_hi = tau.phi[p];
  for (int64_t s = s_lo; s < s_hi; ++s) {
    const int64_t lo = s * kSpan;
    const int64_t hi = min(lo + kSpan, G.d);
    const int64_t k0 = lo + (int64_t)threadIdx.x * kVec;
    if (k0 < G.d) {
      float sv[8], dv[8], xv[8], mh[8];
      if (hi <= p_hi) {
        const float s_ = sscale[tau.pseg[p]];
#pragma unroll
        for (int j = 0; j < 8; ++j) sv[j] = s_;
      } else {
        int32_t js = tau.pseg[p];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (k0 + j < G.d) js = seg_walk(tau.off, js, k0 + j);
          sv[j] = sscale[js];
        }
      }
      const uint32_t byte = sbytes[k0 >> 3];
      load8(denom, k0, G.d, dv);
      load8(x, k0, G.d, xv);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        mh[j] = ((byte >> j) & 1u) ? -sv[j] : sv[j];
        xv[j] = xv[j] - (lr * mh[j]) / dv[j];
      }
      store8(m, k0, G.d, mh);
      store8(x, k0, G.d, xv);
    }
    while (p < p_end && p_hi <= hi) {
      if (++p < p_end) p_hi = tau.phi[p];
    }
  }
}

// ===========================================================================
// launchers
// ===========================================================================
template <typename GT>
static void launch_warmup(const Geo& G, const void* g, float* x, float* m, float* v,
                          const AdamCoef& C, hipStream_t st) {
  hipLaunchKernelGGL(k_adam_warmup<GT>, dim3(G.nblk), dim3(kBlock), 0, st, G,
                     static_cast<const GT*>(g), x, m, v, C);
}

void launch_adam_warmup(const Geo& G, const void* g, bool f16, float* x, float* m, float* v,
                        const AdamCoef& C, hipStream_t st) {
  if (f16)
    launch_warmup<uint16_t>(G, g, x, m, v, C, st);
  else
    launch_warmup<float>(G, g, x, m, v, C, st);
}

void launch_freeze(const Geo& G, const float* v, float* denom, float eta, float bc2,
                   hipStream_t st) {
  hipLaunchKernelGGL(k_freeze, dim3(G.nblk), dim3(kBlock), 0, st, G, v, denom, eta, bc2);
}

template <typename GT, int NB>
static void launch_p1_nb(const Geo& G, const void* g, const float* m, float* delta,
                         uint8_t* wbytes, const SegDev& sig, double* part, float b1, float omb1,
                         hipStream_t st) {
  const int groups = (G.n + NB - 1) / NB;
  hipLaunchKernelGGL((k_compress_p1<GT, NB>), dim3(G.nblk, groups), dim3(kBlock), 0, st, G,
                     static_cast<const GT*>(g), m, delta, wbytes, sig, part, b1, omb1);
}

template <typename GT>
static void launch_p1_t(const Geo& G, const void* g, const float* m, float* delta,
                        uint8_t* wbytes, const SegDev& sig, double* part, float b1, float omb1,
                        hipStream_t st) {
  if (G.n == 1)
    launch_p1_nb<GT, 1>(G, g, m, delta, wbytes, sig, part, b1, omb1, st);
  else if (G.n == 2)
    launch_p1_nb<GT, 2>(G, g, m, delta, wbytes, sig, part, b1, omb1, st);
  else if (G.n <= 4)
    launch_p1_nb<GT, 4>(G, g, m, delta, wbytes, sig, part, b1, omb1, st);
  else
    launch_p1_nb<GT, 8>(G, g, m, delta, wbytes, sig, part, b1, omb1, st);
}

void launch_compress_p1(const Geo& G, const void* g, bool f16, const float* m, float* delta,
                        uint8_t* wbytes, const SegDev& sig, double* part, float b1, float omb1,
                        hipStream_t st) {
  if (f16)
    launch_p1_t<uint16_t>(G, g, m, delta, wbytes, sig, part, b1, omb1, st);
  else
    launch_p1_t<float>(G, g, m, delta, wbytes, sig, part, b1, omb1, st);
}

void launch_finalize(const double* part, int32_t rows, const SegDev& T, float* scale,
                     hipStream_t st) {
  hipLaunchKernelGGL(k_finalize_scales, dim3(T.n_seg, rows), dim3(kBlock), 0, st, part, rows, T,
                     scale);
}

void launch_residual(const Geo& G, float* buf, int64_t ld, int32_t rows, const float* scale,
                     const SegDev& T, hipStream_t st) {
  hipLaunchKernelGGL(k_residual, dim3(G.nblk, rows), dim3(kBlock), 0, st, G, buf, ld, scale, T);
}

void launch_server_p1(const Geo& G, const uint8_t* wbytes, const float* wscale, float* eps,
                      uint8_t* sbytes, const SegDev& sig, const SegDev& tau, double* part,
                      hipStream_t st) {
  hipLaunchKernelGGL(k_server_p1, dim3(G.nblk), dim3(kBlock), 0, st, G, wbytes, wscale, eps,
                     sbytes, sig, tau, part);
}

void launch_decompress_update(const Geo& G, const uint8_t* sbytes, const float* sscale,
                              const float* denom, float* m, float* x, const SegDev& tau, float lr,
                              hipStream_t st) {
  hipLaunchKernelGGL(k_decompress_update, dim3(G.nblk), dim3(kBlock), 0, st, G, sbytes, sscale,
                     denom, m, x, tau, lr);
}

}  // namespace oba
