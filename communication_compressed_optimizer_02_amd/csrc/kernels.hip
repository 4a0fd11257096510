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
// Streamed inputs are read with the nontemporal hint: every byte is used once
// per pass, so there is nothing for the caches to keep.
// -------------------------------------------------------------------------
#ifndef OBA_NT_LOADS
#define OBA_NT_LOADS 1
#endif
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename V>
__device__ __forceinline__ V ldv(const V* p) {
  if constexpr (OBA_NT_LOADS) return __builtin_nontemporal_load(p);
  else return *p;
}

__device__ __forceinline__ void load8(const float* __restrict__ p, int64_t k0, int64_t d,
                                      float (&v)[8]) {
  if (k0 + 8 <= d) {
    const f32x4 a = ldv(reinterpret_cast<const f32x4*>(p + k0));
    const f32x4 b = ldv(reinterpret_cast<const f32x4*>(p + k0 + 4));
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
    const u32x4 a = ldv(reinterpret_cast<const u32x4*>(p + k0));
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

__device__ __forceinline__ float grad_at(const float* p, int64_t k) { return p[k]; }
__device__ __forceinline__ float grad_at(const uint16_t* p, int64_t k) {
  return half_bits_to_float(p[k]);
}

// Full-span loaders: no tail check, so a kernel can issue every load of a
// span before it uses any of them (a checked load is followed by its wait).
__device__ __forceinline__ void load8_full(const float* __restrict__ p, int64_t k0,
                                           float (&v)[8]) {
  const f32x4 a = ldv(reinterpret_cast<const f32x4*>(p + k0));
  const f32x4 b = ldv(reinterpret_cast<const f32x4*>(p + k0 + 4));
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void load8_full(const uint16_t* __restrict__ p, int64_t k0,
                                           float (&v)[8]) {
  const u32x4 a = ldv(reinterpret_cast<const u32x4*>(p + k0));
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = half_bits_to_float(w[j] & 0xFFFFu);
    v[2 * j + 1] = half_bits_to_float(w[j] >> 16);
  }
}

// c = (b1*m + (1-b1)*g) + delta: two products, then two adds (no contraction)
__device__ __forceinline__ float compensate(float b1, float omb1, float m, float g, float dl) {
  const float p = b1 * m + omb1 * g;
  return p + dl;
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

// Same, recomputing c = compensate(m, g, delta) from the inputs.
template <typename GT>
__device__ __forceinline__ double sumsq_range_c(const float* m, const GT* grow, const float* drow,
                                                float b1, float omb1, int64_t k0, int64_t a,
                                                int64_t e) {
  double s = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t k = k0 + j;
    if (k >= a && k < e) {
      const double x = (double)compensate(b1, omb1, m[k], grad_at(grow, k), drow[k]);
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
    const bool full = k0 + 8 <= G.d;
    float sum[8], mv[8], vv[8], xv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) sum[j] = 0.0f;
    for (int32_t i0 = 0; i0 < G.n; i0 += 4) {
      // four rows loaded together (rows past n clamped, their terms skipped)
      float gv[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const GT* row = g + (int64_t)min(i0 + u, G.n - 1) * G.ld;
        if (full)
          load8_full(row, k0, gv[u]);
        else
          load8(row, k0, G.d, gv[u]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (i0 + u < G.n) {
#pragma unroll
          for (int j = 0; j < 8; ++j) sum[j] = sum[j] + gv[u][j];
        }
    }
    if (full) {
      load8_full(m, k0, mv);
      load8_full(v, k0, vv);
      load8_full(x, k0, xv);
    } else {
      load8(m, k0, G.d, mv);
      load8(v, k0, G.d, vv);
      load8(x, k0, G.d, xv);
    }
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
    if (k0 + 8 <= G.d)
      load8_full(v, k0, vv);
    else
      load8(v, k0, G.d, vv);
#pragma unroll
    for (int j = 0; j < 8; ++j) vv[j] = __builtin_sqrtf(vv[j] / bc2) + eta;
    store8(denom, k0, G.d, vv);
  }
}

// ===========================================================================
// Worker side, for NB workers at once (m is read once per coordinate):
//   c = (b1*m + (1-b1)*g_i) + delta_i
// kNorm:  only reduce sum c^2 per (piece, worker) -- reads only;
// kApply: recompute c bit for bit, store the sign byte and
//         delta_i = c - s*sign(c) with the finished scales;
// kDeferred: the state row holds the previous step's c (not delta) and the
//         scale buffer its scales s'; the residual of the last step is formed
//         where it is consumed, delta_i = c' - s'*sign(c'), then
//         c = (b1*m + (1-b1)*g_i) + delta_i is stored over c' with its sign
//         byte and its sum c^2 is reduced -- one pass instead of two.
// The scale needs the whole segment's norm before any residual can be
// written, so c is needed twice.  Recomputing it reads g, m, delta twice but
// never writes c: on this HBM, writes cost more than reads, and storing c in
// a first pass to re-read it was measured 15 % slower per step.
// NB is the exact number of workers of a block: a launch covers workers
// [i0, i0 + gridDim.y*NB); n > 8 takes one launch of NB=8 groups and one
// for the remainder.  Grid: (nblk, groups).
// ===========================================================================
enum { kNorm = 1, kApply = 2, kDeferred = 3 };

template <typename GT, int NB, int MODE>
__global__ __launch_bounds__(kBlock) void k_compress(Geo G, int32_t i0, const GT* __restrict__ g,
                                                     const float* __restrict__ m,
                                                     float* __restrict__ delta,
                                                     uint8_t* __restrict__ wbytes, SegDev sig,
                                                     double* __restrict__ part,
                                                     const float* __restrict__ wscale, float b1,
                                                     float omb1) {
  __shared__ double lds[4 * NB];
  const int32_t b = blockIdx.x;
  i0 += blockIdx.y * NB;  // this block's workers: [i0, i0 + NB)
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
    const bool uniform = hi <= p_hi;  // span inside the current piece
    const bool full = lo + kSpan <= G.d;
    int32_t jseg[8];
    if ((MODE == kApply || MODE == kDeferred) && !uniform) {
      int32_t js = sig.pseg[p];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (k0 + j < G.d) js = seg_walk(sig.off, js, k0 + j);
        jseg[j] = js;
      }
    }
    // every load of the span first (all NB workers), then the arithmetic
    float mv[8], gv[NB][8], c[NB][8];
    if (full) {
      load8_full(m, k0, mv);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int64_t row = (int64_t)(i0 + i) * G.ld;
        load8_full(g + row, k0, gv[i]);
        load8_full(delta + row, k0, c[i]);
      }
    } else {
      load8(m, k0, G.d, mv);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int64_t row = (int64_t)(i0 + i) * G.ld;
        load8(g + row, k0, G.d, gv[i]);
        load8(delta + row, k0, G.d, c[i]);
      }
    }
    double fs[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int64_t row = (int64_t)(i0 + i) * G.ld;
      if (MODE == kDeferred) {  // c[i] holds c' of the last step: form its residual
        const float* sc = wscale + (int64_t)(i0 + i) * sig.n_seg;
        float sv[8];
        if (uniform) {
          const float s_ = sc[sig.pseg[p]];
#pragma unroll
          for (int j = 0; j < 8; ++j) sv[j] = s_;
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) sv[j] = sc[jseg[j]];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) c[i][j] = (c[i][j] < 0.0f) ? c[i][j] + sv[j] : c[i][j] - sv[j];
        if (!full) {  // coordinates past d read as 0 and must stay 0 (no bit, no c^2)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (k0 + j >= G.d) c[i][j] = 0.0f;
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) c[i][j] = compensate(b1, omb1, mv[j], gv[i][j], c[i][j]);
      if (MODE != kNorm && k0 < 64 * G.W)
        wbytes[(int64_t)(i0 + i) * rowbytes + (k0 >> 3)] = (uint8_t)sign_byte(c[i]);
      if (MODE == kDeferred) store8(delta + row, k0, G.d, c[i]);
      fs[i] = (MODE != kApply) ? sumsq8(c[i]) : 0.0;
      if (MODE == kApply) {
        const float* sc = wscale + (int64_t)(i0 + i) * sig.n_seg;
        float sv[8];
        if (uniform) {
          const float s_ = sc[sig.pseg[p]];
#pragma unroll
          for (int j = 0; j < 8; ++j) sv[j] = s_;
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) sv[j] = sc[jseg[j]];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) c[i][j] = (c[i][j] < 0.0f) ? c[i][j] + sv[j] : c[i][j] - sv[j];
        store8(delta + row, k0, G.d, c[i]);
      }
    }
    if (MODE == kApply) {
      while (p < p_end && p_hi <= hi) {
        if (++p < p_end) p_hi = sig.phi[p];
      }
    } else if (uniform) {
#pragma unroll
      for (int i = 0; i < NB; ++i) acc[i] += fs[i];
      if (hi == p_hi) {
        flush_rows<NB>(acc, NB, part + (int64_t)p * G.n + i0, lds);
        if (++p < p_end) p_hi = sig.phi[p];
      }
    } else {  // span crosses piece boundaries: sum this lane's c piece by piece
      int64_t cur = lo;
      while (cur < hi) {
        const int64_t e = min(p_hi, hi);
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const int64_t row = (int64_t)(i0 + i) * G.ld;
          if (MODE == kDeferred)
            acc[i] += sumsq_range(delta + row, k0, cur, e);  // c was stored there
          else
            acc[i] += sumsq_range_c(m, g + row, delta + row, b1, omb1, k0, cur, e);
        }
        if (p_hi <= hi) {
          flush_rows<NB>(acc, NB, part + (int64_t)p * G.n + i0, lds);
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
constexpr int kFinBlock = 1024;  // 16 waves: segments can have 65536 pieces

__global__ __launch_bounds__(kFinBlock) void k_finalize_scales(const double* __restrict__ part,
                                                               int32_t rows, SegDev T,
                                                               float* __restrict__ scale) {
  __shared__ double lds[kFinBlock / 64];
  const int32_t j = blockIdx.x, r = blockIdx.y;
  const int32_t q0 = T.seg_first[j], q1 = T.seg_first[j + 1];
  double t = 0.0;
  for (int32_t q = q0 + threadIdx.x; q < q1; q += kFinBlock) t += part[(int64_t)q * rows + r];
  t = wave_sum(t);
  if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = t;
  __syncthreads();
  if (threadIdx.x == 0) {
    double S = 0.0;
    for (int w = 0; w < kFinBlock / 64; ++w) S += lds[w];  // fixed order
    const double len = (double)(T.off[j + 1] - T.off[j]);
    scale[(int64_t)r * T.n_seg + j] = (float)__builtin_sqrt(S / len);
  }
}

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
      if (lo + kSpan <= G.d)
        load8_full(srow, k0, c);
      else
        load8(srow, k0, G.d, c);
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
      store8(drow, k0, G.d, c);
    }
    while (p < p_end && p_hi <= hi) {
      if (++p < p_end) p_hi = T.phi[p];
    }
  }
}

// ===========================================================================
// Server pass 1: a = (sum_i s_i*sign_i)/n + eps per coordinate (workers in
// order), a stored over eps, server sign byte stored, binary64 sum of a^2
// reduced per server piece.  The sign bytes and scales of NB workers are
// loaded before any is used, so their loads overlap (NB = n for n <= 8, else
// groups of 8).  DEFERRED: the buffer holds the last step's a' and
// sscale_prev its server scales; the server error is formed where it is
// consumed, eps = a' - s'*sign(a'), and a is stored over a'.  Grid: nblk.
// ===========================================================================
template <int NB, bool DEFERRED>
__global__ __launch_bounds__(kBlock) void k_server_p1(Geo G, const uint8_t* __restrict__ wbytes,
                                                      const float* __restrict__ wscale,
                                                      float* __restrict__ eps,
                                                      uint8_t* __restrict__ sbytes, SegDev sig,
                                                      SegDev tau, double* __restrict__ part,
                                                      const float* __restrict__ sscale_prev) {
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
    const int64_t q = k0 >> 3;
    if (hi <= ps_hi && hi <= pt_hi && lo + kSpan <= G.d) {
      // fast path: full span, one worker and one server segment; loads first
      const int32_t js0 = sig.pseg[ps];
      float ev[8], t[8];
      load8_full(eps, k0, ev);
      if (DEFERRED) {
        const float sp = sscale_prev[tau.pseg[pt]];
#pragma unroll
        for (int j = 0; j < 8; ++j) ev[j] = (ev[j] < 0.0f) ? ev[j] + sp : ev[j] - sp;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) t[j] = 0.0f;
      for (int32_t i0 = 0; i0 < G.n; i0 += NB) {  // one pass when n <= NB
        // rows past n are clamped to a valid row and their terms skipped
        uint32_t byte[NB];
        float sw[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          const int64_t r = min(i0 + u, G.n - 1);
          byte[u] = wbytes[r * rowbytes + q];
          sw[u] = wscale[r * sig.n_seg + js0];
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          if (i0 + u < G.n) {
#pragma unroll
            for (int j = 0; j < 8; ++j) t[j] = t[j] + (((byte[u] >> j) & 1u) ? -sw[u] : sw[u]);
          }
        }
      }
      float a[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) a[j] = t[j] / nf + ev[j];
      store8(eps, k0, G.d, a);
      sbytes[q] = (uint8_t)sign_byte(a);
      fs = sumsq8(a);
    } else if (k0 < G.d) {
      // general path (segment boundary in the span, or the tail): one
      // coordinate at a time, same operations in the same order
      uint32_t sb = 0;
      int32_t js = sig.pseg[ps];
      int32_t jt = tau.pseg[pt];
#pragma unroll 1
      for (int j = 0; j < 8; ++j) {
        const int64_t k = k0 + j;
        if (k < G.d) {
          js = seg_walk(sig.off, js, k);
          float e = eps[k];
          if (DEFERRED) {
            jt = seg_walk(tau.off, jt, k);
            const float sp = sscale_prev[jt];
            e = (e < 0.0f) ? e + sp : e - sp;
          }
          float t = 0.0f;
          for (int32_t i = 0; i < G.n; ++i) {
            const uint32_t byte = wbytes[(int64_t)i * rowbytes + q];
            const float s_ = wscale[(int64_t)i * sig.n_seg + js];
            t = t + (((byte >> j) & 1u) ? -s_ : s_);
          }
          const float a = t / nf + e;
          eps[k] = a;
          sb |= (a < 0.0f ? 1u : 0u) << j;
          const double x = (double)a;
          fs = __builtin_fma(x, x, fs);
        }
      }
      sbytes[q] = (uint8_t)sb;
    } else if (k0 < 64 * G.W) {
      sbytes[q] = 0;
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
      if (lo + kSpan <= G.d) {
        load8_full(denom, k0, dv);
        load8_full(x, k0, xv);
      } else {
        load8(denom, k0, G.d, dv);
        load8(x, k0, G.d, xv);
      }
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

template <typename GT, int NB, int MODE>
static void launch_cmp(const Geo& G, int32_t i0, int groups, const void* g, const float* m,
                       float* delta, uint8_t* wbytes, const SegDev& sig, double* part,
                       const float* wscale, float b1, float omb1, hipStream_t st) {
  hipLaunchKernelGGL((k_compress<GT, NB, MODE>), dim3(G.nblk, groups), dim3(kBlock), 0, st, G,
                     i0, static_cast<const GT*>(g), m, delta, wbytes, sig, part, wscale, b1,
                     omb1);
}

// groups of 8 workers, then one launch for the n % 8 remainder
template <typename GT, int MODE>
static void launch_cmp_n(const Geo& G, const void* g, const float* m, float* delta,
                         uint8_t* wbytes, const SegDev& sig, double* part, const float* wscale,
                         float b1, float omb1, hipStream_t st) {
  const int full = G.n / 8, rem = G.n % 8, i0 = full * 8;
  if (full) launch_cmp<GT, 8, MODE>(G, 0, full, g, m, delta, wbytes, sig, part, wscale, b1, omb1, st);
  switch (rem) {
    case 1: launch_cmp<GT, 1, MODE>(G, i0, 1, g, m, delta, wbytes, sig, part, wscale, b1, omb1, st); break;
    case 2: launch_cmp<GT, 2, MODE>(G, i0, 1, g, m, delta, wbytes, sig, part, wscale, b1, omb1, st); break;
    case 3: launch_cmp<GT, 3, MODE>(G, i0, 1, g, m, delta, wbytes, sig, part, wscale, b1, omb1, st); break;
    case 4: launch_cmp<GT, 4, MODE>(G, i0, 1, g, m, delta, wbytes, sig, part, wscale, b1, omb1, st); break;
    case 5: launch_cmp<GT, 5, MODE>(G, i0, 1, g, m, delta, wbytes, sig, part, wscale, b1, omb1, st); break;
    case 6: launch_cmp<GT, 6, MODE>(G, i0, 1, g, m, delta, wbytes, sig, part, wscale, b1, omb1, st); break;
    case 7: launch_cmp<GT, 7, MODE>(G, i0, 1, g, m, delta, wbytes, sig, part, wscale, b1, omb1, st); break;
    default: break;
  }
}

template <int MODE>
static void launch_cmp_t(const Geo& G, const void* g, bool f16, const float* m, float* delta,
                         uint8_t* wbytes, const SegDev& sig, double* part, const float* wscale,
                         float b1, float omb1, hipStream_t st) {
  if (f16)
    launch_cmp_n<uint16_t, MODE>(G, g, m, delta, wbytes, sig, part, wscale, b1, omb1, st);
  else
    launch_cmp_n<float, MODE>(G, g, m, delta, wbytes, sig, part, wscale, b1, omb1, st);
}

void launch_compress_norm(const Geo& G, const void* g, bool f16, const float* m,
                          const float* delta, const SegDev& sig, double* part, float b1,
                          float omb1, hipStream_t st) {
  launch_cmp_t<kNorm>(G, g, f16, m, const_cast<float*>(delta), nullptr, sig, part, nullptr, b1,
                      omb1, st);
}

void launch_compress_deferred(const Geo& G, const void* g, bool f16, const float* m, float* c,
                              uint8_t* wbytes, const SegDev& sig, double* part,
                              const float* wscale_prev, float b1, float omb1, hipStream_t st) {
  launch_cmp_t<kDeferred>(G, g, f16, m, c, wbytes, sig, part, wscale_prev, b1, omb1, st);
}

void launch_compress_apply(const Geo& G, const void* g, bool f16, const float* m, float* delta,
                           uint8_t* wbytes, const SegDev& sig, const float* wscale, float b1,
                           float omb1, hipStream_t st) {
  launch_cmp_t<kApply>(G, g, f16, m, delta, wbytes, sig, nullptr, wscale, b1, omb1, st);
}

void launch_finalize(const double* part, int32_t rows, const SegDev& T, float* scale,
                     hipStream_t st) {
  hipLaunchKernelGGL(k_finalize_scales, dim3(T.n_seg, rows), dim3(kFinBlock), 0, st, part, rows,
                     T, scale);
}

void launch_residual(const Geo& G, const float* src, int64_t src_ld, float* dst, int64_t dst_ld,
                     int32_t rows, const float* scale, const SegDev& T, hipStream_t st) {
  hipLaunchKernelGGL(k_residual, dim3(G.nblk, rows), dim3(kBlock), 0, st, G, src, src_ld, dst,
                     dst_ld, scale, T);
}

template <bool DEFERRED>
static void launch_server_t(const Geo& G, const uint8_t* wbytes, const float* wscale, float* eps,
                            uint8_t* sbytes, const SegDev& sig, const SegDev& tau, double* part,
                            const float* sscale_prev, hipStream_t st) {
#define OBA_SERVER_LAUNCH(NB)                                                                  \
  hipLaunchKernelGGL((k_server_p1<NB, DEFERRED>), dim3(G.nblk), dim3(kBlock), 0, st, G, wbytes, \
                     wscale, eps, sbytes, sig, tau, part, sscale_prev)
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

void launch_decompress_update(const Geo& G, const uint8_t* sbytes, const float* sscale,
                              const float* denom, float* m, float* x, const SegDev& tau, float lr,
                              hipStream_t st) {
  hipLaunchKernelGGL(k_decompress_update, dim3(G.nblk), dim3(kBlock), 0, st, G, sbytes, sscale,
                     denom, m, x, tau, lr);
}

}  // namespace oba
