// kernels.hip -- HIP kernels of the 1-bit Adam compression-stage step, gfx950.
//
// All kernels are HBM-streaming: a few flops per byte, no contraction, so
// no matrix cores.  A block walks a contiguous range of spans of
// kSpan = 8*kBlock coordinates.  Inside a span, thread t owns two quads of
// coordinates, A = [lo+4t, lo+4t+4) and B = [lo+4*kBlock+4t, +4): every
// 16-byte vector instruction of a wave then covers one contiguous kilobyte
// (measured 12-18 % faster on this HBM than 8 consecutive coordinates per
// lane, whose two vectors leave every instruction half-line strided).  The
// 8 sign bits of a lane are two nibbles; lanes 2u and 2u+1 swap theirs with
// one cross-lane exchange, the even lane stores byte u of the A half and the
// odd lane byte u of the B half, so every packed byte has one writer.
// Sums of squares are binary64 per lane (the square of a binary32 value is
// exact there), reduced across the wave by a butterfly and across the waves
// through LDS into one partial per (piece, row); small kernels then sum a
// segment's partials in a fixed order (in two stages when a segment has many
// pieces).  No atomics: results are bitwise reproducible.
//
// Method passages are cited in include/oba.h beside each entry point.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace oba {

namespace {

// -------------------------------------------------------------------------
// Lane layout, loads and stores.  Row bases are 16-byte aligned and
// ld % 8 == 0, so quad starts are 16-byte aligned for binary32 and 8-byte
// aligned for binary16.  Full spans use unchecked vector loads (a checked
// load is followed by its own wait); the tail span checks every element
// (coordinates >= d read as 0 and are never written).
// -------------------------------------------------------------------------
#ifndef OBA_NT_LOADS
#define OBA_NT_LOADS 1
#endif
#ifndef OBA_NT_STORES
#define OBA_NT_STORES 1
#endif
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <typename V>
__device__ __forceinline__ V ldv(const V* p) {
  if constexpr (OBA_NT_LOADS) return __builtin_nontemporal_load(p);
  else return *p;
}

template <typename V>
__device__ __forceinline__ void stv(V v, V* p) {
  if constexpr (OBA_NT_STORES) __builtin_nontemporal_store(v, p);
  else *p = v;
}

struct Quads {
  int64_t kA, kB;  // first coordinates of the lane's two quads
};

__device__ __forceinline__ Quads quads(int64_t lo) {
  const int64_t t = threadIdx.x;
  return {lo + 4 * t, lo + 4 * (int64_t)kBlock + 4 * t};
}

// coordinate of the lane's element j (0..3: quad A, 4..7: quad B); increasing in j
__device__ __forceinline__ int64_t coord(const Quads& q, int j) {
  return j < 4 ? q.kA + j : q.kB + (j - 4);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

// bfloat16 storage: the upper half of a binary32, so decoding is exact
struct bf16_bits {
  uint16_t b;
};

__device__ __forceinline__ float bf16_to_float(uint32_t h) {
  return __builtin_bit_cast(float, h << 16);
}

__device__ __forceinline__ float elem(const float* p, int64_t k) { return p[k]; }
__device__ __forceinline__ float elem(const uint16_t* p, int64_t k) {
  return half_bits_to_float(p[k]);
}
__device__ __forceinline__ float elem(const bf16_bits* p, int64_t k) {
  return bf16_to_float(p[k].b);
}

__device__ __forceinline__ void load_full(const float* __restrict__ p, const Quads& q,
                                          float (&v)[8]) {
  const f32x4 a = ldv(reinterpret_cast<const f32x4*>(p + q.kA));
  const f32x4 b = ldv(reinterpret_cast<const f32x4*>(p + q.kB));
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void load_full(const uint16_t* __restrict__ p, const Quads& q,
                                          float (&v)[8]) {
  const u32x2 a = ldv(reinterpret_cast<const u32x2*>(p + q.kA));
  const u32x2 b = ldv(reinterpret_cast<const u32x2*>(p + q.kB));
  v[0] = half_bits_to_float(a.x & 0xFFFFu);
  v[1] = half_bits_to_float(a.x >> 16);
  v[2] = half_bits_to_float(a.y & 0xFFFFu);
  v[3] = half_bits_to_float(a.y >> 16);
  v[4] = half_bits_to_float(b.x & 0xFFFFu);
  v[5] = half_bits_to_float(b.x >> 16);
  v[6] = half_bits_to_float(b.y & 0xFFFFu);
  v[7] = half_bits_to_float(b.y >> 16);
}

__device__ __forceinline__ void load_full(const bf16_bits* __restrict__ p, const Quads& q,
                                          float (&v)[8]) {
  const u32x2 a = ldv(reinterpret_cast<const u32x2*>(p + q.kA));
  const u32x2 b = ldv(reinterpret_cast<const u32x2*>(p + q.kB));
  v[0] = bf16_to_float(a.x & 0xFFFFu);
  v[1] = bf16_to_float(a.x >> 16);
  v[2] = bf16_to_float(a.y & 0xFFFFu);
  v[3] = bf16_to_float(a.y >> 16);
  v[4] = bf16_to_float(b.x & 0xFFFFu);
  v[5] = bf16_to_float(b.x >> 16);
  v[6] = bf16_to_float(b.y & 0xFFFFu);
  v[7] = bf16_to_float(b.y >> 16);
}

template <typename T>
__device__ __forceinline__ void load_tail(const T* __restrict__ p, const Quads& q, int64_t d,
                                          float (&v)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t k = coord(q, j);
    v[j] = (k < d) ? elem(p, k) : 0.0f;
  }
}

template <typename T>
__device__ __forceinline__ void load8(const T* __restrict__ p, const Quads& q, int64_t d,
                                      bool full, float (&v)[8]) {
  if (full)
    load_full(p, q, v);
  else
    load_tail(p, q, d, v);
}

// ---- tensor lists: each quad's tensor and its offset inside it ------------
struct LaneT {
  int64_t relA, relB;  // quad offsets inside their tensors
  int32_t tA, tB;      // tensors of the quads
  int32_t tu;          // the span's tensor if the whole span lies in one, else -1
  bool okA, okB;       // quad inside [0, d)
};

// Tensor of coordinate k, walking forward from t (k >= off[t]; k < d).
__device__ __forceinline__ int32_t tensor_walk(const int64_t* __restrict__ off, int32_t t,
                                               int64_t k) {
  while (off[t + 1] <= k) ++t;
  return t;
}

// Block-uniform cursor: the tensor holding the current span's first
// coordinate and its range, started from the per-block table (one load) and
// advanced span by span.
struct TCur {
  int64_t lo, hi;
  int32_t t;
};

__device__ __forceinline__ TCur tcur_start(const TList& tl, int32_t b) {
  const TBlk e = tl.blk[b];
  return {e.lo, e.hi, e.t};
}

__device__ __forceinline__ void tcur_advance(const TList& tl, TCur& c, int64_t lo) {
  while (c.hi <= lo) {
    ++c.t;
    c.lo = c.hi;
    c.hi = tl.off[c.t + 1];
  }
}

// The lane's quads for the span [lo, hi) whose first coordinate lies in the
// cursor's tensor (quads past d: ok = false).  A span inside one tensor (the
// common case) needs no lookup and keeps the tensor index block-uniform, so
// its pointers are scalar loads.
__device__ __forceinline__ LaneT lane_tensors(const TList& tl, const TCur& c, const Quads& q,
                                              int64_t hi, int64_t d) {
  LaneT lt;
  lt.okA = q.kA < d;
  lt.okB = q.kB < d;
  if (c.hi >= hi) {
    lt.tu = c.t;
    lt.tA = lt.tB = c.t;
    lt.relA = q.kA - c.lo;
    lt.relB = q.kB - c.lo;
  } else {
    lt.tu = -1;
    lt.tA = lt.okA ? tensor_walk(tl.off, c.t, q.kA) : c.t;
    lt.tB = lt.okB ? tensor_walk(tl.off, lt.tA, q.kB) : lt.tA;
    lt.relA = q.kA - tl.off[lt.tA];
    lt.relB = q.kB - tl.off[lt.tB];
  }
  return lt;
}

// One quad; CHECK: zeros when !ok (the tail span), else an unconditional load
// (a branch around each load would serialise the span's loads).
template <bool CHECK>
__device__ __forceinline__ void load_quad(const float* __restrict__ p, bool ok, float* v) {
  if (!CHECK || ok) {
    const f32x4 a = ldv(reinterpret_cast<const f32x4*>(p));
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  } else {
    v[0] = v[1] = v[2] = v[3] = 0.0f;
  }
}

template <bool CHECK>
__device__ __forceinline__ void load_quad(const uint16_t* __restrict__ p, bool ok, float* v) {
  if (!CHECK || ok) {
    const u32x2 a = ldv(reinterpret_cast<const u32x2*>(p));
    v[0] = half_bits_to_float(a.x & 0xFFFFu);
    v[1] = half_bits_to_float(a.x >> 16);
    v[2] = half_bits_to_float(a.y & 0xFFFFu);
    v[3] = half_bits_to_float(a.y >> 16);
  } else {
    v[0] = v[1] = v[2] = v[3] = 0.0f;
  }
}

template <bool CHECK>
__device__ __forceinline__ void load_quad(const bf16_bits* __restrict__ p, bool ok, float* v) {
  if (!CHECK || ok) {
    const u32x2 a = ldv(reinterpret_cast<const u32x2*>(p));
    v[0] = bf16_to_float(a.x & 0xFFFFu);
    v[1] = bf16_to_float(a.x >> 16);
    v[2] = bf16_to_float(a.y & 0xFFFFu);
    v[3] = bf16_to_float(a.y >> 16);
  } else {
    v[0] = v[1] = v[2] = v[3] = 0.0f;
  }
}

// Row `row` of a listed gradient (rows are workers) at the lane's quads.
template <bool CHECK, typename GT>
__device__ __forceinline__ void load_listed_q(const TList& tl, int64_t row, const LaneT& lt,
                                              float (&v)[8]) {
  const GT* const* tab = reinterpret_cast<const GT* const*>(tl.g) + row * tl.T;
  if (lt.tu >= 0) {  // block-uniform: one pointer for the whole span
    const GT* p = tab[lt.tu];
    load_quad<CHECK>(p + lt.relA, lt.okA, v);
    load_quad<CHECK>(p + lt.relB, lt.okB, v + 4);
  } else {
    load_quad<CHECK>(tab[lt.tA] + lt.relA, lt.okA, v);
    load_quad<CHECK>(tab[lt.tB] + lt.relB, lt.okB, v + 4);
  }
}

template <typename GT>
__device__ __forceinline__ void load_listed(const TList& tl, int64_t row, const LaneT& lt,
                                            bool full, float (&v)[8]) {
  if (full)
    load_listed_q<false, GT>(tl, row, lt, v);
  else
    load_listed_q<true, GT>(tl, row, lt, v);
}

template <bool CHECK>
__device__ __forceinline__ void load_listed_x_q(const TList& tl, const LaneT& lt, float (&v)[8]) {
  if (lt.tu >= 0) {
    const float* p = tl.x[lt.tu];
    load_quad<CHECK>(p + lt.relA, lt.okA, v);
    load_quad<CHECK>(p + lt.relB, lt.okB, v + 4);
  } else {
    load_quad<CHECK>(tl.x[lt.tA] + lt.relA, lt.okA, v);
    load_quad<CHECK>(tl.x[lt.tB] + lt.relB, lt.okB, v + 4);
  }
}

__device__ __forceinline__ void load_listed_x(const TList& tl, const LaneT& lt, bool full,
                                              float (&v)[8]) {
  if (full)
    load_listed_x_q<false>(tl, lt, v);
  else
    load_listed_x_q<true>(tl, lt, v);
}

__device__ __forceinline__ void store_listed_x(const TList& tl, const LaneT& lt, bool full,
                                               const float (&v)[8]) {
  float* pA = lt.tu >= 0 ? tl.x[lt.tu] : tl.x[lt.tA];
  float* pB = lt.tu >= 0 ? pA : tl.x[lt.tB];
  if (full || lt.okA)
    stv(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(pA + lt.relA));
  if (full || lt.okB)
    stv(f32x4{v[4], v[5], v[6], v[7]}, reinterpret_cast<f32x4*>(pB + lt.relB));
}

__device__ __forceinline__ void store8(float* __restrict__ p, const Quads& q, int64_t d,
                                       bool full, const float (&v)[8]) {
  if (full) {
    stv(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(p + q.kA));
    stv(f32x4{v[4], v[5], v[6], v[7]}, reinterpret_cast<f32x4*>(p + q.kB));
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t k = coord(q, j);
      if (k < d) p[k] = v[j];
    }
  }
}

// c = (b1*m + (1-b1)*g) + delta: two products, then two adds (no contraction)
__device__ __forceinline__ float compensate(float b1, float omb1, float m, float g, float dl) {
  const float p = b1 * m + omb1 * g;
  return p + dl;
}

// bit j = (v[j] < 0): -0.0 gives 0 (sign +1).  Bits 0-3 quad A, 4-7 quad B.
__device__ __forceinline__ uint32_t sign_bits(const float (&v)[8]) {
  uint32_t b = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) b |= (v[j] < 0.0f ? 1u : 0u) << j;
  return b;
}

// Store the lane's 8 sign bits into a packed row (little-endian bytes,
// nbytes = 8*W).  Every lane of the wave must call this (cross-lane exchange).
__device__ __forceinline__ void store_sign_bits(uint8_t* __restrict__ row, const Quads& q,
                                                uint32_t b8, int64_t nbytes) {
  const uint32_t p = (uint32_t)__shfl_xor((int)b8, 1, 64);
  const bool odd = threadIdx.x & 1;
  const uint32_t byte = odd ? ((p >> 4) | (b8 & 0xF0u)) : ((b8 & 0xFu) | ((p & 0xFu) << 4));
  const int64_t qi = (odd ? q.kB : q.kA) >> 3;
  if (qi < nbytes) row[qi] = (uint8_t)byte;
}

// The lane's 8 sign bits from a packed row.  FULL: both quads lie inside
// [0, d) (no checks).  Otherwise bytes whose coordinates all lie at or past d
// read as 0.  PAIRS: each lane loads the two bytes holding its quads (no
// cross-lane step, so the bits are not needed until used).  Otherwise the
// even lane loads the A-half byte of the pair, the odd lane the B-half byte
// (one distinct byte per lane), and they swap -- every lane of the wave must
// then call this (cross-lane exchange).  The worker and update passes load
// one row per span and take pairs; the server pass loads n rows and takes the
// exchange (half the load instructions).
#ifndef OBA_PAIRS_CMP
#define OBA_PAIRS_CMP 1
#endif
#ifndef OBA_PAIRS_UPD
#define OBA_PAIRS_UPD 1
#endif
template <bool FULL, bool PAIRS>
__device__ __forceinline__ uint32_t load_sign_bits(const uint8_t* __restrict__ row,
                                                   const Quads& q, int64_t d) {
  const bool odd = threadIdx.x & 1;
  const uint32_t sh = odd ? 4u : 0u;
  uint32_t byte_a, byte_b;
  if constexpr (PAIRS) {
    byte_a = (FULL || q.kA < d) ? (uint32_t)row[q.kA >> 3] : 0u;
    byte_b = (FULL || q.kB < d) ? (uint32_t)row[q.kB >> 3] : 0u;
  } else {
    const int64_t qi = (odd ? q.kB : q.kA) >> 3;
    const uint32_t mine = (FULL || qi * 8 < d) ? (uint32_t)row[qi] : 0u;
    const uint32_t other = (uint32_t)__shfl_xor((int)mine, 1, 64);
    byte_a = odd ? other : mine;
    byte_b = odd ? mine : other;
  }
  return ((byte_a >> sh) & 0xFu) | (((byte_b >> sh) & 0xFu) << 4);
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

// Block-reduce acc[0..nw) and write dst[i*stride], i < nw; resets acc.
// Uniform call.
template <int NB>
__device__ __forceinline__ void flush_rows(double (&acc)[NB], int nw, double* __restrict__ dst,
                                           int64_t stride, double* lds) {
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
    double t = lds[i];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) t += lds[w * NB + i];  // fixed order
    dst[i * stride] = t;
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

// Segments of the lane's 8 coordinates (coordinates >= d keep the last one).
__device__ __forceinline__ void lane_segs(const int64_t* __restrict__ off, int32_t j0,
                                          const Quads& q, int64_t d, int32_t (&js)[8]) {
  int32_t j = j0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int64_t k = coord(q, e);
    if (k < d) j = seg_walk(off, j, k);
    js[e] = j;
  }
}

// Sum of squares of row[k] for the lane's coordinates k in [a, e).
__device__ __forceinline__ double sumsq_range(const float* row, const Quads& q, int64_t a,
                                              int64_t e) {
  double s = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t k = coord(q, j);
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
                                                float b1, float omb1, const Quads& q, int64_t a,
                                                int64_t e) {
  double s = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t k = coord(q, j);
    if (k >= a && k < e) {
      const double x = (double)compensate(b1, omb1, m[k], elem(grow, k), drow[k]);
      s = __builtin_fma(x, x, s);
    }
  }
  return s;
}

// residual c - s*sign(c), sign(c) = -1 iff c < 0
__device__ __forceinline__ float residual(float c, float s) { return (c < 0.0f) ? c + s : c - s; }

}  // namespace

// ===========================================================================
// Warm-up Adam step on the mean gradient.  NORM: also the sum of squares of
// the new v, one binary64 partial per block (part[blockIdx.x]).  NB rows of g
// are loaded together (NB = n for n <= 8; larger n loops over groups of 8),
// after m, v and x, so that all of a span's loads are in flight at once.
// ===========================================================================
template <typename GT, int NB, bool NORM, bool TL>
__global__ __launch_bounds__(kBlock) void k_adam_warmup(Geo G, const GT* __restrict__ g,
                                                        float* __restrict__ x,
                                                        float* __restrict__ m,
                                                        float* __restrict__ v, AdamCoef C,
                                                        double* __restrict__ part, TList tl) {
  __shared__ double lds[kWaves];
  double acc[1] = {0.0};
  const int64_t s_lo = dspan(G.S, G.nblk, blockIdx.x);
  const int64_t s_hi = dspan(G.S, G.nblk, blockIdx.x + 1);
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
    load8(m, q, G.d, full, mv);
    load8(v, q, G.d, full, vv);
    if constexpr (TL)
      load_listed_x(tl, lt, full, xv);
    else
      load8(x, q, G.d, full, xv);
#pragma unroll
    for (int j = 0; j < 8; ++j) sum[j] = 0.0f;
    for (int32_t i0 = 0; i0 < G.n; i0 += NB) {  // one pass when n <= NB
      // rows past n are clamped to a valid row and their terms skipped
      float gv[NB][8];
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        if constexpr (TL)
          load_listed<GT>(tl, min(i0 + u, G.n - 1), lt, full, gv[u]);
        else
          load8(g + (int64_t)min(i0 + u, G.n - 1) * G.ld, q, G.d, full, gv[u]);
      }
#pragma unroll
      for (int u = 0; u < NB; ++u)
        if (i0 + u < G.n) {
#pragma unroll
          for (int j = 0; j < 8; ++j) sum[j] = sum[j] + gv[u][j];
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float gb = pow2 ? sum[j] * inv_n : sum[j] / nf;  // identical for n = 2^k
      const float mk = C.b1 * mv[j] + C.omb1 * gb;
      const float vk = C.b2 * vv[j] + C.omb2 * (gb * gb);
      mv[j] = mk;
      vv[j] = vk;
      xv[j] = xv[j] - (C.lr * (mk / C.bc1)) / (__builtin_sqrtf(vk / C.bc2) + C.eta);
    }
    store8(m, q, G.d, full, mv);
    store8(v, q, G.d, full, vv);
    if constexpr (TL)
      store_listed_x(tl, lt, full, xv);
    else
      store8(x, q, G.d, full, xv);
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
  const int64_t s_lo = dspan(G.S, G.nblk, blockIdx.x);
  const int64_t s_hi = dspan(G.S, G.nblk, blockIdx.x + 1);
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

// ===========================================================================
// Worker side, for NB workers at once (m is read once per coordinate):
//   c = (b1*m + (1-b1)*g_i) + delta_i
// kNorm:  only reduce sum c^2 per (piece, worker) -- reads only;
// kApply: recompute c bit for bit, store the sign bits and
//         delta_i = c - s*sign(c) with the finished scales;
// kDeferred: the state row holds the previous step's c (not delta) and the
//         scale buffer its scales s'; the residual of the last step is formed
//         where it is consumed, delta_i = c' - s'*sign(c'), then
//         c = (b1*m + (1-b1)*g_i) + delta_i is stored over c' with its sign
//         bits and its sum c^2 is reduced -- one pass instead of two;
// kDeferredM: as kDeferred, but m is not read: after a compression step
//         every worker's momentum is the server's m_hat = sbar*sign, so it is
//         rebuilt from the last packed server bits and scales (1/8 byte
//         instead of 4 bytes per coordinate);
// kDeferredLocal: as kDeferred with per-worker momentum: m is [n][ld], each
//         worker's m_i = b1*m_i + (1-b1)*g_i is stored back and
//         c = m_i + delta_i.
// The scale needs the whole segment's norm before any residual can be
// written, so the explicit layout needs c twice.  Recomputing it reads g, m,
// delta twice but never writes c: on this HBM, writes cost more than reads,
// and storing c in a first pass to re-read it was measured 15 % slower per
// step.
// NB is the exact number of workers of a block: a launch covers workers
// [i0, i0 + gridDim.y*NB); larger n takes one launch of full groups and one
// for the remainder.  Grid: (nblk, groups).
// ===========================================================================
enum { kNorm = 1, kApply = 2, kDeferred = 3, kDeferredM = 4, kDeferredLocal = 5 };
#ifndef OBA_WORKER_BATCH
#define OBA_WORKER_BATCH 4
#endif
constexpr int kWorkerBatch = OBA_WORKER_BATCH;

// Optional occupancy target of the worker pass (waves per SIMD), a tuning knob.
#ifdef OBA_CMP_WAVES
#define OBA_CMP_ATTR __attribute__((amdgpu_waves_per_eu(OBA_CMP_WAVES, OBA_CMP_WAVES)))
#else
#define OBA_CMP_ATTR
#endif

template <typename GT, int NB, int MODE, bool TL>
__global__ __launch_bounds__(kBlock) OBA_CMP_ATTR void k_compress(Geo G, int32_t i0, const GT* __restrict__ g,
                                                     float* __restrict__ m,  // read; written by kDeferredLocal
                                                     float* __restrict__ delta,
                                                     uint8_t* __restrict__ wbytes, SegDev sig,
                                                     double* __restrict__ part,
                                                     const float* __restrict__ wscale, float b1,
                                                     float omb1, MomSrc ms, TList tl) {
  __shared__ double lds[kWaves * NB];
  const int32_t b = blockIdx.x;
  i0 += blockIdx.y * NB;  // this block's workers: [i0, i0 + NB)
  const int64_t s_lo = dspan(G.S, G.nblk, b), s_hi = dspan(G.S, G.nblk, b + 1);
  const int32_t p_end = sig.blk_first[b + 1];
  int32_t p = sig.blk_first[b];
  int64_t p_hi = sig.phi[p];
  static_assert(!TL || MODE >= kDeferred, "tensor lists: deferred passes only");
  TCur tcur{};  // tensor cursor (tensor lists)
  if constexpr (TL) tcur = tcur_start(tl, b);
  // kDeferredM: cursor over the server segments (on this grid) for sbar
  int32_t pt = 0, pt_end = 0;
  int64_t pt_hi = 0;
  if (MODE == kDeferredM) {
    pt = ms.tau.blk_first[b];
    pt_end = ms.tau.blk_first[b + 1];
    pt_hi = ms.tau.phi[pt];
  }
  const int64_t rowbytes = G.W * 8;
  double acc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) acc[i] = 0.0;

  for (int64_t s = s_lo; s < s_hi; ++s) {
    const int64_t lo = s * kSpan;
    const int64_t hi = min(lo + kSpan, G.d);
    const Quads q = quads(lo);
    const bool uniform = hi <= p_hi;  // span inside the current piece
    const bool full = lo + kSpan <= G.d;
    int32_t jseg[8];
    if (MODE != kNorm && !uniform) lane_segs(sig.off, sig.pseg[p], q, G.d, jseg);
    LaneT lt{};
    if constexpr (TL) {
      tcur_advance(tl, tcur, lo);
      lt = lane_tensors(tl, tcur, q, min(lo + kSpan, G.d), G.d);
    }
    // every load of the span first (all NB workers), then the arithmetic
    float mv[8];
    if (MODE == kDeferredM) {  // m = sbar*sign from the last server message
      const uint32_t bits = full ? load_sign_bits<true, OBA_PAIRS_CMP>(ms.sbytes, q, G.d)
                                 : load_sign_bits<false, OBA_PAIRS_CMP>(ms.sbytes, q, G.d);
      float sb[8];
      if (hi <= pt_hi) {
        const float s_ = ms.sscale[ms.tau.pseg[pt]];
#pragma unroll
        for (int j = 0; j < 8; ++j) sb[j] = s_;
      } else {
        int32_t jt[8];
        lane_segs(ms.tau.off, ms.tau.pseg[pt], q, G.d, jt);
#pragma unroll
        for (int j = 0; j < 8; ++j) sb[j] = ms.sscale[jt[j]];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        mv[j] = (!full && coord(q, j) >= G.d) ? 0.0f : (((bits >> j) & 1u) ? -sb[j] : sb[j]);
      while (pt < pt_end && pt_hi <= hi) {
        if (++pt < pt_end) pt_hi = ms.tau.phi[pt];
      }
    } else if (MODE == kDeferredLocal) {  // per-worker rows, loaded with g below
#pragma unroll
      for (int j = 0; j < 8; ++j) mv[j] = 0.0f;
    } else if (full) {
      load_full(m, q, mv);
    } else {
      load_tail(m, q, G.d, mv);
    }
    double fs[NB];
    // workers in batches of NBB: all loads of a batch, then its arithmetic
    // and stores (NBB < NB trades loads in flight per wave for occupancy)
    constexpr int NBB = NB < kWorkerBatch ? NB : kWorkerBatch;
#pragma unroll
    for (int ib = 0; ib < NB; ib += NBB) {
      constexpr int NBL = MODE == kDeferredLocal ? NBB : 1;  // per-worker m rows
      float gv[NBB][8], c[NBB][8], ml[NBL][8];
      // ib + u < NB is decided at compile time: a last batch may be partial
      if (full) {
#pragma unroll
        for (int u = 0; u < NBB; ++u) {
          if (ib + u >= NB) break;
          const int64_t row = (int64_t)(i0 + ib + u) * G.ld;
          if constexpr (TL)
            load_listed<GT>(tl, i0 + ib + u, lt, full, gv[u]);
          else
            load_full(g + row, q, gv[u]);
          load_full(delta + row, q, c[u]);
          if (MODE == kDeferredLocal) load_full(m + row, q, ml[u]);
        }
      } else {
#pragma unroll
        for (int u = 0; u < NBB; ++u) {
          if (ib + u >= NB) break;
          const int64_t row = (int64_t)(i0 + ib + u) * G.ld;
          if constexpr (TL)
            load_listed<GT>(tl, i0 + ib + u, lt, full, gv[u]);
          else
            load_tail(g + row, q, G.d, gv[u]);
          load_tail(delta + row, q, G.d, c[u]);
          if (MODE == kDeferredLocal) load_tail(m + row, q, G.d, ml[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < NBB; ++u) {
        const int i = ib + u;
        if (i >= NB) break;
        const int64_t row = (int64_t)(i0 + i) * G.ld;
        const float* sc = wscale + (int64_t)(i0 + i) * sig.n_seg;
        float sv[8];
        if (MODE != kNorm) {
          if (uniform) {
            const float s_ = sc[sig.pseg[p]];
#pragma unroll
            for (int j = 0; j < 8; ++j) sv[j] = s_;
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) sv[j] = sc[jseg[j]];
          }
        }
        if (MODE >= kDeferred) {  // c[u] holds c' of the last step
#pragma unroll
          for (int j = 0; j < 8; ++j) c[u][j] = residual(c[u][j], sv[j]);
          if (!full) {  // coordinates past d read as 0 and must stay 0 (no bit, no c^2)
#pragma unroll
            for (int j = 0; j < 8; ++j)
              if (coord(q, j) >= G.d) c[u][j] = 0.0f;
          }
        }
        if (MODE == kDeferredLocal) {
          // the same two products and two adds as compensate(), m_i kept
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            ml[u][j] = b1 * ml[u][j] + omb1 * gv[u][j];
            c[u][j] = ml[u][j] + c[u][j];
          }
          store8(m + row, q, G.d, full, ml[u]);
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) c[u][j] = compensate(b1, omb1, mv[j], gv[u][j], c[u][j]);
        }
        if (MODE != kNorm) store_sign_bits(wbytes + (int64_t)(i0 + i) * rowbytes, q, sign_bits(c[u]), rowbytes);
        if (MODE >= kDeferred) store8(delta + row, q, G.d, full, c[u]);
        fs[i] = (MODE != kApply) ? sumsq8(c[u]) : 0.0;
        if (MODE == kApply) {
#pragma unroll
          for (int j = 0; j < 8; ++j) c[u][j] = residual(c[u][j], sv[j]);
          store8(delta + row, q, G.d, full, c[u]);
        }
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
        flush_rows<NB>(acc, NB, part + (int64_t)i0 * sig.n_pieces + p, sig.n_pieces, lds);
        if (++p < p_end) p_hi = sig.phi[p];
      }
    } else {  // span crosses piece boundaries: sum this lane's c piece by piece
      int64_t cur = lo;
      while (cur < hi) {
        const int64_t e = min(p_hi, hi);
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const int64_t row = (int64_t)(i0 + i) * G.ld;
          if (MODE >= kDeferred)
            acc[i] += sumsq_range(delta + row, q, cur, e);  // c was stored there
          else
            acc[i] += sumsq_range_c(m, g + row, delta + row, b1, omb1, q, cur, e);
        }
        if (p_hi <= hi) {
          flush_rows<NB>(acc, NB, part + (int64_t)i0 * sig.n_pieces + p, sig.n_pieces, lds);
          if (++p < p_end) p_hi = sig.phi[p];
        }
        cur = e;
      }
    }
  }
}

// ===========================================================================
// Per-segment scale from the binary64 partials: s = sqrt(S / len) in
// binary64, rounded once to binary32.  part: [rows][n_parts]; the parts of
// segment j are [first[j], first[j+1]) (pieces, or items of the two-stage
// sum).  Grid: (n_seg, rows).
// ===========================================================================
constexpr int kFinBlock = 1024;  // 16 waves: at most 8192 parts per segment

__global__ __launch_bounds__(kFinBlock) void k_finalize_scales(const double* __restrict__ part,
                                                               int32_t n_parts,
                                                               const int32_t* __restrict__ first,
                                                               SegDev T,
                                                               float* __restrict__ scale) {
  __shared__ double lds[kFinBlock / 64];
  const int32_t j = blockIdx.x, r = blockIdx.y;
  const double* row = part + (int64_t)r * n_parts;
  const int32_t q0 = first[j], q1 = first[j + 1];
  double t = 0.0;
  for (int32_t q = q0 + threadIdx.x; q < q1; q += kFinBlock) t += row[q];
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

// First stage of a two-stage sum: item it (at most kItem consecutive pieces
// of one segment) of row r.  Grid: (n_items, rows).  part: [rows][n_pieces];
// out: [rows][n_items].
constexpr int kItemBlock = 256;

__global__ __launch_bounds__(kItemBlock) void k_sum_items(const double* __restrict__ part,
                                                          int32_t n_pieces,
                                                          const int32_t* __restrict__ item_q,
                                                          int32_t n_items,
                                                          double* __restrict__ out) {
  __shared__ double lds[kItemBlock / 64];
  const int32_t it = blockIdx.x, r = blockIdx.y;
  const double* row = part + (int64_t)r * n_pieces;
  const int32_t q0 = item_q[it], q1 = item_q[it + 1];
  double t = 0.0;
  for (int32_t q = q0 + threadIdx.x; q < q1; q += kItemBlock) t += row[q];
  t = wave_sum(t);
  if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = t;
  __syncthreads();
  if (threadIdx.x == 0) {
    double S = 0.0;
    for (int w = 0; w < kItemBlock / 64; ++w) S += lds[w];  // fixed order
    out[(int64_t)r * n_items + it] = S;
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
  __shared__ uint2 rows_lds[OBA_SRV_LDS ? NB * 32 : 1];
  const int32_t b = blockIdx.x;
  const int64_t s_lo = dspan(G.S, G.nblk, b), s_hi = dspan(G.S, G.nblk, b + 1);
  const int32_t ps_end = sig.blk_first[b + 1], pt_end = tau.blk_first[b + 1];
  int32_t ps = sig.blk_first[b], pt = tau.blk_first[b];
  int64_t ps_hi = sig.phi[ps], pt_hi = tau.phi[pt];
  const int64_t rowbytes = G.W * 8;
  const float nf = (float)G.n;
  const bool pow2 = (G.n & (G.n - 1)) == 0;
  const float inv_n = 1.0f / nf;
  double acc[1] = {0.0};
  for (int64_t s = s_lo; s < s_hi; ++s) {
    const int64_t lo = s * kSpan;
    const int64_t hi = min(lo + kSpan, G.d);
    const Quads q = quads(lo);
    float a[8];
    if (hi <= ps_hi && hi <= pt_hi && lo + kSpan <= G.d) {
      // fast path: full span, one worker and one server segment; loads first
      const int32_t js0 = sig.pseg[ps];
      float t[8];
      load_full(eps, q, a);
      if (DEFERRED) {
        const float sp = sscale_prev[tau.pseg[pt]];
#pragma unroll
        for (int j = 0; j < 8; ++j) a[j] = residual(a[j], sp);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) t[j] = 0.0f;
      for (int32_t i0 = 0; i0 < G.n; i0 += NB) {  // one pass when n <= NB
        // rows past n are clamped to a valid row and their terms skipped
        uint32_t bits[NB];
        float sw[NB];
        if constexpr (OBA_SRV_LDS != 0) {
          __syncthreads();  // the previous span's reads of rows_lds are done
          if ((int)threadIdx.x < NB * 32) {
            const int u = threadIdx.x >> 5, c = threadIdx.x & 31;
            const int64_t r = min(i0 + u, G.n - 1);
            rows_lds[threadIdx.x] =
                *reinterpret_cast<const uint2*>(wbytes + r * rowbytes + (lo >> 3) + 8 * c);
          }
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
      int32_t js = sig.pseg[ps];
      int32_t jt = tau.pseg[pt];
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
      if (++ps < ps_end) ps_hi = sig.phi[ps];
    }
    // server-segment reduction
    if (hi <= pt_hi) {
      acc[0] += fs;
      if (hi == pt_hi) {
        flush_rows<1>(acc, 1, part + pt, 0, lds);
        if (++pt < pt_end) pt_hi = tau.phi[pt];
      }
    } else {
      int64_t cur = lo;
      while (cur < hi) {
        const int64_t e = min(pt_hi, hi);
        acc[0] += sumsq_range(eps, q, cur, e);
        if (pt_hi <= hi) {
          flush_rows<1>(acc, 1, part + pt, 0, lds);
          if (++pt < pt_end) pt_hi = tau.phi[pt];
        }
        cur = e;
      }
    }
  }
}

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
  const int64_t s_lo = dspan(G.S, G.nblk, b), s_hi = dspan(G.S, G.nblk, b + 1);
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
      load8(denom, q, G.d, full, dv);
      if constexpr (TL)
        load_listed_x(tl, lt, full, xv);
      else
        load8(x, q, G.d, full, xv);
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
    if (WRITE_M) store8(m, q, G.d, full, mh);
    if (UPDATE_X) {
      if constexpr (TL)
        store_listed_x(tl, lt, full, xv);
      else
        store8(x, q, G.d, full, xv);
    }
    while (p < p_end && p_hi <= hi) {
      if (++p < p_end) p_hi = tau.phi[p];
    }
  }
}

// ===========================================================================
// launchers
// ===========================================================================
void launch_norm_finalize(const double* part, int32_t n, double* out, hipStream_t st);

template <typename GT, bool NORM, bool TL>
static void launch_warmup_nb(const Geo& G, const void* g, float* x, float* m, float* v,
                             const AdamCoef& C, double* part, const TList& tl, hipStream_t st) {
#define OBA_WARMUP_LAUNCH(NB)                                                                 \
  hipLaunchKernelGGL((k_adam_warmup<GT, NB, NORM, TL>), dim3(G.nblk), dim3(kBlock), 0, st, G, \
                     static_cast<const GT*>(g), x, m, v, C, part, tl)
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

template <typename GT, int NB, int MODE, bool TL>
static void launch_cmp(const Geo& G, int32_t i0, int groups, const void* g, const float* m,
                       float* delta, uint8_t* wbytes, const SegDev& sig, double* part,
                       const float* wscale, float b1, float omb1, const MomSrc& ms,
                       const TList& tl, hipStream_t st) {
  hipLaunchKernelGGL((k_compress<GT, NB, MODE, TL>), dim3(G.nblk, groups), dim3(kBlock), 0, st,
                     G, i0, static_cast<const GT*>(g), const_cast<float*>(m), delta, wbytes, sig,
                     part, wscale, b1, omb1, ms, tl);
}

// Groups of GROUP workers per block, then one launch for the remainder.  A
// pass that reads m shares it across the block's workers (4 bytes per
// coordinate per group); the implicit momentum costs 1/8 byte per group, so
// that pass can take smaller groups (fewer registers, more blocks).
#ifndef OBA_MAX_NB
#define OBA_MAX_NB 8
#endif
#ifndef OBA_IMPLICIT_NB
#define OBA_IMPLICIT_NB 4
#endif
constexpr int kMaxNB = OBA_MAX_NB;
constexpr int kImplicitNB = OBA_IMPLICIT_NB;
static_assert(kMaxNB >= 1 && kMaxNB <= 8 && kImplicitNB >= 1 && kImplicitNB <= 8,
              "worker groups hold 1 to 8 workers");

template <typename GT, int MODE, bool TL>
static void launch_cmp_n(const Geo& G, const void* g, const float* m, float* delta,
                         uint8_t* wbytes, const SegDev& sig, double* part, const float* wscale,
                         float b1, float omb1, const MomSrc& ms, const TList& tl,
                         hipStream_t st) {
  constexpr int GROUP = (MODE == kDeferredM || MODE == kDeferredLocal) ? kImplicitNB : kMaxNB;
  const int full = G.n / GROUP, rem = G.n % GROUP, i0 = full * GROUP;
#define OBA_CMP(NB_, I0, GROUPS) \
  launch_cmp<GT, NB_, MODE, TL>(G, I0, GROUPS, g, m, delta, wbytes, sig, part, wscale, b1, omb1, \
                                ms, tl, st)
  if (full) OBA_CMP(GROUP, 0, full);
  switch (rem) {
    case 1: OBA_CMP(1, i0, 1); break;
    case 2: OBA_CMP(2, i0, 1); break;
    case 3: OBA_CMP(3, i0, 1); break;
    case 4: OBA_CMP(4, i0, 1); break;
    case 5: OBA_CMP(5, i0, 1); break;
    case 6: OBA_CMP(6, i0, 1); break;
    case 7: OBA_CMP(7, i0, 1); break;
    default: break;
  }
#undef OBA_CMP
}

template <int MODE, bool TL = false>
static void launch_cmp_t(const Geo& G, const void* g, int gdt, const float* m, float* delta,
                         uint8_t* wbytes, const SegDev& sig, double* part, const float* wscale,
                         float b1, float omb1, const MomSrc& ms, hipStream_t st,
                         const TList& tl = TList{}) {
  if (gdt == kGradF16)
    launch_cmp_n<uint16_t, MODE, TL>(G, g, m, delta, wbytes, sig, part, wscale, b1, omb1, ms, tl,
                                     st);
  else if (gdt == kGradBF16)
    launch_cmp_n<bf16_bits, MODE, TL>(G, g, m, delta, wbytes, sig, part, wscale, b1, omb1, ms,
                                      tl, st);
  else
    launch_cmp_n<float, MODE, TL>(G, g, m, delta, wbytes, sig, part, wscale, b1, omb1, ms, tl,
                                  st);
}

void launch_compress_norm(const Geo& G, const void* g, int gdt, const float* m,
                          const float* delta, const SegDev& sig, double* part, float b1,
                          float omb1, hipStream_t st) {
  launch_cmp_t<kNorm>(G, g, gdt, m, const_cast<float*>(delta), nullptr, sig, part, nullptr, b1,
                      omb1, MomSrc{}, st);
}

void launch_compress_deferred(const Geo& G, const void* g, int gdt, const float* m, float* c,
                              uint8_t* wbytes, const SegDev& sig, double* part,
                              const float* wscale_prev, float b1, float omb1, const MomSrc& ms,
                              hipStream_t st) {
  if (ms.sbytes)
    launch_cmp_t<kDeferredM>(G, g, gdt, nullptr, c, wbytes, sig, part, wscale_prev, b1, omb1, ms,
                             st);
  else
    launch_cmp_t<kDeferred>(G, g, gdt, m, c, wbytes, sig, part, wscale_prev, b1, omb1, ms, st);
}

void launch_compress_deferred_listed(const Geo& G, const TList& tl, int gdt, const float* m,
                                     float* c, uint8_t* wbytes, const SegDev& sig, double* part,
                                     const float* wscale_prev, float b1, float omb1,
                                     const MomSrc& ms, hipStream_t st) {
  if (ms.sbytes)
    launch_cmp_t<kDeferredM, true>(G, nullptr, gdt, nullptr, c, wbytes, sig, part, wscale_prev,
                                   b1, omb1, ms, st, tl);
  else
    launch_cmp_t<kDeferred, true>(G, nullptr, gdt, m, c, wbytes, sig, part, wscale_prev, b1,
                                  omb1, ms, st, tl);
}

void launch_compress_deferred_local(const Geo& G, const void* g, int gdt, float* m_local,
                                    float* c, uint8_t* wbytes, const SegDev& sig, double* part,
                                    const float* wscale_prev, float b1, float omb1,
                                    hipStream_t st) {
  launch_cmp_t<kDeferredLocal>(G, g, gdt, m_local, c, wbytes, sig, part, wscale_prev, b1, omb1,
                               MomSrc{}, st);
}

void launch_compress_apply(const Geo& G, const void* g, int gdt, const float* m, float* delta,
                           uint8_t* wbytes, const SegDev& sig, const float* wscale, float b1,
                           float omb1, hipStream_t st) {
  launch_cmp_t<kApply>(G, g, gdt, m, delta, wbytes, sig, nullptr, wscale, b1, omb1, MomSrc{}, st);
}

void launch_finalize(double* part, int32_t rows, const SegDev& T, float* scale,
                     hipStream_t st) {
  if (T.n_items == 0) {
    hipLaunchKernelGGL(k_finalize_scales, dim3(T.n_seg, rows), dim3(kFinBlock), 0, st, part,
                       T.n_pieces, T.seg_first, T, scale);
    return;
  }
  double* items = part + ((size_t)T.n_pieces * rows * 8 + 255) / 256 * 32;
  hipLaunchKernelGGL(k_sum_items, dim3(T.n_items, rows), dim3(kItemBlock), 0, st, part,
                     T.n_pieces, T.item_q, T.n_items, items);
  hipLaunchKernelGGL(k_finalize_scales, dim3(T.n_seg, rows), dim3(kFinBlock), 0, st, items,
                     T.n_items, T.seg_item, T, scale);
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
  if (m)
    hipLaunchKernelGGL((k_decompress_update<true, true, false>), dim3(G.nblk), dim3(kBlock), 0,
                       st, G, sbytes, sscale, denom, m, x, tau, lr, TList{});
  else
    hipLaunchKernelGGL((k_decompress_update<false, true, false>), dim3(G.nblk), dim3(kBlock), 0,
                       st, G, sbytes, sscale, denom, m, x, tau, lr, TList{});
}

void launch_decompress_update_listed(const Geo& G, const TList& tl, const uint8_t* sbytes,
                                     const float* sscale, const float* denom, float* m,
                                     const SegDev& tau, float lr, hipStream_t st) {
  if (m)
    hipLaunchKernelGGL((k_decompress_update<true, true, true>), dim3(G.nblk), dim3(kBlock), 0,
                       st, G, sbytes, sscale, denom, m, nullptr, tau, lr, tl);
  else
    hipLaunchKernelGGL((k_decompress_update<false, true, true>), dim3(G.nblk), dim3(kBlock), 0,
                       st, G, sbytes, sscale, denom, m, nullptr, tau, lr, tl);
}

void launch_server_momentum(const Geo& G, const uint8_t* sbytes, const float* sscale, float* m,
                            const SegDev& tau, hipStream_t st) {
  hipLaunchKernelGGL((k_decompress_update<true, false, false>), dim3(G.nblk), dim3(kBlock), 0, st,
                     G, sbytes, sscale, nullptr, m, nullptr, tau, 0.0f, TList{});
}

}  // namespace oba
