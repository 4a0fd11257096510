// device.hpp -- device helpers shared by the streaming kernels (gfx950):
// the lane layout, vector loads and stores, tensor-list addressing, sign-bit
// packing and the binary64 reductions.  Header-only; every function is
// inline, in an unnamed namespace.
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
#pragma once
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

// ---- 16-bit state rows (binary16 as uint16_t, bfloat16 as bf16_bits) --------
// A lane's 8 values are rounded in pairs with gfx950's packed conversions
// (v_cvt_pk_f16_f32, v_cvt_pk_bf16_f32): nearest, ties to even, subnormals
// kept, overflow to an infinity.  h[i] holds values 2i (low half) and 2i+1.
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack2(const uint16_t*, float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}
__device__ __forceinline__ uint32_t pack2(const bf16_bits*, float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ float lo16(const uint16_t*, uint32_t h) {
  return half_bits_to_float(h & 0xFFFFu);
}
__device__ __forceinline__ float hi16(const uint16_t*, uint32_t h) {
  return half_bits_to_float(h >> 16);
}
__device__ __forceinline__ float lo16(const bf16_bits*, uint32_t h) {
  return __builtin_bit_cast(float, h << 16);
}
__device__ __forceinline__ float hi16(const bf16_bits*, uint32_t h) {
  return __builtin_bit_cast(float, h & 0xFFFF0000u);
}

// The values a row of type T holds for v: v itself for binary32; else v
// rounded to the 16-bit format, whose bit patterns go to h for the store.
template <typename T>
__device__ __forceinline__ void round_to_row(float (&v)[8], uint32_t (&h)[4]) {
  if constexpr (!__is_same(T, float)) {
    const T* tag = nullptr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[i] = pack2(tag, v[2 * i], v[2 * i + 1]);
      v[2 * i] = lo16(tag, h[i]);
      v[2 * i + 1] = hi16(tag, h[i]);
    }
  }
}

// Store a row's values: binary32 from v; a 16-bit row from the patterns h
// that round_to_row made.
__device__ __forceinline__ void store_row(float* __restrict__ p, const Quads& q, int64_t d,
                                          bool full, const float (&v)[8], const uint32_t (&)[4]) {
  store8(p, q, d, full, v);
}

template <typename T16>
__device__ __forceinline__ void store_row(T16* __restrict__ p, const Quads& q, int64_t d,
                                          bool full, const float (&)[8], const uint32_t (&h)[4]) {
  if (full) {
    stv(u32x2{h[0], h[1]}, reinterpret_cast<u32x2*>(p + q.kA));
    stv(u32x2{h[2], h[3]}, reinterpret_cast<u32x2*>(p + q.kB));
  } else {
    uint16_t* e = reinterpret_cast<uint16_t*>(p);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t k = coord(q, j);
      if (k < d) e[k] = (uint16_t)(h[j >> 1] >> (16 * (j & 1)));
    }
  }
}

// ---- full spans through buffer resources ------------------------------------
// OBA_BUF: a full span of one row is read or written through a buffer
// resource whose base is the span's first element (block-uniform, scalar
// registers) and whose size is the span's bytes; each lane adds a 32-bit
// byte offset, so no 64-bit address is formed per lane and one offset
// register serves every row of the same element size.  An access past the
// span's bytes would read 0 and write nothing (the hardware's range check).
#ifndef OBA_BUF
#define OBA_BUF 1
#endif
// the same for the update and the warm-up step
#ifndef OBA_BUF_MISC
#define OBA_BUF_MISC 0
#endif

constexpr int kBufRsrcWord3 = 0x00020000;  // raw (untyped) buffer, gfx9 family
constexpr int kBufLoadAux = OBA_NT_LOADS ? 2 : 0;   // nt
constexpr int kBufStoreAux = OBA_NT_STORES ? 2 : 0;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t span_rsrc(const T* row, int64_t lo) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(row + lo), (short)0,
                                           (int)(kSpan * sizeof(T)), kBufRsrcWord3);
}

__device__ __forceinline__ void load_full_buf(const float* row, int64_t lo, float (&v)[8]) {
  const __amdgpu_buffer_rsrc_t r = span_rsrc(row, lo);
  const f32x4 a = __builtin_bit_cast(
      f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, 16u * threadIdx.x, 0, kBufLoadAux));
  const f32x4 b = __builtin_bit_cast(
      f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, 16u * (kBlock + threadIdx.x), 0, kBufLoadAux));
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <typename T16>
__device__ __forceinline__ void load_full_buf(const T16* row, int64_t lo, float (&v)[8]) {
  const __amdgpu_buffer_rsrc_t r = span_rsrc(row, lo);
  const u32x2 a = __builtin_bit_cast(
      u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, 8u * threadIdx.x, 0, kBufLoadAux));
  const u32x2 b = __builtin_bit_cast(
      u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, 8u * (kBlock + threadIdx.x), 0, kBufLoadAux));
  const T16* tag = nullptr;
  v[0] = lo16(tag, a.x); v[1] = hi16(tag, a.x); v[2] = lo16(tag, a.y); v[3] = hi16(tag, a.y);
  v[4] = lo16(tag, b.x); v[5] = hi16(tag, b.x); v[6] = lo16(tag, b.y); v[7] = hi16(tag, b.y);
}

__device__ __forceinline__ void store_full_buf(float* row, int64_t lo, const float (&v)[8],
                                               const uint32_t (&)[4]) {
  const __amdgpu_buffer_rsrc_t r = span_rsrc(row, lo);
  __builtin_amdgcn_raw_buffer_store_b128(
      __builtin_bit_cast(u32x4, f32x4{v[0], v[1], v[2], v[3]}), r, 16u * threadIdx.x, 0,
      kBufStoreAux);
  __builtin_amdgcn_raw_buffer_store_b128(
      __builtin_bit_cast(u32x4, f32x4{v[4], v[5], v[6], v[7]}), r, 16u * (kBlock + threadIdx.x), 0,
      kBufStoreAux);
}

template <typename T16>
__device__ __forceinline__ void store_full_buf(T16* row, int64_t lo, const float (&)[8],
                                               const uint32_t (&h)[4]) {
  const __amdgpu_buffer_rsrc_t r = span_rsrc(row, lo);
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{h[0], h[1]}, r, 8u * threadIdx.x, 0, kBufStoreAux);
  __builtin_amdgcn_raw_buffer_store_b64(u32x2{h[2], h[3]}, r, 8u * (kBlock + threadIdx.x), 0,
                                        kBufStoreAux);
}

// Full span: buffer form; otherwise the checked loads of load8.
template <bool BUF, typename T>
__device__ __forceinline__ void load8b(const T* __restrict__ p, const Quads& q, int64_t lo,
                                       int64_t d, bool full, float (&v)[8]) {
  if (BUF && full)
    load_full_buf(p, lo, v);
  else
    load8(p, q, d, full, v);
}

template <bool BUF>
__device__ __forceinline__ void store8b(float* __restrict__ p, const Quads& q, int64_t lo,
                                        int64_t d, bool full, const float (&v)[8]) {
  if (BUF && full) {
    const uint32_t none[4] = {0, 0, 0, 0};
    store_full_buf(p, lo, v, none);
  } else {
    store8(p, q, d, full, v);
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

// First span of block b (same split as the host planner's span_begin): a
// multiply and a min, no 64-bit division in the prologue of short blocks.
__device__ __forceinline__ int64_t dspan(const Geo& G, int32_t b) {
  return (int64_t)b * G.q + min(b, G.r);
}

// A block's cursor over the pieces of one segment table: the current piece,
// its end and its segment.  A span peeks at the next piece (pcur_peek) before
// its own loads and steps with that (pcur_step) after its stores.  A table
// load issued after the stores and used by the next span would make that span
// wait for the stores to complete before its own loads go out (one counter
// tracks loads and stores in issue order), and so would a loaded value carried
// from one span to the next in another register.
struct PCur {
  int32_t p, end;  // current piece; one past the block's last piece
  int64_t hi;      // end of piece p
  int32_t js;      // segment of piece p
};
struct PNext {
  int64_t hi;
  int32_t js;
};

// Block-uniform values kept in scalar registers: a cursor value taken
// through a lane read is complete where it is taken, so no later join of
// paths has to wait for the load that produced it.
__device__ __forceinline__ int32_t uni(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int64_t uni(int64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)(v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ PCur pcur_start(const SegDev& T, int32_t b) {
  PCur c;
  c.p = uni(T.blk_first[b]);
  c.end = uni(T.blk_first[b + 1]);
  c.hi = uni(T.phi[c.p]);
  c.js = uni(T.pseg[c.p]);
  return c;
}

// The piece after the current one (the current one if it is the block's last).
__device__ __forceinline__ PNext pcur_peek(const PCur& c, const SegDev& T) {
  const int32_t q = min(c.p + 1, c.end - 1);
  return {T.phi[q], T.pseg[q]};
}

// Step past every piece that ends at or before hi: the first step takes the
// peeked piece, further ones (pieces shorter than a span) load theirs.
__device__ __forceinline__ void pcur_advance(PCur& c, const SegDev& T, const PNext& nx,
                                             int64_t hi) {
  if (c.p < c.end && c.hi <= hi) {
    if (++c.p < c.end) {
      c.hi = uni(nx.hi);
      c.js = uni(nx.js);
    }
    while (c.p < c.end && c.hi <= hi) {
      if (++c.p < c.end) {
        c.hi = uni(T.phi[c.p]);
        c.js = uni(T.pseg[c.p]);
      }
    }
  }
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
template <typename T>
__device__ __forceinline__ double sumsq_range(const T* row, const Quads& q, int64_t a,
                                              int64_t e) {
  double s = 0.0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t k = coord(q, j);
    if (k >= a && k < e) {
      const double x = (double)elem(row, k);
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

}  // namespace oba
