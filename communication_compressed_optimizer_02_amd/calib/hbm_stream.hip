// hbm_stream.hip -- streaming probes that measure what this GPU's HBM delivers
// for the access shapes of the 1-bit Adam kernels (gfx950).  Measurement aid
// only (libhbmstream.so, used by bench.py): no arithmetic of the method.
//
// Every probe walks spans of kSpan = 2048 coordinates, one span per block of
// 256 threads, in the lane layout of the method's streaming kernels (thread t
// owns the quads [lo+4t, lo+4t+4) and [lo+1024+4t, +4)), with non-temporal
// loads and stores, and the same two memory-instruction forms they use:
// global loads and stores, or buffer-resource loads and stores per (row,
// span).  A block handles `NA` rows of A (read only) and `NB` rows of B (not
// touched, written only, or read and written in place) per group; grid.y
// counts the groups, so a shape with groups of 4 rows and grid.y = 2 is the
// deferred worker pass's 8 workers in two groups of 4.  All loads of a block
// are issued before its stores, as in the method's kernels; every stored
// value depends on the values loaded, and every loaded row reaches a stored
// value (a read-only probe sums all of them), so no access can be elided.
//
// C ABI (plain pointers, device memory of the current device):
//   int hbm_stream_shape(int shape, int32_t out[5]);
//     out = {rows of A per group, bytes per A element, rows of B per group,
//            bytes per B element, B mode (0 none, 1 write only, 2 read+write)}
//     Returns 0, or -1 for an unknown shape.
//   int hbm_stream_launch(int shape, int buf, const void* a, void* b, int64_t ld,
//                         int64_t spans, int32_t groups, int32_t blocks_per_cu,
//                         float* sink, hipStream_t stream);
//     a: [groups * rows_a][ld] elements, b: [groups * rows_b][ld] elements,
//     16-byte aligned; ld % 8 == 0 and ld >= spans * 2048; sink: one float
//     (written only by a read-only probe, and only in the improbable case
//     that its loaded values sum to a chosen constant).  buf: bit 0 the
//     buffer forms, bit 1 the worker passes' load order (A and B rows
//     alternating; for read-and-write shapes with as many A as B rows).  blocks_per_cu > 0 caps the resident blocks per compute unit
//     (each block takes 1/blocks_per_cu of the CU's LDS, unused), i.e. the
//     waves per SIMD, since a block is one wave per SIMD; 0 leaves the cap to
//     the kernel's registers.  Enqueues one launch on `stream`; returns 0, -1
//     for a bad argument (checked on the host, nothing launched), -5 for a
//     HIP error.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device.hpp"

namespace oba {
namespace {

enum { kNone = 0, kWrite = 1, kRmw = 2 };

template <typename T>
__device__ __forceinline__ void probe_load(const T* row, const Quads& q, int64_t lo, bool buf,
                                           float (&v)[8]) {
  if (buf)
    load_full_buf(row, lo, v);
  else
    load_full(row, q, v);
}

template <typename T>
__device__ __forceinline__ void probe_store(T* row, const Quads& q, int64_t lo, bool buf,
                                            float (&v)[8]) {
  uint32_t h[4] = {0, 0, 0, 0};
  round_to_row<T>(v, h);
  if (buf)
    store_full_buf(row, lo, v, h);
  else
    store_row(row, q, lo + kSpan, true, v, h);
}

// ILV (read-and-write shapes with as many A as B rows): the loads alternate
// A row u, B row u -- the worker passes' order (gradient, then state, worker
// by worker) -- instead of all A rows, then all B rows.
// SID: the shape's index, so that every shape is a kernel of its own name
// (two shapes may have the same rows and differ in their groups)
template <int SID, typename TA, typename TB, int NA, int NB, int BMODE, bool BUF, bool ILV>
__global__ __launch_bounds__(kBlock) void k_stream(const TA* __restrict__ a, TB* __restrict__ b,
                                                   int64_t ld, float* __restrict__ sink) {
  const int64_t lo = (int64_t)blockIdx.x * kSpan;
  const Quads q = quads(lo);
  const TA* ar = a + (int64_t)blockIdx.y * NA * ld;
  TB* br = b + (int64_t)blockIdx.y * NB * ld;
  float va[NA > 0 ? NA : 1][8];
  float vb[NB > 0 ? NB : 1][8];
  if constexpr (ILV && BMODE == kRmw && NA == NB) {
#pragma unroll
    for (int u = 0; u < NA; ++u) {
      probe_load(ar + u * ld, q, lo, BUF, va[u]);
      probe_load(br + u * ld, q, lo, BUF, vb[u]);
    }
  } else {
#pragma unroll
    for (int u = 0; u < NA; ++u) probe_load(ar + u * ld, q, lo, BUF, va[u]);
    if constexpr (BMODE == kRmw) {
#pragma unroll
      for (int u = 0; u < NB; ++u) probe_load(br + u * ld, q, lo, BUF, vb[u]);
    }
  }
  if constexpr (BMODE == kNone) {
    float s = 0.0f;
#pragma unroll
    for (int u = 0; u < NA; ++u)
#pragma unroll
      for (int j = 0; j < 8; ++j) s = s + va[u][j];
    if (s == 1.25e-37f) sink[0] = s;
  } else {
    // Row u of B takes the A rows u, u + NB, u + 2 NB, ... (so that every
    // loaded A row reaches a store and no load can be dropped), or A row
    // u % NA when there are fewer A rows than B rows.
#pragma unroll
    for (int u = 0; u < NB; ++u) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float acc = BMODE == kRmw ? vb[u][j] : 0.0f;
        if constexpr (NA == 0) {
          acc = acc + (float)j;
        } else if (u >= NA) {
          acc = acc + va[u % (NA > 0 ? NA : 1)][j];
        } else {
#pragma unroll
          for (int k = u; k < NA; k += NB) acc = acc + va[k][j];
        }
        vb[u][j] = acc + 1.0f;
      }
      probe_store(br + u * ld, q, lo, BUF, vb[u]);
    }
  }
}

struct Shape {
  int32_t na, a_bytes, nb, b_bytes, bmode;
};

// Rows per group.  The deferred worker pass at 8 workers with binary16
// gradients is shape 9 with eight groups (one worker per block; shape 3 the
// same with groups of four), with binary32 gradients shape 13; its
// 16-bit-state form shape 12 with eight groups (shape 5 with groups of
// four); the
// warm-up at 8 workers shape 6; the update shape 7; the server pass's a
// shape 8 (its packed rows, n/8 bytes per coordinate, are left out).
constexpr Shape kShapes[] = {
    {8, 4, 0, 4, kNone},   // 0 read: 8 binary32 rows
    {0, 4, 8, 4, kWrite},  // 1 write: 8 binary32 rows
    {4, 4, 4, 4, kWrite},  // 2 copy: 4 rows read, 4 other rows written
    {4, 2, 4, 4, kRmw},    // 3 worker pass, 16-bit gradients: 4 g rows, 4 c rows in place
    {4, 4, 4, 4, kRmw},    // 4 worker pass, binary32 gradients
    {4, 2, 4, 2, kRmw},    // 5 worker pass, 16-bit gradients and 16-bit c rows
    {8, 2, 3, 4, kRmw},    // 6 warm-up, 8 16-bit gradient rows, m v x in place
    {1, 4, 1, 4, kRmw},    // 7 update: denom read, x in place
    {0, 4, 1, 4, kRmw},    // 8 one row in place (the server pass's a)
    {1, 2, 1, 4, kRmw},    // 9 shape 3 with one worker per group
    {2, 2, 2, 4, kRmw},    // 10 shape 3 with two workers per group
    {8, 2, 8, 4, kRmw},    // 11 shape 3 with eight workers per group
    {1, 2, 1, 2, kRmw},    // 12 shape 5 with one worker per group
    {1, 4, 1, 4, kRmw},    // 13 shape 4 with one worker per group
};
constexpr int kNumShapes = sizeof(kShapes) / sizeof(kShapes[0]);

template <int SID, typename TA, typename TB, int NA, int NB, int BMODE, bool ILV>
int launch_t2(bool buf, const void* a, void* b, int64_t ld, int64_t spans, int32_t groups,
              size_t lds, float* sink, hipStream_t st) {
  const dim3 grid((unsigned)spans, (unsigned)groups);
  const TA* pa = static_cast<const TA*>(a);
  TB* pb = static_cast<TB*>(b);
  const void* fn =
      buf ? reinterpret_cast<const void*>(&k_stream<SID, TA, TB, NA, NB, BMODE, true, ILV>)
          : reinterpret_cast<const void*>(&k_stream<SID, TA, TB, NA, NB, BMODE, false, ILV>);
  if (lds > 0 &&
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return -5;
  if (buf)
    hipLaunchKernelGGL((k_stream<SID, TA, TB, NA, NB, BMODE, true, ILV>), grid, dim3(kBlock), lds, st,
                       pa, pb, ld, sink);
  else
    hipLaunchKernelGGL((k_stream<SID, TA, TB, NA, NB, BMODE, false, ILV>), grid, dim3(kBlock), lds,
                       st, pa, pb, ld, sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

template <int SID, typename TA, typename TB, int NA, int NB, int BMODE>
int launch_t(int buf, const void* a, void* b, int64_t ld, int64_t spans, int32_t groups,
             size_t lds, float* sink, hipStream_t st) {
  if (buf & 2)
    return launch_t2<SID, TA, TB, NA, NB, BMODE, true>(buf & 1, a, b, ld, spans, groups, lds, sink,
                                                       st);
  return launch_t2<SID, TA, TB, NA, NB, BMODE, false>(buf & 1, a, b, ld, spans, groups, lds, sink,
                                                      st);
}

}  // namespace
}  // namespace oba

extern "C" {

int hbm_stream_shape(int shape, int32_t* out) {
  if (shape < 0 || shape >= oba::kNumShapes || !out) return -1;
  const oba::Shape& s = oba::kShapes[shape];
  out[0] = s.na;
  out[1] = s.a_bytes;
  out[2] = s.nb;
  out[3] = s.b_bytes;
  out[4] = s.bmode;
  return 0;
}

int hbm_stream_launch(int shape, int buf, const void* a, void* b, int64_t ld, int64_t spans,
                      int32_t groups, int32_t blocks_per_cu, float* sink, hipStream_t st) {
  using namespace oba;
  if (shape < 0 || shape >= kNumShapes) return -1;
  const Shape& s = kShapes[shape];
  if (spans < 1 || spans > 0x7fffffffLL || groups < 1 || groups > 65535) return -1;
  if (ld % 8 != 0 || ld < spans * kSpan) return -1;
  if ((s.na > 0 && (!a || ((uintptr_t)a & 15))) || (s.nb > 0 && (!b || ((uintptr_t)b & 15))) ||
      !sink)
    return -1;
  if (blocks_per_cu < 0 || blocks_per_cu > 32) return -1;
  size_t lds = 0;
  if (blocks_per_cu > 0) {  // an LDS share per block that lets blocks_per_cu blocks fit a CU
    int dev = 0, per_cu = 0, per_block = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                              dev) != hipSuccess ||
        hipDeviceGetAttribute(&per_block, hipDeviceAttributeSharedMemPerBlockOptin, dev) !=
            hipSuccess)
      return -5;
    lds = (size_t)(per_cu / blocks_per_cu) / 512 * 512;
    if (lds == 0 || (int)lds > per_block) return -1;
  }
  if (buf < 0 || buf > 3) return -1;
  const int bf = buf;
  switch (shape) {
    case 0: return launch_t<0, float, float, 8, 0, kNone>(bf, a, b, ld, spans, groups, lds, sink, st);
    case 1: return launch_t<1, float, float, 0, 8, kWrite>(bf, a, b, ld, spans, groups, lds, sink, st);
    case 2: return launch_t<2, float, float, 4, 4, kWrite>(bf, a, b, ld, spans, groups, lds, sink, st);
    case 3: return launch_t<3, uint16_t, float, 4, 4, kRmw>(bf, a, b, ld, spans, groups, lds, sink, st);
    case 4: return launch_t<4, float, float, 4, 4, kRmw>(bf, a, b, ld, spans, groups, lds, sink, st);
    case 5:
      return launch_t<5, uint16_t, uint16_t, 4, 4, kRmw>(bf, a, b, ld, spans, groups, lds, sink, st);
    case 6: return launch_t<6, uint16_t, float, 8, 3, kRmw>(bf, a, b, ld, spans, groups, lds, sink, st);
    case 7: return launch_t<7, float, float, 1, 1, kRmw>(bf, a, b, ld, spans, groups, lds, sink, st);
    case 8: return launch_t<8, float, float, 0, 1, kRmw>(bf, a, b, ld, spans, groups, lds, sink, st);
    case 9: return launch_t<9, uint16_t, float, 1, 1, kRmw>(bf, a, b, ld, spans, groups, lds, sink, st);
    case 10:
      return launch_t<10, uint16_t, float, 2, 2, kRmw>(bf, a, b, ld, spans, groups, lds, sink, st);
    case 11:
      return launch_t<11, uint16_t, float, 8, 8, kRmw>(bf, a, b, ld, spans, groups, lds, sink, st);
    case 12:
      return launch_t<12, uint16_t, uint16_t, 1, 1, kRmw>(bf, a, b, ld, spans, groups, lds, sink, st);
    default: return launch_t<13, float, float, 1, 1, kRmw>(bf, a, b, ld, spans, groups, lds, sink, st);
  }
}

}  // extern "C"
