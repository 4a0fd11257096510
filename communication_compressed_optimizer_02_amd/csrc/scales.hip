// scales.hip -- per-segment scales from the binary64 partials (gfx950).
// Method passages are cited in include/oba.h beside each entry point.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device.hpp"

namespace oba {

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

// ---- launchers ----------------------------------------------------------------

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

}  // namespace oba
