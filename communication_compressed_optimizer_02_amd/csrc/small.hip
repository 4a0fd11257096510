// small.hip -- the whole deferred compression step in one thread block, for
// layouts small enough that launch latency, not HBM, bounds the step
// (gfx950).  The arithmetic of every coordinate is that of the streaming
// kernels, in the same order; only the norms are summed in another fixed
// order (one block reduction per segment and row).
// Method passages are cited in include/oba.h beside each entry point.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device.hpp"

namespace oba {

namespace {

constexpr int kSmallWaves = kSmallBlock / 64;

// Sum of v over the block in a fixed order; every thread gets the sum.
__device__ __forceinline__ double block_sum(double v, double* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double s = 0.0;
  for (int w = 0; w < kSmallWaves; ++w) s += red[w];
  __syncthreads();  // red is reused by the next call
  return s;
}

__device__ __forceinline__ int bit_at(const uint64_t* row, int64_t k) {
  return (int)((row[k >> 6] >> (k & 63)) & 1u);
}

// Packs (v[k] < 0) of row `vals` into words[0, W): wave w packs words
// w, w + kSmallWaves, ... with one ballot each; lane 0 stores the word.
__device__ __forceinline__ void pack_row(const float* vals, int64_t d, int64_t W,
                                         uint64_t* words) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int64_t w = wv; w < W; w += kSmallWaves) {
    const int64_t k = w * 64 + lane;
    const bool neg = k < d && vals[k] < 0.0f;
    const uint64_t mask = __ballot(neg);
    if (lane == 0) words[w] = mask;
  }
}

}  // namespace

template <typename GT>
__global__ __launch_bounds__(kSmallBlock) void k_step_small(SmallArgs A) {
  __shared__ double red[kSmallWaves];
  __shared__ int64_t woff[kSmallMaxSeg + 1], soff[kSmallMaxSeg + 1];
  const int tid = threadIdx.x;
  for (int j = tid; j <= A.n_wseg; j += kSmallBlock) woff[j] = A.wseg[j];
  for (int j = tid; j <= A.n_sseg; j += kSmallBlock) soff[j] = A.sseg[j];
  __syncthreads();
  const GT* g = static_cast<const GT*>(A.g);

  // 1. worker side: the last step's residual, then this step's c
  for (int32_t i = 0; i < A.n; ++i) {
    float* ci = A.c + (int64_t)i * A.ld;
    const float* si = A.wscale + (int64_t)i * A.n_wseg;
    const GT* gi = g + (int64_t)i * A.ld;
    int32_t js = 0, jt = 0;
    for (int64_t k = tid; k < A.d; k += kSmallBlock) {
      js = seg_walk(woff, js, k);
      float mk;
      if (A.m_in) {
        mk = A.m_in[k];
      } else {  // m = sbar*sign from the last server message
        jt = seg_walk(soff, jt, k);
        mk = bit_at(A.sbits, k) ? -A.sscale[jt] : A.sscale[jt];
      }
      const float dl = residual(ci[k], si[js]);
      ci[k] = compensate(A.b1, A.omb1, mk, elem(gi, k), dl);
    }
  }
  __syncthreads();  // every read of the last scales and message is done

  // 2. worker scales and bits
  for (int32_t i = 0; i < A.n; ++i) {
    const float* ci = A.c + (int64_t)i * A.ld;
    for (int32_t j = 0; j < A.n_wseg; ++j) {
      double s = 0.0;
      for (int64_t k = woff[j] + tid; k < woff[j + 1]; k += kSmallBlock) {
        const double x = (double)ci[k];
        s = __builtin_fma(x, x, s);
      }
      s = block_sum(s, red);
      if (tid == 0)
        A.wscale[(int64_t)i * A.n_wseg + j] =
            (float)__builtin_sqrt(s / (double)(woff[j + 1] - woff[j]));
    }
    pack_row(ci, A.d, A.W, A.wbits + (int64_t)i * A.W);
  }
  __syncthreads();

  // 3. server: the last server residual, the mean of the messages, a
  const float nf = (float)A.n;
  const bool pow2 = (A.n & (A.n - 1)) == 0;
  const float inv_n = 1.0f / nf;
  {
    int32_t js = 0, jt = 0;
    for (int64_t k = tid; k < A.d; k += kSmallBlock) {
      js = seg_walk(woff, js, k);
      jt = seg_walk(soff, jt, k);
      const float e = residual(A.a[k], A.sscale[jt]);
      float t = 0.0f;
      for (int32_t i = 0; i < A.n; ++i) {
        const float s_ = A.wscale[(int64_t)i * A.n_wseg + js];
        t = t + (bit_at(A.wbits + (int64_t)i * A.W, k) ? -s_ : s_);
      }
      A.a[k] = (pow2 ? t * inv_n : t / nf) + e;
    }
  }
  __syncthreads();  // every read of the last server scales is done
  for (int32_t j = 0; j < A.n_sseg; ++j) {
    double s = 0.0;
    for (int64_t k = soff[j] + tid; k < soff[j + 1]; k += kSmallBlock) {
      const double x = (double)A.a[k];
      s = __builtin_fma(x, x, s);
    }
    s = block_sum(s, red);
    if (tid == 0) A.sscale[j] = (float)__builtin_sqrt(s / (double)(soff[j + 1] - soff[j]));
  }
  pack_row(A.a, A.d, A.W, A.sbits);
  __syncthreads();

  // 4. decompress, precondition, update
  {
    int32_t jt = 0;
    for (int64_t k = tid; k < A.d; k += kSmallBlock) {
      jt = seg_walk(soff, jt, k);
      const float mh = (A.a[k] < 0.0f) ? -A.sscale[jt] : A.sscale[jt];
      if (A.m_out) A.m_out[k] = mh;
      A.x[k] = A.x[k] - (A.lr * mh) / A.denom[k];
    }
  }
}

// ---- launchers ----------------------------------------------------------------

void launch_step_small(const SmallArgs& A, int gdt, hipStream_t st) {
  if (gdt == kGradF16)
    hipLaunchKernelGGL(k_step_small<uint16_t>, dim3(1), dim3(kSmallBlock), 0, st, A);
  else if (gdt == kGradBF16)
    hipLaunchKernelGGL(k_step_small<bf16_bits>, dim3(1), dim3(kSmallBlock), 0, st, A);
  else
    hipLaunchKernelGGL(k_step_small<float>, dim3(1), dim3(kSmallBlock), 0, st, A);
}

}  // namespace oba
