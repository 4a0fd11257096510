/* oracle_driver.c -- runs every oracle function on small, awkward inputs
 * (d not a multiple of 64, segment boundaries inside 64-bit words, n = 3,
 * binary16 and bfloat16 gradients, zero-length and one-coordinate cases) so
 * that the test suite can build the oracle with address and
 * undefined-behaviour sanitizers.  Prints a checksum; exit 0 on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static uint64_t state = 88172645463325252ull;
static double urand(void) { /* xorshift64 */
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return (double)(state >> 11) * (1.0 / 9007199254740992.0);
}

static double run(int64_t d, int32_t n, int g_kind) {
  const int64_t ld = (d + 7) / 8 * 8, W = (d + 63) / 64;
  int64_t wseg[4] = {0, d / 3, d / 3 + 1, d}, sseg[3] = {0, d / 2 + 5, d};
  int32_t nw = 3, ns = 2;
  if (d < 8) { wseg[1] = d; nw = 1; sseg[1] = d; ns = 1; }
  float* x = calloc((size_t)d + 1, 4);
  float* m = calloc((size_t)d + 1, 4);
  float* v = calloc((size_t)d + 1, 4);
  float* den = calloc((size_t)d + 1, 4);
  float* eps = calloc((size_t)d + 1, 4);
  float* delta = calloc((size_t)(n * ld) + 1, 4);
  float* ml = calloc((size_t)(n * ld) + 1, 4);
  float* g32 = calloc((size_t)(n * ld) + 1, 4);
  uint16_t* g16 = calloc((size_t)(n * ld) + 1, 2);
  uint64_t* wb = calloc((size_t)(n * W) + 1, 8);
  uint64_t* sb = calloc((size_t)W + 1, 8);
  float* wsc = calloc((size_t)(n * nw), 4);
  float* ssc = calloc((size_t)ns, 4);
  const void* g = g_kind ? (const void*)g16 : (const void*)g32;
  for (int64_t k = 0; k < d; ++k) x[k] = (float)(0.02 * (urand() - 0.5));
  double sum = 0.0;
  for (int t = 0; t < 4; ++t) {
    for (int64_t r = 0; r < (int64_t)n * ld; ++r) {
      g32[r] = (float)(urand() - 0.5);
      /* moderate magnitudes (about 2^-6 .. 2^1) with random sign and fraction */
      const uint32_t sgn = urand() < 0.5 ? 0x8000u : 0u;
      if (g_kind == 1)
        g16[r] = (uint16_t)(sgn | ((uint32_t)(9 + 8 * urand()) << 10) | (uint32_t)(urand() * 1023));
      else
        g16[r] = (uint16_t)(sgn | ((uint32_t)(121 + 8 * urand()) << 7) | (uint32_t)(urand() * 127));
    }
    if (t < 2) {
      oracle_adam_warmup_step(d, n, ld, g, g_kind, x, m, v, 1e-3, 0.9, 0.999, 1e-8, 1.0, 1.0);
      sum += oracle_l2norm(d, v);
      if (t == 1) {
        oracle_freeze_variance(d, v, den, 1e-8, 1.0);
        for (int64_t r = 0; r < (int64_t)n * ld; ++r) ml[r] = m[r % ld < d ? r % ld : 0];
      }
      continue;
    }
    oracle_compress(d, n, ld, wseg, nw, g, g_kind, m, delta, wb, wsc, 0.9);
    oracle_server_reduce_recompress(d, n, wseg, nw, sseg, ns, wb, wsc, eps, sb, ssc);
    oracle_decompress_update(0, d, sseg, ns, sb, ssc, den, m, x, 1e-3);
    oracle_compress_local(d, n, ld, wseg, nw, g, g_kind, ml, delta, wb, wsc, 0.9);
    for (int64_t k = 0; k < d; ++k) sum += x[k] + (oracle_bit(sb, k) ? 1.0 : 0.0);
  }
  double h[40];
  for (int i = 0; i < 40; ++i) h[i] = 1.0 - pow(0.9, i + 1);
  sum += (double)oracle_plateau_first(40, h, 5, 0.05, 0) + oracle_plateau_first(0, h, 1, 0.1, 0);
  sum += oracle_half_to_double(0x3c00) + oracle_bfloat16_to_double(0x3f80);
  free(x); free(m); free(v); free(den); free(eps); free(delta); free(ml); free(g32); free(g16);
  free(wb); free(sb); free(wsc); free(ssc);
  return sum;
}

int main(void) {
  double s = 0.0;
  const int64_t ds[] = {1, 7, 64, 65, 130, 1000, 4099};
  for (size_t i = 0; i < sizeof(ds) / sizeof(ds[0]); ++i)
    for (int kind = 0; kind < 3; ++kind) s += run(ds[i], 3, kind);
  printf("checksum %.17g\n", s);
  return isfinite(s) ? 0 : 1;
}
