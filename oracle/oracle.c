/*
 * oracle.c -- plain, slow, single-threaded CPU oracle of the 1-bit Adam
 * compression-stage step.  TEST INFRASTRUCTURE ONLY (see oracle.h): nothing
 * in the GPU library includes or calls it, and it includes nothing of that
 * library.  Scalar loops, written in the order the method's steps are stated
 * on the pages; page abbreviations [Tang], [AIMech], [CwP] are defined in
 * oracle.h.
 *
 * Readings taken where the pages leave a step open (each is listed with its
 * reason in the design notes of the repository):
 *   R1  the broadcast server momentum replaces every worker's momentum
 *       (m <- m_hat), so one momentum vector exists in the compression stage;
 *   R2  no bias correction unless the caller passes bc1, bc2 != 1;
 *   R3  the preconditioner divides by sqrt(v) + eta;
 *   R4  the scale is ||c||_2 / ||sign(c)||_2 with sign(0) = +1, so the
 *       denominator is sqrt(segment length);
 *   R5  the server averages the n decompressed worker messages (mean), adds
 *       its error, and recompresses with the same 1-bit compressor.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* IEEE 754 binary16 decoded from its definition: sign, 5-bit biased exponent
 * (bias 15), 10-bit fraction; exponent 0 is subnormal (f * 2^-24).  Every
 * binary16 value is exactly representable in binary32 and binary64. */
double oracle_half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int f = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25);
  return sign ? -v : v;
}

/* bfloat16 decoded from its definition: sign, 8-bit biased exponent (bias
 * 127), 7-bit fraction; exponent 0 is subnormal (f * 2^-133).  Every
 * bfloat16 value is exactly representable in binary32. */
double oracle_bfloat16_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 7) & 255;
  int f = h & 127;
  double v;
  if (e == 0)
    v = ldexp((double)f, -133);
  else if (e == 255)
    v = f ? NAN : INFINITY;
  else
    v = ldexp((double)(128 + f), e - 134);
  return sign ? -v : v;
}

/* Round x to the nearest value of a binary floating-point format with p
 * significand bits (the leading bit included), smallest normal exponent
 * emin and largest finite value maxv; a tie goes to the even significand
 * (IEEE 754 roundTiesToEven).  Below 2^emin the grid is the subnormal one,
 * 2^(emin - p + 1).  A result above maxv becomes an infinity of x's sign;
 * zeros keep their sign.  The result is a double that the format holds
 * exactly. */
static double round_to_format(double x, int p, int emin, double maxv) {
  if (isnan(x) || isinf(x) || x == 0.0) return x;
  int e;
  frexp(fabs(x), &e); /* |x| = f * 2^e with 1/2 <= f < 1: x's exponent is e - 1 */
  int ex = e - 1 < emin ? emin : e - 1;
  const double ulp = ldexp(1.0, ex - (p - 1));
  const double r = nearbyint(x / ulp) * ulp; /* x / ulp is exact: a power-of-two scaling */
  return fabs(r) > maxv ? copysign(INFINITY, x) : r;
}

/* The bit pattern of v, a value of a 16-bit binary format (fraction bits fb,
 * exponent bias bias, all-ones exponent for inf and NaN), from its parts. */
static uint16_t format_bits(double v, int fb, int bias) {
  const uint16_t sign = signbit(v) ? 0x8000u : 0u;
  const int emax_field = (1 << (15 - fb)) - 1;
  if (isnan(v)) return (uint16_t)(sign | (emax_field << fb) | (1u << (fb - 1)));
  if (isinf(v)) return (uint16_t)(sign | (emax_field << fb));
  const double a = fabs(v);
  if (a < ldexp(1.0, 1 - bias)) /* zero or subnormal: a = f * 2^(1 - bias - fb) */
    return (uint16_t)(sign | (uint16_t)ldexp(a, bias - 1 + fb));
  int e;
  const double f = frexp(a, &e); /* a = (2f) * 2^(e-1), 1 <= 2f < 2 */
  const uint16_t frac = (uint16_t)ldexp(2.0 * f - 1.0, fb);
  return (uint16_t)(sign | (uint16_t)((e - 1 + bias) << fb) | frac);
}

/* binary32 -> binary16 (p = 11, emin = -14, max 65504), nearest, ties even */
uint16_t oracle_float_to_half(float x) {
  return format_bits(round_to_format((double)x, 11, -14, 65504.0), 10, 15);
}

/* binary32 -> bfloat16 (p = 8, emin = -126, max (2 - 2^-7) 2^127), nearest,
 * ties even */
uint16_t oracle_float_to_bfloat16(float x) {
  return format_bits(round_to_format((double)x, 8, -126, ldexp(255.0, 120)), 7, 127);
}

/* kind 1: binary16, kind 2: bfloat16 */
void oracle_round16(int64_t len, const float* x, uint16_t* out, int kind) {
  for (int64_t k = 0; k < len; ++k)
    out[k] = kind == 1 ? oracle_float_to_half(x[k]) : oracle_float_to_bfloat16(x[k]);
}

/* g_kind: 0 binary32, 1 binary16, 2 bfloat16 */
static float grad_at(const void* g, int g_kind, int64_t idx) {
  if (g_kind == 1) return (float)oracle_half_to_double(((const uint16_t*)g)[idx]);
  if (g_kind == 2) return (float)oracle_bfloat16_to_double(((const uint16_t*)g)[idx]);
  return ((const float*)g)[idx];
}

/* ---------------------------------------------------------------------------
 * Warm-up: one uncompressed Adam step on the mean gradient.
 * [AIMech] definition paragraph: v_t = b2 v_{t-1} + (1-b2) g_t^2 and
 * m_t = b1 m_{t-1} + (1-b1) g_t; [Tang] 1 and 4.3: plain Adam runs during the
 * warm-up, with an uncompressed exchange, so g_t is the mean of the workers'
 * gradients.  Per coordinate k, in this order:
 *   gbar = (((0 + g_0) + g_1) + ... + g_{n-1}) / n
 *   m = b1*m + (1-b1)*gbar
 *   v = b2*v + (1-b2)*(gbar*gbar)
 *   x = x - (lr*(m/bc1)) / (sqrt(v/bc2) + eta)
 * The binary32 coefficients are the binary64 hyperparameters rounded once;
 * (1-b1) and (1-b2) are formed in binary64 before that rounding.
 * ------------------------------------------------------------------------- */
void oracle_adam_warmup_step(int64_t d, int32_t n, int64_t ld, const void* g, int g_kind,
                             float* x, float* m, float* v, double lr_, double beta1_,
                             double beta2_, double eta_, double bc1_, double bc2_) {
  const float lr = (float)lr_, beta1 = (float)beta1_, beta2 = (float)beta2_;
  const float eta = (float)eta_, bc1 = (float)bc1_, bc2 = (float)bc2_;
  const float omb1 = (float)(1.0 - beta1_);
  const float omb2 = (float)(1.0 - beta2_);
  for (int64_t k = 0; k < d; ++k) {
    float sum = 0.0f;
    for (int32_t i = 0; i < n; ++i) sum = sum + grad_at(g, g_kind, (int64_t)i * ld + k);
    float gbar = sum / (float)n;
    float mk = beta1 * m[k] + omb1 * gbar;
    float vk = beta2 * v[k] + omb2 * (gbar * gbar);
    m[k] = mk;
    v[k] = vk;
    x[k] = x[k] - (lr * (mk / bc1)) / (sqrtf(vk / bc2) + eta);
  }
}

/* Norm of the fused variance vector, the quantity whose levelling-off
 * motivates the freeze ([Tang] 3.3, Figure 2): the plain definition
 * sqrt(sum_k v_k^2), every square exact in binary64, summed in index order. */
double oracle_l2norm(int64_t d, const float* v) {
  double s = 0.0;
  for (int64_t k = 0; k < d; ++k) {
    const double x = (double)v[k];
    s += x * x;
  }
  return sqrt(s);
}

/* When the warm-up may stop: the pages show the variance levelling off
 * ([Tang] 3.3, Figure 2; [AIMech] definition: run Adam until v stabilises)
 * but give no test.  Reading: at step t (1-based) the series h has levelled
 * off when t > window, t >= min_steps and |h_t - h_{t-window}| <= rtol*|h_t|.
 * Returns the first such t among h_1..h_len, or 0. */
int64_t oracle_plateau_first(int64_t len, const double* h, int32_t window, double rtol,
                             int32_t min_steps) {
  for (int64_t t = 1; t <= len; ++t) {
    if (t <= window || t < min_steps) continue;
    const double now = h[t - 1], before = h[t - 1 - window];
    if (fabs(now - before) <= rtol * fabs(now)) return t;
  }
  return 0;
}

/* Freeze: the variance stops changing and becomes the fixed preconditioner
 * V = diag(sqrt(v_Tw) + eta) ([AIMech] definition paragraph; [Tang] 3.3 and
 * 5).  denom = sqrt(v/bc2) + eta, stored once. */
void oracle_freeze_variance(int64_t d, const float* v, float* denom, double eta_, double bc2_) {
  const float eta = (float)eta_, bc2 = (float)bc2_;
  for (int64_t k = 0; k < d; ++k) denom[k] = sqrtf(v[k] / bc2) + eta;
}

/* ---------------------------------------------------------------------------
 * The 1-bit compressor with error compensation ([Tang] 4.3: sign of each
 * element plus one scale that keeps the magnitude; [CwP]: scale = magnitude
 * of the compensated vector / magnitude of its sign vector; [AIMech]
 * gather-broadcast mechanism: worker and server error memories).
 * ------------------------------------------------------------------------- */

/* sum of c^2 over a segment, each square exact in binary64 */
double oracle_sumsq(int64_t len, const float* c) {
  double s = 0.0;
  for (int64_t k = 0; k < len; ++k) s += (double)c[k] * (double)c[k];
  return s;
}

/* ||c||_2 / ||sign(c)||_2 where every sign is +-1, so ||sign(c)||_2^2 = len */
float oracle_scale(double sumsq, int64_t len) { return (float)sqrt(sumsq / (double)len); }

/* bit k (global index bit0+k) = 1 iff c[k] < 0; -0.0 and +0.0 give 0 (+1) */
void oracle_pack_signs(int64_t len, const float* c, uint64_t* bits, int64_t bit0) {
  for (int64_t k = 0; k < len; ++k) {
    int64_t b = bit0 + k;
    if (c[k] < 0.0f) bits[b >> 6] |= (uint64_t)1 << (b & 63);
  }
}

int oracle_bit(const uint64_t* bits, int64_t k) { return (int)((bits[k >> 6] >> (k & 63)) & 1); }

/* err = c - s*sign(c), sign(c) = -1 if c < 0 else +1 */
void oracle_residual(int64_t len, const float* c, float s, float* err) {
  for (int64_t k = 0; k < len; ++k) {
    float sg = (c[k] < 0.0f) ? -1.0f : 1.0f;
    err[k] = c[k] - s * sg;
  }
}

/* Compress one vector c of length d with segment table seg: per segment a
 * scale, signs into bits (row of W words, cleared here), residual into err. */
static void ec_onebit(int64_t d, const int64_t* seg, int32_t n_seg, const float* c,
                      uint64_t* bits, float* scale, float* err) {
  int64_t W = (d + 63) / 64;
  memset(bits, 0, (size_t)W * sizeof(uint64_t));
  for (int32_t j = 0; j < n_seg; ++j) {
    int64_t lo = seg[j], hi = seg[j + 1];
    float s = oracle_scale(oracle_sumsq(hi - lo, c + lo), hi - lo);
    scale[j] = s;
    oracle_pack_signs(hi - lo, c + lo, bits, lo);
    oracle_residual(hi - lo, c + lo, s, err + lo);
  }
}

/* Worker side, per coordinate ([Tang] 11: each worker updates its momentum
 * locally and applies error-compensated compression; [AIMech] definition
 * paragraph for the momentum recurrence):
 *   c = (b1*m + (1-b1)*g) + delta      two products, then two adds
 * with b1 and (1-b1) rounded to binary32 from binary64 as in the warm-up. */
void oracle_compensate(int64_t len, double beta1_, const float* m, const void* g, int g_kind,
                       int64_t g_off, const float* delta, float* c) {
  const float beta1 = (float)beta1_;
  const float omb1 = (float)(1.0 - beta1_);
  for (int64_t k = 0; k < len; ++k) {
    float p = beta1 * m[k] + omb1 * grad_at(g, g_kind, g_off + k);
    c[k] = p + delta[k];
  }
}

void oracle_compress(int64_t d, int32_t n, int64_t ld, const int64_t* wseg, int32_t n_wseg,
                     const void* g, int g_kind, const float* m, float* delta, uint64_t* wbits,
                     float* wscale, double beta1) {
  int64_t W = (d + 63) / 64;
  float* c = (float*)malloc((size_t)(d > 0 ? d : 1) * sizeof(float));
  for (int32_t i = 0; i < n; ++i) {
    float* di = delta + (int64_t)i * ld;
    oracle_compensate(d, beta1, m, g, g_kind, (int64_t)i * ld, di, c);
    ec_onebit(d, wseg, n_wseg, c, wbits + (int64_t)i * W, wscale + (int64_t)i * n_wseg, di);
  }
  free(c);
}

/* The worker pass with each worker's compensated momentum held in a 16-bit
 * format, c_kind 1 (binary16) or 2 (bfloat16): the deferred layout of the
 * state, where c16 [n][ld] holds each worker's last compressed vector and
 * wscale_prev its scales.  Worker i, coordinate k:
 *   c'    = c16 decoded;  delta = c' - s'*sign(c')   (s' the scale of k's segment)
 *   c     = (b1*m + (1-b1)*g) + delta                 (binary32, as above)
 *   c~    = c rounded to the 16-bit format, nearest, ties to even
 * then c~ is the vector compressed ([Tang] 4.3; [CwP] scale) and stored as
 * the new c16.  The rounding c - c~ is this variant's own loss and is not
 * fed back; the residual the next step feeds back is exact for what was
 * sent.  wbits, wscale as for oracle_compress. */
void oracle_compress_deferred16(int64_t d, int32_t n, int64_t ld, const int64_t* wseg,
                                int32_t n_wseg, const void* g, int g_kind, const float* m,
                                uint16_t* c16, int c_kind, const float* wscale_prev,
                                uint64_t* wbits, float* wscale, double beta1) {
  int64_t W = (d + 63) / 64;
  size_t bytes = (size_t)(d > 0 ? d : 1) * sizeof(float);
  float* cp = (float*)malloc(bytes);
  float* delta = (float*)malloc(bytes);
  float* c = (float*)malloc(bytes);
  float* unused = (float*)malloc(bytes);
  for (int32_t i = 0; i < n; ++i) {
    uint16_t* row = c16 + (int64_t)i * ld;
    for (int64_t k = 0; k < d; ++k)
      cp[k] = (float)(c_kind == 1 ? oracle_half_to_double(row[k])
                                  : oracle_bfloat16_to_double(row[k]));
    for (int32_t j = 0; j < n_wseg; ++j)
      oracle_residual(wseg[j + 1] - wseg[j], cp + wseg[j],
                      wscale_prev[(int64_t)i * n_wseg + j], delta + wseg[j]);
    oracle_compensate(d, beta1, m, g, g_kind, (int64_t)i * ld, delta, c);
    for (int64_t k = 0; k < d; ++k) {
      row[k] = c_kind == 1 ? oracle_float_to_half(c[k]) : oracle_float_to_bfloat16(c[k]);
      c[k] = (float)(c_kind == 1 ? oracle_half_to_double(row[k])
                                 : oracle_bfloat16_to_double(row[k]));
    }
    ec_onebit(d, wseg, n_wseg, c, wbits + (int64_t)i * W, wscale + (int64_t)i * n_wseg, unused);
  }
  free(cp);
  free(delta);
  free(c);
  free(unused);
}

/* Per-worker momentum: the other reading of [Tang] 4.3 (each worker keeps
 * and updates its own momentum, the broadcast m_hat only moves x).  Worker i:
 *   m_i = b1*m_i + (1-b1)*g_i      (kept by the worker)
 *   c   = m_i + delta_i
 * then the same compressor.  m_local, delta: [n][ld], updated in place. */
void oracle_compress_local(int64_t d, int32_t n, int64_t ld, const int64_t* wseg, int32_t n_wseg,
                           const void* g, int g_kind, float* m_local, float* delta,
                           uint64_t* wbits, float* wscale, double beta1_) {
  const float beta1 = (float)beta1_;
  const float omb1 = (float)(1.0 - beta1_);
  int64_t W = (d + 63) / 64;
  float* c = (float*)malloc((size_t)(d > 0 ? d : 1) * sizeof(float));
  for (int32_t i = 0; i < n; ++i) {
    float* mi = m_local + (int64_t)i * ld;
    float* di = delta + (int64_t)i * ld;
    for (int64_t k = 0; k < d; ++k) {
      mi[k] = beta1 * mi[k] + omb1 * grad_at(g, g_kind, (int64_t)i * ld + k);
      c[k] = mi[k] + di[k];
    }
    ec_onebit(d, wseg, n_wseg, c, wbits + (int64_t)i * W, wscale + (int64_t)i * n_wseg, di);
  }
  free(c);
}

/* Server side, per coordinate k in [k0, k1) ([Tang] 11: the server averages
 * the workers' messages, then compresses again; [AIMech] gather-broadcast
 * mechanism: server error memory):
 *   t = ((0 + s_0*sg_0) + s_1*sg_1) + ... + s_{n-1}*sg_{n-1}
 *   a = t / n + eps
 * where s_i is worker i's scale for the worker segment holding k and sg_i its
 * decoded sign.  eps and a are indexed by the global coordinate. */
void oracle_server_average(int64_t k0, int64_t k1, int64_t d, int32_t n, const int64_t* wseg,
                           int32_t n_wseg, const uint64_t* wbits, const float* wscale,
                           const float* eps, float* a) {
  int64_t W = (d + 63) / 64;
  int32_t j = 0;
  for (int64_t k = k0; k < k1; ++k) {
    while (wseg[j + 1] <= k) ++j;
    float t = 0.0f;
    for (int32_t i = 0; i < n; ++i) {
      float s = wscale[(int64_t)i * n_wseg + j];
      float sg = oracle_bit(wbits + (int64_t)i * W, k) ? -1.0f : 1.0f;
      t = t + s * sg;
    }
    a[k] = t / (float)n + eps[k];
  }
}

void oracle_server_reduce_recompress(int64_t d, int32_t n, const int64_t* wseg, int32_t n_wseg,
                                     const int64_t* sseg, int32_t n_sseg, const uint64_t* wbits,
                                     const float* wscale, float* eps, uint64_t* sbits,
                                     float* sscale) {
  float* a = (float*)malloc((size_t)(d > 0 ? d : 1) * sizeof(float));
  oracle_server_average(0, d, d, n, wseg, n_wseg, wbits, wscale, eps, a);
  ec_onebit(d, sseg, n_sseg, a, sbits, sscale, eps);
  free(a);
}

/* Broadcast and update ([Tang] 11: the server broadcasts the momentum and
 * workers update their models; [AIMech] definition paragraph:
 * x_t = x_{t-1} - gamma V^{-1} m_hat_t), per coordinate k in [k0, k1):
 *   m_hat = s_tau * sign        (s_tau: scale of the server segment of k)
 *   m = m_hat                   (reading R1)
 *   x = x - (lr*m_hat) / denom */
void oracle_decompress_update(int64_t k0, int64_t k1, const int64_t* sseg, int32_t n_sseg,
                              const uint64_t* sbits, const float* sscale, const float* denom,
                              float* m, float* x, double lr_) {
  const float lr = (float)lr_;
  int32_t j = 0;
  (void)n_sseg;
  for (int64_t k = k0; k < k1; ++k) {
    while (sseg[j + 1] <= k) ++j;
    float mh = sscale[j] * (oracle_bit(sbits, k) ? -1.0f : 1.0f);
    m[k] = mh;
    x[k] = x[k] - (lr * mh) / denom[k];
  }
}
