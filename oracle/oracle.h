/*
 * oracle.h -- plain CPU oracle of the 1-bit Adam compression-stage step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * includes, links or calls anything here, and this file includes nothing of
 * the GPU library.
 *
 * Pages cited (by title and section):
 *   [Tang]   "1-bit Adam: Communication Efficient Large-Scale Training with
 *            Adam's Convergence Speed" -- paper summary page, sections as
 *            numbered on that page (4.3 algorithm, 6 system design,
 *            11 proof to the updating form, 12 proof to Theorem 1).
 *   [AIMech] "1-bit Adam (Two-Stage Preconditioner-Frozen Error-Compensated
 *            Adam)" -- curated algorithm page: definition paragraph, and the
 *            claims "Mechanism: nonlinear variance / preconditioner freeze"
 *            and "Mechanism: custom compressed allreduce gather-broadcast".
 *   [CwP]    "1-bit Adam" -- method description page (scale factor, volume).
 *
 * Numerics contract (all functions): hyperparameters arrive in binary64 and
 * each binary32 coefficient is rounded from binary64 once (b1 = fl32(beta1),
 * fl32(1 - beta1) with the subtraction in binary64, likewise beta2, lr, eta,
 * bc1, bc2).  State is binary32; every elementwise
 * operation is one IEEE binary32 operation, rounded to nearest, in the order
 * written in the function's comment; sums of squares are accumulated in
 * binary64 (each square is exact there) and the square root of a scale is
 * taken in binary64 then rounded once to binary32.  Build with
 * -ffp-contract=off and without fast-math so that no product is fused into a
 * following add.
 *
 * Layouts: a "row" array [n][ld] holds worker i's vector at offset i*ld.
 * Packed signs: bit j of 64-bit word w is coordinate 64*w+j (least
 * significant bit first), bit = 1 means negative; a packed row has
 * W = ceil(d/64) words and the bits past d are 0.  A segment table is an
 * array of n_seg+1 strictly increasing offsets from 0 to d.
 */
#ifndef ORACLE_H
#define ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- gradient element access: binary32, or binary16 / bfloat16 decoded
 * exactly; g_kind 0, 1, 2 respectively ----------------------------------- */
double oracle_half_to_double(uint16_t h);
double oracle_bfloat16_to_double(uint16_t h);

/* ---- binary32 rounded to a 16-bit format (nearest, ties to even), from
 * the formats' definitions; kind 1 binary16, 2 bfloat16 ------------------- */
uint16_t oracle_float_to_half(float x);
uint16_t oracle_float_to_bfloat16(float x);
void oracle_round16(int64_t len, const float* x, uint16_t* out, int kind);

/* ---- warm-up and freeze -------------------------------------------------- */
void oracle_adam_warmup_step(int64_t d, int32_t n, int64_t ld, const void* g, int g_kind,
                             float* x, float* m, float* v, double lr, double beta1,
                             double beta2, double eta, double bc1, double bc2);
void oracle_freeze_variance(int64_t d, const float* v, float* denom, double eta, double bc2);
double oracle_l2norm(int64_t d, const float* v);
int64_t oracle_plateau_first(int64_t len, const double* h, int32_t window, double rtol,
                             int32_t min_steps);

/* ---- the 1-bit error-compensated compressor, one segment at a time ------ */
double oracle_sumsq(int64_t len, const float* c);
float oracle_scale(double sumsq, int64_t len);
void oracle_pack_signs(int64_t len, const float* c, uint64_t* bits, int64_t bit0);
int oracle_bit(const uint64_t* bits, int64_t k);
void oracle_residual(int64_t len, const float* c, float s, float* err);

/* ---- the step, composed ------------------------------------------------- */
void oracle_compensate(int64_t len, double beta1, const float* m, const void* g, int g_kind,
                       int64_t g_off, const float* delta, float* c);
void oracle_compress(int64_t d, int32_t n, int64_t ld, const int64_t* wseg, int32_t n_wseg,
                     const void* g, int g_kind, const float* m, float* delta, uint64_t* wbits,
                     float* wscale, double beta1);
void oracle_compress_deferred16(int64_t d, int32_t n, int64_t ld, const int64_t* wseg,
                                int32_t n_wseg, const void* g, int g_kind, const float* m,
                                uint16_t* c16, int c_kind, const float* wscale_prev,
                                uint64_t* wbits, float* wscale, double beta1);
void oracle_compress_local(int64_t d, int32_t n, int64_t ld, const int64_t* wseg, int32_t n_wseg,
                           const void* g, int g_kind, float* m_local, float* delta,
                           uint64_t* wbits, float* wscale, double beta1);
void oracle_server_average(int64_t k0, int64_t k1, int64_t d, int32_t n, const int64_t* wseg,
                           int32_t n_wseg, const uint64_t* wbits, const float* wscale,
                           const float* eps, float* a);
void oracle_server_reduce_recompress(int64_t d, int32_t n, const int64_t* wseg, int32_t n_wseg,
                                     const int64_t* sseg, int32_t n_sseg, const uint64_t* wbits,
                                     const float* wscale, float* eps, uint64_t* sbits,
                                     float* sscale);
void oracle_decompress_update(int64_t k0, int64_t k1, const int64_t* sseg, int32_t n_sseg,
                              const uint64_t* sbits, const float* sscale, const float* denom,
                              float* m, float* x, double lr);

#ifdef __cplusplus
}
#endif
#endif
