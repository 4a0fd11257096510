/*
 * oba.h -- C ABI of the 1-bit Adam compression-stage step on AMD MI355X
 * (gfx950).  All arithmetic runs in the library's HIP kernels; the caller
 * owns every buffer and the stream.
 *
 * Method (pages cited by title and section):
 *   [Tang]   "1-bit Adam: Communication Efficient Large-Scale Training with
 *            Adam's Convergence Speed" (paper summary page), sections 3.3,
 *            4.1-4.3, 5, 6, 11, 12 as numbered there.
 *   [AIMech] "1-bit Adam (Two-Stage Preconditioner-Frozen Error-Compensated
 *            Adam)" (curated algorithm page): definition paragraph and the
 *            mechanism claims (preconditioner freeze; compressed
 *            gather-broadcast allreduce with worker and server errors).
 *   [CwP]    "1-bit Adam" (method description page): the scale factor and
 *            the volume reduction of the packed message.
 *
 * Two stages: plain Adam for a warm-up ([Tang] 4.3), then the variance is
 * frozen into a fixed preconditioner and the momentum is exchanged in a
 * 1-bit, error-compensated form ([Tang] 4.3, 6; [AIMech] definition).  The
 * n data-parallel workers are n rows of device buffers; the gather to the
 * servers and the broadcast back become packed sign words in device memory.
 *
 * ---- Conventions (every entry point) ----------------------------------
 * Sizes: d parameters, n workers, ld = row stride (elements) of the [n][ld]
 *   buffers g and delta, W = ceil(d/64) packed words per row.
 * Memory: every pointer named in a call is DEVICE memory of the current HIP
 *   device, except the segment tables of oba_layout_create/validate, which
 *   are HOST arrays copied by the call.  float/half buffers must be 16-byte
 *   aligned (the 16-bit state rows of oba_compress_deferred16: 8-byte),
 *   packed words 8-byte aligned, scales 4-byte aligned.
 * Packed signs: bit j of word w is coordinate 64*w+j (least significant bit
 *   first); bit 1 = negative, bit 0 = non-negative (sign(0) = +1, also for
 *   -0.0); bits past d in the last word are written as 0.
 * Segments: a segment table holds n_seg+1 strictly increasing offsets from 0
 *   to d; each segment carries one scale.  Worker segments (sigma) give the
 *   scales of the workers' messages, server segments (tau) those of the
 *   server's.  Boundaries may fall anywhere, also inside a 64-bit word.
 * Numerics: hyperparameters are binary64 and each binary32 coefficient is
 *   rounded from them once (1-beta is formed in binary64 first).  Elementwise
 *   work is binary32 in the order given per call, no fused multiply-add,
 *   subnormals kept, division and square root correctly rounded.  Sums of
 *   squares are binary64, reduced in a fixed order (results are bitwise
 *   reproducible run to run on one device).
 * Asynchrony: a call validates its arguments on the host, enqueues its
 *   kernels on `stream` and returns; nothing is synchronised.  Faults from a
 *   kernel surface at the caller's next synchronisation.
 * Errors: 0 on success, a negative OBA_E* code otherwise; argument errors are
 *   found before any HIP call and leave every buffer untouched.
 *   oba_status_string gives a message (for OBA_EHIP it includes the HIP
 *   error text of the failing launch on this thread).
 * Aliasing: the in/out buffers named below are updated in place; no other
 *   two buffer arguments of a call may overlap.
 * Threads: calls are reentrant.  One workspace must not be used by two
 *   calls that can run at the same time (two streams).
 */
#ifndef OBA_H
#define OBA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  OBA_OK = 0,
  OBA_EINVAL = -1,     /* null pointer, bad size, bad dtype, bad hyperparameter */
  OBA_EALIGN = -2,     /* a buffer is not aligned as required */
  OBA_ESEG = -3,       /* a segment table is not 0 = o_0 < o_1 < ... < o_k = d */
  OBA_EWORKSPACE = -4, /* workspace smaller than oba_workspace_bytes() */
  OBA_EHIP = -5,       /* a HIP call failed (see oba_status_string) */
  OBA_ENOMEM = -6,     /* host or device allocation of the layout failed */
  OBA_ESCRATCH = -7    /* the layout needs more than OBA_NOALLOC_SCRATCH_BYTES */
};

/* gradient dtype: binary32, binary16, or bfloat16 (the upper half of a
 * binary32; decoded exactly).  All arithmetic is binary32 and so is all
 * state, except the workers' compensated vectors of the 16-bit-state pass
 * (oba_compress_deferred16), whose format is OBA_F16 or OBA_BF16. */
enum { OBA_F32 = 0, OBA_F16 = 1, OBA_BF16 = 2 };

typedef struct oba_layout_s* oba_layout;

/* Library version, 100*major + minor. */
int oba_version(void);

/* Message for a status code (static storage; OBA_EHIP's text is per thread). */
const char* oba_status_string(int status);

/* ---- layout --------------------------------------------------------------
 * Checks, on the host only, that (d, n, ld) and both segment tables are
 * valid: d >= 0, 1 <= n <= 4096, ld >= d, ld % 8 == 0, and each table rises
 * strictly from 0 to d (for d = 0 the table is the single offset {0} and
 * n_seg = 0).  Pure function: no HIP call, no allocation. */
int oba_layout_validate(int64_t d, int32_t n, int64_t ld, const int64_t* wseg, int32_t n_wseg,
                        const int64_t* sseg, int32_t n_sseg);

/* Validates as above, then builds the handle: small device copies of the
 * segment tables and of the per-block piece lists the kernels walk (five
 * tables, each about 16 bytes per thread block of its grid plus 20 bytes per
 * segment; the worker and update grids have at most 2^21 blocks and the
 * server grid 2^18, so about 9 MB at 336M parameters).  Allocates on the current device; the handle must be used on that
 * device only.  *out is set only on success. */
int oba_layout_create(oba_layout* out, int64_t d, int32_t n, int64_t ld, const int64_t* wseg,
                      int32_t n_wseg, const int64_t* sseg, int32_t n_sseg);

/* Frees the handle's device tables (synchronises the device first). */
void oba_layout_destroy(oba_layout layout);

/* Bytes of device workspace that oba_compress and
 * oba_server_reduce_recompress need (per-block binary64 partial sums). */
size_t oba_workspace_bytes(oba_layout layout);

/* ---- warm-up (plain Adam on the mean gradient) --------------------------
 * [AIMech] definition paragraph (the two moment recurrences, the update
 * x -= lr * m / (sqrt(v) + eta)); [Tang] 1 and 4.3 (Adam, uncompressed,
 * during the warm-up).  g: [n][ld] of dtype g_dtype (rows are workers).
 * x, m, v: [d] binary32, updated in place.  Per coordinate:
 *   gbar = (((0 + g_0) + g_1) + ... + g_{n-1}) / n
 *   m = b1*m + (1-b1)*gbar;  v = b2*v + (1-b2)*(gbar*gbar)
 *   x = x - (lr*(m/bc1)) / (sqrt(v/bc2) + eta)
 * bc1 = bc2 = 1 gives the bare recurrences; pass 1-b1^t, 1-b2^t for
 * Kingma-Ba bias correction.  Requires 0 <= beta < 1, bc > 0, eta >= 0. */
int oba_adam_warmup_step(oba_layout layout, const void* g, int g_dtype, float* x, float* m,
                         float* v, double lr, double beta1, double beta2, double eta, double bc1,
                         double bc2, hipStream_t stream);

/* ---- variance norm and the freeze trigger ---------------------------------
 * [Tang] 3.3 and Figure 2 (the norm of the fused -- all-parameter -- variance
 * vector levels off early in training, which motivates the freeze);
 * [AIMech] definition (the warm-up runs until v stabilises) and limitations
 * (v must be quasi-stationary by the end of the warm-up).
 *
 * The warm-up step of oba_adam_warmup_step that also writes vnorm[0] =
 * ||v||_2 of the updated v over all d coordinates (binary64 sum of squares
 * in a fixed order, then sqrt), computed in the same pass.  vnorm: one
 * double of device memory (8-byte aligned); ws as for oba_compress (unused
 * when d = 0, where vnorm[0] = 0). */
int oba_adam_warmup_step_vnorm(oba_layout layout, const void* g, int g_dtype, float* x, float* m,
                               float* v, double lr, double beta1, double beta2, double eta,
                               double bc1, double bc2, double* vnorm, void* ws, size_t ws_bytes,
                               hipStream_t stream);

/* Plateau test on a scalar series, host only (no HIP call, no allocation).
 * The pages show the plateau but give no rule; this one: the t-th observed
 * value h_t (t = 1, 2, ...) passes when t > window, t >= min_steps and
 * |h_t - h_{t-window}| <= rtol * |h_t|.  oba_plateau_observe returns 1 from
 * the first step that passes onward (latched), 0 before, OBA_EINVAL for a
 * null state or a non-finite value.  The caller owns the struct; init
 * requires 1 <= window <= OBA_PLATEAU_MAX_WINDOW, rtol >= 0, min_steps >= 0.
 * Observe ||v/bc2|| = vnorm/bc2 when the warm-up is bias corrected. */
#define OBA_PLATEAU_MAX_WINDOW 1024
typedef struct {
  int32_t window, min_steps, steps, fired;
  double rtol;
  double ring[OBA_PLATEAU_MAX_WINDOW];
} oba_plateau;
int oba_plateau_init(oba_plateau* p, int32_t window, double rtol, int32_t min_steps);
int oba_plateau_observe(oba_plateau* p, double value);

/* ---- variance freeze ------------------------------------------------------
 * [AIMech] definition paragraph (V = diag(sqrt(v_Tw) + eps) is frozen);
 * [Tang] 3.3, 5.  denom[k] = sqrt(v[k]/bc2) + eta, once, at the end of the
 * warm-up.  v, denom: [d] binary32 (distinct buffers).  The caller zeroes
 * the worker errors delta and the server error eps before the first
 * compression step; the momentum m carries over. */
int oba_freeze_variance(oba_layout layout, const float* v, float* denom, double eta, double bc2,
                        hipStream_t stream);

/* ---- worker side: momentum, error compensation, 1-bit compression -------
 * [Tang] 4.3 and 11 (each worker updates its momentum and compresses it
 * with error compensation, sign plus a magnitude-keeping scale); [CwP]
 * (scale = ||c|| / ||sign(c)||); [AIMech] gather-broadcast mechanism
 * (worker error memory delta_i).  For every worker i and coordinate k:
 *   c = (b1*m + (1-b1)*g_i) + delta_i
 *   s_{i,sigma} = sqrt(sum_{k in sigma} c^2 / |sigma|)   (binary64 sum)
 *   bit = (c < 0);  delta_i = c - s*sign(c)
 * g: [n][ld] (g_dtype); m: [d]; delta: [n][ld] in/out; wbits: [n][W] out;
 * wscale: [n][n_wseg] out.  ws: workspace of at least
 * oba_workspace_bytes(layout) bytes (contents on entry are ignored). */
int oba_compress(oba_layout layout, const void* g, int g_dtype, const float* m, float* delta,
                 uint64_t* wbits, float* wscale, double beta1, void* ws, size_t ws_bytes,
                 hipStream_t stream);

/* ---- server side: average, server error, recompression ------------------
 * [Tang] 6 and 11 (the server averages the workers' compressed messages and
 * compresses the result again); [AIMech] gather-broadcast mechanism (server
 * error memory eps).  For every coordinate k (s_i = worker i's scale of the
 * worker segment holding k, sg_i its sign):
 *   a = (((0 + s_0*sg_0) + s_1*sg_1) + ... + s_{n-1}*sg_{n-1}) / n + eps
 *   sbar_tau = sqrt(sum_{k in tau} a^2 / |tau|)          (binary64 sum)
 *   sbit = (a < 0);  eps = a - sbar*sign(a)
 * wbits: [n][W]; wscale: [n][n_wseg]; eps: [d] in/out; sbits: [W] out;
 * sscale: [n_sseg] out.  ws as for oba_compress. */
int oba_server_reduce_recompress(oba_layout layout, const uint64_t* wbits, const float* wscale,
                                 float* eps, uint64_t* sbits, float* sscale, void* ws,
                                 size_t ws_bytes, hipStream_t stream);

/* ---- broadcast: decompress, precondition, update --------------------------
 * [Tang] 11 (the server broadcasts the momentum, workers update their
 * models); [AIMech] definition paragraph (x_t = x_{t-1} - gamma V^-1 m_hat).
 * Every worker holds the same momentum afterwards.  Per coordinate:
 *   m_hat = sbar_tau * sign;  m = m_hat;  x = x - (lr*m_hat) / denom
 * sbits: [W]; sscale: [n_sseg]; denom: [d]; m: [d] out; x: [d] in/out.
 * m may be NULL: the momentum is then not stored, since it is fully given by
 * (sbits, sscale) -- the implicit momentum of oba_compress_deferred. */
int oba_decompress_update(oba_layout layout, const uint64_t* sbits, const float* sscale,
                          const float* denom, float* m, float* x, double lr, hipStream_t stream);

/* m[k] = sbar_tau * sign (the momentum every worker holds after a step,
 * [Tang] 11), materialised from the server message: for checkpoints,
 * inspection, or to return to a layout that reads m.  sbits: [W]; sscale:
 * [n_sseg]; m: [d] out. */
int oba_server_momentum(oba_layout layout, const uint64_t* sbits, const float* sscale, float* m,
                        hipStream_t stream);

/* ---- deferred-residual state layout --------------------------------------
 * The same step with a cheaper state: instead of the residuals delta_i and
 * eps, the state keeps the last step's compensated vectors c_i and a, and the
 * scale buffers keep the last step's scales.  A residual is formed only where
 * it is consumed -- in the next step's pass -- as delta_i = c_i - s_i*sign(c_i)
 * and eps = a - sbar*sign(a) ([Tang] 4.1: each step's compression error is
 * fed back at the next step; [AIMech] limitations: the error buffers are the
 * memory cost).  Every operation, its binary32 rounding and its order are
 * those of oba_compress / oba_server_reduce_recompress, so the results are
 * identical; the worker side is one pass over g, m, c instead of two, and the
 * server residual pass disappears.
 *
 * Start of the compression stage: zero c, a, wscale and sscale (then every
 * residual is 0, as after the freeze).  A step is oba_compress_deferred ->
 * oba_server_reduce_recompress_deferred -> oba_decompress_update.  With the
 * implicit momentum, the first step reads the warm-up's m and every later
 * one the last server message, and the update is called with m = NULL;
 * oba_server_momentum writes m out when it is wanted.
 * oba_deferred_errors writes delta and/or eps out of place (for checkpoints
 * or inspection); it does not change the state. */

/* c: [n][ld] in (last c) / out (this c); wscale: [n][n_wseg] in (last
 * scales) / out (this step's); g, wbits, ws as for oba_compress.
 *   delta_i = c_i - s_i*sign(c_i);  c_i = (b1*m + (1-b1)*g_i) + delta_i;
 *   s_{i,sigma} = sqrt(sum c^2 / |sigma|);  bit = (c < 0).
 * The momentum m comes from exactly one source:
 *   - m != NULL, sbits_prev = sscale_prev = NULL: m is read ([d]); the first
 *     step after the freeze, whose m is the warm-up's;
 *   - m == NULL, sbits_prev: [W] and sscale_prev: [n_sseg] the last step's
 *     server message: m[k] = sscale_prev[tau] * sign, which is what
 *     oba_decompress_update stored (implicit momentum: 1/8 byte per
 *     coordinate read instead of 4, and the update need not write m).
 * Any other combination is OBA_EINVAL. */
int oba_compress_deferred(oba_layout layout, const void* g, int g_dtype, const float* m,
                          const uint64_t* sbits_prev, const float* sscale_prev, float* c,
                          uint64_t* wbits, float* wscale, double beta1, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* oba_compress_deferred for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same checks, kernels and results (bit for bit), but no
 * workspace argument: the worker pass's binary64 partial sums go to a fixed
 * device array of OBA_NOALLOC_SCRATCH_BYTES that the library holds on every
 * GPU it runs on, until the process ends.  The call allocates nothing and
 * records no memset (no part of the array needs to start at zero: every
 * partial is written before it is read).  OBA_ESCRATCH if the layout's
 * partials, n * (worker pieces + items) binary64 values, exceed the array (a
 * layout whose oba_workspace_bytes() is at most OBA_NOALLOC_SCRATCH_BYTES
 * always fits: 10.5 MB at 336M parameters and 8 workers).  All calls on one
 * GPU share its array: two such calls that can run at the same time (two
 * streams) race.  The array's device address is looked up when the first
 * layout is created on a device. */
#define OBA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int oba_compress_deferred_noalloc(oba_layout layout, const void* g, int g_dtype, const float* m,
                                  const uint64_t* sbits_prev, const float* sscale_prev, float* c,
                                  uint64_t* wbits, float* wscale, double beta1,
                                  hipStream_t stream);

/* Per-worker momentum (the other reading of [Tang] 4.3: every worker keeps
 * its own momentum and the broadcast m_hat only moves x), in the deferred
 * layout.  m_local: [n][ld] in/out, worker i's momentum (set every row to the
 * warm-up's m at the freeze); c, wscale, g, wbits, ws as for
 * oba_compress_deferred.  Per worker i and coordinate:
 *   delta_i = c_i - s_i*sign(c_i);  m_i = b1*m_i + (1-b1)*g_i;
 *   c_i = m_i + delta_i;  s_{i,sigma} = sqrt(sum c^2 / |sigma|);  bit = (c < 0).
 * The step continues with oba_server_reduce_recompress_deferred and
 * oba_decompress_update with m = NULL. */
int oba_compress_deferred_local(oba_layout layout, const void* g, int g_dtype, float* m_local,
                                float* c, uint64_t* wbits, float* wscale, double beta1, void* ws,
                                size_t ws_bytes, hipStream_t stream);

/* The worker pass of the deferred layout with each worker's compensated
 * vector held in a 16-bit format (c_dtype OBA_F16 binary16 or OBA_BF16
 * bfloat16): half the bytes of the largest state and of its two streams per
 * step ([AIMech] limitations: the error buffers are the method's memory
 * cost; [Tang] 4.3 and [CwP] fix the compressor, which is unchanged).
 * c: [n][ld] 16-bit elements, 8-byte aligned, in (last c, exactly as stored)
 * / out; every other argument as for oba_compress_deferred.  Per worker i
 * and coordinate, in binary32:
 *   c'  = c_i decoded (exact);  delta_i = c' - s_i*sign(c');
 *   c   = (b1*m + (1-b1)*g_i) + delta_i;
 *   c~  = c rounded to the format (nearest, ties to even; overflow gives an
 *         infinity, as the format's conversion does);
 * then c~ is compressed (scale sqrt(sum c~^2 / |sigma|), bit = (c~ < 0), so a
 * c that rounds to -0 encodes +1) and stored as the new c_i.  The residual
 * the next step feeds back is exact for the message sent; the rounding c - c~
 * is this variant's own loss and is not fed back.  The step continues with
 * oba_server_reduce_recompress_deferred and oba_decompress_update, unchanged.
 * Start of the compression stage: zero c (all-zero bits) and wscale.
 * OBA_EINVAL for another c_dtype; otherwise the errors of
 * oba_compress_deferred. */
int oba_compress_deferred16(oba_layout layout, const void* g, int g_dtype, const float* m,
                            const uint64_t* sbits_prev, const float* sscale_prev, void* c,
                            int c_dtype, uint64_t* wbits, float* wscale, double beta1, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/* a: [d] in (last a) / out (this a); sscale: [n_sseg] in (last) / out (this);
 * wbits, wscale: this step's worker messages; sbits, ws as for
 * oba_server_reduce_recompress.
 *   eps = a' - sbar'*sign(a');  a = (sum_i s_i*sg_i)/n + eps;
 *   sbar_tau = sqrt(sum a^2 / |tau|);  sbit = (a < 0). */
int oba_server_reduce_recompress_deferred(oba_layout layout, const uint64_t* wbits,
                                          const float* wscale, float* a, uint64_t* sbits,
                                          float* sscale, void* ws, size_t ws_bytes,
                                          hipStream_t stream);

/* delta = c - s*sign(c) ([n][ld], if delta != NULL) and eps = a - sbar*sign(a)
 * ([d], if eps != NULL): the errors of the state (c, wscale, a, sscale), out
 * of place.  At least one output must be given. */
int oba_deferred_errors(oba_layout layout, const float* c, const float* wscale, const float* a,
                        const float* sscale, float* delta, float* eps, hipStream_t stream);

/* ---- tensor lists ----------------------------------------------------------
 * The parameters x and the n workers' gradients may live in T separate
 * tensors instead of flat buffers ([AIMech] definition: x and g are the
 * model's parameters and gradients; [Tang] 11: the implementation works per
 * tensor chunk).  Tensor t covers the flat coordinates [o_t, o_t + len_t),
 * o_0 = 0, o_{t+1} = o_t + len_t, and the lengths sum to the layout's d.
 * Every length must be a positive multiple of 4.  Segment tables, messages,
 * scales and all other state (m, v, denom, c, a) keep the flat coordinates.
 *
 * x_ptrs: host array [T] of device pointers to binary32 tensors (16-byte
 * aligned); g_ptrs: host array [n][T] of device pointers, row i = worker i
 * (16-byte aligned for OBA_F32, 8 for OBA_F16 and OBA_BF16).  The tables are copied to
 * the device at creation: the tensors must stay allocated (and at the same
 * addresses) while the handle is used.  *out is set only on success. */
typedef struct oba_tensors_s* oba_tensors;
int oba_tensors_create(oba_tensors* out, oba_layout layout, int32_t n_tensors,
                       const int64_t* lengths, float* const* x_ptrs, const void* const* g_ptrs,
                       int g_dtype);
/* Frees the device tables (synchronises the device first). */
void oba_tensors_destroy(oba_tensors tensors);

/* oba_adam_warmup_step (vnorm == NULL) or oba_adam_warmup_step_vnorm on the
 * listed x and g; m, v: [d] flat. */
int oba_adam_warmup_step_listed(oba_layout layout, oba_tensors tensors, float* m, float* v,
                                double lr, double beta1, double beta2, double eta, double bc1,
                                double bc2, double* vnorm, void* ws, size_t ws_bytes,
                                hipStream_t stream);

/* oba_compress_deferred16 on the listed gradients: c (16-bit, c_dtype) and
 * everything else as there. */
int oba_compress_deferred16_listed(oba_layout layout, oba_tensors tensors, const float* m,
                                   const uint64_t* sbits_prev, const float* sscale_prev, void* c,
                                   int c_dtype, uint64_t* wbits, float* wscale, double beta1,
                                   void* ws, size_t ws_bytes, hipStream_t stream);

/* oba_compress_deferred on the listed gradients (same momentum sources). */
int oba_compress_deferred_listed(oba_layout layout, oba_tensors tensors, const float* m,
                                 const uint64_t* sbits_prev, const float* sscale_prev, float* c,
                                 uint64_t* wbits, float* wscale, double beta1, void* ws,
                                 size_t ws_bytes, hipStream_t stream);

/* oba_decompress_update on the listed x (m may be NULL as there). */
int oba_decompress_update_listed(oba_layout layout, oba_tensors tensors, const uint64_t* sbits,
                                 const float* sscale, const float* denom, float* m, double lr,
                                 hipStream_t stream);

/* ---- the whole deferred step in one launch (small layouts) ------------------
 * For layouts whose step is bound by launch latency rather than HBM
 * (d <= 65536, n <= 64, at most 64 worker and 64 server segments; OBA_EINVAL
 * otherwise): oba_compress_deferred, oba_server_reduce_recompress_deferred and
 * oba_decompress_update in one launch of one thread block, with the same
 * arguments and per-coordinate arithmetic.  m: the momentum ([d]), or NULL
 * for the implicit momentum held in (sbits, sscale); c, wscale, a, sbits,
 * sscale: the deferred state, last step's in and this step's out; m_out: [d]
 * or NULL (m not stored); x updated in place.  No workspace.  The norms are
 * summed in another fixed order than the streaming kernels', so scales may
 * differ from theirs in the last bit (results are still reproducible). */
int oba_step_small(oba_layout layout, const void* g, int g_dtype, const float* m, float* c,
                   uint64_t* wbits, float* wscale, float* a, uint64_t* sbits, float* sscale,
                   const float* denom, float* m_out, float* x, double beta1, double lr,
                   hipStream_t stream);

/* ---- kernel timing (measurement aid) ---------------------------------------
 * While enabled, every kernel the library launches is bracketed by two HIP
 * events on the launch stream (up to `capacity` launches are kept).
 * oba_timing_read synchronises on the recorded events and returns the summed
 * duration in milliseconds and the launch count of the kernels whose name
 * equals `kernel` ("compress_p1", "compress_p2", "finalize_scales",
 * "server_p1", "server_p2", "decompress_update", "adam_warmup",
 * "freeze_variance", "compress_deferred", "server_deferred",
 * "deferred_errors", "server_momentum", "compress_deferred_local",
 * "step_small"; the listed entry points record under the names of their flat
 * forms; "adam_warmup" includes the norm kernel of
 * oba_adam_warmup_step_vnorm).  oba_timing_reset drops all records. */
int oba_timing_enable(int on, int32_t capacity);
int oba_timing_read(const char* kernel, double* total_ms, int64_t* launches);
int oba_timing_reset(void);

#ifdef __cplusplus
}
#endif
#endif /* OBA_H */
