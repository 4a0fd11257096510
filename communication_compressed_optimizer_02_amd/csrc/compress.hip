// compress.hip -- the worker pass: momentum, error feedback, 1-bit compression (gfx950).
// Method passages are cited in include/oba.h beside each entry point.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "device.hpp"
#include "occupancy.hpp"

namespace oba {

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
// CT is the type of the state rows (delta, or c in the deferred modes):
// binary32, or -- kDeferred and kDeferredM only -- a 16-bit format (uint16_t
// binary16, bf16_bits bfloat16).  With a 16-bit row, c is rounded to the
// format (nearest, ties to even) before its bits, its sum of squares and its
// store, so the vector compressed is the one the next step reads back, and
// the residual fed back is exact for what was sent.
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

// Workers loaded together by the pass with 16-bit state rows (a span of such
// rows holds less data per worker, so it can take more workers per load batch
// or fewer registers), a tuning knob.
#ifndef OBA_WORKER_BATCH16
#define OBA_WORKER_BATCH16 4
#endif
constexpr int kWorkerBatch16 = OBA_WORKER_BATCH16;
// The binary32 deferred worker pass with the implicit momentum in the body of
// the 16-bit pass (two spans per iteration, cursors in registers) with one
// worker per block on blocks of two spans (1), or in compress_body with
// groups of four on the one-span grid (0, with OBA_IMPLICIT_NB=4 and
// OBA_CMP_SPANS=1): 4.54-4.57 -> 4.46-4.51 ms at bert_large (same-box A/B;
// four spans per block 4.85 ms, two workers per block 4.68 ms).
#ifndef OBA_CMP_SPANSBODY
#define OBA_CMP_SPANSBODY 1
#endif
constexpr bool kSpansBody = OBA_CMP_SPANSBODY != 0;
// The 16-bit-state pass takes two full spans per iteration where a block lies
// inside one worker piece and one server piece (1), or one span at a time (0):
// 2.868/2.845 -> 2.854/2.820 ms at bert_large (same-box A/B, two runs each; the
// registers stay at 2 waves per SIMD either way).
#ifndef OBA_CMP16_PAIR
#define OBA_CMP16_PAIR 1
#endif

// Optional occupancy targets (waves per SIMD) of the worker pass and of its
// 16-bit-state instances, tuning knobs.
#ifdef OBA_CMP_WAVES
#define OBA_CMP_ATTR __attribute__((amdgpu_waves_per_eu(OBA_CMP_WAVES, OBA_CMP_WAVES)))
#else
#define OBA_CMP_ATTR
#endif
#ifdef OBA_CMP16_WAVES
#define OBA_CMP16_ATTR __attribute__((amdgpu_waves_per_eu(OBA_CMP16_WAVES, OBA_CMP16_WAVES)))
#else
#define OBA_CMP16_ATTR
#endif

template <typename GT, typename CT, int NB, int MODE, bool TL>
__device__ __forceinline__ void compress_body(Geo G, int32_t i0, const GT* __restrict__ g,
                                              float* __restrict__ m,  // read; written by kDeferredLocal
                                              CT* __restrict__ delta,
                                              uint8_t* __restrict__ wbytes, SegDev sig,
                                              double* __restrict__ part,
                                              const float* __restrict__ wscale, float b1,
                                              float omb1, MomSrc ms, TList tl) {
  __shared__ double lds[kWaves * NB];
  const int32_t b = blockIdx.x;
  i0 += blockIdx.y * NB;  // this block's workers: [i0, i0 + NB)
  const int64_t s_lo = dspan(G, b), s_hi = dspan(G, b + 1);
  const int32_t p_end = sig.blk_first[b + 1];
  int32_t p = sig.blk_first[b];
  int64_t p_hi = sig.phi[p];
  static_assert(!TL || MODE >= kDeferred, "tensor lists: deferred passes only");
  static_assert(__is_same(CT, float) || MODE == kDeferred || MODE == kDeferredM,
                "16-bit state rows: the deferred passes with the shared momentum only");
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
    constexpr int kBatch = __is_same(CT, float) ? kWorkerBatch : kWorkerBatch16;
    // buffer-resource loads and stores in the deferred passes (the explicit
    // passes keep the plain form: their read-only norm pass ran 1.6x slower
    // through buffers)
    constexpr bool kBuf = OBA_BUF != 0 && MODE >= kDeferred;
    constexpr int NBB = NB < kBatch ? NB : kBatch;
#pragma unroll
    for (int ib = 0; ib < NB; ib += NBB) {
      constexpr int NBL = MODE == kDeferredLocal ? NBB : 1;  // per-worker m rows
      float gv[NBB][8], c[NBB][8], ml[NBL][8];
      uint32_t h16[NBB][4];  // a 16-bit state row's patterns
      // ib + u < NB is decided at compile time: a last batch may be partial
      if (full) {
#pragma unroll
        for (int u = 0; u < NBB; ++u) {
          if (ib + u >= NB) break;
          const int64_t row = (int64_t)(i0 + ib + u) * G.ld;
          if constexpr (TL)
            load_listed<GT>(tl, i0 + ib + u, lt, full, gv[u]);
          else if constexpr (kBuf)
            load_full_buf(g + row, lo, gv[u]);
          else
            load_full(g + row, q, gv[u]);
          if constexpr (kBuf)
            load_full_buf(delta + row, lo, c[u]);
          else
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
          round_to_row<CT>(c[u], h16[u]);  // a 16-bit state: c as the row holds it
        }
        if (MODE != kNorm) store_sign_bits(wbytes + (int64_t)(i0 + i) * rowbytes, q, sign_bits(c[u]), rowbytes);
        if (MODE >= kDeferred) {
          if (kBuf && full)
            store_full_buf(delta + row, lo, c[u], h16[u]);
          else
            store_row(delta + row, q, G.d, full, c[u], h16[u]);
        }
        fs[i] = (MODE != kApply) ? sumsq8(c[u]) : 0.0;
        if (MODE == kApply) {
#pragma unroll
          for (int j = 0; j < 8; ++j) c[u][j] = residual(c[u][j], sv[j]);
          store_row(delta + row, q, G.d, full, c[u], h16[u]);
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
          if constexpr (MODE >= kDeferred)
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

// The same pass for blocks of several spans (the grid of the 16-bit-state
// pass): the block's piece cursors and each worker's scale stay in registers
// (reloaded only when a piece ends, with the next piece peeked before the
// span's stores), and a span's arithmetic has a fast path for spans inside
// one piece apart from the general one.  In compress_body a table load issued
// after a worker's or a span's stores is waited for before the next worker or
// span proceeds, which waits for those stores too (one counter tracks loads
// and stores in issue order): 16-bit-state pass 3.27 -> 2.87 ms at bert_large.
// The binary32 pass at one span per block measured 1-5 % slower in this form
// (same-box A/B), so it keeps compress_body.
template <typename GT, typename CT, int NB, int MODE, bool TL>
__device__ __forceinline__ void compress_body_spans(Geo G, int32_t i0, const GT* __restrict__ g,
                                              float* __restrict__ m,  // read; written by kDeferredLocal
                                              CT* __restrict__ delta,
                                              uint8_t* __restrict__ wbytes, SegDev sig,
                                              double* __restrict__ part,
                                              const float* __restrict__ wscale, float b1,
                                              float omb1, MomSrc ms, TList tl) {
  __shared__ double lds[kWaves * NB];
  const int32_t b = blockIdx.x;
  i0 += blockIdx.y * NB;  // this block's workers: [i0, i0 + NB)
  const int64_t s_lo = dspan(G, b), s_hi = dspan(G, b + 1);
  static_assert(!TL || MODE >= kDeferred, "tensor lists: deferred passes only");
  static_assert(__is_same(CT, float) || MODE == kDeferred || MODE == kDeferredM,
                "16-bit state rows: the deferred passes with the shared momentum only");
  TCur tcur{};  // tensor cursor (tensor lists)
  if constexpr (TL) tcur = tcur_start(tl, b);
  // worker pieces; each worker's scale of the current piece's segment, kept
  // in registers and reloaded only when the piece changes (a reload per
  // worker would be a load after the previous worker's stores)
  PCur pc = pcur_start(sig, b);
  float sw[NB];
  auto load_scales = [&]() {
    if (MODE != kNorm) {
#pragma unroll
      for (int i = 0; i < NB; ++i) sw[i] = wscale[(int64_t)(i0 + i) * sig.n_seg + pc.js];
    }
  };
  load_scales();
  // kDeferredM: cursor over the server segments (on this grid) and sbar of
  // the current one
  PCur tc{};
  float sbar = 0.0f;
  if (MODE == kDeferredM) {
    tc = pcur_start(ms.tau, b);
    sbar = ms.sscale[tc.js];
  }
  const int64_t rowbytes = G.W * 8;
  double acc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) acc[i] = 0.0;

  // a block inside one worker piece (and one server piece) has every full
  // span inside it: known from the block's piece range alone
  const bool one_piece = pc.end - pc.p == 1;
  const bool one_tpiece = MODE != kDeferredM || tc.end - tc.p == 1;

  // Two full spans at once, in a block inside one worker piece and one
  // server piece: both spans' loads are issued before the first span's
  // arithmetic, so each wave has twice the bytes in flight.  Per coordinate
  // the operations are those of the one-span fast path below, and each
  // worker's sums of squares are added span by span in the same order.
  constexpr bool kPair = OBA_CMP16_PAIR != 0 && !TL && (MODE == kDeferred || MODE == kDeferredM);
  constexpr bool kBufP = OBA_BUF != 0;
  // (one span's data per set of named arrays: arrays indexed by the span
  // would be placed in LDS by the compiler before its loops are unrolled)
  auto span_loads = [&](int64_t l, const Quads& q, uint32_t& mb, float(&mv)[8],
                        float(&gv)[NB][8], float(&c)[NB][8]) {
    if constexpr (MODE == kDeferredM)
      mb = load_sign_bits<true, OBA_PAIRS_CMP>(ms.sbytes, q, G.d);
    else
      load_full(m, q, mv);
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int64_t row = (int64_t)(i0 + u) * G.ld;
      if constexpr (kBufP) {
        load_full_buf(g + row, l, gv[u]);
        load_full_buf(delta + row, l, c[u]);
      } else {
        load_full(g + row, q, gv[u]);
        load_full(delta + row, q, c[u]);
      }
    }
  };
  auto span_work = [&](int64_t l, const Quads& q, uint32_t mb, float(&mv)[8], float(&gv)[NB][8],
                       float(&c)[NB][8], double(&fs)[NB]) {
    if constexpr (MODE == kDeferredM) {  // m = sbar*sign from the last server message
#pragma unroll
      for (int j = 0; j < 8; ++j) mv[j] = ((mb >> j) & 1u) ? -sbar : sbar;
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int64_t row = (int64_t)(i0 + u) * G.ld;
      uint32_t h16[4];
#pragma unroll
      for (int j = 0; j < 8; ++j) c[u][j] = residual(c[u][j], sw[u]);
#pragma unroll
      for (int j = 0; j < 8; ++j) c[u][j] = compensate(b1, omb1, mv[j], gv[u][j], c[u][j]);
      round_to_row<CT>(c[u], h16);
      store_sign_bits(wbytes + (int64_t)(i0 + u) * rowbytes, q, sign_bits(c[u]), rowbytes);
      if constexpr (kBufP)
        store_full_buf(delta + row, l, c[u], h16);
      else
        store_row(delta + row, q, G.d, true, c[u], h16);
      fs[u] = sumsq8(c[u]);
    }
  };
  auto two_spans = [&](int64_t lo0) {
    const int64_t lo1 = lo0 + kSpan;
    const Quads qa = quads(lo0), qb = quads(lo1);
    uint32_t mba = 0u, mbb = 0u;
    float mva[8], mvb[8], ga[NB][8], ca[NB][8], gb[NB][8], cb[NB][8];
    double fsa[NB], fsb[NB];
    span_loads(lo0, qa, mba, mva, ga, ca);
    span_loads(lo1, qb, mbb, mvb, gb, cb);
    span_work(lo0, qa, mba, mva, ga, ca, fsa);
    span_work(lo1, qb, mbb, mvb, gb, cb, fsb);
#pragma unroll
    for (int u = 0; u < NB; ++u) acc[u] += fsa[u];
#pragma unroll
    for (int u = 0; u < NB; ++u) acc[u] += fsb[u];
    const int64_t hi1 = lo1 + kSpan;
    if (hi1 == pc.hi) {  // the block's one piece ends here
      flush_rows<NB>(acc, NB, part + (int64_t)i0 * sig.n_pieces + pc.p, sig.n_pieces, lds);
      pcur_advance(pc, sig, PNext{pc.hi, pc.js}, hi1);
    }
    if (MODE == kDeferredM) pcur_advance(tc, ms.tau, PNext{tc.hi, tc.js}, hi1);
  };

  for (int64_t s = s_lo; s < s_hi; ++s) {
    const int64_t lo = s * kSpan;
    if constexpr (kPair) {
      if (one_piece && one_tpiece && s + 1 < s_hi && lo + 2 * kSpan <= G.d) {
        two_spans(lo);
        ++s;
        continue;
      }
    }
    const int64_t hi = min(lo + kSpan, G.d);
    const Quads q = quads(lo);
    const bool full = lo + kSpan <= G.d;
    int32_t jseg[8];
    LaneT lt{};
    if constexpr (TL) {
      tcur_advance(tl, tcur, lo);
      lt = lane_tensors(tl, tcur, q, min(lo + kSpan, G.d), G.d);
    }
    // every load of the span first (all NB workers), then the arithmetic
    float mv[8];
    uint32_t mbits = 0;  // kDeferredM: the last server message's sign bits
    if (MODE == kDeferredM) {
      mbits = full ? load_sign_bits<true, OBA_PAIRS_CMP>(ms.sbytes, q, G.d)
                   : load_sign_bits<false, OBA_PAIRS_CMP>(ms.sbytes, q, G.d);
    } else if (MODE == kDeferredLocal) {  // per-worker rows, loaded with g below
#pragma unroll
      for (int j = 0; j < 8; ++j) mv[j] = 0.0f;
    } else if (full) {
      load_full(m, q, mv);
    } else {
      load_tail(m, q, G.d, mv);
    }
    // the next pieces, used after the span's stores (blocks of several spans)
    PNext pnx{}, tnx{};
    if (s + 1 < s_hi) {
      pnx = pcur_peek(pc, sig);
      if (MODE == kDeferredM) tnx = pcur_peek(tc, ms.tau);
    }
    double fs[NB];
    bool uniform = true;  // span inside the current piece
    // workers in batches of NBB: all loads of a batch, then its arithmetic
    // and stores (NBB < NB trades loads in flight per wave for occupancy)
    constexpr int kBatch = __is_same(CT, float) ? kWorkerBatch : kWorkerBatch16;
    // buffer-resource loads and stores in the deferred passes (the explicit
    // passes keep the plain form: their read-only norm pass ran 1.6x slower
    // through buffers)
    constexpr bool kBuf = OBA_BUF != 0 && MODE >= kDeferred;
    constexpr int NBB = NB < kBatch ? NB : kBatch;
#pragma unroll
    for (int ib = 0; ib < NB; ib += NBB) {
      constexpr int NBL = MODE == kDeferredLocal ? NBB : 1;  // per-worker m rows
      float gv[NBB][8], c[NBB][8], ml[NBL][8];
      uint32_t h16[NBB][4];  // a 16-bit state row's patterns
      // ib + u < NB is decided at compile time: a last batch may be partial
      if (full) {
#pragma unroll
        for (int u = 0; u < NBB; ++u) {
          if (ib + u >= NB) break;
          const int64_t row = (int64_t)(i0 + ib + u) * G.ld;
          if constexpr (TL)
            load_listed<GT>(tl, i0 + ib + u, lt, true, gv[u]);
          else if constexpr (kBuf)
            load_full_buf(g + row, lo, gv[u]);
          else
            load_full(g + row, q, gv[u]);
          if constexpr (kBuf)
            load_full_buf(delta + row, lo, c[u]);
          else
            load_full(delta + row, q, c[u]);
          if (MODE == kDeferredLocal) load_full(m + row, q, ml[u]);
        }
      } else {
#pragma unroll
        for (int u = 0; u < NBB; ++u) {
          if (ib + u >= NB) break;
          const int64_t row = (int64_t)(i0 + ib + u) * G.ld;
          if constexpr (TL)
            load_listed<GT>(tl, i0 + ib + u, lt, false, gv[u]);
          else
            load_tail(g + row, q, G.d, gv[u]);
          load_tail(delta + row, q, G.d, c[u]);
          if (MODE == kDeferredLocal) load_tail(m + row, q, G.d, ml[u]);
        }
      }
      // The batch's arithmetic and stores.  FAST (a full span inside one
      // worker piece and, for the implicit momentum, one server piece --
      // nearly every span) takes the scales from registers; the general path
      // looks each coordinate's segment up.  Kept apart, so that no load of
      // the general path is pending where the fast path continues (a wait
      // for it there would also wait for the stores issued before it: one
      // counter tracks loads and stores in issue order).
      auto work = [&](auto fast_tag) {
        constexpr bool FAST = decltype(fast_tag)::value;
        if (ib == 0) {
          if (!FAST && MODE != kNorm && !uniform) lane_segs(sig.off, pc.js, q, G.d, jseg);
          if (MODE == kDeferredM) {  // m = sbar*sign from the last server message
            float sb[8];
            if (FAST || hi <= tc.hi) {
#pragma unroll
              for (int j = 0; j < 8; ++j) sb[j] = sbar;
            } else {
              int32_t jt[8];
              lane_segs(ms.tau.off, tc.js, q, G.d, jt);
#pragma unroll
              for (int j = 0; j < 8; ++j) sb[j] = ms.sscale[jt[j]];
            }
#pragma unroll
            for (int j = 0; j < 8; ++j)
              mv[j] = (!FAST && !full && coord(q, j) >= G.d)
                          ? 0.0f
                          : (((mbits >> j) & 1u) ? -sb[j] : sb[j]);
          }
        }
#pragma unroll
        for (int u = 0; u < NBB; ++u) {
          const int i = ib + u;
          if (i >= NB) break;
          const int64_t row = (int64_t)(i0 + i) * G.ld;
          float sv[8];
          if (MODE != kNorm) {
            if (FAST || uniform) {
#pragma unroll
              for (int j = 0; j < 8; ++j) sv[j] = sw[i];
            } else {
              const float* sc = wscale + (int64_t)(i0 + i) * sig.n_seg;
#pragma unroll
              for (int j = 0; j < 8; ++j) sv[j] = sc[jseg[j]];
            }
          }
          if (MODE >= kDeferred) {  // c[u] holds c' of the last step
#pragma unroll
            for (int j = 0; j < 8; ++j) c[u][j] = residual(c[u][j], sv[j]);
            if (!FAST && !full) {  // coordinates past d read as 0 and must stay 0 (no bit, no c^2)
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
            store8(m + row, q, G.d, FAST || full, ml[u]);
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) c[u][j] = compensate(b1, omb1, mv[j], gv[u][j], c[u][j]);
            round_to_row<CT>(c[u], h16[u]);  // a 16-bit state: c as the row holds it
          }
          if (MODE != kNorm) store_sign_bits(wbytes + (int64_t)(i0 + i) * rowbytes, q, sign_bits(c[u]), rowbytes);
          if (MODE >= kDeferred) {
            if (kBuf && (FAST || full))
              store_full_buf(delta + row, lo, c[u], h16[u]);
            else
              store_row(delta + row, q, G.d, FAST || full, c[u], h16[u]);
          }
          fs[i] = (MODE != kApply) ? sumsq8(c[u]) : 0.0;
          if (MODE == kApply) {
#pragma unroll
            for (int j = 0; j < 8; ++j) c[u][j] = residual(c[u][j], sv[j]);
            store_row(delta + row, q, G.d, FAST || full, c[u], h16[u]);
          }
        }
      };
      if (ib == 0) uniform = one_piece || hi <= pc.hi;
      if (full && uniform && (one_tpiece || hi <= tc.hi))
        work(std::true_type{});
      else
        work(std::false_type{});
    }
    const int32_t p0 = pc.p;
    if (MODE == kApply) {
      pcur_advance(pc, sig, pnx, hi);
    } else if (uniform) {
#pragma unroll
      for (int i = 0; i < NB; ++i) acc[i] += fs[i];
      if (hi == pc.hi) {
        flush_rows<NB>(acc, NB, part + (int64_t)i0 * sig.n_pieces + pc.p, sig.n_pieces, lds);
        pcur_advance(pc, sig, pnx, hi);
      }
    } else {  // span crosses piece boundaries: sum this lane's c piece by piece
      int64_t cur = lo;
      while (cur < hi) {
        const int64_t e = min(pc.hi, hi);
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const int64_t row = (int64_t)(i0 + i) * G.ld;
          if constexpr (MODE >= kDeferred)
            acc[i] += sumsq_range(delta + row, q, cur, e);  // c was stored there
          else
            acc[i] += sumsq_range_c(m, g + row, delta + row, b1, omb1, q, cur, e);
        }
        if (pc.hi <= hi) {
          flush_rows<NB>(acc, NB, part + (int64_t)i0 * sig.n_pieces + pc.p, sig.n_pieces, lds);
          if (++pc.p < pc.end) {  // the rare path: load the next piece here
            pc.hi = uni(sig.phi[pc.p]);
            pc.js = uni(sig.pseg[pc.p]);
          }
        }
        cur = e;
      }
    }
    if (pc.p != p0 && pc.p < pc.end) load_scales();  // used from the next span on
    if (MODE == kDeferredM) {
      const int32_t t0 = tc.p;
      pcur_advance(tc, ms.tau, tnx, hi);
      if (tc.p != t0 && tc.p < tc.end) sbar = ms.sscale[tc.js];
    }
  }
}

template <typename GT, typename CT, int NB, int MODE, bool TL>
__global__ __launch_bounds__(kBlock) OBA_CMP_ATTR void k_compress(
    Geo G, int32_t i0, const GT* __restrict__ g, float* __restrict__ m, CT* __restrict__ delta,
    uint8_t* __restrict__ wbytes, SegDev sig, double* __restrict__ part,
    const float* __restrict__ wscale, float b1, float omb1, MomSrc ms, TList tl) {
  if constexpr (kSpansBody && MODE == kDeferredM && !TL) {
    compress_body_spans<GT, CT, NB, MODE, TL>(G, i0, g, m, delta, wbytes, sig, part, wscale, b1,
                                              omb1, ms, tl);
    return;
  }
  compress_body<GT, CT, NB, MODE, TL>(G, i0, g, m, delta, wbytes, sig, part, wscale, b1, omb1,
                                      ms, tl);
}

// the 16-bit-state instances (their own occupancy knob)
template <typename GT, typename CT, int NB, int MODE, bool TL>
__global__ __launch_bounds__(kBlock) OBA_CMP16_ATTR void k_compress16(
    Geo G, int32_t i0, const GT* __restrict__ g, float* __restrict__ m, CT* __restrict__ delta,
    uint8_t* __restrict__ wbytes, SegDev sig, double* __restrict__ part,
    const float* __restrict__ wscale, float b1, float omb1, MomSrc ms, TList tl) {
  compress_body_spans<GT, CT, NB, MODE, TL>(G, i0, g, m, delta, wbytes, sig, part, wscale, b1,
                                            omb1, ms, tl);
}

// ---- launchers ----------------------------------------------------------------

// Occupancy caps (blocks per CU, 0: none) of the deferred worker passes with
// binary32 and with 16-bit state rows, tuning knobs (2 blocks: binary32 pass
// 4.55 -> 5.39 ms, 16-bit pass equal at bert_large; none kept).
#ifndef OBA_CMP_BPC
#define OBA_CMP_BPC 0
#endif
#ifndef OBA_CMP16_BPC
#define OBA_CMP16_BPC 0
#endif

template <typename GT, typename CT, int NB, int MODE, bool TL>
static void launch_cmp(const Geo& G, int32_t i0, int groups, const void* g, const float* m,
                       void* delta, uint8_t* wbytes, const SegDev& sig, double* part,
                       const float* wscale, float b1, float omb1, const MomSrc& ms,
                       const TList& tl, hipStream_t st) {
  if constexpr (__is_same(CT, float)) {
    const size_t lds = MODE >= kDeferred ? occupancy_lds(OBA_CMP_BPC) : 0;
    allow_lds(reinterpret_cast<const void*>(&k_compress<GT, CT, NB, MODE, TL>), lds);
    hipLaunchKernelGGL((k_compress<GT, CT, NB, MODE, TL>), dim3(G.nblk, groups), dim3(kBlock),
                       lds, st, G, i0, static_cast<const GT*>(g), const_cast<float*>(m),
                       static_cast<CT*>(delta), wbytes, sig, part, wscale, b1, omb1, ms, tl);
  } else {
    const size_t lds = occupancy_lds(OBA_CMP16_BPC);
    allow_lds(reinterpret_cast<const void*>(&k_compress16<GT, CT, NB, MODE, TL>), lds);
    hipLaunchKernelGGL((k_compress16<GT, CT, NB, MODE, TL>), dim3(G.nblk, groups), dim3(kBlock),
                       lds, st, G, i0, static_cast<const GT*>(g), const_cast<float*>(m),
                       static_cast<CT*>(delta), wbytes, sig, part, wscale, b1, omb1, ms, tl);
  }
}

// Groups of GROUP workers per block, then one launch for the remainder.  A
// pass that reads m shares it across the block's workers (4 bytes per
// coordinate per group); the implicit momentum costs 1/8 byte per group, so
// that pass can take smaller groups (fewer registers, more blocks).
#ifndef OBA_MAX_NB
#define OBA_MAX_NB 8
#endif
#ifndef OBA_IMPLICIT_NB
#define OBA_IMPLICIT_NB 1
#endif
// Workers per block of the 16-bit-state pass with the implicit momentum, a
// tuning knob: one worker per block (its spans two at a time) took the pass
// from 2.85 to 2.72 ms at bert_large (two: 2.75 ms; same-box A/B; occupancy
// caps of 2 or 3 blocks per CU made it slower).  The first step after the
// freeze reads m, shared by the workers of a block, so it keeps groups of
// OBA_READ_NB16.
#ifndef OBA_IMPLICIT_NB16
#define OBA_IMPLICIT_NB16 1
#endif
#ifndef OBA_READ_NB16
#define OBA_READ_NB16 4
#endif
constexpr int kMaxNB = OBA_MAX_NB;
constexpr int kImplicitNB16 = OBA_IMPLICIT_NB16;
constexpr int kReadNB16 = OBA_READ_NB16;
constexpr int kImplicitNB = OBA_IMPLICIT_NB;
// the tensor-list form of that pass (compress_body: no two-span path) keeps
// groups of four
#ifndef OBA_LISTED_NB
#define OBA_LISTED_NB 4
#endif
constexpr int kListedNB = OBA_LISTED_NB;
// Workers per block of the per-worker-momentum pass (three rows per worker),
// a tuning knob: one worker per block took the pass from 8.38-8.47 to
// 8.08-8.23 ms at bert_large (two: equal to four; same-box A/B).
#ifndef OBA_LOCAL_NB
#define OBA_LOCAL_NB 1
#endif
constexpr int kLocalNB = OBA_LOCAL_NB;
static_assert(kMaxNB >= 1 && kMaxNB <= 8 && kImplicitNB >= 1 && kImplicitNB <= 8 &&
                  kImplicitNB16 >= 1 && kImplicitNB16 <= 8 && kReadNB16 >= 1 &&
                  kReadNB16 <= 8,
              "worker groups hold 1 to 8 workers");

template <typename GT, typename CT, int MODE, bool TL>
static void launch_cmp_n(const Geo& G, const void* g, const float* m, void* delta,
                         uint8_t* wbytes, const SegDev& sig, double* part, const float* wscale,
                         float b1, float omb1, const MomSrc& ms, const TList& tl,
                         hipStream_t st) {
  // (the tensor-list 16-bit pass has no two-span path, without which one
  // worker per block was slower: it keeps groups of OBA_READ_NB16)
  constexpr int GROUP = !__is_same(CT, float)
                            ? (MODE == kDeferredM && !TL ? kImplicitNB16 : kReadNB16)
                        : MODE == kDeferredM                  ? (TL ? kListedNB : kImplicitNB)
                        : MODE == kDeferredLocal                         ? kLocalNB
                                                                         : kMaxNB;
  const int full = G.n / GROUP, rem = G.n % GROUP, i0 = full * GROUP;
#define OBA_CMP(NB_, I0, GROUPS) \
  launch_cmp<GT, CT, NB_, MODE, TL>(G, I0, GROUPS, g, m, delta, wbytes, sig, part, wscale, b1, omb1, \
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

template <int MODE, bool TL = false, typename CT = float>
static void launch_cmp_t(const Geo& G, const void* g, int gdt, const float* m, void* delta,
                         uint8_t* wbytes, const SegDev& sig, double* part, const float* wscale,
                         float b1, float omb1, const MomSrc& ms, hipStream_t st,
                         const TList& tl = TList{}) {
  if (gdt == kGradF16)
    launch_cmp_n<uint16_t, CT, MODE, TL>(G, g, m, delta, wbytes, sig, part, wscale, b1, omb1, ms,
                                         tl, st);
  else if (gdt == kGradBF16)
    launch_cmp_n<bf16_bits, CT, MODE, TL>(G, g, m, delta, wbytes, sig, part, wscale, b1, omb1,
                                          ms, tl, st);
  else
    launch_cmp_n<float, CT, MODE, TL>(G, g, m, delta, wbytes, sig, part, wscale, b1, omb1, ms,
                                      tl, st);
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

void launch_compress_deferred16(const Geo& G, const void* g, int gdt, const float* m, void* c,
                                int cdt, uint8_t* wbytes, const SegDev& sig, double* part,
                                const float* wscale_prev, float b1, float omb1, const MomSrc& ms,
                                hipStream_t st) {
  const TList none{};
  if (cdt == kGradBF16) {
    if (ms.sbytes)
      launch_cmp_t<kDeferredM, false, bf16_bits>(G, g, gdt, nullptr, c, wbytes, sig, part,
                                                 wscale_prev, b1, omb1, ms, st, none);
    else
      launch_cmp_t<kDeferred, false, bf16_bits>(G, g, gdt, m, c, wbytes, sig, part, wscale_prev,
                                                b1, omb1, ms, st, none);
  } else {
    if (ms.sbytes)
      launch_cmp_t<kDeferredM, false, uint16_t>(G, g, gdt, nullptr, c, wbytes, sig, part,
                                                wscale_prev, b1, omb1, ms, st, none);
    else
      launch_cmp_t<kDeferred, false, uint16_t>(G, g, gdt, m, c, wbytes, sig, part, wscale_prev,
                                               b1, omb1, ms, st, none);
  }
}

void launch_compress_deferred16_listed(const Geo& G, const TList& tl, int gdt, const float* m,
                                       void* c, int cdt, uint8_t* wbytes, const SegDev& sig,
                                       double* part, const float* wscale_prev, float b1,
                                       float omb1, const MomSrc& ms, hipStream_t st) {
  if (cdt == kGradBF16) {
    if (ms.sbytes)
      launch_cmp_t<kDeferredM, true, bf16_bits>(G, nullptr, gdt, nullptr, c, wbytes, sig, part,
                                                wscale_prev, b1, omb1, ms, st, tl);
    else
      launch_cmp_t<kDeferred, true, bf16_bits>(G, nullptr, gdt, m, c, wbytes, sig, part,
                                               wscale_prev, b1, omb1, ms, st, tl);
  } else {
    if (ms.sbytes)
      launch_cmp_t<kDeferredM, true, uint16_t>(G, nullptr, gdt, nullptr, c, wbytes, sig, part,
                                               wscale_prev, b1, omb1, ms, st, tl);
    else
      launch_cmp_t<kDeferred, true, uint16_t>(G, nullptr, gdt, m, c, wbytes, sig, part,
                                              wscale_prev, b1, omb1, ms, st, tl);
  }
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

}  // namespace oba
