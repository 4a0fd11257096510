// layout.hpp -- host-only planning of the streaming grid and segment pieces.
//
// The streaming kernels cut [0, d) into spans of kSpan coordinates (one span
// = one pass of a 256-thread block, 8 coordinates per lane) and give each
// block a contiguous range of spans: floor(S/nblk) each, one more for the
// first S mod nblk blocks (span_begin).  A segment
// table is then cut at block boundaries into "pieces": each piece lies in one
// block and one segment, so a block can reduce its part of a segment's sum of
// squares into one binary64 partial per piece without atomics, and a segment's
// pieces are consecutive (its partials are summed in a fixed order).
//
// No HIP here: this file is also compiled by the host compiler for tests.
#pragma once
#include <cstdint>
#include <vector>

namespace oba {

#ifndef OBA_BLOCK
#define OBA_BLOCK 256
#endif
constexpr int kBlock = OBA_BLOCK;           // threads per block of the streaming kernels
constexpr int kWaves = kBlock / 64;         // wave64s per block
constexpr int kVec = 8;                     // consecutive coordinates per lane
constexpr int64_t kSpan = kBlock * kVec;    // coordinates per block pass
#ifndef OBA_MAX_BLOCKS
#define OBA_MAX_BLOCKS 262144
#endif
#ifndef OBA_MAX_BLOCKS_WORKER
#define OBA_MAX_BLOCKS_WORKER 2097152
#endif
// Streaming grids: the worker-side kernels and the update run best with one
// span per block (up to 2^21 blocks, 4.3e9 coordinates), the server pass (n
// packed rows per span) with four spans per block (up to 2^18 blocks).
#ifndef OBA_SERVER_SPANS
#define OBA_SERVER_SPANS 4
#endif
constexpr int kMaxBlocks = OBA_MAX_BLOCKS;
constexpr int kServerSpans = OBA_SERVER_SPANS;  // least spans per block of the server grid
constexpr int kMaxBlocksWorker = OBA_MAX_BLOCKS_WORKER;
// Spans per block of the compress grid, the grid of the deferred worker
// passes, a tuning knob: their binary32 form takes one worker per block and a
// block's two spans at once, so blocks of two spans.
#ifndef OBA_CMP_SPANS
#define OBA_CMP_SPANS 2
#endif
inline int32_t compress_spans(int32_t) { return OBA_CMP_SPANS; }
// Spans per block of the explicit grid (the explicit apply pass and the
// per-worker-momentum pass): one when a block holds four workers or more;
// with fewer workers per block a block does too little work per span, and 4/n
// spans per block measured 16 % faster for one worker.
inline int32_t explicit_spans(int32_t n) { return n >= 4 ? 1 : 4 / n; }
constexpr int32_t kMaxWorkers = 4096;

// A segment cut into more than kSplitAbove pieces has its partials summed in
// two stages: runs of at most kItem consecutive pieces ("items") first, in
// parallel, then the items of each segment.  Both orders are fixed.
constexpr int32_t kItem = 2048;
constexpr int32_t kSplitAbove = 8192;

struct Pieces {
  std::vector<int64_t> lo, hi;      // piece [lo, hi)
  std::vector<int32_t> seg;         // segment of the piece
  std::vector<int32_t> blk_first;   // [nblk+1] first piece of each block
  std::vector<int32_t> seg_first;   // [n_seg+1] first piece of each segment
  // empty unless some segment has more than kSplitAbove pieces:
  std::vector<int32_t> item_q;      // [n_items+1] first piece of each item
  std::vector<int32_t> seg_item;    // [n_seg+1] first item of each segment
};

struct Plan {
  int64_t d = 0, ld = 0, W = 0, S = 0;
  int32_t n = 0;
  int32_t nblk = 0;    // grid of the server, residual, warm-up, freeze, norm kernels
  int32_t nblk_w = 0;  // grid of the update (one span per block)
  int32_t nblk_c = 0;  // grid of the deferred worker passes (compress grid)
  int32_t nblk_e = 0;  // grid of the explicit apply and per-worker-momentum passes
  std::vector<int64_t> wseg, sseg;  // offsets, n_seg+1 each
  Pieces wp;    // worker segments cut on the compress grid
  Pieces wp_s;  // worker segments cut on the server grid (scale lookups there)
  Pieces sp;    // server segments cut on the server grid
  Pieces sp_w;  // server segments cut on the update grid
  Pieces sp_c;  // server segments cut on the compress grid (implicit momentum)
  Pieces wp_e;  // worker segments cut on the explicit grid
};

// Status codes mirror the C ABI (0 ok, negative error).
int validate(int64_t d, int32_t n, int64_t ld, const int64_t* wseg, int32_t n_wseg,
             const int64_t* sseg, int32_t n_sseg);

int make_plan(int64_t d, int32_t n, int64_t ld, const int64_t* wseg, int32_t n_wseg,
              const int64_t* sseg, int32_t n_sseg, Plan* out);

// First span of block b: every block takes S / nblk spans and the first
// S % nblk blocks one more.
inline int64_t span_begin(int64_t S, int32_t nblk, int32_t b) {
  const int64_t q = S / nblk, r = S % nblk;
  return (int64_t)b * q + std::min<int64_t>(b, r);
}

// Tensor lists: checks lengths (each a positive multiple of 4, summing to d)
// and fills off [T+1] and, for a grid of nblk blocks, the tensor holding
// each block's first coordinate.
int tensor_offsets(const Plan& P, int32_t T, const int64_t* lengths, std::vector<int64_t>* off);
void tensor_blocks(const Plan& P, int32_t nblk, const std::vector<int64_t>& off,
                   std::vector<int32_t>* first);

}  // namespace oba
