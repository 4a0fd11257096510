// kernels.hpp -- launch interface between the C ABI and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "layout.hpp"

namespace oba {

// Grid geometry shared by all streaming kernels of a layout.
struct Geo {
  int64_t d, ld, W, S;
  int32_t n, nblk;
  int64_t q;  // S / nblk: spans per block (the first r blocks take one more)
  int32_t r;  // S % nblk
};

// Device view of one segmentation (see layout.hpp for pieces).
struct SegDev {
  const int64_t* off;        // [n_seg+1] segment offsets
  const int64_t* phi;        // [n_pieces] piece ends
  const int32_t* pseg;       // [n_pieces] piece segment
  const int32_t* blk_first;  // [nblk+1]
  const int32_t* seg_first;  // [n_seg+1]
  const int32_t* item_q;     // [n_items+1] (two-stage sums only)
  const int32_t* seg_item;   // [n_seg+1] (two-stage sums only)
  int32_t n_seg;
  int32_t n_pieces;
  int32_t n_items;           // 0: one-stage sums
};

// Bytes of binary64 partials for table T with `rows` rows: [rows][pieces],
// then (two-stage) [rows][items], each part 256-byte aligned.
inline size_t partial_bytes(const SegDev& T, int32_t rows) {
  auto al = [](size_t b) { return (b + 255) / 256 * 256; };
  return al((size_t)T.n_pieces * rows * 8) + al((size_t)T.n_items * rows * 8);
}

// Model tensors given as a list (x and the gradient rows live in separate
// allocations).  Tensor t covers flat coordinates [off[t], off[t+1]); every
// length is a multiple of 4, so a lane's 4-coordinate quads never straddle
// two tensors.
// gradient element types (the ABI's OBA_F32, OBA_F16, OBA_BF16)
constexpr int kGradF32 = 0, kGradF16 = 1, kGradBF16 = 2;

struct TBlk {      // the tensor holding a block's first coordinate
  int64_t lo, hi;  // its flat range [off[t], off[t+1])
  int32_t t, pad;
};

struct TList {
  const int64_t* off;    // [T+1]
  const TBlk* blk;       // [nblk] per block of the grid in use
  const void* const* g;  // [n][T] gradient tensors (g dtype)
  float* const* x;       // [T] parameter tensors
  int32_t T;
};

// The whole deferred step in one block (small layouts, latency bound).
constexpr int kSmallBlock = 1024;
constexpr int64_t kSmallMaxD = 65536;
constexpr int32_t kSmallMaxN = 64;
constexpr int32_t kSmallMaxSeg = 64;
struct SmallArgs {
  int64_t d, ld, W;
  int32_t n, n_wseg, n_sseg;
  const int64_t* wseg;  // device segment offsets
  const int64_t* sseg;
  const void* g;
  const float* m_in;    // null: m = sscale * sign(sbits) (implicit momentum)
  float* c;
  uint64_t* wbits;
  float* wscale;
  float* a;
  uint64_t* sbits;
  float* sscale;
  const float* denom;
  float* m_out;         // null: m not stored
  float* x;
  float b1, omb1, lr;
};
void launch_step_small(const SmallArgs& A, int gdt, hipStream_t st);

// Momentum source of the deferred worker pass: null sbytes = read m;
// otherwise m = sbar*sign from the last packed server bits and scales, with
// the server segments cut on the worker pass's grid.
struct MomSrc {
  const uint8_t* sbytes;
  const float* sscale;
  SegDev tau;
};

struct AdamCoef {
  float lr, b1, omb1, b2, omb2, eta, bc1, bc2;
};

// out[0] = sqrt(part[0] + ... + part[n-1]) in a fixed order (0 for n = 0)
void launch_norm_finalize(const double* part, int32_t n, double* out, hipStream_t st);
// vnorm != nullptr: also ||v_new||_2 into vnorm[0] (part: nblk doubles)
void launch_adam_warmup(const Geo& G, const void* g, int gdt, float* x, float* m, float* v,
                        const AdamCoef& C, double* part, double* vnorm, hipStream_t st);
void launch_freeze(const Geo& G, const float* v, float* denom, float eta, float bc2,
                   hipStream_t st);
// Worker compression: read-only norm pass, then recompute c and store.
void launch_compress_norm(const Geo& G, const void* g, int gdt, const float* m,
                          const float* delta, const SegDev& sig, double* part, float b1,
                          float omb1, hipStream_t st);
// Tensor lists (x and g rows listed; everything else flat).  The listed
// worker pass supports the deferred modes (m read, or implicit with ms).
void launch_adam_warmup_listed(const Geo& G, const TList& tl, int gdt, float* m, float* v,
                               const AdamCoef& C, double* part, double* vnorm, hipStream_t st);
void launch_compress_deferred_listed(const Geo& G, const TList& tl, int gdt, const float* m,
                                     float* c, uint8_t* wbytes, const SegDev& sig, double* part,
                                     const float* wscale_prev, float b1, float omb1,
                                     const MomSrc& ms, hipStream_t st);
void launch_decompress_update_listed(const Geo& G, const TList& tl, const uint8_t* sbytes,
                                     const float* sscale, const float* denom, float* m,
                                     const SegDev& tau, float lr, hipStream_t st);
// per-worker momentum: m_local [n][ld] in/out
void launch_compress_deferred_local(const Geo& G, const void* g, int gdt, float* m_local,
                                    float* c, uint8_t* wbytes, const SegDev& sig, double* part,
                                    const float* wscale_prev, float b1, float omb1,
                                    hipStream_t st);
void launch_compress_apply(const Geo& G, const void* g, int gdt, const float* m, float* delta,
                           uint8_t* wbytes, const SegDev& sig, const float* wscale, float b1,
                           float omb1, hipStream_t st);
void launch_finalize(double* part, int32_t rows, const SegDev& T, float* scale,
                     hipStream_t st);
void launch_residual(const Geo& G, const float* src, int64_t src_ld, float* dst, int64_t dst_ld,
                     int32_t rows, const float* scale, const SegDev& T, hipStream_t st);
// Deferred-residual state: rows hold the last step's c (worker) / a (server)
// and the scale buffers its scales; see compress.hip.
void launch_compress_deferred(const Geo& G, const void* g, int gdt, const float* m, float* c,
                              uint8_t* wbytes, const SegDev& sig, double* part,
                              const float* wscale_prev, float b1, float omb1, const MomSrc& ms,
                              hipStream_t st);
// The same pass with 16-bit state rows c (cdt: kGradF16 binary16, kGradBF16
// bfloat16): c is rounded to the format before it is compressed and stored.
void launch_compress_deferred16(const Geo& G, const void* g, int gdt, const float* m, void* c,
                                int cdt, uint8_t* wbytes, const SegDev& sig, double* part,
                                const float* wscale_prev, float b1, float omb1, const MomSrc& ms,
                                hipStream_t st);
void launch_compress_deferred16_listed(const Geo& G, const TList& tl, int gdt, const float* m,
                                       void* c, int cdt, uint8_t* wbytes, const SegDev& sig,
                                       double* part, const float* wscale_prev, float b1,
                                       float omb1, const MomSrc& ms, hipStream_t st);
void launch_server_deferred(const Geo& G, const uint8_t* wbytes, const float* wscale, float* a,
                            uint8_t* sbytes, const SegDev& sig, const SegDev& tau, double* part,
                            const float* sscale_prev, hipStream_t st);
void launch_server_p1(const Geo& G, const uint8_t* wbytes, const float* wscale, float* eps,
                      uint8_t* sbytes, const SegDev& sig, const SegDev& tau, double* part,
                      hipStream_t st);
// m == nullptr: m is not written (the momentum stays implicit in sbits, sscale)
void launch_server_momentum(const Geo& G, const uint8_t* sbytes, const float* sscale, float* m,
                            const SegDev& tau, hipStream_t st);
void launch_decompress_update(const Geo& G, const uint8_t* sbytes, const float* sscale,
                              const float* denom, float* m, float* x, const SegDev& tau, float lr,
                              hipStream_t st);

}  // namespace oba
