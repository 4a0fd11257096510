// layout.cpp -- host-only validation and piece planning (see layout.hpp).
#include "layout.hpp"

#include <algorithm>
#include <climits>

namespace oba {

namespace {

constexpr int kOk = 0, kEInval = -1, kESeg = -3, kENoMem = -6;

int check_table(int64_t d, const int64_t* seg, int32_t n_seg) {
  if (!seg) return kEInval;
  if (d == 0) return (n_seg == 0 && seg[0] == 0) ? kOk : kESeg;
  if (n_seg < 1 || n_seg > INT32_MAX - 1) return kESeg;
  if (seg[0] != 0 || seg[n_seg] != d) return kESeg;
  for (int32_t j = 0; j < n_seg; ++j)
    if (seg[j + 1] <= seg[j]) return kESeg;
  return kOk;
}

// Cut segment table `off` at the block boundaries of a grid of nblk blocks.
int cut(const Plan& P, int32_t nblk, const std::vector<int64_t>& off, Pieces* out) {
  const int32_t n_seg = (int32_t)off.size() - 1;
  out->lo.clear();
  out->hi.clear();
  out->seg.clear();
  out->blk_first.assign((size_t)nblk + 1, 0);
  out->seg_first.assign((size_t)n_seg + 1, 0);
  int32_t j = 0;
  for (int32_t b = 0; b < nblk; ++b) {
    out->blk_first[b] = (int32_t)out->lo.size();
    const int64_t r0 = span_begin(P.S, nblk, b) * kSpan;
    const int64_t r1 = std::min(span_begin(P.S, nblk, b + 1) * kSpan, P.d);
    while (off[j + 1] <= r0) ++j;
    for (int32_t jj = j; jj < n_seg && off[jj] < r1; ++jj) {
      if (out->lo.size() >= (size_t)INT32_MAX - 1) return kESeg;
      out->lo.push_back(std::max(r0, off[jj]));
      out->hi.push_back(std::min(r1, off[jj + 1]));
      out->seg.push_back(jj);
    }
  }
  out->blk_first[nblk] = (int32_t)out->lo.size();
  // pieces are in coordinate order, so each segment's pieces are consecutive
  int32_t q = 0;
  for (int32_t s = 0; s < n_seg; ++s) {
    while (out->seg[q] < s) ++q;
    out->seg_first[s] = q;
  }
  out->seg_first[n_seg] = (int32_t)out->lo.size();
  out->item_q.clear();
  out->seg_item.clear();
  int32_t most = 0;
  for (int32_t s = 0; s < n_seg; ++s)
    most = std::max(most, out->seg_first[s + 1] - out->seg_first[s]);
  if (most > kSplitAbove) {
    out->seg_item.assign((size_t)n_seg + 1, 0);
    for (int32_t s = 0; s < n_seg; ++s) {
      out->seg_item[s] = (int32_t)out->item_q.size();
      for (int32_t q = out->seg_first[s]; q < out->seg_first[s + 1]; q += kItem)
        out->item_q.push_back(q);
    }
    out->seg_item[n_seg] = (int32_t)out->item_q.size();
    out->item_q.push_back((int32_t)out->lo.size());
  }
  return kOk;
}

}  // namespace

int validate(int64_t d, int32_t n, int64_t ld, const int64_t* wseg, int32_t n_wseg,
             const int64_t* sseg, int32_t n_sseg) {
  if (d < 0 || d > ((int64_t)1 << 46)) return kEInval;
  if (n < 1 || n > kMaxWorkers) return kEInval;
  if (ld < d || ld % 8 != 0 || ld > ((int64_t)1 << 46)) return kEInval;
  int rc = check_table(d, wseg, n_wseg);
  if (rc) return rc;
  return check_table(d, sseg, n_sseg);
}

int make_plan(int64_t d, int32_t n, int64_t ld, const int64_t* wseg, int32_t n_wseg,
              const int64_t* sseg, int32_t n_sseg, Plan* out) {
  int rc = validate(d, n, ld, wseg, n_wseg, sseg, n_sseg);
  if (rc) return rc;
  try {
    Plan P;
    P.d = d;
    P.n = n;
    P.ld = ld;
    P.W = (d + 63) / 64;
    P.S = (d + kSpan - 1) / kSpan;
    P.nblk = (int32_t)std::min<int64_t>((P.S + kServerSpans - 1) / kServerSpans, kMaxBlocks);
    P.nblk_w = (int32_t)std::min<int64_t>(P.S, kMaxBlocksWorker);
    const int32_t spc = compress_spans(n);
    P.nblk_c = (int32_t)std::min<int64_t>((P.S + spc - 1) / spc, kMaxBlocksWorker);
    const int32_t spe = explicit_spans(n);
    P.nblk_e = (int32_t)std::min<int64_t>((P.S + spe - 1) / spe, kMaxBlocksWorker);
    P.wseg.assign(wseg, wseg + n_wseg + 1);
    P.sseg.assign(sseg, sseg + n_sseg + 1);
    if ((rc = cut(P, P.nblk_c, P.wseg, &P.wp))) return rc;
    if ((rc = cut(P, P.nblk, P.wseg, &P.wp_s))) return rc;
    if ((rc = cut(P, P.nblk, P.sseg, &P.sp))) return rc;
    if ((rc = cut(P, P.nblk_w, P.sseg, &P.sp_w))) return rc;
    if ((rc = cut(P, P.nblk_c, P.sseg, &P.sp_c))) return rc;
    if ((rc = cut(P, P.nblk_e, P.wseg, &P.wp_e))) return rc;
    *out = std::move(P);
  } catch (...) {
    return kENoMem;
  }
  return kOk;
}

int tensor_offsets(const Plan& P, int32_t T, const int64_t* lengths, std::vector<int64_t>* off) {
  if (!lengths || T < 1 || T > INT32_MAX - 1) return kEInval;
  try {
    off->assign((size_t)T + 1, 0);
  } catch (...) {
    return kENoMem;
  }
  for (int32_t t = 0; t < T; ++t) {
    const int64_t len = lengths[t];
    if (len <= 0 || len % 4 != 0 || len > P.d - (*off)[t]) return kEInval;
    (*off)[t + 1] = (*off)[t] + len;
  }
  return (*off)[T] == P.d ? kOk : kEInval;
}

void tensor_blocks(const Plan& P, int32_t nblk, const std::vector<int64_t>& off,
                   std::vector<int32_t>* first) {
  first->assign((size_t)nblk, 0);
  int32_t t = 0;
  for (int32_t b = 0; b < nblk; ++b) {
    const int64_t k = span_begin(P.S, nblk, b) * kSpan;
    while (off[t + 1] <= k) ++t;
    (*first)[b] = t;
  }
}

}  // namespace oba
