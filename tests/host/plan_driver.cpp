// plan_driver.cpp -- test driver for the host-only piece planner.
// Usage: plan_driver d n ld n_wseg o_0 .. o_nw n_sseg o_0 .. o_ns
// Prints "rc <status>", then "G d W S nblk nblk_w nblk_c nblk_e", then for the
// worker segments on the compress grid, the worker segments on the server
// grid, the server segments on the server grid, on the update grid and on the
// compress grid, and the worker segments on the explicit grid:
// "T <n_pieces> <n_seg>", one
// "P lo hi seg" line per piece, "B" + blk_first, "S" + seg_first, "I" +
// item_q, "J" + seg_item (the last two empty for one-stage sums).  With a
// tensor list appended ("nt l_0 .. l_{nt-1}"): "TO <status>", then for the
// update, server and compress grids "TB" + the first tensor of each block.  Built by the test suite with the host compiler and
// sanitizers; it calls nothing of HIP.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "layout.hpp"

static void dump(const oba::Pieces& p, int n_seg) {
  std::printf("T %zu %d\n", p.lo.size(), n_seg);
  for (size_t i = 0; i < p.lo.size(); ++i)
    std::printf("P %lld %lld %d\n", (long long)p.lo[i], (long long)p.hi[i], p.seg[i]);
  std::printf("B");
  for (int v : p.blk_first) std::printf(" %d", v);
  std::printf("\nS");
  for (int v : p.seg_first) std::printf(" %d", v);
  std::printf("\nI");
  for (int v : p.item_q) std::printf(" %d", v);
  std::printf("\nJ");
  for (int v : p.seg_item) std::printf(" %d", v);
  std::printf("\n");
}

int main(int argc, char** argv) {
  int a = 1;
  auto next = [&]() { return a < argc ? std::atoll(argv[a++]) : 0LL; };
  const long long d = next(), n = next(), ld = next();
  const int nw = (int)next();
  std::vector<int64_t> w(nw + 1);
  for (auto& x : w) x = next();
  const int ns = (int)next();
  std::vector<int64_t> s(ns + 1);
  for (auto& x : s) x = next();
  oba::Plan P;
  int rc = oba::make_plan(d, (int32_t)n, ld, w.data(), nw, s.data(), ns, &P);
  std::printf("rc %d\n", rc);
  if (rc) return 0;
  std::printf("G %lld %lld %lld %d %d %d %d\n", (long long)P.d, (long long)P.W, (long long)P.S,
              P.nblk, P.nblk_w, P.nblk_c, P.nblk_e);
  dump(P.wp, nw);
  dump(P.wp_s, nw);
  dump(P.sp, ns);
  dump(P.sp_w, ns);
  dump(P.sp_c, ns);
  dump(P.wp_e, nw);
  // optional tensor list: nt l_0 .. l_{nt-1}
  if (a < argc) {
    const int nt = (int)next();
    std::vector<int64_t> len(nt > 0 ? nt : 1);
    for (int t = 0; t < nt; ++t) len[t] = next();
    std::vector<int64_t> off;
    const int trc = oba::tensor_offsets(P, nt, len.data(), &off);
    std::printf("TO %d\n", trc);
    if (trc == 0) {
      for (int32_t nb : {P.nblk_w, P.nblk, P.nblk_c}) {
        std::vector<int32_t> first;
        oba::tensor_blocks(P, nb, off, &first);
        std::printf("TB");
        for (int v : first) std::printf(" %d", v);
        std::printf("\n");
      }
    }
  }
  return 0;
}
