// Host check of the persistent MFMA kernels' block ranges (layout.cpp): on
// seeded random launch shapes, every unit of the work sequence belongs to
// exactly one block, positions are normalized and monotone; without a piece
// set-up cost the weight of a block's range is within one unit of the mean,
// with one the largest block cost (weights plus set-up per piece) is no larger
// than under the plain split; and replaying the kernels' walk (first / last
// piece flags, as for_each_piece in kmfma.h computes them) finds each piece's
// partial tile at the offset listed for that block in the tile's
// contributions, in block order, with disjoint offsets.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>

#include "layout.h"

using lora::LayoutHost;
using lora::kPosInts;

namespace {
struct P {
  int j, t, k;
};
bool lt(P a, P b) { return a.j < b.j || (a.j == b.j && (a.t < b.t || (a.t == b.t && a.k < b.k))); }
P at(const int32_t* tab, int L) { return P{tab[kPosInts * L], tab[kPosInts * L + 1], tab[kPosInts * L + 2]}; }
}  // namespace

int main(int argc, char** argv) {
  const int trials = argc > 1 ? atoi(argv[1]) : 2000;
  std::mt19937 rng(20261203);
  int bad = 0;
  auto fail = [&](const char* what, int trial) {
    if (bad++ < 10) printf("FAIL trial %d: %s\n", trial, what);
  };
  for (int trial = 0; trial < trials; ++trial) {
    const int T = 1 + rng() % 300, J = 1 + rng() % 8, G = 8 * (1 + rng() % 64);
    std::vector<int32_t> ws(T), we(T), tu(T), nst(J), nch(J);
    for (int t = 0; t < T; ++t) {
      ws[t] = 1 + rng() % ((trial % 3 == 0) ? 1000 : 50);
      we[t] = 1 + rng() % 300;
      tu[t] = 64 * (1 + rng() % 32);
    }
    for (int j = 0; j < J; ++j) {
      nst[j] = 1 + rng() % ((trial % 5 == 0) ? 3 : 400);
      nch[j] = 1 + rng() % 400;
    }
    const int64_t ov_s = (trial % 2) ? 0 : 1 + rng() % 2000;
    const int64_t ov_e = (trial % 4 == 1) ? 0 : 1 + rng() % 3000;
    // every third trial with two or more slices leaves an expand pool
    const double pool_frac = (trial % 3 == 2) ? 0.05 + 0.05 * (rng() % 5) : 0.0;
    LayoutHost h;
    if (!lora::layout_host(ws, we, tu, nst, nch, G, ov_s, ov_e, h, false, pool_frac)) {
      fail("layout_host refused", trial);
      continue;
    }
    const int32_t* fl = h.buf.data() + h.o_fl;
    const int32_t* coff = h.buf.data() + h.o_off;
    const int32_t* cent = h.buf.data() + h.o_ent;
    const int32_t* pool = h.buf.data() + h.o_pool;
    if (h.pool != (pool_frac > 0 && J >= 2)) fail("pool presence", trial);
    // the pool: whole tiles at the end of the last slice
    const int pool_t0 = h.pool ? T - pool[0] / nch[J - 1] : T;
    if (h.pool && (pool[0] % nch[J - 1] != 0 || pool_t0 < 0 || pool_t0 >= T ||
                   pool[1] < std::min(8, nch[J - 1]) || pool[1] > nch[J - 1]))
      fail("pool shape", trial);
    for (int pass = 0; pass < 2; ++pass) {
      const int32_t* tab = h.buf.data() + (pass ? h.o_be : h.o_bs);
      const std::vector<int32_t>& n = pass ? nch : nst;
      const std::vector<int32_t>& w = pass ? we : ws;
      const int64_t ov = pass ? ov_e : ov_s;
      double max_cost = 0;
      std::vector<std::vector<int>> cover((size_t)J * T);
      for (int j = 0; j < J; ++j)
        for (int t = 0; t < T; ++t) cover[(size_t)j * T + t].assign(n[j], 0);
      const P a0 = at(tab, 0), aG = at(tab, G);
      // the expand ranges end where the pool starts
      const P end = (pass && h.pool) ? P{J - 1, pool_t0, 0} : P{J, 0, 0};
      if (!(aG.j == end.j && aG.t == end.t && aG.k == end.k)) fail("ends", trial);
      if (lt(P{0, 0, 0}, end) && !(a0.j == 0 && a0.t == 0 && a0.k == 0)) fail("start", trial);
      if (pass && h.pool)  // the pool's chunks, each claimed once
        for (int t = pool_t0; t < T; ++t)
          for (int kk = 0; kk < nch[J - 1]; ++kk) cover[(size_t)(J - 1) * T + t][kk]++;
      double total = 0, wmax = 0;
      for (int j = 0; j < J; ++j)
        for (int t = 0; t < T; ++t)
          if (lt(P{j, t, 0}, end)) total += (double)n[j] * w[t];
      for (int x : w) wmax = std::max(wmax, (double)x);
      for (int L = 0; L < G; ++L) {
        const P a = at(tab, L), b = at(tab, L + 1);
        if (lt(b, a)) fail("not monotone", trial);
        if (b.j < J && !(b.t < T && b.k < n[b.j])) fail("not normalized", trial);
        // the kernels' walk
        int j = a.j, t = a.t, k = a.k;
        bool first = true;
        double wsum = 0, cost = 0;
        while (lt(P{j, t, k}, b)) {
          const bool ends_here = j == b.j && t == b.t;
          const int k1 = ends_here ? b.k : n[j];
          int nj = j, nt = t + 1;
          if (nt == T) {
            nt = 0;
            ++nj;
          }
          const bool last = ends_here || !lt(P{nj, nt, 0}, b);
          if (!(k < k1)) fail("empty piece", trial);
          for (int kk = k; kk < k1; ++kk) cover[(size_t)j * T + t][kk]++;
          wsum += (double)(k1 - k) * w[t];
          cost += (double)(k1 - k) * w[t] + ov;
          if (pass == 0) {
            const int32_t off = first ? fl[2 * L] : last ? fl[2 * L + 1] : cent[coff[j * (T + 1) + t]];
            // block L's index among the tile's contributors (blocks whose
            // non-empty ranges meet the tile), in block order
            int idx = 0, found = -1;
            for (int M = 0; M < G; ++M) {
              const P c = at(tab, M), d = at(tab, M + 1);
              if (lt(c, d) && lt(c, P{j, t, n[j]}) && lt(P{j, t, 0}, d)) {
                if (M == L) found = idx;
                ++idx;
              }
            }
            const int c0 = coff[j * (T + 1) + t], c1 = coff[j * (T + 1) + t + 1];
            if (found < 0 || c1 - c0 != idx || cent[c0 + found] != off) fail("contribution offset", trial);
            if (!first && !last && c1 - c0 != 1) fail("middle piece shared", trial);
          }
          first = false;
          j = nj;
          t = nt;
          k = 0;
        }
        if (ov == 0 && wsum > total / G + wmax + 1e-6) fail("imbalance", trial);
        max_cost = std::max(max_cost, cost);
      }
      if (ov > 0 && (int64_t)J * T <= lora::kMaxPiecesOv && !(pass && h.pool)) {
        // the plain split (no set-up cost) under the same cost: never better
        std::vector<int32_t> plain((size_t)kPosInts * (G + 1));
        lora::balance_ranges(w, n, G, 0, plain.data());
        double plain_max = 0;
        for (int L = 0; L < G; ++L) {
          const P a = at(plain.data(), L), b = at(plain.data(), L + 1);
          double c = 0;
          int j = a.j, t = a.t, k = a.k;
          while (lt(P{j, t, k}, b)) {
            const int k1 = (j == b.j && t == b.t) ? b.k : n[j];
            c += (double)(k1 - k) * w[t] + ov;
            k = 0;
            if (++t == T) {
              t = 0;
              ++j;
            }
          }
          plain_max = std::max(plain_max, c);
        }
        if (max_cost > plain_max + 1e-6) fail("set-up-aware split worse than the plain one", trial);
      }
      for (auto& c : cover)
        for (int x : c)
          if (x != 1) {
            fail("unit not covered exactly once", trial);
            break;
          }
    }
    int64_t expect = 0;
    for (int j = 0; j < J; ++j)
      for (int t = 0; t < T; ++t)
        for (int c = coff[j * (T + 1) + t]; c < coff[j * (T + 1) + t + 1]; ++c) {
          if (cent[c] != expect) fail("partial offsets not disjoint", trial);
          expect += tu[t];
        }
    if (h.pool && pool[2] != expect) fail("pool counter offset", trial);
    if (expect + (h.pool ? 1 : 0) != h.part_units || (size_t)coff[J * (T + 1) - 1] != h.buf.size() - h.o_ent)
      fail("partial units", trial);
  }
  printf("%d trials, %d failures\n", trials, bad);
  return bad != 0;
}
