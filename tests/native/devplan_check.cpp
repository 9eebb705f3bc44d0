// Host check of the device planner (csrc/devplan.h), run sequentially on the
// CPU: on seeded random batches (repeated, invalid and non-resident ids,
// mixed ranks, several slices, grids of 8 to 1024 blocks) its output must be
// bit-identical to the plan built the host planner's way -- a stable sort of
// the tokens by adapter, tiles of at most 64 tokens ordered by rank band and
// size, the shared tile weights -- laid out by the host layout (layout.cpp)
// with the ranges cut by spread_ranges; and its partial tiles must fit the
// workspace bound.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "devplan.h"
#include "layout.h"

using namespace lora;

namespace {

struct HostCtx {
  template <class F>
  void par(int n, F&& f) {
    for (int i = 0; i < n; ++i) f(i);
  }
  void sync() {}
  bool leader() const { return true; }
  void scan(int32_t* a, int32_t*, int n) {
    for (int i = 1; i < n; ++i) a[i] += a[i - 1];
  }
};

int g_bad = 0;
int g_multi_chunk = 0;  // trials with more contributions than one scan chunk
void fail(int trial, const char* what) {
  if (g_bad++ < 20) printf("FAIL trial %d: %s\n", trial, what);
}

}  // namespace

int main(int argc, char** argv) {
  const int trials = argc > 1 ? atoi(argv[1]) : 300;
  std::mt19937 rng(20261204);
  for (int trial = 0; trial < trials; ++trial) {
    const int NA = 1 + (int)(rng() % 3000);
    const int J = 1 + (int)(rng() % 4);
    const int G = 8 * (1 + (int)(rng() % 128));
    const int n = trial % 7 == 0 ? 1 + (int)(rng() % 8) : 1 + (int)(rng() % kDpMaxTokens);
    const int rs_per16 = 8;
    const int max_rank = 128;
    // adapter table: J slices x NA adapters; some adapters absent from a slice
    std::vector<DevEntry> entries((size_t)J * NA);
    const int ranks[] = {8, 16, 24, 32, 40, 64, 100, 128};
    for (int a = 0; a < NA; ++a) {
      const int r = ranks[rng() % 8];
      for (int j = 0; j < J; ++j) {
        DevEntry e{};
        e.rank = (rng() % 10 == 0) ? 0 : (trial % 3 == 0 ? ranks[rng() % 8] : r);
        entries[(size_t)j * NA + a] = e;
      }
    }
    // ids: a few popular adapters (Zipf-like), uniform ones, -1 and out of range
    std::vector<int32_t> ids((size_t)n);
    const int hot = 1 + (int)(rng() % 8);
    for (int i = 0; i < n; ++i) {
      const unsigned u = rng() % 100;
      if (u < 5) ids[(size_t)i] = -1;
      else if (u < 8) ids[(size_t)i] = NA + (int)(rng() % 5);
      else if (u < 50) ids[(size_t)i] = (int)(rng() % (unsigned)std::min(NA, hot));
      else ids[(size_t)i] = (int)(rng() % (unsigned)NA);
    }
    DevPlanShape sh{};
    sh.n = n;
    sh.J = J;
    sh.G = G;
    sh.rs_per16 = rs_per16;
    sh.cap = n;
    sh.ov_s = trial % 4 == 0 ? 0 : (int)(rng() % 2000);
    sh.ov_e = trial % 4 == 1 ? 0 : (int)(rng() % 3000);
    std::vector<int32_t> nst((size_t)J), nch((size_t)J);
    for (int j = 0; j < J; ++j) {
      sh.slice[j] = j;
      sh.nst[j] = nst[(size_t)j] = 1 + (int)(rng() % (trial % 5 == 0 ? 3 : 200));
      sh.nch[j] = nch[(size_t)j] = 1 + (int)(rng() % 500);
    }
    PoolView pv{};
    pv.entries = entries.data();
    pv.max_adapters = NA;
    // ---- device planner, run on the host
    DevPlanWs w;
    if (!devplan_ws(J, n, G, max_rank, w)) {
      fail(trial, "workspace bound overflow");
      continue;
    }
    std::vector<char> ws(w.bytes, 0x5A);
    const DevPlanOut o = devplan_out(ws.data(), w);
    DevPlanLds* lds = new DevPlanLds;
    HostCtx cx;
    devplan_run(cx, pv, sh, ids.data(), o, *lds);
    delete lds;
    // ---- the host planner's way
    auto resident_any = [&](int a) {
      for (int j = 0; j < J; ++j)
        if (entries[(size_t)j * NA + a].rank > 0) return true;
      return false;
    };
    std::vector<int32_t> perm;
    for (int i = 0; i < n; ++i) {
      const int a = ids[(size_t)i];
      if (a >= 0 && a < NA && resident_any(a)) perm.push_back(i);
    }
    std::stable_sort(perm.begin(), perm.end(), [&](int x, int y) { return ids[(size_t)x] < ids[(size_t)y]; });
    struct Tile {
      PlanItem it;
      int band, rmax;
    };
    std::vector<Tile> tiles;
    int groups = 0;
    for (size_t p = 0; p < perm.size();) {
      size_t q = p;
      const int a = ids[(size_t)perm[p]];
      while (q < perm.size() && ids[(size_t)perm[q]] == a) ++q;
      ++groups;
      const int L = (int)(q - p);
      int rmax = 0;
      for (int j = 0; j < J; ++j) rmax = std::max(rmax, (int)entries[(size_t)j * NA + a].rank);
      const int nt = (L + kTileM - 1) / kTileM;
      int off = 0;
      for (int t = 0; t < nt; ++t) {
        const int c = L / nt + (t < L % nt ? 1 : 0);
        tiles.push_back({{a, (int32_t)p + off, c, 1}, (rmax + 15) / 16, rmax});
        off += c;
      }
      p = q;
    }
    std::stable_sort(tiles.begin(), tiles.end(), [](const Tile& x, const Tile& y) {
      if (x.band != y.band) return x.band > y.band;
      return x.it.count > y.it.count;
    });
    const int T = (int)tiles.size();
    std::vector<int32_t> wsv((size_t)T), wev((size_t)T), tuv((size_t)T);
    for (int t = 0; t < T; ++t) {
      const int rs = (tiles[(size_t)t].rmax + rs_per16 - 1) / rs_per16 * rs_per16;
      const TileCost tc = tile_cost(tiles[(size_t)t].it.count, tiles[(size_t)t].rmax, rs);
      wsv[(size_t)t] = tc.ws;
      wev[(size_t)t] = tc.we;
      tuv[(size_t)t] = tc.tu;
    }
    // ---- compare
    if (o.counts[0] != T) fail(trial, "tile count");
    if (o.counts[1] != (int)perm.size()) fail(trial, "token count");
    if (o.counts[2] != groups) fail(trial, "group count");
    for (size_t p = 0; p < perm.size(); ++p)
      if (o.perm[p] != perm[p]) {
        fail(trial, "perm");
        break;
      }
    for (int t = 0; t < T && t < o.counts[0]; ++t) {
      const PlanItem& a = o.items[t];
      const PlanItem& b = tiles[(size_t)t].it;
      if (a.adapter != b.adapter || a.start != b.start || a.count != b.count || a.kind != 1) {
        fail(trial, "items");
        break;
      }
    }
    if (T == 0) {
      // no tile: every range is the end position
      for (int L = 0; L <= G; ++L)
        if (o.bs[4 * L] != J || o.be[4 * L] != J || o.bs[4 * L + 2] || o.be[4 * L + 2]) {
          fail(trial, "empty ranges");
          break;
        }
      continue;
    }
    LayoutHost h;
    if (!layout_host(wsv, wev, tuv, nst, nch, G, sh.ov_s, sh.ov_e, h, true)) {
      fail(trial, "layout_host refused");
      continue;
    }
    const int NC = (int)(h.buf.size() - h.o_ent);
    if (NC > kDpThreads) ++g_multi_chunk;
    if (o.counts[3] != NC) fail(trial, "contribution count");
    if (o.counts[4] != h.part_units) fail(trial, "partial units");
    if (h.part_units > w.part_units) fail(trial, "partial tiles above the workspace bound");
    for (int i = 0; i < 4 * (G + 1); ++i) {
      if (o.bs[i] != h.buf[h.o_bs + (size_t)i]) {
        fail(trial, "shrink ranges");
        break;
      }
    }
    for (int i = 0; i < 4 * (G + 1); ++i) {
      if (o.be[i] != h.buf[h.o_be + (size_t)i]) {
        fail(trial, "expand ranges");
        break;
      }
    }
    for (int i = 0; i < 2 * G; ++i)
      if (o.fl[i] != h.buf[h.o_fl + (size_t)i]) {
        fail(trial, "first / last partial tiles");
        break;
      }
    for (int i = 0; i < J * (T + 1); ++i)
      if (o.c_off[i] != h.buf[h.o_off + (size_t)i]) {
        fail(trial, "contribution offsets");
        break;
      }
    for (int c = 0; c < NC && c < o.counts[3]; ++c)
      if (o.c_ent[c] != h.buf[h.o_ent + (size_t)c]) {
        fail(trial, "contribution entries");
        break;
      }
  }
  printf("%d trials (%d with several contribution chunks), %d failures\n", trials, g_multi_chunk, g_bad);
  return g_bad ? 1 : 0;
}
