// Block ranges and split-K contributions of the persistent MFMA kernels (see
// layout.h).  The kernels walk the same ranges (kmfma.h, for_each_piece); a
// CPU test replays that walk against this image.
#include "layout.h"

#include <algorithm>
#include <climits>

namespace lora {

namespace {

struct Pos {
  int j, tile, k;
};
bool pos_lt(Pos a, Pos b) {
  return a.j < b.j || (a.j == b.j && (a.tile < b.tile || (a.tile == b.tile && a.k < b.k)));
}
Pos pos_at(const int32_t* tab, int L) {
  return Pos{tab[kPosInts * L], tab[kPosInts * L + 1], tab[kPosInts * L + 2]};
}

// The non-empty pieces (slice j, tile t, units [k0, k1)) of the range [a, b).
template <class F>
void for_pieces(Pos a, Pos b, int T, const std::vector<int32_t>& n, F&& f) {
  Pos p = a;
  while (pos_lt(p, b)) {
    const int k1 = (p.j == b.j && p.tile == b.tile) ? b.k : n[(size_t)p.j];
    f(p.j, p.tile, p.k, k1);
    p.k = 0;
    if (++p.tile == T) {
      p.tile = 0;
      ++p.j;
    }
  }
}

}  // namespace

namespace {

void set_pos(int32_t* out, int L, int j, int t, int k) {
  int32_t* o = out + kPosInts * L;
  o[0] = j;
  o[1] = t;
  o[2] = k;
  o[3] = 0;
}

// Blocks needed when each takes units in sequence until its cost (units times
// their weight, plus ov for every tile piece it touches) would pass `cap`; a
// block always takes at least one unit.  Stops counting past G.  out (if
// given): the start of every used block.  Only the tiles before sequence
// index seq_end (j T + t) are cut.
int greedy_ranges(const std::vector<int32_t>& w, const std::vector<int32_t>& n, int G, int64_t ov,
                  int64_t cap, int32_t* out, int seq_end) {
  const int T = (int)w.size();
  int used = 0;
  bool open = false;
  int64_t cost = 0;
  for (int sq = 0; sq < seq_end; ++sq) {
    const int j = sq / T, t = sq - j * T;
    {
      const int64_t nn = n[(size_t)j], wt = w[(size_t)t];
      int64_t k = 0;
      while (k < nn) {
        if (!open) {
          if (used == G) return G + 1;
          if (out) set_pos(out, used, j, t, (int)k);
          ++used;
          open = true;
          cost = 0;
        }
        const int64_t avail = cap - cost - ov;
        int64_t take = avail >= wt ? std::min(nn - k, avail / wt) : 0;
        if (take == 0) {
          if (cost > 0) {  // full: the next block starts here
            open = false;
            continue;
          }
          take = 1;
        }
        cost += ov + take * wt;
        k += take;
        if (k < nn) open = false;  // full inside the tile
      }
    }
  }
  return used;
}

}  // namespace

void balance_ranges(const std::vector<int32_t>& w, const std::vector<int32_t>& n, int G, int64_t ov,
                    int32_t* out, int seq_end) {
  const int T = (int)w.size(), J = (int)n.size();
  if (seq_end < 0) seq_end = J * T;
  const int ej = seq_end / T, et = seq_end - ej * T;  // the end position {ej, et, 0}
  int64_t total = 0;
  for (int sq = 0; sq < seq_end; ++sq) total += (int64_t)n[(size_t)(sq / T)] * w[(size_t)(sq % T)];
  if (ov > 0 && (int64_t)J * T <= kMaxPiecesOv) {
    // smallest per-block cap that G blocks cover (binary search)
    int64_t wmax = 0;
    for (int32_t x : w) wmax = std::max<int64_t>(wmax, x);
    int64_t lo = std::max<int64_t>(1, total / G), hi = total + ov * (int64_t)seq_end + ov + wmax;
    while (lo < hi) {
      const int64_t mid = lo + (hi - lo) / 2;
      if (greedy_ranges(w, n, G, ov, mid, nullptr, seq_end) <= G) hi = mid;
      else lo = mid + 1;
    }
    const int used = greedy_ranges(w, n, G, ov, lo, out, seq_end);
    for (int L = used; L <= G; ++L) set_pos(out, L, ej, et, 0);
    return;
  }
  int j = 0, t = 0;
  int64_t before = 0;  // weight of the units before tile t of slice j
  for (int L = 0; L <= G; ++L) {
    const int64_t target = total * L / G;
    set_pos(out, L, ej, et, 0);
    while (j * T + t < seq_end) {
      const int64_t wt = w[(size_t)t];
      const int64_t k = std::max<int64_t>(0, (target - before + wt - 1) / wt);
      if (k < n[(size_t)j]) {
        set_pos(out, L, j, t, (int)k);
        break;
      }
      before += wt * n[(size_t)j];
      if (++t == T) {
        t = 0;
        ++j;
      }
    }
  }
}

void spread_ranges(const std::vector<int32_t>& w, const std::vector<int32_t>& n, int G, int64_t ov,
                   int32_t* out) {
  const int T = (int)w.size(), J = (int)n.size();
  int64_t per = 0, units = 0;
  for (int32_t x : w) per += x;
  for (int32_t nj : n) units += nj;
  const int64_t total = per * units + ov * J * T;
  int j = 0, t = 0;
  int64_t b = 0;  // start of tile t of slice j, the set-ups of the tiles before it included
  for (int L = 0; L <= G; ++L) {
    const int64_t target = total * L / G;
    set_pos(out, L, J, 0, 0);
    while (j < J) {
      const int64_t wt = w[(size_t)t];
      const int64_t nj = n[(size_t)j];
      // unit 0 starts at b, unit k >= 1 at b + ov + k wt
      int64_t k = 0;
      if (target > b) {
        k = 1;
        while (k < nj && b + ov + k * wt < target) ++k;
      }
      if (k < nj) {
        set_pos(out, L, j, t, (int)k);
        break;
      }
      b += ov + wt * nj;
      if (++t == T) {
        t = 0;
        ++j;
      }
    }
  }
}

bool layout_host(const std::vector<int32_t>& ws, const std::vector<int32_t>& we,
                 const std::vector<int32_t>& tu, const std::vector<int32_t>& nst,
                 const std::vector<int32_t>& nch, int G, int64_t ov_s, int64_t ov_e,
                 LayoutHost& h, bool spread, double pool_frac) {
  const int J = (int)nst.size();
  const int T = (int)ws.size();
  h.o_bs = 0;
  h.o_be = (size_t)kPosInts * ((size_t)G + 1);
  h.o_fl = 2 * (size_t)kPosInts * ((size_t)G + 1);
  h.o_pool = (h.o_fl + 2 * (size_t)G + 3) & ~(size_t)3;
  h.o_off = h.o_pool + 4;
  h.o_ent = (h.o_off + (size_t)J * ((size_t)T + 1) + 3) & ~(size_t)3;
  std::vector<int32_t>& buf = h.buf;
  buf.assign(h.o_ent, 0);
  // the expand pool: whole tiles at the end of the last slice, about
  // pool_frac of the expand weight
  int pool_t0 = T;
  if (!spread && pool_frac > 0 && J >= 2 && T > 0) {
    int64_t total = 0, acc = 0;
    for (int j = 0; j < J; ++j)
      for (int t = 0; t < T; ++t) total += (int64_t)nch[(size_t)j] * we[(size_t)t];
    while (pool_t0 > 0 && (double)acc < pool_frac * (double)total) {
      --pool_t0;
      acc += (int64_t)nch[(size_t)(J - 1)] * we[(size_t)pool_t0];
    }
  }
  h.pool = pool_t0 < T;
  if (spread) {
    spread_ranges(ws, nst, G, ov_s, buf.data() + h.o_bs);
    spread_ranges(we, nch, G, ov_e, buf.data() + h.o_be);
  } else {
    balance_ranges(ws, nst, G, ov_s, buf.data() + h.o_bs);
    balance_ranges(we, nch, G, ov_e, buf.data() + h.o_be, (J - 1) * T + pool_t0);
  }
  // per (j, tile) the blocks whose shrink ranges meet it, in block order; each
  // block's first and last piece
  std::vector<std::vector<int32_t>> lists((size_t)J * (size_t)T);
  std::vector<Pos> first((size_t)G, Pos{-1, -1, 0}), last((size_t)G, Pos{-1, -1, 0});
  for (int L = 0; L < G; ++L) {
    const int32_t* bs = buf.data() + h.o_bs;
    for_pieces(pos_at(bs, L), pos_at(bs, L + 1), T, nst, [&](int j, int t, int, int) {
      lists[(size_t)j * T + t].push_back(L);
      if (first[(size_t)L].j < 0) first[(size_t)L] = Pos{j, t, 0};
      last[(size_t)L] = Pos{j, t, 0};
    });
  }
  int64_t units = 0;
  std::vector<int32_t> ent;
  for (int j = 0; j < J; ++j) {
    for (int t = 0; t < T; ++t) {
      buf[h.o_off + (size_t)j * (T + 1) + t] = (int32_t)ent.size();
      for (int32_t L : lists[(size_t)j * T + t]) {
        if (units > INT32_MAX) return false;
        if (first[(size_t)L].j == j && first[(size_t)L].tile == t) buf[h.o_fl + 2 * (size_t)L] = (int32_t)units;
        if (last[(size_t)L].j == j && last[(size_t)L].tile == t) buf[h.o_fl + 2 * (size_t)L + 1] = (int32_t)units;
        ent.push_back((int32_t)units);
        units += tu[(size_t)t];
      }
    }
    buf[h.o_off + (size_t)j * (T + 1) + T] = (int32_t)ent.size();
  }
  if (h.pool) {
    // claims of about three set-ups' worth of chunks (at least 8, at most a
    // tile); the counter after the partial tiles
    int64_t wsum = 0;
    for (int t = pool_t0; t < T; ++t) wsum += we[(size_t)t];
    const int64_t wavg = std::max<int64_t>(1, wsum / (T - pool_t0));
    const int64_t n_last = nch[(size_t)(J - 1)];
    const int64_t pool_units = (int64_t)(T - pool_t0) * n_last;
    const int64_t batch = std::min<int64_t>(n_last, std::max<int64_t>(8, (3 * ov_e + wavg - 1) / wavg));
    if (pool_units > INT32_MAX) return false;
    buf[h.o_pool] = (int32_t)pool_units;
    buf[h.o_pool + 1] = (int32_t)batch;
    buf[h.o_pool + 2] = (int32_t)units;
    units += 1;
  }
  if (units > INT32_MAX) return false;
  buf.insert(buf.end(), ent.begin(), ent.end());
  h.part_units = units;
  return true;
}

}  // namespace lora
