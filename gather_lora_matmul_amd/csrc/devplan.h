// Decode plan built on the device from device-resident adapter ids.
//
// Groups the tokens of a batch by adapter -- the index vector of the
// multi-LoRA serving article's SGMV section sends tokens to adapters in any
// order, and tokens sharing one adapter form one segment -- and lays the
// groups out for the persistent MFMA kernels exactly as the host planner
// does: a stable sort of the tokens by adapter, tiles of at most 64 tokens,
// tiles ordered by rank band and size (the article's FAQ on mixed ranks), the
// tiles' weights, block ranges over the launch's work sequence, and the
// split-K contributions with their partial-tile offsets.  One difference from
// the host planner: the host cuts the ranges greedily under the smallest cap
// that also counts a set-up cost per tile piece (a sequential bisection);
// here every block boundary is found on its own, at equal shares of the
// sequence's weight with one set-up cost added at the start of every tile
// (layout.h, spread_ranges).
//
// One workgroup runs the whole plan.  The algorithm is written as a sequence
// of phases over a context: ctx.par(n, f) runs f(i) for i in [0, n) spread
// over the workgroup's threads, ctx.sync() separates phases, ctx.scan(a, tmp,
// n) replaces a[0, n) by its inclusive prefix sums.  Within a phase no i reads
// what another i writes, so the same code runs sequentially on the host (the
// CPU check of this planner against the host planner).
#pragma once

#include "lora_internal.h"

namespace lora {

constexpr int kDpMaxTokens = 1024;  // tokens per device-planned batch, at most
constexpr int kDpMaxBlocks = 1024;  // persistent grid, at most
constexpr int kDpThreads = 1024;

// Launch shape of a device-planned batch (a kernel argument).
struct DevPlanShape {
  int32_t n;                   // tokens
  int32_t J;                   // launch slices
  int32_t G;                   // persistent grid of the MFMA kernels
  int32_t rs_per16;            // elements per 16 bytes of a page (rank rounding of stored B rows)
  int32_t cap;                 // token capacity the workspace was sized for
  int32_t ov_s, ov_e;          // set-up cost of a tile piece (shrink, expand weight units)
  int32_t slice[LORA_MAX_IO];  // pool slice of launch slice j
  int32_t nst[LORA_MAX_IO];    // shrink stages of launch slice j (64 columns of d_in)
  int32_t nch[LORA_MAX_IO];    // expand chunks of launch slice j (64 rows of d_out)
};

// Where the plan goes (device pointers into the caller's workspace).  The
// layout arrays have the formats of the host layout (layout.h).
struct DevPlanOut {
  int32_t* counts;   // [0] tiles, [1] tokens with an adapter, [2] groups,
                     // [3] contributions, [4] float4 units of partial tiles
  int32_t* perm;     // [cap]            tokens grouped by adapter
  PlanItem* items;   // [cap]            tiles
  int32_t* bs;       // [(G + 1) * 4]    shrink ranges
  int32_t* be;       // [(G + 1) * 4]    expand ranges
  int32_t* fl;       // [2 G]            first / last partial tile of each shrink range
  int32_t* c_off;    // [J (cap + 1)]    first contribution of (slice, tile); stride tiles + 1
  int32_t* c_ent;    // [J cap + G]      partial-tile offset of each contribution
};

// Workgroup-shared state (49 KB).  The grouping arrays are dead once the
// tiles are written, so the range arrays reuse their memory.
struct DevPlanLds {
  union {
    struct {
      alignas(16) uint32_t key[kDpMaxTokens];  // token keys (adapter << 10 | token), sorted
      int32_t gstart[kDpMaxTokens + 1];  // group starts in the sorted order
      int32_t grmax[kDpMaxTokens];       // per group: largest rank over the launch slices
      int32_t tb[kDpMaxTokens];          // per group: its first tile (before ordering)
      int32_t tg[kDpMaxTokens];          // per tile (before ordering): its group
      alignas(16) uint32_t tkey[kDpMaxTokens];  // unsorted keys: tokens, then tiles (band, size, tile)
      uint32_t tsort[kDpMaxTokens];      // tile keys, sorted
    } g;
    struct {
      int32_t cw_s[kDpMaxTokens + 1];    // exclusive prefix sums of w_s, w_e
      int32_t cw_e[kDpMaxTokens + 1];
      int32_t seq_s[kDpMaxBlocks + 1];   // shrink range starts: sequence index j T + t
      int32_t k_s[kDpMaxBlocks + 1];     //   ... and unit within the tile
      int32_t np[kDpMaxBlocks + 1];      // first contribution of each shrink range
      int32_t c_blk[kDpThreads];         // per contribution of the current chunk: its block
      int32_t c_sq[kDpThreads];          //   ... and its (slice, tile) sequence index
    } r;
  } u;
  int32_t w_s[kDpMaxTokens];             // per tile: shrink stage weight
  int32_t w_e[kDpMaxTokens];             // per tile: expand chunk weight
  int32_t tu[kDpMaxTokens];              // per tile: partial tile size
  int32_t sc0[kDpThreads], sc1[kDpThreads];  // scan buffers
  int32_t scal[8];                       // valid tokens; carry and last tile of the chunked scan
  int32_t wtot[kDpThreads / 64];         // per-wave totals of a scan
};

// Byte offsets of a device plan's arrays in the caller's workspace, and the
// float4 units reserved for its partial tiles.  Bound on the partial tiles:
// every (slice, tile) has one contribution plus one per block boundary inside
// it (at most G - 1 boundaries); a tile of c tokens whose adapter has rank
// r <= max_rank holds ceil(r / 16) * ceil(c / 16) * 64 units, and
// ceil(c / 16) <= c, so J tiles' worth sums to at most ceil(max_rank / 16) *
// 64 * J * n, and each extra contribution to at most ceil(max_rank / 16) * 4 * 64.
struct DevPlanWs {
  size_t counts, perm, items, bs, be, fl, c_off, c_ent, part, bytes;
  int64_t part_units;
};
inline bool devplan_ws(int J, int n, int G, int max_rank, DevPlanWs& w) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t o = 0;
  w.counts = o;
  o = up(o + 8 * sizeof(int32_t));
  w.perm = o;
  o = up(o + sizeof(int32_t) * (size_t)n);
  w.items = o;
  o = up(o + sizeof(PlanItem) * (size_t)n);
  w.bs = o;
  o = up(o + sizeof(RangePos) * ((size_t)G + 1));
  w.be = o;
  o = up(o + sizeof(RangePos) * ((size_t)G + 1));
  w.fl = o;
  o = up(o + 2 * sizeof(int32_t) * (size_t)G);
  w.c_off = o;
  o = up(o + sizeof(int32_t) * (size_t)J * ((size_t)n + 1));
  w.c_ent = o;
  o = up(o + sizeof(int32_t) * ((size_t)J * n + G));
  const int64_t rb = (max_rank + 15) / 16;
  w.part_units = rb * 64 * ((int64_t)J * n + 4 * (int64_t)G);
  w.part = o;
  o = up(o + 16 * (size_t)w.part_units);
  w.bytes = o;
  return w.part_units <= 0x7FFFFFFF;
}

inline DevPlanOut devplan_out(char* ws, const DevPlanWs& w) {
  DevPlanOut o;
  o.counts = reinterpret_cast<int32_t*>(ws + w.counts);
  o.perm = reinterpret_cast<int32_t*>(ws + w.perm);
  o.items = reinterpret_cast<PlanItem*>(ws + w.items);
  o.bs = reinterpret_cast<int32_t*>(ws + w.bs);
  o.be = reinterpret_cast<int32_t*>(ws + w.be);
  o.fl = reinterpret_cast<int32_t*>(ws + w.fl);
  o.c_off = reinterpret_cast<int32_t*>(ws + w.c_off);
  o.c_ent = reinterpret_cast<int32_t*>(ws + w.c_ent);
  return o;
}

// Launchers (k_devplan.hip), all on stream s; ws holds w.bytes bytes.  The
// plan alone (one workgroup); the planned MFMA apply from a plan in ws; both.
hipError_t launch_devplan(const PoolView& pv, const int32_t* ids, const DevPlanShape& sh,
                          const DevPlanWs& w, char* ws, hipStream_t s);
hipError_t launch_devplan_mfma(const Types& ty, const PoolView& pv, const IoSet& ios,
                               const DevPlanShape& sh, const DevPlanWs& w, char* ws, hipStream_t s);
hipError_t launch_devplan_apply(const Types& ty, const PoolView& pv, const IoSet& ios,
                                const int32_t* ids, const DevPlanShape& sh, const DevPlanWs& w,
                                char* ws, hipStream_t s);

constexpr uint32_t kDpNone = 0xFFFFFFFFu;  // padding key (above every key)
// A token without a (resident) adapter gets key kDpSkip | token: distinct, and
// above every token with one (adapter ids < 2^21, so those keys are < 2^31).
constexpr uint32_t kDpSkip = 0x80000000u;
constexpr int kDpTokBits = 10;             // token index bits of a key
static_assert(kDpMaxTokens <= (1 << kDpTokBits), "token index must fit the key");

__host__ __device__ inline int dp_pow2(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// Sort of n distinct keys a[0, n) into out[0, n), ascending: each key goes to
// its rank, the count of keys below it, counted by R threads per key (each
// over one part of a) into cnt[R n] (at most kDpThreads words).  a is padded
// with kDpNone up to a multiple of 4 (read 16 bytes at a time; the padding
// never counts, every key being below it).
template <class Ctx>
__host__ __device__ inline void dp_rank_sort(Ctx& cx, const uint32_t* a, uint32_t* out, int n,
                                             int32_t* cnt) {
  const int q4 = (n + 3) / 4;  // 16-byte groups of a
  int R = kDpThreads / n;
  R = R < 1 ? 1 : (R > 8 ? 8 : R);
  const int per = (q4 + R - 1) / R;
  const uint4* a4 = reinterpret_cast<const uint4*>(a);
  cx.par(n * R, [&](int idx) {
    const int r = idx / n, i = idx - r * n;
    const uint32_t v = a[i];
    const int g1 = (r + 1) * per < q4 ? (r + 1) * per : q4;
    int below = 0;
#pragma unroll 8
    for (int g = r * per; g < g1; ++g) {
      const uint4 q = a4[g];
      below += (q.x < v) + (q.y < v) + (q.z < v) + (q.w < v);
    }
    cnt[idx] = below;
  });
  cx.sync();
  cx.par(n, [&](int i) {
    int below = 0;
    for (int r = 0; r < R; ++r) below += cnt[r * n + i];
    out[below] = a[i];
  });
  cx.sync();
}

// Start of the range of block L (of G) over a work sequence of J slices x T
// tiles, slice j having n[j] units of weight w[t] in tile t (cw: exclusive
// prefix of w, per = sum of w), with a set-up cost ov at the start of every
// tile: the first unit whose start, counting the set-up costs before it, is
// at or past total * L / G (total = all units and set-ups).  Unit 0 of a tile
// spans its set-up and its own weight.  Out: sequence index j T + t and unit
// k, or (J T, 0).  With ov = 0 this is the host's plain equal-weight split.
__host__ __device__ inline void dp_range_start(int L, int G, int J, int T, const int32_t* n,
                                               const int32_t* w, const int32_t* cw, int64_t per,
                                               int64_t ov, int32_t& seq, int32_t& k) {
  int64_t units = 0;
  for (int j = 0; j < J; ++j) units += n[j];
  const int64_t num = (per * units + ov * J * T) * L;
  int lg = 0;  // the grid is a power of two in practice: a shift instead of a 64-bit division
  while ((1 << lg) < G) ++lg;
  const int64_t target = (1 << lg) == G ? num >> lg : num / G;
  // the slice: the first whose last unit starts at or past target
  int j = 0;
  int64_t sj = 0;  // start of slice j, set-ups included
  for (; j < J; ++j) {
    const int64_t end = sj + n[j] * per + ov * T;  // start of slice j + 1
    // last unit of its last tile (a tile of one unit starts at its set-up)
    const int64_t last = end - w[T - 1] - (n[j] > 1 ? 0 : ov);
    if (last >= target) break;
    sj = end;
  }
  seq = J * T;
  k = 0;
  if (j == J) return;
  // the tile: the first whose last unit starts at or past target
  const int64_t nj = n[j];
  auto start = [&](int t) { return sj + nj * cw[t] + ov * t; };
  auto last_start = [&](int t) { return start(t) + (nj > 1 ? ov + (nj - 1) * w[t] : 0); };
  int lo = 0, hi = T - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (last_start(mid) >= target) hi = mid;
    else lo = mid + 1;
  }
  seq = j * T + lo;
  const int64_t b = start(lo);
  if (target > b) {  // past the tile's set-up and first unit: 32-bit quotient
    const int32_t num = (int32_t)(target - b - ov);
    const int32_t kk = (num + w[lo] - 1) / w[lo];
    k = kk > 1 ? kk : 1;
  }
}

// The whole plan.  pv: the adapter table the launches will read; ids: n
// device ids (outside [0, max_adapters) or not resident in any launch slice:
// the token is left out).
template <class Ctx>
__host__ __device__ inline void devplan_run(Ctx& cx, const PoolView& pv, const DevPlanShape& sh,
                                            const int32_t* ids, const DevPlanOut& o,
                                            DevPlanLds& s) {
  const int n = sh.n, J = sh.J, G = sh.G, NA = pv.max_adapters;
  uint32_t* const key = s.u.g.key;
  int32_t* const gstart = s.u.g.gstart;
  int32_t* const grmax = s.u.g.grmax;
  int32_t* const tb = s.u.g.tb;
  int32_t* const tg = s.u.g.tg;
  uint32_t* const tkey = s.u.g.tkey;
  uint32_t* const tsort = s.u.g.tsort;
  int32_t* const cw_s = s.u.r.cw_s;
  int32_t* const cw_e = s.u.r.cw_e;
  int32_t* const seq_s = s.u.r.seq_s;
  int32_t* const k_s = s.u.r.k_s;
  int32_t* const np = s.u.r.np;
  int32_t* const c_blk = s.u.r.c_blk;
  int32_t* const c_sq = s.u.r.c_sq;
  constexpr uint32_t kTokMask = (1u << kDpTokBits) - 1;
  // (1) keys: adapter and token of every token with a resident adapter,
  //     sorted (tokens of one adapter together, in batch order)
  cx.par((n + 3) & ~3, [&](int i) {
    uint32_t kv = i < n ? kDpSkip | (uint32_t)i : kDpNone;
    if (i < n) {
      const int a = ids[i];
      if (a >= 0 && a < NA) {
        bool res = false;
        for (int j = 0; j < J; ++j) res = res || pv.entries[sh.slice[j] * NA + a].rank > 0;
        if (res) kv = ((uint32_t)a << kDpTokBits) | (uint32_t)i;
      }
    }
    tkey[i] = kv;
  });
  cx.sync();
  dp_rank_sort(cx, tkey, key, n, s.sc1);
  // (2) perm, group heads (a token whose adapter differs from the previous one)
  cx.par(n, [&](int p) {
    const uint32_t k = key[p];
    const bool valid = k < kDpSkip;
    if (valid && (p + 1 == n || key[p + 1] >= kDpSkip)) s.scal[0] = p + 1;
    if (p == 0 && !valid) s.scal[0] = 0;
    if (valid) o.perm[p] = (int32_t)(k & kTokMask);
    s.sc0[p] = valid && (p == 0 || (k >> kDpTokBits) != (key[p - 1] >> kDpTokBits)) ? 1 : 0;
  });
  cx.sync();
  const int nv = s.scal[0];
  cx.scan(s.sc0, s.wtot, n);
  const int NG = s.sc0[n - 1];
  cx.par(n, [&](int p) {
    if (s.sc0[p] != (p ? s.sc0[p - 1] : 0)) gstart[s.sc0[p] - 1] = p;
    if (p == 0) gstart[NG] = nv;
  });
  cx.sync();
  // (3) per group: largest rank over the launch slices, tiles of <= 64 tokens
  cx.par(NG, [&](int g) {
    const int a = (int)(key[gstart[g]] >> kDpTokBits);
    int rmax = 0;
    for (int j = 0; j < J; ++j) {
      const int r = pv.entries[sh.slice[j] * NA + a].rank;
      rmax = r > rmax ? r : rmax;
    }
    grmax[g] = rmax;
    s.sc1[g] = (gstart[g + 1] - gstart[g] + kTileM - 1) / kTileM;
  });
  cx.sync();
  if (NG > 0) cx.scan(s.sc1, s.wtot, NG);
  const int T = NG > 0 ? s.sc1[NG - 1] : 0;
  cx.par(NG, [&](int g) { tb[g] = g ? s.sc1[g - 1] : 0; });
  cx.sync();
  // (4) tile keys: rank band (descending), token count (descending), then
  //     group order (adapter id) and position in the group
  cx.par(NG, [&](int g) {
    const int L = gstart[g + 1] - gstart[g];
    const int ntg = (L + kTileM - 1) / kTileM;
    const int band = (grmax[g] + 15) / 16;
    for (int q = 0; q < ntg; ++q) {
      const int seq = tb[g] + q;
      const int count = L / ntg + (q < L % ntg ? 1 : 0);
      tg[seq] = g;
      tkey[seq] = ((uint32_t)(15 - band) << 20) | ((uint32_t)(kTileM - count) << kDpTokBits) |
                  (uint32_t)seq;
    }
  });
  cx.par(((T + 3) & ~3) - T, [&](int i) { tkey[T + i] = kDpNone; });
  cx.sync();
  if (T > 0) dp_rank_sort(cx, tkey, tsort, T, s.sc0);
  // (5) items and weights in tile order
  cx.par(T, [&](int i) {
    const int seq = (int)(tsort[i] & kTokMask);
    const int g = tg[seq];
    const int q = seq - tb[g];
    const int L = gstart[g + 1] - gstart[g];
    const int ntg = (L + kTileM - 1) / kTileM;
    const int base = L / ntg, rem = L % ntg;
    const int count = base + (q < rem ? 1 : 0);
    const int off = q * base + (q < rem ? q : rem);
    PlanItem it;
    it.adapter = (int32_t)(key[gstart[g]] >> kDpTokBits);
    it.start = gstart[g] + off;
    it.count = count;
    it.kind = 1;
    o.items[i] = it;
    const int rmax = grmax[g];
    const int rs = (rmax + sh.rs_per16 - 1) / sh.rs_per16 * sh.rs_per16;
    const TileCost tc = tile_cost(count, rmax, rs);
    s.w_s[i] = tc.ws;
    s.w_e[i] = tc.we;
    s.tu[i] = tc.tu;
    s.sc0[i] = tc.ws;
    s.sc1[i] = tc.we;
  });
  cx.sync();
  // exclusive prefix sums of the weights (the grouping arrays are dead now)
  if (T > 0) {
    cx.scan(s.sc0, s.wtot, T);
    cx.scan(s.sc1, s.wtot, T);
  }
  cx.par(T + 1, [&](int i) {
    cw_s[i] = i ? s.sc0[i - 1] : 0;
    cw_e[i] = i ? s.sc1[i - 1] : 0;
  });
  cx.sync();
  // (6) block ranges: shrink (stages) and expand (chunks)
  const int64_t per_s = cw_s[T], per_e = cw_e[T];
  cx.par(2 * G, [&](int i) {
    const bool ex = i >= G;
    const int L = ex ? i - G : i;
    int32_t seq = J * T, k = 0;
    if (T > 0) {
      if (ex) dp_range_start(L, G, J, T, sh.nch, s.w_e, cw_e, per_e, sh.ov_e, seq, k);
      else dp_range_start(L, G, J, T, sh.nst, s.w_s, cw_s, per_s, sh.ov_s, seq, k);
    }
    const int j = T > 0 ? seq / T : J, t = T > 0 ? seq - j * T : 0;
    int32_t* pos = (ex ? o.be : o.bs) + 4 * L;
    pos[0] = j;
    pos[1] = t;
    pos[2] = k;
    pos[3] = 0;
    if (!ex) {
      seq_s[L] = seq;
      k_s[L] = k;
    }
  });
  if (cx.leader()) {  // both tables end at the end position
    for (int q = 0; q < 4; ++q) {
      o.bs[4 * G + q] = q == 0 ? J : 0;
      o.be[4 * G + q] = q == 0 ? J : 0;
    }
    seq_s[G] = J * T;
    k_s[G] = 0;
  }
  cx.sync();
  // (7) pieces of every shrink range: the (slice, tile) pairs it meets;
  //     np[L] becomes the first contribution of block L (np[G]: their count)
  cx.par(G, [&](int L) {
    const int sa = seq_s[L], ka = k_s[L], sb = seq_s[L + 1], kb = k_s[L + 1];
    s.sc0[L] = (sa == sb && ka == kb) ? 0 : sb - sa + (kb > 0 ? 1 : 0);
  });
  cx.sync();
  cx.scan(s.sc0, s.wtot, G);
  const int NC = s.sc0[G - 1];
  cx.par(G + 1, [&](int L) { np[L] = L ? s.sc0[L - 1] : 0; });
  if (cx.leader()) s.scal[4] = 0;  // carry of the chunked scan below (scal[5]: last sequence index)
  cx.sync();
  // (8) contributions in (slice, tile, block) order are in block order, a
  //     block's pieces in sequence order.  Per chunk of contributions: each
  //     block lists its own (block, sequence index), then a scan of the tile
  //     sizes gives each partial tile's float4 offset; the first contribution
  //     of each (slice, tile) and each block's first and last partial tile
  cx.par(G, [&](int L) {
    if (np[L + 1] == np[L]) {
      o.fl[2 * L] = 0;
      o.fl[2 * L + 1] = 0;
    }
  });
  for (int c0 = 0; c0 < NC; c0 += kDpThreads) {
    const int m = NC - c0 < kDpThreads ? NC - c0 : kDpThreads;
    cx.par(G, [&](int L) {
      const int a = np[L] > c0 ? np[L] : c0;
      const int b = np[L + 1] < c0 + m ? np[L + 1] : c0 + m;
      for (int c = a; c < b; ++c) {
        c_blk[c - c0] = L;
        c_sq[c - c0] = seq_s[L] + (c - np[L]);
      }
    });
    cx.sync();
    cx.par(m, [&](int i) {
      const int sq = c_sq[i];
      const int32_t tu = s.tu[sq - (sq / T) * T];
      s.sc0[i] = tu;
      s.sc1[i] = tu;
    });
    cx.sync();
    cx.scan(s.sc0, s.wtot, m);
    const int carry = s.scal[4];
    const int prev_sq = s.scal[5];
    cx.par(m, [&](int i) {
      const int c = c0 + i;
      const int32_t off = carry + s.sc0[i] - s.sc1[i];
      o.c_ent[c] = off;
      const int L = c_blk[i], sq = c_sq[i];
      if (c == np[L]) o.fl[2 * L] = off;
      if (c == np[L + 1] - 1) o.fl[2 * L + 1] = off;
      const int sqp = i ? c_sq[i - 1] : (c ? prev_sq : -1);
      if (sqp != sq) {
        const int j = sq / T, t = sq - j * T;
        o.c_off[j * (T + 1) + t] = c;
        if (t == 0 && j > 0) o.c_off[(j - 1) * (T + 1) + T] = c;
      }
    });
    cx.sync();
    if (cx.leader()) {
      s.scal[4] = carry + s.sc0[m - 1];
      s.scal[5] = c_sq[m - 1];
    }
    cx.sync();
  }
  // (9) counts
  cx.par(J, [&](int j) {
    if (T == 0) o.c_off[j] = 0;
  });
  if (cx.leader()) {
    if (T > 0) o.c_off[(J - 1) * (T + 1) + T] = NC;
    o.counts[0] = T;
    o.counts[1] = nv;
    o.counts[2] = NG;
    o.counts[3] = NC;
    o.counts[4] = s.scal[4];
  }
  cx.sync();
}

}  // namespace lora
