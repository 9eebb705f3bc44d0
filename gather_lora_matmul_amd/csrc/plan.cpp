// SGMV batch planner (host, once per batch).
//
// Tokens are grouped by adapter with a stable counting sort: every group is a
// segment of tokens sharing one adapter (multi-LoRA serving article, SGMV
// section), whether its tokens were contiguous in the batch or not (the
// article's index-vector diagram sends tokens 1 and 4 to the same adapter).
// Groups of at least l_long tokens (default 1: all of them, on 16-bit pools)
// become MFMA tiles of up to 64 tokens; the rest, and every group of an fp32
// pool, become short items of up to four tokens that run on the vector ALUs.  Items are ordered by rank band (rank rounded up to 16, the MFMA tile
// width), largest first, so that the biggest items start first -- the "bands
// of uniform granularity with little padding" of the article's FAQ on mixed
// ranks.
#include <algorithm>
#include <cstring>

#include "runtime.h"

using namespace lora;

namespace {

// Split the weighted tile list w[0..n) into G contiguous ranges of equal
// weight (persistent kernels: logical block L takes [out[L], out[L+1])).
// Range boundaries fall inside tiles; a kernel rounds them to the stage or
// chunk grid of the slice it runs.
void balance_blocks(const std::vector<int32_t>& w, int G, BlockStart* out) {
  const int n = (int)w.size();
  int64_t total = 0;
  for (int32_t x : w) total += x;
  int i = 0;
  int64_t before = 0;  // weight of tiles [0, i)
  for (int L = 0; L <= G; ++L) {
    const int64_t pos = total * L / G;
    while (i < n && before + w[(size_t)i] <= pos) before += w[(size_t)i++];
    if (i >= n) {
      out[L] = BlockStart{n, 0, 1, 0};
    } else {
      out[L] = BlockStart{i, (int32_t)(pos - before), w[(size_t)i], 0};
    }
  }
}

// First unit of logical block L in a slice whose tiles have n units: the
// kernels' rounding of the BlockStart table, replicated exactly.
struct HPos {
  int tile, k;
};
HPos range_start_host(const BlockStart* bs, int L, int n, int n_tiles) {
  const BlockStart b = bs[L];
  if (b.tile >= n_tiles) return HPos{n_tiles, 0};
  const int k = (int)(((uint32_t)n * (uint32_t)b.off + (uint32_t)b.w - 1u) / (uint32_t)b.w);
  if (k >= n) return HPos{b.tile + 1, 0};
  return HPos{b.tile, k};
}
bool hpos_lt(HPos a, HPos b) { return a.tile < b.tile || (a.tile == b.tile && a.k < b.k); }

// Contributor lists of the split-K shrink for every pool slice (its d_in fixes
// the stage count): per tile, the blocks whose ranges meet it, in block order,
// as {(L << 1) | side, offset of the contribution's partial tile} (side 0: the
// tile is the first of the block's range).  A partial tile holds
// ceil(rank / 16) * ceil(count / 16) * 64 float4 units; the offsets of a slice
// run from 0 to at most part_stride.
void shrink_contributors(lora_plan* pl, int n_tiles, const std::vector<int32_t>& tile_units) {
  const lora_pool* p = pl->pool;
  const int G = pl->G;
  const size_t offn = (size_t)pl->max_tokens + 1;
  pl->h_contrib.assign((size_t)p->n_slices * (offn + 2 * (size_t)pl->contrib_cap), 0);
  pl->part_stride = 0;
  std::vector<std::vector<int32_t>> lists((size_t)n_tiles);
  for (int s = 0; s < p->n_slices; ++s) {
    const int nst = (p->d_in[(size_t)s] + 63) / 64;
    for (auto& l : lists) l.clear();
    HPos a = range_start_host(pl->h_bs.data(), 0, nst, n_tiles);
    for (int L = 0; L < G; ++L) {
      const HPos b = range_start_host(pl->h_bs.data(), L + 1, nst, n_tiles);
      for (int i = a.tile; i < n_tiles && hpos_lt(HPos{i, 0}, b); ++i) {
        const int k0 = i == a.tile ? a.k : 0;
        const int k1 = i == b.tile ? b.k : nst;
        if (k0 < k1) lists[(size_t)i].push_back((L << 1) | (i == a.tile ? 0 : 1));
      }
      a = b;
    }
    int32_t* off = pl->h_contrib.data() + (size_t)s * offn;
    int32_t* ent = pl->h_contrib.data() + (size_t)p->n_slices * offn + (size_t)s * 2 * pl->contrib_cap;
    int32_t pos = 0;
    int64_t units = 0;
    for (int i = 0; i < n_tiles; ++i) {
      off[i] = pos;
      for (int32_t x : lists[(size_t)i]) {
        ent[2 * pos] = x;
        ent[2 * pos + 1] = (int32_t)units;
        units += tile_units[(size_t)i];
        ++pos;
      }
    }
    off[n_tiles] = pos;
    pl->part_stride = std::max(pl->part_stride, units);
  }
}

}  // namespace

namespace lora {
lora_status plan_reserve_part(lora_plan* pl, int n_io) {
  const size_t need = (size_t)n_io * (size_t)pl->part_stride * 4;  // floats
  if (need <= pl->part_cap) return LORA_OK;
  if (pl->d_part) {
    LORA_HIP(hipDeviceSynchronize());  // earlier launches may still use the old buffer
    (void)hipFree(pl->d_part);
    pl->d_part = nullptr;
    pl->part_cap = 0;
  }
  LORA_HIP(hipMalloc((void**)&pl->d_part, sizeof(float) * need));
  pl->part_cap = need;
  return LORA_OK;
}
}  // namespace lora

extern "C" {

lora_status lora_plan_create(lora_pool* pool, int32_t max_tokens, lora_plan** out) {
  clear_error();
  if (!pool || !out || max_tokens <= 0) return fail(LORA_E_ARG, "bad argument");
  *out = nullptr;
  lora_plan* pl = new (std::nothrow) lora_plan();
  if (!pl) return fail(LORA_E_NOMEM, "out of host memory");
  pl->pool = pool;
  pl->max_tokens = max_tokens;
  pl->h_perm.reserve((size_t)max_tokens);
  pl->h_items.reserve((size_t)max_tokens);
  if (!pool->host_only) {
    // persistent MFMA kernels run two blocks per compute unit
    int ncu = 0;
    hipError_t e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, pool->device);
    if (e != hipSuccess || ncu <= 0) {
      lora_plan_destroy(pl);
      return fail(LORA_E_HIP, "plan: compute unit count: %s", hipGetErrorString(e));
    }
    pl->G = ((2 * ncu + 7) / 8) * 8;
    const size_t tok = (size_t)max_tokens;
    pl->contrib_cap = 2 * pl->G + max_tokens + 8;
    const size_t ncontrib = (size_t)pool->n_slices * ((size_t)max_tokens + 1 + 2 * (size_t)pl->contrib_cap);
    const size_t need = sizeof(int32_t) * tok + sizeof(PlanItem) * tok + 256 +
                        sizeof(BlockStart) * 2 * ((size_t)pl->G + 1) + 256 + sizeof(int32_t) * ncontrib + 256;
    e = hipHostMalloc((void**)&pl->h_pinned, need, hipHostMallocDefault);
    if (e == hipSuccess) e = hipMalloc((void**)&pl->d_perm, sizeof(int32_t) * tok);
    if (e == hipSuccess) e = hipMalloc((void**)&pl->d_items, sizeof(PlanItem) * tok);
    if (e == hipSuccess) e = hipMalloc((void**)&pl->d_bs, sizeof(BlockStart) * 2 * ((size_t)pl->G + 1));
    if (pool->dtype != LORA_F32) {  // MFMA tiles exist only on 16-bit pools
      if (e == hipSuccess) e = hipMalloc((void**)&pl->d_contrib, sizeof(int32_t) * ncontrib);
    }
    if (e == hipSuccess) e = hipEventCreateWithFlags(&pl->ev, hipEventDisableTiming);
    if (e != hipSuccess) {
      lora_plan_destroy(pl);
      return fail(LORA_E_HIP, "plan allocation: %s", hipGetErrorString(e));
    }
    pl->pinned_cap = need;
  }
  *out = pl;
  return LORA_OK;
}

lora_status lora_plan_destroy(lora_plan* pl) {
  clear_error();
  if (!pl) return LORA_OK;
  if (pl->ev) {
    (void)hipEventSynchronize(pl->ev);
    (void)hipEventDestroy(pl->ev);
  }
  if (pl->h_pinned) (void)hipHostFree(pl->h_pinned);
  if (pl->d_perm || pl->d_part) (void)hipDeviceSynchronize();  // launches may still read them
  if (pl->d_perm) (void)hipFree(pl->d_perm);
  if (pl->d_items) (void)hipFree(pl->d_items);
  if (pl->d_bs) (void)hipFree(pl->d_bs);
  if (pl->d_part) (void)hipFree(pl->d_part);
  if (pl->d_contrib) (void)hipFree(pl->d_contrib);
  delete pl;
  return LORA_OK;
}

lora_status lora_plan_build(lora_plan* pl, const int32_t* ids, int32_t n, int32_t l_long,
                            void* stream) {
  clear_error();
  if (!pl || (n > 0 && !ids) || n < 0) return fail(LORA_E_ARG, "bad argument");
  if (n > pl->max_tokens) return fail(LORA_E_ARG, "%d tokens exceed plan capacity %d", n, pl->max_tokens);
  lora_pool* p = pl->pool;
  if (l_long <= 0) l_long = 1;  // 16-bit pools: every group runs on MFMA tiles
  const int NA = p->max_adapters;
  // validate and count (bucket NA holds the tokens without an adapter)
  std::vector<int32_t> count((size_t)NA + 1, 0);
  for (int i = 0; i < n; ++i) {
    const int a = ids[i];
    if (a >= NA) return fail(LORA_E_ARG, "token %d: adapter id %d >= max_adapters %d", i, a, NA);
    if (a >= 0) {
      for (int s = 0; s < p->n_slices; ++s)
        if (!p->slot(s, a).rank)
          return fail(LORA_E_NOT_RESIDENT, "token %d: adapter %d is not resident in slice %d", i, a, s);
      ++count[(size_t)a];
    } else {
      ++count[(size_t)NA];
    }
  }
  // stable counting sort -> perm; groups in increasing adapter id, then no-adapter
  std::vector<int32_t> start((size_t)NA + 2, 0);
  for (int a = 0; a <= NA; ++a) start[(size_t)a + 1] = start[(size_t)a] + count[(size_t)a];
  pl->h_perm.assign((size_t)n, 0);
  {
    std::vector<int32_t> cur(start.begin(), start.end() - 1);
    for (int i = 0; i < n; ++i) {
      const int b = ids[i] >= 0 ? ids[i] : NA;
      pl->h_perm[(size_t)cur[(size_t)b]++] = i;
    }
  }
  const bool mfma_ok = (p->dtype != LORA_F32);
  struct Keyed {
    PlanItem it;
    int band;
  };
  std::vector<Keyed> items;
  int groups = 0, mfma_tokens = 0, n_mfma = 0;
  for (int b = 0; b <= NA; ++b) {
    const int L = count[(size_t)b];
    if (!L) continue;
    ++groups;
    const int a = b < NA ? b : -1;
    int rmax = 0;
    if (a >= 0)
      for (int s = 0; s < p->n_slices; ++s) rmax = std::max(rmax, p->slot(s, a).rank);
    const int band = (rmax + 15) / 16;
    const int s0 = start[(size_t)b];
    // MFMA tiles read the A page ids of a tile from LDS (at most kMaxNpa pages
    // per A row) and B rows with wave-uniform page ids (at least 16 B rows per
    // page); other layouts run as short items.
    bool tile_ok = mfma_ok && a >= 0 && p->P / p->rs_of(rmax) >= 16;
    for (int s = 0; s < p->n_slices && tile_ok; ++s) tile_ok = p->npa[(size_t)s] <= kMaxNpa;
    if (tile_ok && L >= l_long) {
      const int nt = (L + kTileM - 1) / kTileM;
      int off = 0;
      for (int t = 0; t < nt; ++t) {
        const int c = L / nt + (t < L % nt ? 1 : 0);
        items.push_back({{a, s0 + off, c, 1}, band});
        off += c;
      }
      n_mfma += nt;
      mfma_tokens += L;
    } else {
      for (int off = 0; off < L; off += kShortG)
        items.push_back({{a, s0 + off, std::min(kShortG, L - off), 0}, band});
    }
  }
  std::stable_sort(items.begin(), items.end(), [](const Keyed& x, const Keyed& y) {
    if (x.it.kind != y.it.kind) return x.it.kind > y.it.kind;
    if (x.band != y.band) return x.band > y.band;
    return x.it.count > y.it.count;
  });
  pl->h_items.clear();
  for (const Keyed& k : items) pl->h_items.push_back(k.it);
  if (pl->G > 0) {
    // Weights of the MFMA tiles (items [0, n_mfma)) per shrink stage and per
    // expand chunk, in 128-byte rows moved: x rows (16 per token block) plus A
    // rows for a shrink stage; y rows read and written plus B rows for an
    // expand chunk; +16 for the fixed per-step cost.
    std::vector<int32_t> ws((size_t)n_mfma), we((size_t)n_mfma), tu((size_t)n_mfma);
    for (int i = 0; i < n_mfma; ++i) {
      const PlanItem& it = pl->h_items[(size_t)i];
      int rmax = 0;
      for (int s = 0; s < p->n_slices; ++s) rmax = std::max(rmax, p->slot(s, it.adapter).rank);
      const int rp = (rmax + 15) / 16 * 16;
      // a stage costs about one memory round trip whatever it moves: a large
      // fixed part plus half the rows
      ws[(size_t)i] = 64 + (16 * ((it.count + 15) / 16) + rp) / 2;
      // an expand chunk: likewise a large fixed part, plus y and B rows
      we[(size_t)i] = 256 + 2 * it.count + p->rs_of(rmax) / 2;
      tu[(size_t)i] = (rp / 16) * ((it.count + 15) / 16) * 64;
    }
    pl->h_bs.assign(2 * ((size_t)pl->G + 1), BlockStart{0, 0, 1, 0});
    balance_blocks(ws, pl->G, pl->h_bs.data());
    balance_blocks(we, pl->G, pl->h_bs.data() + pl->G + 1);
    if (pl->d_contrib) shrink_contributors(pl, n_mfma, tu);
  }
  pl->n_tokens = n;
  pl->n_groups = groups;
  pl->n_items = (int32_t)pl->h_items.size();
  pl->n_mfma = n_mfma;
  pl->mfma_tokens = mfma_tokens;
  pl->l_long = l_long;
  pl->pool_generation = p->generation;
  if (!p->host_only && n > 0) {
    hipStream_t s = (hipStream_t)stream;
    if (pl->ev_pending) LORA_HIP(hipEventSynchronize(pl->ev));  // pinned buffer reuse
    const size_t pb = sizeof(int32_t) * (size_t)n;
    const size_t ioff = (pb + 255) & ~(size_t)255;
    const size_t ib = sizeof(PlanItem) * pl->h_items.size();
    const size_t boff = (ioff + ib + 255) & ~(size_t)255;
    const size_t bb = sizeof(BlockStart) * pl->h_bs.size();
    memcpy(pl->h_pinned, pl->h_perm.data(), pb);
    memcpy(pl->h_pinned + ioff, pl->h_items.data(), ib);
    memcpy(pl->h_pinned + boff, pl->h_bs.data(), bb);
    LORA_HIP(hipMemcpyAsync(pl->d_perm, pl->h_pinned, pb, hipMemcpyHostToDevice, s));
    LORA_HIP(hipMemcpyAsync(pl->d_items, pl->h_pinned + ioff, ib, hipMemcpyHostToDevice, s));
    LORA_HIP(hipMemcpyAsync(pl->d_bs, pl->h_pinned + boff, bb, hipMemcpyHostToDevice, s));
    if (pl->d_contrib && n_mfma > 0) {
      const size_t coff = (boff + bb + 255) & ~(size_t)255;
      const size_t cb = sizeof(int32_t) * pl->h_contrib.size();
      memcpy(pl->h_pinned + coff, pl->h_contrib.data(), cb);
      LORA_HIP(hipMemcpyAsync(pl->d_contrib, pl->h_pinned + coff, cb, hipMemcpyHostToDevice, s));
    }
    LORA_HIP(hipEventRecord(pl->ev, s));
    pl->ev_pending = true;
  }
  pl->built = true;
  return LORA_OK;
}

lora_status lora_plan_get_stats(const lora_plan* pl, lora_plan_stats* out) {
  clear_error();
  if (!pl || !out) return fail(LORA_E_ARG, "null argument");
  out->n_tokens = pl->n_tokens;
  out->n_groups = pl->n_groups;
  out->n_items = pl->n_items;
  out->n_mfma_items = pl->n_mfma;
  out->mfma_tokens = pl->mfma_tokens;
  out->l_long = pl->l_long;
  return LORA_OK;
}

// Host copy of the plan (items as 4 int32 each), for tests of the planner.
lora_status lora_plan_export(const lora_plan* pl, int32_t* perm, int32_t* items4) {
  clear_error();
  if (!pl) return fail(LORA_E_ARG, "null plan");
  if (perm) memcpy(perm, pl->h_perm.data(), sizeof(int32_t) * pl->h_perm.size());
  if (items4) memcpy(items4, pl->h_items.data(), sizeof(PlanItem) * pl->h_items.size());
  return LORA_OK;
}

}  // extern "C"
