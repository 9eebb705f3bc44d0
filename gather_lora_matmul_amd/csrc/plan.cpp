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

#include "layout.h"
#include "runtime.h"

using namespace lora;

static_assert(sizeof(RangePos) == kPosInts * sizeof(int32_t), "device positions are 4 int32");

namespace lora {

// Fused launches of two or more slices leave about this fraction of the
// expand weight (whole tiles at the end of the last slice) to a pool claimed
// by the blocks that finish their ranges first: measured block durations
// spread by 1.1-1.4x around the weights' prediction, which a static split
// cannot absorb.  Only where the MFMA tiles hold at least kPoolMinFill tokens
// on average: pieces of one- or two-token tiles are mostly set-up, and there
// the claims cost more than the balance gains.
constexpr double kExpandPoolFrac = 0.15;
constexpr int kPoolMinFill = 8;

std::vector<int32_t> layout_key(const IoSet& ios) {
  std::vector<int32_t> key;
  key.push_back(ios.n_io);
  for (int j = 0; j < ios.n_io; ++j) {
    key.push_back((ios.io[j].d_in + 63) / 64);
    key.push_back((ios.io[j].d_out + 63) / 64);
  }
  return key;
}

const PlanLayout* plan_find_layout(const lora_plan* pl, const IoSet& ios) {
  const std::vector<int32_t> key = layout_key(ios);
  for (const PlanLayout& l : pl->layouts)
    if (l.valid && l.key == key) {
      const_cast<PlanLayout&>(l).used = ++pl->layout_clock;
      return &l;
    }
  return nullptr;
}

lora_status plan_prepare_layout(lora_plan* pl, const IoSet& ios, hipStream_t s) {
  if (plan_find_layout(pl, ios)) return LORA_OK;
  const int J = ios.n_io;
  const int G = pl->G;
  std::vector<int32_t> nst((size_t)J), nch((size_t)J);
  for (int j = 0; j < J; ++j) {
    nst[(size_t)j] = (ios.io[j].d_in + 63) / 64;
    nch[(size_t)j] = (ios.io[j].d_out + 63) / 64;
  }
  // build into the least recently used slot
  PlanLayout* lay = &pl->layouts[0];
  for (PlanLayout& l : pl->layouts)
    if (!l.valid || l.used < lay->used) lay = &l;
  lay->valid = false;
  LayoutHost h;
  if (!layout_host(pl->h_ws, pl->h_we, pl->h_tu, nst, nch, G, kPieceSetupShrink,
                   kPieceSetupExpand, h, false, J >= 2 && pl->mfma_tokens >= kPoolMinFill * pl->n_mfma ? kExpandPoolFrac : 0.0))
    return fail(LORA_E_ARG, "plan: partial-tile workspace exceeds 2^31 float4 units");
  const std::vector<int32_t>& buf = h.buf;
  const size_t bytes = sizeof(int32_t) * buf.size();
  if (pl->pool->host_only) {  // sizes only: nothing runs on a host-only pool
    lay->key = layout_key(ios);
    lay->part_units = h.part_units;
    lay->pool = h.pool;
    lay->valid = true;
    lay->used = ++pl->layout_clock;
    return LORA_OK;
  }
  if (lay->ev_pending) {  // the staging buffer of this slot may still be copied from
    LORA_HIP(hipEventSynchronize(lay->ev));
    lay->ev_pending = false;
  }
  if (bytes > lay->cap) {
    if (lay->d_buf) {
      LORA_HIP(hipDeviceSynchronize());  // earlier launches may still read it
      (void)hipFree(lay->d_buf);
      lay->d_buf = nullptr;
    }
    if (lay->h_buf) (void)hipHostFree(lay->h_buf);
    lay->h_buf = nullptr;
    lay->cap = 0;
    const size_t cap = bytes + bytes / 2 + 4096;
    LORA_HIP(hipMalloc((void**)&lay->d_buf, cap));
    hipError_t e = hipHostMalloc((void**)&lay->h_buf, cap, hipHostMallocDefault);
    if (e != hipSuccess) {
      (void)hipFree(lay->d_buf);
      lay->d_buf = nullptr;
      return fail(LORA_E_HIP, "plan layout staging: %s", hipGetErrorString(e));
    }
    lay->cap = cap;
  }
  if (!lay->ev) LORA_HIP(hipEventCreateWithFlags(&lay->ev, hipEventDisableTiming));
  memcpy(lay->h_buf, buf.data(), bytes);
  LORA_HIP(hipMemcpyAsync(lay->d_buf, lay->h_buf, bytes, hipMemcpyHostToDevice, s));
  LORA_HIP(hipEventRecord(lay->ev, s));
  lay->ev_pending = true;
  lay->key = layout_key(ios);
  lay->part_units = h.part_units;
  lay->o_bs = h.o_bs;
  lay->o_be = h.o_be;
  lay->o_fl = h.o_fl;
  lay->o_pool = h.o_pool;
  lay->pool = h.pool;
  lay->o_off = h.o_off;
  lay->o_ent = h.o_ent;
  lay->valid = true;
  lay->used = ++pl->layout_clock;
  return LORA_OK;
}

// Launch shape of a prepare / workspace-size call: the slices of io (x and y
// are not read).
lora_status shape_of(const lora_plan* pl, int32_t n_io, const lora_io* io, IoSet& ios) {
  if (!pl || !pl->built) return fail(LORA_E_ARG, "plan not built");
  if (n_io < 1 || n_io > LORA_MAX_IO || !io) return fail(LORA_E_ARG, "n_io must be in [1, %d]", LORA_MAX_IO);
  const lora_pool* p = pl->pool;
  memset(&ios, 0, sizeof(ios));
  ios.n_io = n_io;
  for (int k = 0; k < n_io; ++k) {
    if (io[k].slice < 0 || io[k].slice >= p->n_slices)
      return fail(LORA_E_ARG, "io %d: slice %d out of range", k, io[k].slice);
    ios.io[k] = p->io(io[k].slice, nullptr, nullptr);
  }
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
  // host-only pools (layout tests): the nominal grid of a 256-CU device
  if (pool->host_only) pl->G = 512;
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
    const size_t need = sizeof(int32_t) * tok + sizeof(PlanItem) * tok + 256;
    e = hipHostMalloc((void**)&pl->h_pinned, need, hipHostMallocDefault);
    if (e == hipSuccess) e = hipMalloc((void**)&pl->d_perm, sizeof(int32_t) * tok);
    if (e == hipSuccess) e = hipMalloc((void**)&pl->d_items, sizeof(PlanItem) * tok);
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
  for (PlanLayout& l : pl->layouts)
    if (l.ev) {
      (void)hipEventSynchronize(l.ev);
      (void)hipEventDestroy(l.ev);
    }
  if (pl->h_pinned) (void)hipHostFree(pl->h_pinned);
  if (pl->d_perm) (void)hipDeviceSynchronize();  // launches may still read the plan's buffers
  if (pl->d_perm) (void)hipFree(pl->d_perm);
  if (pl->d_items) (void)hipFree(pl->d_items);
  for (PlanLayout& l : pl->layouts) {
    if (l.d_buf) (void)hipFree(l.d_buf);
    if (l.h_buf) (void)hipHostFree(l.h_buf);
  }
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
  // MFMA tiles for 16-bit pages; fp32 and FP8 pages run as short VALU items
  const bool mfma_ok = (p->dtype == LORA_F16 || p->dtype == LORA_BF16);
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
  {
    // Weights of the MFMA tiles (items [0, n_mfma)) per shrink stage and per
    // expand chunk (each in its own unit, consistent with the per-piece set-up
    // costs of plan_layout), and the size of a partial tile.  The range tables
    // and contributions are built per launch shape (plan_layout); the plan's
    // old ones are dropped here.
    std::vector<int32_t>& ws = pl->h_ws;
    std::vector<int32_t>& we = pl->h_we;
    std::vector<int32_t>& tu = pl->h_tu;
    ws.assign((size_t)n_mfma, 0);
    we.assign((size_t)n_mfma, 0);
    tu.assign((size_t)n_mfma, 0);
    for (PlanLayout& l : pl->layouts) l.valid = false;
    for (int i = 0; i < n_mfma; ++i) {
      const PlanItem& it = pl->h_items[(size_t)i];
      int rmax = 0;
      for (int s = 0; s < p->n_slices; ++s) rmax = std::max(rmax, p->slot(s, it.adapter).rank);
      const TileCost tc = tile_cost(it.count, rmax, p->rs_of(rmax));
      ws[(size_t)i] = tc.ws;
      we[(size_t)i] = tc.we;
      tu[(size_t)i] = tc.tu;
    }
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
    memcpy(pl->h_pinned, pl->h_perm.data(), pb);
    memcpy(pl->h_pinned + ioff, pl->h_items.data(), ib);
    LORA_HIP(hipMemcpyAsync(pl->d_perm, pl->h_pinned, pb, hipMemcpyHostToDevice, s));
    LORA_HIP(hipMemcpyAsync(pl->d_items, pl->h_pinned + ioff, ib, hipMemcpyHostToDevice, s));
    LORA_HIP(hipEventRecord(pl->ev, s));
    pl->ev_pending = true;
  }
  pl->built = true;
  return LORA_OK;
}

lora_status lora_plan_prepare(lora_plan* pl, int32_t n_io, const lora_io* io, void* stream) {
  clear_error();
  IoSet ios;
  lora_status st = shape_of(pl, n_io, io, ios);
  if (st) return st;
  if (pl->n_mfma == 0) return LORA_OK;  // nothing to lay out
  return plan_prepare_layout(pl, ios, (hipStream_t)stream);
}

lora_status lora_workspace_size(const lora_plan* pl, int32_t n_io, const lora_io* io,
                                size_t* bytes) {
  clear_error();
  if (!bytes) return fail(LORA_E_ARG, "null bytes");
  IoSet ios;
  lora_status st = shape_of(pl, n_io, io, ios);
  if (st) return st;
  *bytes = 0;
  if (pl->n_mfma == 0) return LORA_OK;
  const PlanLayout* lay = plan_find_layout(pl, ios);
  if (!lay) return fail(LORA_E_STATE, "launch shape not prepared: call lora_plan_prepare");
  *bytes = 16 * (size_t)lay->part_units;
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
