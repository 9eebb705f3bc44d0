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
    const size_t need = sizeof(int32_t) * (size_t)max_tokens + sizeof(PlanItem) * (size_t)max_tokens + 256;
    hipError_t e = hipHostMalloc((void**)&pl->h_pinned, need, hipHostMallocDefault);
    if (e == hipSuccess) e = hipMalloc((void**)&pl->d_perm, sizeof(int32_t) * (size_t)max_tokens);
    if (e == hipSuccess) e = hipMalloc((void**)&pl->d_items, sizeof(PlanItem) * (size_t)max_tokens);
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
  if (pl->d_perm) (void)hipFree(pl->d_perm);
  if (pl->d_items) (void)hipFree(pl->d_items);
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
    if (a >= 0 && mfma_ok && L >= l_long) {
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
    memcpy(pl->h_pinned, pl->h_perm.data(), pb);
    memcpy(pl->h_pinned + ioff, pl->h_items.data(), sizeof(PlanItem) * pl->h_items.size());
    LORA_HIP(hipMemcpyAsync(pl->d_perm, pl->h_pinned, pb, hipMemcpyHostToDevice, s));
    LORA_HIP(hipMemcpyAsync(pl->d_items, pl->h_pinned + ioff, sizeof(PlanItem) * pl->h_items.size(),
                            hipMemcpyHostToDevice, s));
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
