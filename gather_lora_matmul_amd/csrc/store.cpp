// Host adapter store and on-demand residency.
//
// Every adapter lives in host memory; its pages are loaded into the unified
// pool when a batch needs it, and the least recently used adapters go back out
// when pages run short (S-LoRA paper explainer, "Unified Paging").  Loads run
// on a dedicated upload stream so they overlap the compute already enqueued
// (multi-LoRA serving article, unified paged pool section: prefetch over PCIe
// on dedicated streams).
//
// The store keeps each registered adapter slice as ready-made page images in
// pinned host memory, so a load is a DMA into a device staging area (slices
// registered one after the other go out as one copy) and one scatter kernel
// per batch.  Ordering, all on the GPU streams
// (the host never waits for the compute stream):
//   upload stream:  ids -> staging; slices bound for free pages -> staging;
//                   scatter | [if pages were evicted: wait for the compute
//                   stream to pass the eviction point; slices bound for the
//                   evicted pages; scatter; NaN refill of evicted pages not
//                   reused] | new page table into the inactive table buffer
//   compute stream: waits for the new table; launches enqueued after the call
//                   read it, launches enqueued before it keep the old one.
#include <algorithm>
#include <cstring>

#include "runtime.h"

using namespace lora;

namespace {

// Pinned host memory handed out in large chunks (one registration per slice
// would pin thousands of small buffers).
struct PinnedArena {
  std::vector<char*> chunks;
  size_t used = 0;  // bytes used in the last chunk
  size_t chunk_bytes = 0;
  static constexpr size_t kChunk = size_t(64) << 20;

  char* take(size_t bytes, lora_status* st) {
    bytes = (bytes + 255) & ~size_t(255);
    if (chunks.empty() || used + bytes > chunk_bytes) {
      const size_t cap = std::max(kChunk, bytes);
      char* c = nullptr;
      const hipError_t e = hipHostMalloc((void**)&c, cap, hipHostMallocDefault);
      if (e != hipSuccess) {
        *st = fail(LORA_E_NOMEM, "pinned host store: %s", hipGetErrorString(e));
        return nullptr;
      }
      chunks.push_back(c);
      used = 0;
      chunk_bytes = cap;
    }
    char* p = chunks.back() + used;
    used += bytes;
    return p;
  }
  void release() {
    for (char* c : chunks) (void)hipHostFree(c);
    chunks.clear();
  }
};

struct StoredSlice {
  int32_t rank = 0;  // 0: not registered
  float scale = 0.f;
  std::vector<float> qs;   // FP8 pools: a_scale, then b_scale
  const char* image = nullptr;  // pinned page images (pages_of(slice, rank) pages)
  int64_t npages = 0;
};

}  // namespace

struct lora_store {
  lora_pool* pool = nullptr;
  std::vector<StoredSlice> slices;  // [slice * max_adapters + adapter]
  std::vector<uint64_t> last_use;   // per adapter: clock of the last ensure naming it
  uint64_t clock = 0;
  PinnedArena arena;
  // staging of one ensure: device page images + page ids, pinned ids
  char* d_stage = nullptr;
  size_t d_cap = 0;
  int32_t* h_ids = nullptr;
  size_t h_ids_cap = 0;  // int32 words
  hipEvent_t done = nullptr;  // the last ensure's copies and scatters are complete
  bool done_pending = false;
  hipEvent_t retire = nullptr;  // compute stream passed an eviction point
  lora_store_stats st{};
  StoredSlice& at(int slice, int adapter) { return slices[(size_t)slice * pool->max_adapters + adapter]; }
};

namespace {

bool registered(lora_store* s, int a) {
  for (int sl = 0; sl < s->pool->n_slices; ++sl)
    if (!s->at(sl, a).rank) return false;
  return true;
}
bool resident(const lora_pool* p, int a) {
  for (int sl = 0; sl < p->n_slices; ++sl)
    if (!p->slot(sl, a).rank) return false;
  return true;
}
bool any_resident(const lora_pool* p, int a) {
  for (int sl = 0; sl < p->n_slices; ++sl)
    if (p->slot(sl, a).rank) return true;
  return false;
}

// One slice load: its image goes to the pool pages `pages`; into_evicted:
// some of them were freed by this call's evictions.
struct Load {
  int adapter, slice;
  std::vector<int32_t> pages;
  bool into_evicted;
};

}  // namespace

extern "C" {

lora_status lora_store_create(lora_pool* pool, lora_store** out) {
  clear_error();
  if (!pool || !out) return fail(LORA_E_ARG, "null argument");
  if (pool->host_only) return fail(LORA_E_STATE, "a store needs a device pool");
  *out = nullptr;
  lora_store* s = new (std::nothrow) lora_store();
  if (!s) return fail(LORA_E_NOMEM, "out of host memory");
  s->pool = pool;
  s->slices.resize((size_t)pool->n_slices * pool->max_adapters);
  s->last_use.assign((size_t)pool->max_adapters, 0);
  hipError_t e = hipEventCreateWithFlags(&s->done, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&s->retire, hipEventDisableTiming);
  if (e != hipSuccess) {
    lora_store_destroy(s);
    return fail(LORA_E_HIP, "store events: %s", hipGetErrorString(e));
  }
  *out = s;
  return LORA_OK;
}

lora_status lora_store_destroy(lora_store* s) {
  clear_error();
  if (!s) return LORA_OK;
  if (s->done_pending) (void)hipEventSynchronize(s->done);
  if (s->d_stage) (void)hipFree(s->d_stage);
  if (s->h_ids) (void)hipHostFree(s->h_ids);
  if (s->done) (void)hipEventDestroy(s->done);
  if (s->retire) (void)hipEventDestroy(s->retire);
  s->arena.release();
  delete s;
  return LORA_OK;
}

lora_status lora_store_add(lora_store* s, int32_t adapter, int32_t slice, int32_t rank, float scale,
                           const void* A, const float* a_scale, const void* B,
                           const float* b_scale) {
  clear_error();
  if (!s || !A || !B) return fail(LORA_E_ARG, "null argument");
  lora_pool* p = s->pool;
  if (adapter < 0 || adapter >= p->max_adapters) return fail(LORA_E_ARG, "adapter %d out of range", adapter);
  if (slice < 0 || slice >= p->n_slices) return fail(LORA_E_ARG, "slice %d out of range", slice);
  if (rank < 1 || rank > p->max_rank) return fail(LORA_E_RANK, "rank %d outside [1, %d]", rank, p->max_rank);
  if (p->quant() != (a_scale && b_scale))
    return fail(LORA_E_ARG, p->quant() ? "FP8 pool: scales required" : "scales need an FP8 pool");
  StoredSlice& ss = s->at(slice, adapter);
  if (ss.rank) return fail(LORA_E_STATE, "adapter %d slice %d already registered", adapter, slice);
  const int64_t np = pages_of(p, slice, rank);
  lora_status st = LORA_OK;
  char* img = s->arena.take((size_t)(np * p->page_bytes), &st);
  if (!img) return st;
  pack_slice(p, slice, rank, A, B, img);
  ss.rank = rank;
  ss.scale = scale;
  ss.image = img;
  ss.npages = np;
  ss.qs.clear();
  if (p->quant()) {
    ss.qs.assign(a_scale, a_scale + rank);
    ss.qs.insert(ss.qs.end(), b_scale, b_scale + rank);
  }
  return LORA_OK;
}

lora_status lora_store_ensure(lora_store* s, int32_t n, const int32_t* adapters, void* upload_stream,
                              void* compute_stream) {
  clear_error();
  if (!s || n < 0 || (n > 0 && !adapters)) return fail(LORA_E_ARG, "bad argument");
  lora_pool* p = s->pool;
  hipStream_t up = (hipStream_t)upload_stream, cs = (hipStream_t)compute_stream;
  const int NA = p->max_adapters;
  // the request: distinct registered adapters (negative ids: no adapter)
  std::vector<char> want((size_t)NA, 0);
  std::vector<int> req;
  for (int i = 0; i < n; ++i) {
    const int a = adapters[i];
    if (a < 0) continue;
    if (a >= NA) return fail(LORA_E_ARG, "adapter %d out of range", a);
    if (want[(size_t)a]) continue;
    if (!resident(p, a)) {
      if (!registered(s, a)) return fail(LORA_E_NOT_RESIDENT, "adapter %d is not in the store", a);
      if (any_resident(p, a))
        return fail(LORA_E_STATE, "adapter %d is partly resident outside the store", a);
    }
    want[(size_t)a] = 1;
    req.push_back(a);
  }
  ++s->clock;
  // slices to load and the pages they need
  std::vector<std::pair<int, int>> todo;  // (adapter, slice)
  int64_t need = 0;
  for (int a : req)
    if (!resident(p, a))
      for (int sl = 0; sl < p->n_slices; ++sl) {
        todo.push_back({a, sl});
        need += s->at(sl, a).npages;
      }
  reclaim_pages(p);
  int64_t have = (int64_t)p->free_list.size();
  // eviction candidates: store adapters resident in full, not requested, least
  // recently used first
  std::vector<int> victims;
  if (have < need) {
    std::vector<int> cand;
    for (int a = 0; a < NA; ++a)
      if (!want[(size_t)a] && registered(s, a) && resident(p, a)) cand.push_back(a);
    std::sort(cand.begin(), cand.end(), [&](int x, int y) {
      return s->last_use[(size_t)x] < s->last_use[(size_t)y] ||
             (s->last_use[(size_t)x] == s->last_use[(size_t)y] && x < y);
    });
    int64_t gain = 0;
    for (int a : cand) {
      if (have + gain >= need) break;
      victims.push_back(a);
      for (int sl = 0; sl < p->n_slices; ++sl) gain += (int64_t)p->slot(sl, a).pages.size();
    }
    if (have + gain < need) {
      // pages still retiring from earlier evictions: wait for them
      for (Quarantine& q : p->quarantine) LORA_HIP(hipEventSynchronize(q.ev));
      reclaim_pages(p);
      have = (int64_t)p->free_list.size();
      if (have + gain < need)
        return fail(LORA_E_NOMEM, "request needs %lld pages: %lld free, %lld evictable",
                    (long long)need, (long long)have, (long long)gain);
    }
  }
  // staging of the previous ensure may still be in use
  if (s->done_pending) {
    LORA_HIP(hipEventSynchronize(s->done));
    s->done_pending = false;
  }
  // host and device staging for this call, sized before any pool state
  // changes (a failed allocation leaves the pool as it was): page ids of every
  // load (free pages first, then evicted ones) and of the evicted pages no load
  // takes, and the page images of every load
  int64_t gain_pages = 0;
  for (int a : victims)
    for (int sl = 0; sl < p->n_slices; ++sl) gain_pages += (int64_t)p->slot(sl, a).pages.size();
  const int64_t from_evicted = std::max<int64_t>(0, need - (int64_t)p->free_list.size());
  const int64_t n_ids = need + (gain_pages - from_evicted);
  if ((size_t)n_ids > s->h_ids_cap) {
    if (s->h_ids) (void)hipHostFree(s->h_ids);
    s->h_ids = nullptr;
    s->h_ids_cap = 0;
    const size_t cap = (size_t)n_ids + (size_t)n_ids / 2 + 1024;
    const hipError_t e = hipHostMalloc((void**)&s->h_ids, cap * sizeof(int32_t), hipHostMallocDefault);
    if (e != hipSuccess) {
      s->h_ids = nullptr;
      return fail(LORA_E_NOMEM, "pinned staging of %zu page ids: %s", cap, hipGetErrorString(e));
    }
    s->h_ids_cap = cap;
  }
  const size_t img_bytes = (size_t)(need * p->page_bytes);
  const size_t ids_off = (img_bytes + 255) & ~size_t(255);
  const size_t stage_bytes = ids_off + sizeof(int32_t) * (size_t)std::max<int64_t>(n_ids, 1);
  if (stage_bytes > s->d_cap) {
    if (s->d_stage) (void)hipFree(s->d_stage);  // the last ensure's use of it has completed
    s->d_stage = nullptr;
    s->d_cap = 0;
    const size_t cap = stage_bytes + stage_bytes / 4 + (1 << 20);
    const hipError_t e = hipMalloc((void**)&s->d_stage, cap);
    if (e != hipSuccess) {
      s->d_stage = nullptr;
      return fail(LORA_E_NOMEM, "device staging of %zu bytes: %s", cap, hipGetErrorString(e));
    }
    s->d_cap = cap;
  }
  // evict (host state): their pages become this call's second pool of pages
  std::vector<int32_t> evicted;
  for (int a : victims)
    for (int sl = 0; sl < p->n_slices; ++sl) {
      Slot& slot = p->slot(sl, a);
      evicted.insert(evicted.end(), slot.pages.begin(), slot.pages.end());
      slot = Slot();
      ++s->st.evictions;
    }
  // assign pages: free pages first (loads that need not wait), then evicted
  std::vector<Load> loads;
  int64_t stage_pages = 0;
  size_t ev_next = 0;
  for (auto [a, sl] : todo) {
    const StoredSlice& ss = s->at(sl, a);
    Load ld{a, sl, {}, false};
    for (int64_t i = 0; i < ss.npages; ++i) {
      if (!p->free_list.empty()) {
        ld.pages.push_back(p->free_list.back());
        p->free_list.pop_back();
      } else {
        ld.pages.push_back(evicted[ev_next++]);
        ld.into_evicted = true;
      }
    }
    stage_pages += ss.npages;
    loads.push_back(std::move(ld));
  }
  // (loads into free pages come first: pages are assigned in that order)
  std::vector<int32_t> leftover(evicted.begin() + (ptrdiff_t)ev_next, evicted.end());
  // ids: [free loads' pages | evicted loads' pages | leftover evicted pages]
  int64_t k = 0, n_free_pages = 0;
  for (const Load& ld : loads) {
    for (int32_t pg : ld.pages) s->h_ids[k++] = pg;
    if (!ld.into_evicted) n_free_pages += (int64_t)ld.pages.size();
  }
  for (int32_t pg : leftover) s->h_ids[k++] = pg;
  if (k != n_ids || stage_pages != need)
    return fail(LORA_E_STATE, "internal: %lld page ids staged, %lld expected", (long long)k,
                (long long)n_ids);
  const int32_t* d_ids = (const int32_t*)(s->d_stage + ids_off);
  if (n_ids > 0)
    LORA_HIP(hipMemcpyAsync(s->d_stage + ids_off, s->h_ids, sizeof(int32_t) * (size_t)n_ids,
                            hipMemcpyHostToDevice, up));
  // (1) loads into free pages.  Images of slices registered one after the
  // other are adjacent in the pinned store, as are their staging places:
  // adjacent loads go out as one copy.
  int64_t staged = 0;
  const char* run_src = nullptr;
  char* run_dst = nullptr;
  size_t run_bytes = 0;
  auto flush = [&]() -> lora_status {
    if (run_bytes) LORA_HIP(hipMemcpyAsync(run_dst, run_src, run_bytes, hipMemcpyHostToDevice, up));
    run_bytes = 0;
    return LORA_OK;
  };
  auto copy_load = [&](const Load& ld) -> lora_status {
    const StoredSlice& ss = s->at(ld.slice, ld.adapter);
    const size_t bytes = (size_t)(ss.npages * p->page_bytes);
    char* dst = s->d_stage + staged * p->page_bytes;
    if (run_bytes && ss.image == run_src + run_bytes && dst == run_dst + run_bytes) {
      run_bytes += bytes;
    } else {
      lora_status st = flush();
      if (st) return st;
      run_src = ss.image;
      run_dst = dst;
      run_bytes = bytes;
    }
    staged += ss.npages;
    return LORA_OK;
  };
  size_t li = 0;
  for (; li < loads.size() && !loads[li].into_evicted; ++li) {
    lora_status st = copy_load(loads[li]);
    if (st) return st;
  }
  {
    lora_status st = flush();
    if (st) return st;
  }
  if (n_free_pages > 0)
    LORA_HIP(launch_scatter_pages(p->pages, p->page_bytes, s->d_stage, d_ids, n_free_pages, up));
  // (2) loads into evicted pages, after the compute stream has passed this point
  if (!evicted.empty()) {
    LORA_HIP(hipEventRecord(s->retire, cs));
    LORA_HIP(hipStreamWaitEvent(up, s->retire, 0));
    const int64_t first = staged;
    for (; li < loads.size(); ++li) {
      lora_status st = copy_load(loads[li]);
      if (st) return st;
    }
    {
      lora_status st = flush();
      if (st) return st;
    }
    if (staged > first)
      LORA_HIP(launch_scatter_pages(p->pages, p->page_bytes, s->d_stage + first * p->page_bytes,
                                    d_ids + first, staged - first, up));
    if (!leftover.empty()) {
      if (p->flags & LORA_POOL_POISON)
        LORA_HIP(launch_fill_pages(p->pages, p->page_bytes, d_ids + staged, (int64_t)leftover.size(),
                                   nan_pattern(p->dtype), p->elt, up));
      Quarantine q;
      q.pages = leftover;
      for (int32_t pg : leftover) p->state[(size_t)pg] = 3;
      LORA_HIP(hipEventCreateWithFlags(&q.ev, hipEventDisableTiming));
      LORA_HIP(hipEventRecord(q.ev, up));
      p->quarantine.push_back(std::move(q));
    }
  }
  LORA_HIP(hipEventRecord(s->done, up));
  s->done_pending = true;
  // host state of the loaded slices
  for (Load& ld : loads) {
    const StoredSlice& ss = s->at(ld.slice, ld.adapter);
    Slot& slot = p->slot(ld.slice, ld.adapter);
    for (int32_t pg : ld.pages) p->state[(size_t)pg] = 1;
    slot.rank = ss.rank;
    slot.rs = p->rs_of(ss.rank);
    slot.scale = ss.scale;
    slot.pages = std::move(ld.pages);
    slot.qs = ss.qs;
    ++s->st.uploads;
    s->st.bytes_uploaded += ss.npages * p->page_bytes;
  }
  for (int a : req) s->last_use[(size_t)a] = s->clock;
  if (!loads.empty() || !victims.empty()) {
    ++p->generation;
    p->dirty = true;
  }
  // (3) the new page table, ordered after the loads; compute waits for it
  if (p->dirty) return publish_table(p, up, cs);
  return LORA_OK;
}

lora_status lora_store_get_stats(const lora_store* s, lora_store_stats* out) {
  clear_error();
  if (!s || !out) return fail(LORA_E_ARG, "null argument");
  *out = s->st;
  out->resident = 0;
  out->registered = 0;
  for (int a = 0; a < s->pool->max_adapters; ++a) {
    if (registered(const_cast<lora_store*>(s), a)) ++out->registered;
    if (resident(s->pool, a)) ++out->resident;
  }
  return LORA_OK;
}

}  // extern "C"
