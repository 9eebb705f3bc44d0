// Unified page pool: free list, adapter upload/evict, page-table build.
//
// One pool of fixed-size pages holds every adapter's rows next to pages owned
// by other users such as KV-cache blocks (S-LoRA paper explainer, "Unified
// Paging"; multi-LoRA serving article, unified paged pool section).  An adapter
// slice occupies whole pages only, so loading and unloading adapters never
// fragments the pool; the only waste is the unused tail of a slice's last page
// of each kind.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "runtime.h"

namespace lora {

static thread_local std::string g_err;

lora_status fail(lora_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}
void clear_error() { g_err.clear(); }

static uint64_t splitmix64(uint64_t& s) {
  uint64_t z = (s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static void fill_pattern(char* dst, size_t bytes, uint32_t pattern, int elt) {
  if (elt == 1) {
    memset(dst, (int)(pattern & 0xffu), bytes);
  } else if (elt == 4) {
    for (size_t i = 0; i + 4 <= bytes; i += 4) memcpy(dst + i, &pattern, 4);
  } else {
    const uint16_t p16 = (uint16_t)pattern;
    for (size_t i = 0; i + 2 <= bytes; i += 2) memcpy(dst + i, &p16, 2);
  }
}

static lora_status ensure_host_stage(lora_pool* p, size_t bytes) {
  if (p->h_stage_cap >= bytes) return LORA_OK;
  if (p->h_stage) {
    if (p->host_only) free(p->h_stage);
    else (void)hipHostFree(p->h_stage);
    p->h_stage = nullptr;
    p->h_stage_cap = 0;
  }
  const size_t cap = std::max<size_t>(bytes, 1 << 20);
  if (p->host_only) {
    p->h_stage = (char*)malloc(cap);
    if (!p->h_stage) return fail(LORA_E_NOMEM, "host staging allocation of %zu bytes failed", cap);
  } else {
    LORA_HIP(hipHostMalloc((void**)&p->h_stage, cap, hipHostMallocDefault));
  }
  p->h_stage_cap = cap;
  return LORA_OK;
}

static lora_status ensure_dev_stage(lora_pool* p, size_t bytes) {
  if (p->d_stage_cap >= bytes) return LORA_OK;
  if (p->d_stage) {
    (void)hipFree(p->d_stage);
    p->d_stage = nullptr;
    p->d_stage_cap = 0;
  }
  const size_t cap = std::max<size_t>(bytes, 1 << 20);
  LORA_HIP(hipMalloc((void**)&p->d_stage, cap));
  p->d_stage_cap = cap;
  return LORA_OK;
}

int64_t pages_of(const lora_pool* p, int slice, int rank) {
  return (int64_t)rank * p->npa[(size_t)slice] + p->npb_of(slice, rank);
}

void pack_slice(const lora_pool* p, int slice, int rank, const void* A, const void* B, char* dst) {
  const int d_in = p->d_in[(size_t)slice], d_out = p->d_out[(size_t)slice], npa = p->npa[(size_t)slice];
  const int rs = p->rs_of(rank), rpp = p->P / rs;
  const size_t data_bytes = (size_t)(pages_of(p, slice, rank) * p->page_bytes);
  // page tails (and A pages past d_in) keep the pool's fill: NaN when poisoned
  if (p->flags & LORA_POOL_POISON) fill_pattern(dst, data_bytes, nan_pattern(p->dtype), p->elt);
  else memset(dst, 0, data_bytes);
  const int elt = p->elt;
  const char* Ab = (const char*)A;
  const char* Bb = (const char*)B;
  for (int k = 0; k < rank; ++k)
    for (int c = 0; c < npa; ++c) {
      const int j0 = c * p->P, j1 = std::min(d_in, j0 + p->P);
      memcpy(dst + ((int64_t)k * npa + c) * p->page_bytes, Ab + ((int64_t)k * d_in + j0) * elt,
             (size_t)(j1 - j0) * elt);
    }
  char* bstg = dst + (int64_t)rank * npa * p->page_bytes;
  for (int m = 0; m < d_out; ++m) {
    char* row = bstg + (int64_t)(m / rpp) * p->page_bytes + (int64_t)(m % rpp) * rs * elt;
    memcpy(row, Bb + (int64_t)m * rank * elt, (size_t)rank * elt);
    memset(row + (size_t)rank * elt, 0, (size_t)(rs - rank) * elt);
  }
}

void reclaim_pages(lora_pool* p) {
  if (p->host_only) return;
  size_t keep = 0;
  for (size_t i = 0; i < p->quarantine.size(); ++i) {
    Quarantine& q = p->quarantine[i];
    if (hipEventQuery(q.ev) == hipSuccess) {
      for (int32_t pg : q.pages) {
        p->state[(size_t)pg] = 0;
        p->free_list.push_back(pg);
      }
      (void)hipEventDestroy(q.ev);
    } else {
      p->quarantine[keep++] = std::move(q);
    }
  }
  p->quarantine.resize(keep);
}

lora_status publish_table(lora_pool* p, hipStream_t upload, hipStream_t compute) {
  std::vector<DevEntry> ent(p->slots.size());
  std::vector<int32_t> ids;
  ids.reserve((size_t)p->n_pages);
  int r_min = 0, r_max = 0;
  for (int s = 0; s < p->n_slices; ++s)
    for (int a = 0; a < p->max_adapters; ++a) {
      const Slot& sl = p->slot(s, a);
      DevEntry& e = ent[(size_t)s * p->max_adapters + a];
      memset(&e, 0, sizeof(e));
      if (!sl.rank) continue;
      r_min = r_min ? std::min(r_min, sl.rank) : sl.rank;
      r_max = std::max(r_max, sl.rank);
      e.rank = sl.rank;
      e.rs = sl.rs;
      e.scale = sl.scale;
      e.rpp = p->P / sl.rs;
      e.inv_rpp = 1.0f / (float)e.rpp;
      e.a_off = (int32_t)ids.size();
      e.b_off = e.a_off + sl.rank * p->npa[s];
      ids.insert(ids.end(), sl.pages.begin(), sl.pages.end());
      if (p->quant()) {  // a_scale, then b_scale, as float bits
        e.q_off = (int32_t)ids.size();
        for (float f : sl.qs) {
          int32_t w;
          memcpy(&w, &f, 4);
          ids.push_back(w);
        }
      }
    }
  if (p->host_only) {
    p->dirty = false;
    return LORA_OK;
  }
  if (ids.size() > p->page_ids_cap)
    return fail(LORA_E_STATE, "page table of %zu words exceeds its %zu", ids.size(), p->page_ids_cap);
  DevTable& t = p->tables[1 - p->cur];
  t.mixed_ranks = r_min != r_max;
  const size_t eb = sizeof(DevEntry) * ent.size();
  const size_t ib = sizeof(int32_t) * ids.size();
  const size_t ioff = (eb + 255) & ~(size_t)255;
  if (t.staged_pending) {  // the last copy out of this staging buffer
    LORA_HIP(hipEventSynchronize(t.staged));
    t.staged_pending = false;
  }
  if (t.h_cap < ioff + ib) {
    if (t.h_stage) (void)hipHostFree(t.h_stage);
    t.h_stage = nullptr;
    t.h_cap = 0;
    const size_t cap = ioff + ib + (ioff + ib) / 4 + 4096;
    LORA_HIP(hipHostMalloc((void**)&t.h_stage, cap, hipHostMallocDefault));
    t.h_cap = cap;
  }
  memcpy(t.h_stage, ent.data(), eb);
  if (ib) memcpy(t.h_stage + ioff, ids.data(), ib);
  // launches that read this buffer before it became inactive must be done
  if (t.retired_pending) LORA_HIP(hipStreamWaitEvent(upload, t.retired, 0));
  LORA_HIP(hipMemcpyAsync(t.entries, t.h_stage, eb, hipMemcpyHostToDevice, upload));
  if (ib) LORA_HIP(hipMemcpyAsync(t.page_ids, t.h_stage + ioff, ib, hipMemcpyHostToDevice, upload));
  LORA_HIP(hipEventRecord(t.staged, upload));
  t.staged_pending = true;
  if (compute != upload) {
    LORA_HIP(hipEventRecord(p->pub_ev, upload));
    LORA_HIP(hipStreamWaitEvent(compute, p->pub_ev, 0));
  }
  // launches enqueued on `compute` so far read the current buffer
  DevTable& old = p->tables[p->cur];
  LORA_HIP(hipEventRecord(old.retired, compute));
  old.retired_pending = true;
  p->cur = 1 - p->cur;
  p->dirty = false;
  return LORA_OK;
}

}  // namespace lora

using namespace lora;

extern "C" {

const char* lora_last_error(void) { return lora::g_err.c_str(); }

lora_status lora_pool_create(const lora_pool_desc* d, lora_pool** out) {
  clear_error();
  if (!d || !out) return fail(LORA_E_ARG, "null argument");
  *out = nullptr;
  if (d->dtype < LORA_F32 || d->dtype > LORA_FP8_E4M3) return fail(LORA_E_ARG, "bad dtype %d", d->dtype);
  const bool quant = d->dtype == LORA_FP8_E4M3;
  if (quant ? (d->act_dtype != LORA_F16 && d->act_dtype != LORA_BF16) : d->act_dtype != d->dtype)
    return fail(LORA_E_ARG, "act_dtype %d: the page dtype, or f16/bf16 for FP8 pages", d->act_dtype);
  const int elt = elt_bytes(d->dtype);
  if (d->page_elems <= 0 || ((int64_t)d->page_elems * elt) % 16 != 0)
    return fail(LORA_E_ARG, "page_elems %d: page size must be a positive multiple of 16 bytes",
                d->page_elems);
  if (d->n_pages <= 0 || d->n_pages >= (1ll << 31)) return fail(LORA_E_ARG, "n_pages out of range");
  if (d->max_adapters <= 0) return fail(LORA_E_ARG, "max_adapters must be positive");
  if (d->max_rank < 1 || d->max_rank > LORA_MAX_RANK)
    return fail(LORA_E_RANK, "max_rank %d outside [1, %d]", d->max_rank, LORA_MAX_RANK);
  if (d->n_slices < 1 || d->n_slices > LORA_MAX_SLICES || !d->slice_d_in || !d->slice_d_out)
    return fail(LORA_E_ARG, "n_slices must be in [1, %d] with dims", LORA_MAX_SLICES);
  const bool host_only = (d->flags & LORA_POOL_HOST_ONLY) != 0;
  if (host_only && d->pages_dev) return fail(LORA_E_ARG, "host-only pool takes no device pages");
  for (int s = 0; s < d->n_slices; ++s) {
    if (d->slice_d_in[s] <= 0 || d->slice_d_out[s] <= 0 || d->slice_d_in[s] % 8 ||
        d->slice_d_out[s] % 8 || d->slice_d_out[s] >= (1 << 20) || d->slice_d_in[s] >= (1 << 24) ||
        (quant && d->slice_d_in[s] % 16))
      return fail(LORA_E_ARG, "slice %d dims %dx%d: need positive multiples of 8 (d_in of 16 on "
                  "FP8 pools), d_out < 2^20", s, d->slice_d_in[s], d->slice_d_out[s]);
  }
  {
    // the largest rank must fit one B row per page
    const int per16 = 16 / elt;
    const int rs = (d->max_rank + per16 - 1) / per16 * per16;
    if (rs > d->page_elems) return fail(LORA_E_RANK, "max_rank %d does not fit a page", d->max_rank);
  }
  lora_pool* p = new (std::nothrow) lora_pool();
  if (!p) return fail(LORA_E_NOMEM, "out of host memory");
  p->P = d->page_elems;
  p->dtype = d->dtype;
  p->act = d->act_dtype;
  p->n_pages = d->n_pages;
  p->max_adapters = d->max_adapters;
  p->max_rank = d->max_rank;
  p->n_slices = d->n_slices;
  p->flags = d->flags;
  p->elt = elt;
  p->page_bytes = (int64_t)p->P * elt;
  p->host_only = host_only;
  for (int s = 0; s < d->n_slices; ++s) {
    p->d_in.push_back(d->slice_d_in[s]);
    p->d_out.push_back(d->slice_d_out[s]);
    p->npa.push_back((d->slice_d_in[s] + p->P - 1) / p->P);
  }
  p->slots.resize((size_t)p->n_slices * p->max_adapters);
  p->state.assign((size_t)p->n_pages, 0);
  // free list: a seeded permutation of the page ids (pages of one adapter end
  // up scattered over the pool, interleaved with other users' pages)
  p->free_list.resize((size_t)p->n_pages);
  for (int64_t i = 0; i < p->n_pages; ++i) p->free_list[(size_t)i] = (int32_t)(p->n_pages - 1 - i);
  if (d->shuffle_seed) {
    uint64_t st = d->shuffle_seed;
    for (int64_t i = p->n_pages - 1; i > 0; --i) {
      const int64_t j = (int64_t)(splitmix64(st) % (uint64_t)(i + 1));
      std::swap(p->free_list[(size_t)i], p->free_list[(size_t)j]);
    }
  }
  const int64_t bytes = p->n_pages * p->page_bytes;
  const bool poison = (d->flags & LORA_POOL_POISON) != 0;
  if (host_only) {
    p->pages = (char*)malloc((size_t)bytes);
    if (!p->pages) {
      delete p;
      return fail(LORA_E_NOMEM, "host pool of %lld bytes", (long long)bytes);
    }
    p->owns_pages = true;
    if (poison) fill_pattern(p->pages, (size_t)bytes, nan_pattern(p->dtype), elt);
    else memset(p->pages, 0, (size_t)bytes);
    *out = p;
    return LORA_OK;
  }
  hipError_t e = hipGetDevice(&p->device);
  if (e == hipSuccess)
    e = hipDeviceGetAttribute(&p->n_cu, hipDeviceAttributeMultiprocessorCount, p->device);
  if (e != hipSuccess || p->n_cu <= 0) {
    delete p;
    return fail(LORA_E_HIP, "device query: %s", hipGetErrorString(e));
  }
  if (d->pages_dev) {
    if ((uintptr_t)d->pages_dev % 256) {
      delete p;
      return fail(LORA_E_ARG, "pages_dev must be 256-byte aligned");
    }
    p->pages = (char*)d->pages_dev;
  } else {
    e = hipMalloc((void**)&p->pages, (size_t)bytes);
    if (e != hipSuccess) {
      delete p;
      return fail(LORA_E_NOMEM, "hipMalloc of %lld pool bytes: %s", (long long)bytes,
                  hipGetErrorString(e));
    }
    p->owns_pages = true;
  }
  {
    const lora_status st = scratch_init(p->device);
    if (st) {
      if (p->owns_pages) (void)hipFree(p->pages);
      delete p;
      return st;
    }
  }
  // page ids of every page, plus (FP8) 2 * max_rank scale words per slot
  p->page_ids_cap = (size_t)p->n_pages + (quant ? 2 * (size_t)p->max_rank * p->slots.size() : 0);
  e = hipEventCreateWithFlags(&p->pub_ev, hipEventDisableTiming);
  for (DevTable& t : p->tables) {
    if (e == hipSuccess) e = hipMalloc((void**)&t.entries, sizeof(DevEntry) * p->slots.size());
    if (e == hipSuccess) e = hipMalloc((void**)&t.page_ids, sizeof(int32_t) * p->page_ids_cap);
    if (e == hipSuccess) e = hipMemset(t.entries, 0, sizeof(DevEntry) * p->slots.size());
    if (e == hipSuccess) e = hipEventCreateWithFlags(&t.staged, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&t.retired, hipEventDisableTiming);
  }
  if (e == hipSuccess && poison) e = launch_fill_all(p->pages, bytes, nan_pattern(p->dtype), elt, nullptr);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    lora_pool_destroy(p);
    return fail(LORA_E_HIP, "pool setup: %s", hipGetErrorString(e));
  }
  *out = p;
  return LORA_OK;
}

lora_status lora_pool_destroy(lora_pool* p) {
  clear_error();
  if (!p) return LORA_OK;
  if (p->host_only) {
    if (p->owns_pages) free(p->pages);
    free(p->h_stage);
  } else {
    (void)hipDeviceSynchronize();
    if (p->owns_pages && p->pages) (void)hipFree(p->pages);
    for (DevTable& t : p->tables) {
      if (t.entries) (void)hipFree(t.entries);
      if (t.page_ids) (void)hipFree(t.page_ids);
      if (t.h_stage) (void)hipHostFree(t.h_stage);
      if (t.staged) (void)hipEventDestroy(t.staged);
      if (t.retired) (void)hipEventDestroy(t.retired);
    }
    for (Quarantine& q : p->quarantine)
      if (q.ev) (void)hipEventDestroy(q.ev);
    if (p->pub_ev) (void)hipEventDestroy(p->pub_ev);
    if (p->d_stage) (void)hipFree(p->d_stage);
    if (p->h_stage) (void)hipHostFree(p->h_stage);
  }
  delete p;
  return LORA_OK;
}

lora_status lora_pool_info(const lora_pool* p, int64_t* free_pages, void** base) {
  clear_error();
  if (!p) return fail(LORA_E_ARG, "null pool");
  reclaim_pages(const_cast<lora_pool*>(p));
  if (free_pages) *free_pages = (int64_t)p->free_list.size();
  if (base) *base = p->pages;
  return LORA_OK;
}

lora_status lora_pool_alloc_pages(lora_pool* p, int64_t n, int32_t* ids) {
  clear_error();
  if (!p || (n > 0 && !ids) || n < 0) return fail(LORA_E_ARG, "bad argument");
  reclaim_pages(p);
  if ((int64_t)p->free_list.size() < n)
    return fail(LORA_E_NOMEM, "%lld pages requested, %zu free", (long long)n, p->free_list.size());
  for (int64_t i = 0; i < n; ++i) {
    ids[i] = p->free_list.back();
    p->free_list.pop_back();
    p->state[(size_t)ids[i]] = 2;
  }
  return LORA_OK;
}

lora_status lora_pool_free_pages(lora_pool* p, int64_t n, const int32_t* ids) {
  clear_error();
  if (!p || (n > 0 && !ids) || n < 0) return fail(LORA_E_ARG, "bad argument");
  std::vector<int32_t> seen;
  for (int64_t i = 0; i < n; ++i) {
    if (ids[i] < 0 || ids[i] >= p->n_pages) return fail(LORA_E_ARG, "page id %d out of range", ids[i]);
    if (p->state[(size_t)ids[i]] != 2)
      return fail(LORA_E_STATE, "page %d is not held by a pool user", ids[i]);
    seen.push_back(ids[i]);
  }
  std::sort(seen.begin(), seen.end());
  if (std::adjacent_find(seen.begin(), seen.end()) != seen.end())
    return fail(LORA_E_STATE, "page listed twice");
  for (int64_t i = 0; i < n; ++i) {
    p->state[(size_t)ids[i]] = 0;
    p->free_list.push_back(ids[i]);
  }
  return LORA_OK;
}

}  // extern "C"

namespace lora {
static lora_status upload_impl(lora_pool* p, int32_t adapter, int32_t slice, int32_t rank,
                               float scale, const void* A, const float* sa, const void* B,
                               const float* sb, void* stream) {
  if (!p || !A || !B) return fail(LORA_E_ARG, "null argument");
  if (adapter < 0 || adapter >= p->max_adapters) return fail(LORA_E_ARG, "adapter %d out of range", adapter);
  if (slice < 0 || slice >= p->n_slices) return fail(LORA_E_ARG, "slice %d out of range", slice);
  if (rank < 1 || rank > p->max_rank) return fail(LORA_E_RANK, "rank %d outside [1, %d]", rank, p->max_rank);
  Slot& sl = p->slot(slice, adapter);
  if (sl.rank) return fail(LORA_E_STATE, "adapter %d slice %d already resident", adapter, slice);
  reclaim_pages(p);
  const int rs = p->rs_of(rank);
  const int64_t need = pages_of(p, slice, rank);
  if ((int64_t)p->free_list.size() < need)
    return fail(LORA_E_NOMEM, "adapter %d slice %d needs %lld pages, %zu free", adapter, slice,
                (long long)need, p->free_list.size());
  const size_t data_bytes = (size_t)(need * p->page_bytes);
  const size_t ids_off = (data_bytes + 255) & ~(size_t)255;
  lora_status st = ensure_host_stage(p, ids_off + sizeof(int32_t) * (size_t)need);
  if (st) return st;
  char* stg = p->h_stage;
  pack_slice(p, slice, rank, A, B, stg);
  // take the pages
  std::vector<int32_t> pages((size_t)need);
  for (int64_t i = 0; i < need; ++i) {
    pages[(size_t)i] = p->free_list.back();
    p->free_list.pop_back();
  }
  auto give_back = [&]() {
    for (int64_t i = need - 1; i >= 0; --i) p->free_list.push_back(pages[(size_t)i]);
  };
  if (p->host_only) {
    for (int64_t i = 0; i < need; ++i)
      memcpy(p->pages + (int64_t)pages[(size_t)i] * p->page_bytes, stg + i * p->page_bytes,
             (size_t)p->page_bytes);
  } else {
    memcpy(stg + ids_off, pages.data(), sizeof(int32_t) * (size_t)need);
    st = ensure_dev_stage(p, ids_off + sizeof(int32_t) * (size_t)need);
    if (st) {
      give_back();
      return st;
    }
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipMemcpyAsync(p->d_stage, stg, ids_off + sizeof(int32_t) * (size_t)need,
                                  hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
      e = launch_scatter_pages(p->pages, p->page_bytes, p->d_stage,
                               (const int32_t*)(p->d_stage + ids_off), need, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
      give_back();
      return fail(LORA_E_HIP, "upload copy: %s", hipGetErrorString(e));
    }
  }
  for (int32_t pg : pages) p->state[(size_t)pg] = 1;
  sl.rank = rank;
  sl.rs = rs;
  sl.scale = scale;
  sl.pages = std::move(pages);
  sl.qs.clear();
  if (p->quant()) {
    sl.qs.assign(sa, sa + rank);
    sl.qs.insert(sl.qs.end(), sb, sb + rank);
  }
  p->dirty = true;
  ++p->generation;
  return LORA_OK;
}
}  // namespace lora

extern "C" {

lora_status lora_pool_upload(lora_pool* p, int32_t adapter, int32_t slice, int32_t rank,
                             float scale, const void* A, const void* B, void* stream) {
  clear_error();
  if (p && p->quant())
    return fail(LORA_E_ARG, "FP8 pool: upload codes with their scales (lora_pool_upload_scaled)");
  return upload_impl(p, adapter, slice, rank, scale, A, nullptr, B, nullptr, stream);
}

lora_status lora_pool_upload_scaled(lora_pool* p, int32_t adapter, int32_t slice, int32_t rank,
                                    float scale, const void* A, const float* a_scale,
                                    const void* B, const float* b_scale, void* stream) {
  clear_error();
  if (!p) return fail(LORA_E_ARG, "null pool");
  if (!p->quant()) return fail(LORA_E_ARG, "scaled upload needs an FP8 pool");
  if (!a_scale || !b_scale) return fail(LORA_E_ARG, "null scale array");
  return upload_impl(p, adapter, slice, rank, scale, A, a_scale, B, b_scale, stream);
}



lora_status lora_pool_evict(lora_pool* p, int32_t adapter, int32_t slice, void* stream) {
  clear_error();
  if (!p) return fail(LORA_E_ARG, "null pool");
  if (adapter < 0 || adapter >= p->max_adapters) return fail(LORA_E_ARG, "adapter %d out of range", adapter);
  if (slice < 0 || slice >= p->n_slices) return fail(LORA_E_ARG, "slice %d out of range", slice);
  Slot& sl = p->slot(slice, adapter);
  if (!sl.rank) return fail(LORA_E_STATE, "adapter %d slice %d is not resident", adapter, slice);
  const int64_t n = (int64_t)sl.pages.size();
  if (p->flags & LORA_POOL_POISON) {
    if (p->host_only) {
      for (int32_t pg : sl.pages)
        fill_pattern(p->pages + (int64_t)pg * p->page_bytes, (size_t)p->page_bytes,
                     nan_pattern(p->dtype), p->elt);
    } else {
      lora_status st = ensure_host_stage(p, sizeof(int32_t) * (size_t)n);
      if (st) return st;
      st = ensure_dev_stage(p, sizeof(int32_t) * (size_t)n);
      if (st) return st;
      memcpy(p->h_stage, sl.pages.data(), sizeof(int32_t) * (size_t)n);
      hipStream_t s = (hipStream_t)stream;
      hipError_t e = hipMemcpyAsync(p->d_stage, p->h_stage, sizeof(int32_t) * (size_t)n,
                                    hipMemcpyHostToDevice, s);
      if (e == hipSuccess)
        e = launch_fill_pages(p->pages, p->page_bytes, (const int32_t*)p->d_stage, n,
                              nan_pattern(p->dtype), p->elt, s);
      if (e == hipSuccess) e = hipStreamSynchronize(s);
      if (e != hipSuccess) return fail(LORA_E_HIP, "evict fill: %s", hipGetErrorString(e));
    }
  }
  for (int64_t i = n - 1; i >= 0; --i) {
    p->state[(size_t)sl.pages[(size_t)i]] = 0;
    p->free_list.push_back(sl.pages[(size_t)i]);
  }
  sl = Slot();
  p->dirty = true;
  ++p->generation;
  return LORA_OK;
}

lora_status lora_page_table_build(lora_pool* p, void* stream) {
  clear_error();
  if (!p) return fail(LORA_E_ARG, "null pool");
  hipStream_t s = (hipStream_t)stream;
  lora_status st = publish_table(p, s, s);
  if (st) return st;
  if (!p->host_only) LORA_HIP(hipStreamSynchronize(s));
  return LORA_OK;
}

lora_status lora_pool_export_entry(const lora_pool* p, int32_t adapter, int32_t slice,
                                   int32_t* rank, float* scale, int32_t* n_a, int32_t* a_pages,
                                   int32_t* n_b, int32_t* b_pages) {
  clear_error();
  if (!p) return fail(LORA_E_ARG, "null pool");
  if (adapter < 0 || adapter >= p->max_adapters) return fail(LORA_E_ARG, "adapter %d out of range", adapter);
  if (slice < 0 || slice >= p->n_slices) return fail(LORA_E_ARG, "slice %d out of range", slice);
  const Slot& sl = p->slot(slice, adapter);
  const int na = sl.rank * p->npa[slice];
  const int nb = sl.rank ? p->npb_of(slice, sl.rank) : 0;
  if (rank) *rank = sl.rank;
  if (scale) *scale = sl.scale;
  if (n_a) *n_a = na;
  if (n_b) *n_b = nb;
  if (a_pages && na) memcpy(a_pages, sl.pages.data(), sizeof(int32_t) * (size_t)na);
  if (b_pages && nb) memcpy(b_pages, sl.pages.data() + na, sizeof(int32_t) * (size_t)nb);
  return LORA_OK;
}

lora_status lora_pool_export_scales(const lora_pool* p, int32_t adapter, int32_t slice,
                                    float* a_scale, float* b_scale) {
  clear_error();
  if (!p) return fail(LORA_E_ARG, "null pool");
  if (!p->quant()) return fail(LORA_E_ARG, "pool is not FP8: no scales");
  if (adapter < 0 || adapter >= p->max_adapters) return fail(LORA_E_ARG, "adapter %d out of range", adapter);
  if (slice < 0 || slice >= p->n_slices) return fail(LORA_E_ARG, "slice %d out of range", slice);
  const Slot& sl = p->slot(slice, adapter);
  if (!sl.rank) return fail(LORA_E_NOT_RESIDENT, "adapter %d slice %d is not resident", adapter, slice);
  if (a_scale) memcpy(a_scale, sl.qs.data(), sizeof(float) * (size_t)sl.rank);
  if (b_scale) memcpy(b_scale, sl.qs.data() + sl.rank, sizeof(float) * (size_t)sl.rank);
  return LORA_OK;
}

lora_status lora_pool_read_pages(const lora_pool* p, int64_t first, int64_t count, void* dst) {
  clear_error();
  if (!p || (count > 0 && !dst)) return fail(LORA_E_ARG, "null argument");
  if (first < 0 || count < 0 || first + count > p->n_pages) return fail(LORA_E_ARG, "page range out of bounds");
  const size_t bytes = (size_t)(count * p->page_bytes);
  if (p->host_only) {
    memcpy(dst, p->pages + first * p->page_bytes, bytes);
  } else {
    LORA_HIP(hipMemcpy(dst, p->pages + first * p->page_bytes, bytes, hipMemcpyDeviceToHost));
  }
  return LORA_OK;
}

}  // extern "C"
