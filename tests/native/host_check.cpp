// Host paths of the library under AddressSanitizer / UndefinedBehaviorSanitizer
// (built with g++ by tests/test_sanitizers.py; no GPU): host-only pools of
// every dtype, uploads of odd ranks and ragged shapes, KV pages, eviction,
// page-table builds, plans over seeded id vectors, launch-shape preparation,
// workspace sizes and every error path reachable without a device.  The
// device kernels are replaced by stubs that fail: a host-only pool never
// launches one, and a call that tried would fail the check.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "devplan.h"
#include "lora_internal.h"

namespace lora {
static int g_launches = 0;
#define STUB(...) \
  {               \
    ++g_launches; \
    return hipErrorNotSupported; \
  }
hipError_t launch_fill_pages(char*, int64_t, const int32_t*, int64_t, uint32_t, int, hipStream_t) STUB()
hipError_t launch_fill_all(char*, int64_t, uint32_t, int, hipStream_t) STUB()
hipError_t launch_scatter_pages(char*, int64_t, const char*, const int32_t*, int64_t, hipStream_t) STUB()
hipError_t launch_bgmv_shrink(const Types&, const PoolView&, const IoDesc&, const int32_t*, int32_t,
                              float*, int32_t, hipStream_t) STUB()
hipError_t launch_bgmv_expand(const Types&, const PoolView&, const IoDesc&, const float*, int32_t,
                              const int32_t*, int32_t, const float*, hipStream_t) STUB()
hipError_t launch_bgmv_apply(const Types&, const PoolView&, const IoSet&, const int32_t*, int32_t,
                             hipStream_t) STUB()
hipError_t read_block_timeline(void*, size_t) STUB()
hipError_t launch_sgmv_shrink(const Types&, const PoolView&, const PlanView&, const IoDesc&, float*,
                              int32_t, hipStream_t) STUB()
hipError_t launch_sgmv_expand(const Types&, const PoolView&, const PlanView&, const IoDesc&,
                              const float*, int32_t, hipStream_t) STUB()
hipError_t launch_apply(const Types&, const PoolView&, const PlanView&, const IoSet&, hipStream_t) STUB()
hipError_t launch_devplan_apply(const Types&, const PoolView&, const IoSet&, const int32_t*,
                                const DevPlanShape&, const DevPlanWs&, char*, hipStream_t) STUB()
hipError_t launch_devplan(const PoolView&, const int32_t*, const DevPlanShape&, const DevPlanWs&,
                          char*, hipStream_t) STUB()
hipError_t launch_devplan_mfma(const Types&, const PoolView&, const IoSet&, const DevPlanShape&,
                               const DevPlanWs&, char*, hipStream_t) STUB()
hipError_t launch_debug_decode(int, const void*, int64_t, float*, hipStream_t) STUB()
hipError_t launch_debug_resolve(const PoolView&, const IoDesc&, int32_t, int, const int32_t*, int32_t,
                                int64_t*, int64_t*, hipStream_t) STUB()
hipError_t launch_debug_gather(int, const PoolView&, const IoDesc&, int32_t, int32_t, void*, void*,
                               hipStream_t) STUB()
lora_status scratch_init(int) {
  ++g_launches;
  return LORA_E_UNSUPPORTED;
}
}  // namespace lora

static int g_bad = 0;
#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      ++g_bad;                                                       \
      printf("FAIL %s:%d: %s (%s)\n", __FILE__, __LINE__, #cond, lora_last_error()); \
    }                                                                \
  } while (0)

static int elt_of(int dt) { return dt == LORA_F32 ? 4 : (dt == LORA_FP8_E4M3 ? 1 : 2); }

static void one_case(std::mt19937& rng, int dt, int P, int d_in, int d_out, int n_slices,
                     int n_adapters) {
  const int elt = elt_of(dt);
  std::vector<int32_t> din(n_slices, d_in), dout(n_slices, d_out);
  const int max_rank = std::min(128, P * elt / 16 * 16 / elt);
  lora_pool_desc d;
  memset(&d, 0, sizeof(d));
  d.page_elems = P;
  d.dtype = dt;
  d.n_pages = 4096;
  d.max_adapters = n_adapters;
  d.max_rank = max_rank;
  d.n_slices = n_slices;
  d.slice_d_in = din.data();
  d.slice_d_out = dout.data();
  d.shuffle_seed = rng();
  d.flags = LORA_POOL_HOST_ONLY | LORA_POOL_POISON;
  d.act_dtype = dt == LORA_FP8_E4M3 ? (int)(LORA_F16 + rng() % 2) : dt;
  lora_pool* pool = nullptr;
  CHECK(lora_pool_create(&d, &pool) == LORA_OK);
  if (!pool) return;
  std::vector<int> rank(n_adapters);
  for (int a = 0; a < n_adapters; ++a) {
    rank[a] = 1 + (int)(rng() % (unsigned)max_rank);
    std::vector<char> A((size_t)rank[a] * d_in * elt), B((size_t)d_out * rank[a] * elt);
    for (auto& c : A) c = (char)(rng() & 0x3f);
    for (auto& c : B) c = (char)(rng() & 0x3f);
    std::vector<float> sa(rank[a], 0.25f), sb(rank[a], 2.0f);
    int up = 0;
    for (; up < n_slices; ++up) {
      const lora_status st =
          dt == LORA_FP8_E4M3
              ? lora_pool_upload_scaled(pool, a, up, rank[a], 0.5f, A.data(), sa.data(), B.data(),
                                        sb.data(), nullptr)
              : lora_pool_upload(pool, a, up, rank[a], 0.5f, A.data(), B.data(), nullptr);
      CHECK(st == LORA_OK || st == LORA_E_NOMEM);
      if (st != LORA_OK) break;
    }
    if (up < n_slices) {  // the pool is full: take the adapter out again
      for (int s = 0; s < up; ++s) CHECK(lora_pool_evict(pool, a, s, nullptr) == LORA_OK);
      rank[a] = 0;
    }
    if (rng() % 3 == 0) {  // KV users between adapters
      int32_t ids[7];
      if (lora_pool_alloc_pages(pool, 7, ids) == LORA_OK) {
        CHECK(lora_pool_free_pages(pool, 7, ids) == LORA_OK);
        CHECK(lora_pool_free_pages(pool, 1, ids) == LORA_E_STATE);
      }
    }
  }
  CHECK(lora_page_table_build(pool, nullptr) == LORA_OK);
  // exported entries: page lists of the documented sizes, all distinct
  std::vector<char> seen((size_t)d.n_pages, 0);
  for (int s = 0; s < n_slices; ++s)
    for (int a = 0; a < n_adapters; ++a) {
      int32_t r = -1, na = -1, nb = -1;
      float sc = 0;
      CHECK(lora_pool_export_entry(pool, a, s, &r, &sc, &na, nullptr, &nb, nullptr) == LORA_OK);
      std::vector<int32_t> ap((size_t)std::max(na, 0) + 1), bp((size_t)std::max(nb, 0) + 1);
      CHECK(lora_pool_export_entry(pool, a, s, nullptr, nullptr, nullptr, ap.data(), nullptr,
                                   bp.data()) == LORA_OK);
      for (int i = 0; i < na; ++i) {
        CHECK(ap[i] >= 0 && ap[i] < d.n_pages && !seen[ap[i]]);
        if (ap[i] >= 0 && ap[i] < d.n_pages) seen[ap[i]] = 1;
      }
      for (int i = 0; i < nb; ++i) {
        CHECK(bp[i] >= 0 && bp[i] < d.n_pages && !seen[bp[i]]);
        if (bp[i] >= 0 && bp[i] < d.n_pages) seen[bp[i]] = 1;
      }
      if (dt == LORA_FP8_E4M3 && r > 0) {
        std::vector<float> qa((size_t)r), qb((size_t)r);
        CHECK(lora_pool_export_scales(pool, a, s, qa.data(), qb.data()) == LORA_OK);
        for (int k = 0; k < r; ++k) CHECK(qa[k] == 0.25f && qb[k] == 2.0f);
      }
    }
  std::vector<char> img((size_t)d.n_pages * P * elt);
  CHECK(lora_pool_read_pages(pool, 0, d.n_pages, img.data()) == LORA_OK);
  CHECK(lora_pool_read_pages(pool, 1, d.n_pages, img.data()) == LORA_E_ARG);
  // plans over seeded id vectors (some ids -1, some repeated, some long groups)
  for (int trial = 0; trial < 6; ++trial) {
    const int n = 1 + (int)(rng() % 600);
    std::vector<int32_t> ids(n);
    for (int i = 0; i < n; ++i) {
      int a = (int)(rng() % (unsigned)(n_adapters + 1)) - 1;
      if (a >= 0 && !rank[a]) a = -1;
      if (i > 0 && rng() % 4) a = ids[i - 1];
      ids[i] = a;
    }
    lora_plan* plan = nullptr;
    CHECK(lora_plan_create(pool, n, &plan) == LORA_OK);
    if (!plan) continue;
    CHECK(lora_plan_build(plan, ids.data(), n, trial % 3 == 0 ? 16 : 0, nullptr) == LORA_OK);
    lora_plan_stats st;
    CHECK(lora_plan_get_stats(plan, &st) == LORA_OK);
    std::vector<int32_t> perm(n), items((size_t)st.n_items * 4 + 4);
    CHECK(lora_plan_export(plan, perm.data(), items.data()) == LORA_OK);
    std::vector<int> cover(n, 0);
    for (int i = 0; i < n; ++i)
      if (perm[i] >= 0 && perm[i] < n) cover[perm[i]]++;
    for (int i = 0; i < n; ++i) CHECK(cover[i] == 1);
    std::vector<lora_io> io(n_slices);
    for (int s = 0; s < n_slices; ++s) io[s] = lora_io{s, 0, nullptr, nullptr};
    for (int k = 1; k <= n_slices && k <= LORA_MAX_IO; ++k) {
      CHECK(lora_plan_prepare(plan, k, io.data(), nullptr) == LORA_OK);
      size_t ws = 1;
      CHECK(lora_workspace_size(plan, k, io.data(), &ws) == LORA_OK);
      CHECK(st.n_mfma_items > 0 || ws == 0);
    }
    // compute calls on a host-only pool: refused on the host, nothing launched
    lora_io bad[2] = {{0, 0, (void*)16, (void*)16}, {n_slices, 0, (void*)16, (void*)16}};
    CHECK(lora_apply(pool, plan, 2, bad, d.act_dtype, (void*)16, 1 << 30, nullptr) == LORA_E_ARG);
    CHECK(lora_apply(pool, plan, 1, bad, d.act_dtype, (void*)16, (size_t)1 << 30, nullptr) != LORA_OK);
    CHECK(lora_bgmv_apply(pool, 1, bad, (const int32_t*)16, n, d.act_dtype, nullptr) == LORA_E_STATE);
    CHECK(lora_bgmv_apply(pool, 2, bad, (const int32_t*)16, n, d.act_dtype, nullptr) == LORA_E_ARG);
    int32_t over = n_adapters;
    CHECK(lora_plan_build(plan, &over, 1, 0, nullptr) == LORA_E_ARG);
    CHECK(lora_plan_build(plan, ids.data(), n + 1, 0, nullptr) == LORA_E_ARG);
    CHECK(lora_plan_destroy(plan) == LORA_OK);
  }
  // evict half the adapters, rebuild, re-upload one
  for (int a = 0; a < n_adapters; a += 2)
    for (int s = 0; s < n_slices; ++s)
      CHECK(lora_pool_evict(pool, a, s, nullptr) == (rank[a] ? LORA_OK : LORA_E_STATE));
  CHECK(lora_page_table_build(pool, nullptr) == LORA_OK);
  CHECK(lora_pool_evict(pool, 0, 0, nullptr) == LORA_E_STATE);
  CHECK(lora_pool_evict(pool, n_adapters, 0, nullptr) == LORA_E_ARG);
  CHECK(lora_pool_destroy(pool) == LORA_OK);
}

int main(int argc, char** argv) {
  const int trials = argc > 1 ? atoi(argv[1]) : 20;
  std::mt19937 rng(77);
  for (int t = 0; t < trials; ++t) {
    const int dt = (int)(rng() % 4);
    const int P = (dt == LORA_F32 ? 64 : 128) * (1 + (int)(rng() % 4));
    const int d_in = (dt == LORA_FP8_E4M3 ? 16 : 8) * (1 + (int)(rng() % 64));
    const int d_out = 8 * (1 + (int)(rng() % 96));
    one_case(rng, dt, P, d_in, d_out, 1 + (int)(rng() % 3), 2 + (int)(rng() % 12));
  }
  // bad descriptions
  lora_pool_desc d;
  memset(&d, 0, sizeof(d));
  lora_pool* p = nullptr;
  CHECK(lora_pool_create(&d, &p) == LORA_E_ARG);
  CHECK(lora_pool_create(nullptr, &p) == LORA_E_ARG);
  CHECK(lora::g_launches == 0);
  printf("%d trials, %d failures\n", trials, g_bad);
  return g_bad ? 1 : 0;
}
