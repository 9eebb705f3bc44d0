// Host-side runtime objects behind the opaque handles of the C ABI.
#pragma once

#include <cstdarg>
#include <string>
#include <vector>

#include "lora_internal.h"

namespace lora {

// One buffer of the device page table with its pinned staging.
struct DevTable {
  DevEntry* entries = nullptr;
  int32_t* page_ids = nullptr;    // page ids (and FP8 scales) of every resident slice
  char* h_stage = nullptr;        // pinned image of the table being written
  size_t h_cap = 0;
  hipEvent_t staged = nullptr;    // the copy from h_stage has completed
  bool staged_pending = false;
  hipEvent_t retired = nullptr;   // launches that read this table have completed
  bool retired_pending = false;
  bool mixed_ranks = false;       // the resident adapters have more than one rank
};

struct Quarantine {
  std::vector<int32_t> pages;
  hipEvent_t ev = nullptr;        // completes once the pages may be handed out again
};

struct Slot {
  int32_t rank = 0;   // 0: not resident
  int32_t rs = 0;
  float scale = 0.f;
  std::vector<int32_t> pages;  // rank*npa A pages, then npb B pages
  std::vector<float> qs;       // FP8 pools: a_scale [rank], then b_scale [rank]
};

lora_status fail(lora_status st, const char* fmt, ...);
void clear_error();
// Look up the device address of `device`'s static scratch array (device
// current); done once per device, at pool creation.
lora_status scratch_init(int device);

#define LORA_HIP(expr)                                                                     \
  do {                                                                                     \
    hipError_t _e = (expr);                                                                \
    if (_e != hipSuccess) return ::lora::fail(LORA_E_HIP, "%s failed: %s", #expr,          \
                                               hipGetErrorString(_e));                     \
  } while (0)

inline int elt_bytes(int dtype) { return dtype == LORA_F32 ? 4 : (dtype == LORA_FP8_E4M3 ? 1 : 2); }
inline uint32_t nan_pattern(int dtype) {
  switch (dtype) {
    case LORA_F32: return 0x7FC00000u;
    case LORA_F16: return 0x7E00u;
    case LORA_FP8_E4M3: return 0x7Fu;
    default: return 0x7FC0u;
  }
}

}  // namespace lora

struct lora_pool {
  int32_t P = 0;
  int32_t dtype = 0;
  int32_t act = 0;                 // activation dtype of x (16-bit y)
  int64_t n_pages = 0;
  int32_t max_adapters = 0;
  int32_t max_rank = 0;
  int32_t n_slices = 0;
  uint32_t flags = 0;
  int elt = 2;
  int64_t page_bytes = 0;
  bool host_only = false;
  bool owns_pages = false;
  char* pages = nullptr;
  std::vector<int32_t> d_in, d_out, npa;
  std::vector<lora::Slot> slots;   // [slice * max_adapters + adapter]
  std::vector<int32_t> free_list;  // stack, allocation pops from the back
  std::vector<uint8_t> state;      // per page: 0 free, 1 adapter, 2 other user
  bool dirty = true;
  uint64_t generation = 0;         // bumped by every residency change
  // Device page table, double-buffered: launches read tables[cur]; a rebuild
  // writes the other one, on a stream ordered after the launches that last
  // read it, and becomes current only for launches enqueued after it.
  lora::DevTable tables[2];
  int cur = 0;
  hipEvent_t pub_ev = nullptr;     // a rebuilt table has been written
  size_t page_ids_cap = 0;         // int32 words of each table's page-id list
  // Pages of evicted slices waiting for the launches that may still read them
  // (and their NaN refill) to finish before they return to the free list.
  std::vector<lora::Quarantine> quarantine;
  char* h_stage = nullptr;
  size_t h_stage_cap = 0;
  char* d_stage = nullptr;
  size_t d_stage_cap = 0;
  int device = 0;
  int32_t n_cu = 256;              // compute units of the device

  lora::Slot& slot(int slice, int adapter) { return slots[(size_t)slice * max_adapters + adapter]; }
  const lora::Slot& slot(int slice, int adapter) const {
    return slots[(size_t)slice * max_adapters + adapter];
  }
  bool quant() const { return dtype == LORA_FP8_E4M3; }
  lora::Types types(int y_dtype) const { return lora::Types{dtype, act, y_dtype}; }
  int rs_of(int rank) const {
    const int per16 = 16 / elt;
    return (rank + per16 - 1) / per16 * per16;
  }
  int npb_of(int slice, int rank) const {
    const int rpp = P / rs_of(rank);
    return (d_out[slice] + rpp - 1) / rpp;
  }
  lora::PoolView view() const {
    lora::PoolView v;
    v.pages = pages;
    v.entries = tables[cur].entries;
    v.page_ids = tables[cur].page_ids;
    v.P = P;
    v.max_adapters = max_adapters;
    v.max_nch = rs_of(max_rank) * elt / 16;
    v.n_cu = n_cu;
    v.mixed_ranks = tables[cur].mixed_ranks ? 1 : 0;
    return v;
  }
  lora::IoDesc io(int slice, const void* x, void* y) const {
    lora::IoDesc d;
    d.x = x;
    d.y = y;
    d.slice = slice;
    d.d_in = d_in[slice];
    d.d_out = d_out[slice];
    d.npa = npa[slice];
    return d;
  }
};

namespace lora {
// Write the page table of the pool's current residency into the inactive
// buffer on `upload` (after the launches that last read that buffer), make
// `compute` wait for it and switch launches to it.  compute == upload for the
// synchronous build.
lora_status publish_table(lora_pool* p, hipStream_t upload, hipStream_t compute);
// Return quarantined pages whose readers have finished to the free list.
void reclaim_pages(lora_pool* p);
// Page images of one adapter slice as the pool lays them out (rank * npa A
// pages, then the B pages); dst holds pages_of(slice, rank) pages.
void pack_slice(const lora_pool* p, int slice, int rank, const void* A, const void* B, char* dst);
int64_t pages_of(const lora_pool* p, int slice, int rank);
}  // namespace lora

struct lora_plan;
namespace lora {
// The range tables and split-K contributions of one launch shape (n_io, then
// the stage and chunk counts of each launch slice), built on the host by
// lora_plan_prepare and copied to the device on its stream.
struct PlanLayout {
  std::vector<int32_t> key;
  bool valid = false;
  uint64_t used = 0;          // LRU clock
  int32_t* d_buf = nullptr;   // device copy: ranges, part_fl, c_off, c_ent
  char* h_buf = nullptr;      // pinned staging of the same
  size_t cap = 0;             // bytes of each
  hipEvent_t ev = nullptr;    // the staging copy has been consumed
  bool ev_pending = false;
  int64_t part_units = 0;     // float4 units of partial tiles (and the pool counter)
  bool pool = false;          // the expand ranges leave a pool (fused launches of >= 2 slices)
  size_t o_bs = 0, o_be = 0, o_fl = 0, o_pool = 0, o_off = 0, o_ent = 0;  // int32 offsets
};
constexpr int kPlanLayouts = 8;

// Key of a launch shape: n_io, then per launch slice its shrink stage and
// expand chunk counts.
std::vector<int32_t> layout_key(const IoSet& ios);
// Build (or find) the layout of this launch shape: host work, may allocate and
// synchronise (lora_plan_prepare only).
lora_status plan_prepare_layout(lora_plan* pl, const IoSet& ios, hipStream_t s);
// The prepared layout of this launch shape, or null (compute calls: no
// allocation, no synchronisation).
const PlanLayout* plan_find_layout(const lora_plan* pl, const IoSet& ios);
}  // namespace lora

struct lora_plan {
  lora_pool* pool = nullptr;
  int32_t max_tokens = 0;
  int32_t n_tokens = 0;
  int32_t n_groups = 0;
  int32_t n_items = 0;
  int32_t n_mfma = 0;
  int32_t mfma_tokens = 0;
  int32_t l_long = 1;
  uint64_t pool_generation = ~0ull;
  bool built = false;
  std::vector<int32_t> h_perm;
  std::vector<lora::PlanItem> h_items;
  char* h_pinned = nullptr;
  size_t pinned_cap = 0;
  hipEvent_t ev = nullptr;
  bool ev_pending = false;
  int32_t* d_perm = nullptr;
  lora::PlanItem* d_items = nullptr;
  // persistent MFMA kernels: grid, per-tile weights and launch-shape layouts
  int32_t G = 0;
  std::vector<int32_t> h_ws;  // per MFMA tile: weight of one shrink stage
  std::vector<int32_t> h_we;  //   ... of one expand chunk
  std::vector<int32_t> h_tu;  //   ... float4 units of one partial tile
  // Launch shapes prepared for this build (lora_plan_prepare).  The LRU stamp
  // is bumped by compute calls, which take the plan as const.
  lora::PlanLayout layouts[lora::kPlanLayouts];
  mutable uint64_t layout_clock = 0;
  // part: the caller's workspace for the partial tiles of this call
  lora::PlanView view(const lora::PlanLayout* lay, void* part) const {
    lora::PlanView v;
    v.items = d_items;
    v.perm = d_perm;
    v.bs_shrink = lay ? reinterpret_cast<const lora::RangePos*>(lay->d_buf + lay->o_bs) : nullptr;
    v.bs_expand = lay ? reinterpret_cast<const lora::RangePos*>(lay->d_buf + lay->o_be) : nullptr;
    v.part_fl = lay ? reinterpret_cast<const int2*>(lay->d_buf + lay->o_fl) : nullptr;
    v.c_off = lay ? lay->d_buf + lay->o_off : nullptr;
    v.c_ent = lay ? lay->d_buf + lay->o_ent : nullptr;
    v.part = reinterpret_cast<float*>(part);
    v.n_tiles_dev = nullptr;
    v.pool = lay && lay->pool ? lay->d_buf + lay->o_pool : nullptr;
    v.n_items = n_items;
    v.n_tokens = n_tokens;
    v.n_mfma = n_mfma;
    v.G = G;
    return v;
  }
};
