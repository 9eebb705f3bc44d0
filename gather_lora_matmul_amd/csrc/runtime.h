// Host-side runtime objects behind the opaque handles of the C ABI.
#pragma once

#include <cstdarg>
#include <string>
#include <vector>

#include "lora_internal.h"

namespace lora {

struct Slot {
  int32_t rank = 0;   // 0: not resident
  int32_t rs = 0;
  float scale = 0.f;
  std::vector<int32_t> pages;  // rank*npa A pages, then npb B pages
};

lora_status fail(lora_status st, const char* fmt, ...);
void clear_error();

#define LORA_HIP(expr)                                                                     \
  do {                                                                                     \
    hipError_t _e = (expr);                                                                \
    if (_e != hipSuccess) return ::lora::fail(LORA_E_HIP, "%s failed: %s", #expr,          \
                                               hipGetErrorString(_e));                     \
  } while (0)

inline int elt_bytes(int dtype) { return dtype == LORA_F32 ? 4 : 2; }
inline uint32_t nan_pattern(int dtype) {
  return dtype == LORA_F32 ? 0x7FC00000u : (dtype == LORA_F16 ? 0x7E00u : 0x7FC0u);
}

}  // namespace lora

struct lora_pool {
  int32_t P = 0;
  int32_t dtype = 0;
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
  lora::DevEntry* d_entries = nullptr;
  int32_t* d_page_ids = nullptr;
  char* h_stage = nullptr;
  size_t h_stage_cap = 0;
  char* d_stage = nullptr;
  size_t d_stage_cap = 0;
  int device = 0;

  lora::Slot& slot(int slice, int adapter) { return slots[(size_t)slice * max_adapters + adapter]; }
  const lora::Slot& slot(int slice, int adapter) const {
    return slots[(size_t)slice * max_adapters + adapter];
  }
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
    v.entries = d_entries;
    v.page_ids = d_page_ids;
    v.P = P;
    v.max_adapters = max_adapters;
    v.max_nch = rs_of(max_rank) * elt / 16;
    v.pad = 0;
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

struct lora_plan;
namespace lora {
// The range tables and split-K contributions of one launch shape (n_io, then
// the stage and chunk counts of each launch slice), built on the host at the
// first launch of that shape after a plan build and copied to the device on
// the launch stream.
struct PlanLayout {
  std::vector<int32_t> key;
  bool valid = false;
  uint64_t used = 0;          // LRU clock
  int32_t* d_buf = nullptr;   // device copy: ranges, part_fl, c_off, c_ent
  char* h_buf = nullptr;      // pinned staging of the same
  size_t cap = 0;             // bytes of each
  hipEvent_t ev = nullptr;    // the staging copy has been consumed
  bool ev_pending = false;
  int64_t part_units = 0;     // float4 units of partial tiles
  size_t o_bs = 0, o_be = 0, o_fl = 0, o_off = 0, o_ent = 0;  // int32 offsets
};
constexpr int kPlanLayouts = 4;

// Layout for the launch slices of `ios` (built and uploaded on `s` if the plan
// has none of that shape), with the plan's partial-tile workspace grown to it.
lora_status plan_layout(const lora_plan* pl, const IoSet& ios, hipStream_t s, const PlanLayout** out);
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
  // Launch-time state of a built plan (compute calls take the plan as const):
  // the cache of launch-shape layouts and the partial-tile workspace.
  mutable lora::PlanLayout layouts[lora::kPlanLayouts];
  mutable uint64_t layout_clock = 0;
  mutable float* d_part = nullptr;  // partial tiles, grown on demand
  mutable size_t part_cap = 0;      // floats
  lora::PlanView view(const lora::PlanLayout* lay) const {
    lora::PlanView v;
    v.items = d_items;
    v.perm = d_perm;
    v.bs_shrink = lay ? reinterpret_cast<const lora::RangePos*>(lay->d_buf + lay->o_bs) : nullptr;
    v.bs_expand = lay ? reinterpret_cast<const lora::RangePos*>(lay->d_buf + lay->o_be) : nullptr;
    v.part_fl = lay ? reinterpret_cast<const int2*>(lay->d_buf + lay->o_fl) : nullptr;
    v.c_off = lay ? lay->d_buf + lay->o_off : nullptr;
    v.c_ent = lay ? lay->d_buf + lay->o_ent : nullptr;
    v.part = d_part;
    v.n_items = n_items;
    v.n_tokens = n_tokens;
    v.n_mfma = n_mfma;
    v.G = G;
    return v;
  }
};
