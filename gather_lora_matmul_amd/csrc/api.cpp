// Compute entry points of the C ABI: argument and state checks, then
// stream-ordered launches.  Nothing here allocates memory or waits for the
// device: planned calls find their launch shape's layout among those the plan
// prepared (lora_plan_prepare) and take the partial-tile workspace from the
// caller.
#include <algorithm>
#include <cstring>
#include <new>

#include "devplan.h"
#include "runtime.h"

using namespace lora;

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

lora_status check_pool(const lora_pool* p) {
  if (!p) return fail(LORA_E_ARG, "null pool");
  if (p->host_only) return fail(LORA_E_STATE, "host-only pool cannot run kernels");
  if (p->dirty) return fail(LORA_E_STATE, "page table is stale: call lora_page_table_build");
  return LORA_OK;
}

lora_status check_slice(const lora_pool* p, int32_t slice) {
  if (slice < 0 || slice >= p->n_slices) return fail(LORA_E_ARG, "slice %d out of range", slice);
  return LORA_OK;
}

lora_status check_ydt(const lora_pool* p, int32_t y_dtype) {
  if (y_dtype != p->act && y_dtype != LORA_F32)
    return fail(LORA_E_ARG, "y dtype %d must be the activation dtype or LORA_F32", y_dtype);
  return LORA_OK;
}

lora_status check_plan(const lora_pool* p, const lora_plan* pl) {
  if (!pl || !pl->built) return fail(LORA_E_ARG, "plan not built");
  if (pl->pool != p) return fail(LORA_E_ARG, "plan belongs to another pool");
  if (pl->pool_generation != p->generation)
    return fail(LORA_E_STATE, "residency changed since the plan was built");
  return LORA_OK;
}

lora_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(LORA_E_HIP, "%s launch: %s", what, hipGetErrorString(e));
  return LORA_OK;
}

// The io entries of a call; with `groups`, entries sharing an x_group are
// made contiguous and described by grp_start (n_groups stays 0 when no group
// has two members).
lora_status build_ioset(const lora_pool* p, int32_t n_io, const lora_io* io, IoSet& ios,
                        bool groups = false) {
  if (n_io < 1 || n_io > LORA_MAX_IO || !io) return fail(LORA_E_ARG, "n_io must be in [1, %d]", LORA_MAX_IO);
  memset(&ios, 0, sizeof(ios));
  ios.n_io = n_io;
  bool shared = false;
  for (int k = 0; k < n_io; ++k) {
    lora_status st = check_slice(p, io[k].slice);
    if (st) return st;
    if (!io[k].x_dev || !io[k].y_dev) return fail(LORA_E_ARG, "io %d: null x or y", k);
    if (!aligned16(io[k].x_dev) || !aligned16(io[k].y_dev)) return fail(LORA_E_ARG, "io %d: x/y not 16-byte aligned", k);
    if (io[k].x_group < 0) return fail(LORA_E_ARG, "io %d: negative x_group", k);
    for (int j = 0; j < k; ++j)
      if (io[k].x_group && io[j].x_group == io[k].x_group) {
        if (io[j].x_dev != io[k].x_dev || p->d_in[(size_t)io[j].slice] != p->d_in[(size_t)io[k].slice])
          return fail(LORA_E_ARG, "io %d and %d: x_group %d needs one x and one d_in", j, k,
                      io[k].x_group);
        shared = true;
      }
    ios.io[k] = p->io(io[k].slice, io[k].x_dev, io[k].y_dev);
    ios.max_d_in = std::max(ios.max_d_in, ios.io[k].d_in);
    ios.max_d_out = std::max(ios.max_d_out, ios.io[k].d_out);
  }
  if (groups && shared) {
    // group members contiguous, groups in first-appearance order; an entry
    // without a group is a group of its own
    std::vector<char> taken((size_t)n_io, 0);
    IoDesc ord[LORA_MAX_IO];
    int m = 0;
    for (int k = 0; k < n_io; ++k) {
      if (taken[(size_t)k]) continue;
      ios.grp_start[ios.n_groups++] = m;
      for (int j = k; j < n_io; ++j)
        if (!taken[(size_t)j] && (j == k || (io[k].x_group && io[j].x_group == io[k].x_group))) {
          taken[(size_t)j] = 1;
          ord[m++] = ios.io[j];
        }
    }
    ios.grp_start[ios.n_groups] = m;
    for (int k = 0; k < n_io; ++k) ios.io[k] = ord[k];
  }
  return LORA_OK;
}

// A launch of one slice (split API): its layout has the same key as a fused
// launch of that slice alone.
IoSet single_io(const IoDesc& io) {
  IoSet s;
  memset(&s, 0, sizeof(s));
  s.n_io = 1;
  s.io[0] = io;
  s.max_d_in = io.d_in;
  s.max_d_out = io.d_out;
  return s;
}

// The prepared layout of a planned call's launch shape and the check of the
// caller's workspace against it (none needed without MFMA tiles).
lora_status find_layout(const lora_plan* pl, const IoSet& ios, const void* ws, size_t ws_bytes,
                        bool needs_ws, const PlanLayout** out) {
  *out = nullptr;
  if (pl->n_mfma == 0) return LORA_OK;
  const PlanLayout* lay = plan_find_layout(pl, ios);
  if (!lay) return fail(LORA_E_STATE, "launch shape not prepared: call lora_plan_prepare after lora_plan_build");
  if (needs_ws) {
    const size_t need = 16 * (size_t)lay->part_units;
    if (ws_bytes < need || (need && !ws))
      return fail(LORA_E_ARG, "workspace of %zu bytes, this launch needs %zu (lora_workspace_size)",
                  ws_bytes, need);
    if ((uintptr_t)ws & 15u) return fail(LORA_E_ARG, "workspace not 16-byte aligned");
  }
  *out = lay;
  return LORA_OK;
}

// Launch shape and workspace layout of a device-planned decode call; refuses
// what the MFMA tiles cannot take.
lora_status devplan_shape(const lora_pool* p, const IoSet& ios, int32_t n, DevPlanShape& sh,
                          DevPlanWs& w) {
  if (p->dtype != LORA_F16 && p->dtype != LORA_BF16)
    return fail(LORA_E_UNSUPPORTED, "device-planned decode needs 16-bit pages (use lora_bgmv_apply)");
  if (p->P / p->rs_of(p->max_rank) < 16)
    return fail(LORA_E_UNSUPPORTED, "device-planned decode needs >= 16 B rows per page");
  if (n > kDpMaxTokens) return fail(LORA_E_ARG, "%d tokens exceed %d per device-planned call", n, kDpMaxTokens);
  if (p->max_adapters > (1 << 21)) return fail(LORA_E_UNSUPPORTED, "max_adapters above 2^21");
  memset(&sh, 0, sizeof(sh));
  sh.n = n;
  sh.J = ios.n_io;
  sh.G = ((2 * p->n_cu + 7) / 8) * 8;
  if (sh.G > kDpMaxBlocks) sh.G = kDpMaxBlocks;
  sh.rs_per16 = 16 / p->elt;
  sh.cap = n;
  sh.ov_s = (int32_t)kPieceSetupShrink;
  sh.ov_e = (int32_t)kPieceSetupExpand;
  for (int j = 0; j < ios.n_io; ++j) {
    if (ios.io[j].npa > kMaxNpa)
      return fail(LORA_E_UNSUPPORTED, "io %d: A rows span more than %d pages", j, kMaxNpa);
    sh.slice[j] = ios.io[j].slice;
    sh.nst[j] = (ios.io[j].d_in + 63) / 64;
    sh.nch[j] = (ios.io[j].d_out + 63) / 64;
  }
  if (!devplan_ws(sh.J, n, sh.G, p->max_rank, w))
    return fail(LORA_E_ARG, "partial tiles exceed 2^31 float4 units");
  return LORA_OK;
}

}  // namespace

// A device plan kept between calls: built from device ids by lora_dplan_build,
// applied by lora_dplan_apply to any launch whose slices have the shapes it
// was created for (the layers of a model whose LoRA calls share one decode
// step's ids).  Owns its device workspace.
struct lora_dplan {
  lora_pool* pool = nullptr;
  int32_t max_tokens = 0;
  int32_t n_io = 0;
  int32_t d_in[LORA_MAX_IO] = {}, d_out[LORA_MAX_IO] = {};
  lora::DevPlanShape sh{};   // shape of the last build (slices, token count)
  lora::DevPlanWs w{};       // workspace layout for max_tokens
  char* ws = nullptr;
  bool built = false;
  uint64_t generation = ~0ull;  // pool residency the plan was built against
};

#define LORA_TRY(expr)          \
  do {                          \
    lora_status _s = (expr);    \
    if (_s != LORA_OK) return _s; \
  } while (0)

extern "C" {

lora_status lora_bgmv_shrink(lora_pool* p, int32_t slice, const void* x, const int32_t* ids,
                             int32_t n, float* v, int32_t v_ld, void* stream) {
  clear_error();
  LORA_TRY(check_pool(p));
  LORA_TRY(check_slice(p, slice));
  if (n < 0) return fail(LORA_E_ARG, "n < 0");
  if (n == 0) return LORA_OK;
  if (!x || !ids || !v) return fail(LORA_E_ARG, "null device pointer");
  if (!aligned16(x)) return fail(LORA_E_ARG, "x not 16-byte aligned");
  if (v_ld < p->max_rank) return fail(LORA_E_ARG, "v_ld %d < max_rank %d", v_ld, p->max_rank);
  return hip_status(launch_bgmv_shrink(p->types(p->act), p->view(), p->io(slice, x, nullptr), ids, n,
                                       v, v_ld, (hipStream_t)stream),
                    "bgmv_shrink");
}

lora_status lora_bgmv_expand(lora_pool* p, int32_t slice, const float* v, int32_t v_ld,
                             const int32_t* ids, int32_t n, const float* tok_scale, void* y,
                             int32_t y_dtype, void* stream) {
  clear_error();
  LORA_TRY(check_pool(p));
  LORA_TRY(check_slice(p, slice));
  LORA_TRY(check_ydt(p, y_dtype));
  if (n < 0) return fail(LORA_E_ARG, "n < 0");
  if (n == 0) return LORA_OK;
  if (!v || !ids || !y) return fail(LORA_E_ARG, "null device pointer");
  if (!aligned16(y)) return fail(LORA_E_ARG, "y not 16-byte aligned");
  if (v_ld < p->max_rank) return fail(LORA_E_ARG, "v_ld %d < max_rank %d", v_ld, p->max_rank);
  return hip_status(launch_bgmv_expand(p->types(y_dtype), p->view(), p->io(slice, nullptr, y), v,
                                       v_ld, ids, n, tok_scale, (hipStream_t)stream),
                    "bgmv_expand");
}

lora_status lora_bgmv_apply(lora_pool* p, int32_t n_io, const lora_io* io, const int32_t* ids,
                            int32_t n, int32_t y_dtype, void* stream) {
  clear_error();
  if (!p) return fail(LORA_E_ARG, "null pool");
  LORA_TRY(check_ydt(p, y_dtype));
  IoSet ios;
  LORA_TRY(build_ioset(p, n_io, io, ios, true));
  if (n < 0) return fail(LORA_E_ARG, "n < 0");
  if (n == 0) return LORA_OK;
  if (!ids) return fail(LORA_E_ARG, "null ids");
  LORA_TRY(check_pool(p));
  return hip_status(launch_bgmv_apply(p->types(y_dtype), p->view(), ios, ids, n, (hipStream_t)stream),
                    "bgmv_apply");
}

lora_status lora_bgmv_planned_workspace_size(lora_pool* p, int32_t n_io, const lora_io* io,
                                             int32_t n, size_t* bytes) {
  clear_error();
  if (!p || !bytes) return fail(LORA_E_ARG, "null argument");
  if (n_io < 1 || n_io > LORA_MAX_IO || !io) return fail(LORA_E_ARG, "n_io must be in [1, %d]", LORA_MAX_IO);
  if (n < 0) return fail(LORA_E_ARG, "n < 0");
  IoSet ios;
  memset(&ios, 0, sizeof(ios));
  ios.n_io = n_io;
  for (int k = 0; k < n_io; ++k) {
    LORA_TRY(check_slice(p, io[k].slice));
    ios.io[k] = p->io(io[k].slice, nullptr, nullptr);
  }
  DevPlanShape sh;
  DevPlanWs w;
  LORA_TRY(devplan_shape(p, ios, n, sh, w));
  *bytes = w.bytes;
  return LORA_OK;
}

lora_status lora_bgmv_apply_planned(lora_pool* p, int32_t n_io, const lora_io* io,
                                    const int32_t* ids, int32_t n, int32_t y_dtype, void* ws,
                                    size_t ws_bytes, void* stream) {
  clear_error();
  if (!p) return fail(LORA_E_ARG, "null pool");
  LORA_TRY(check_ydt(p, y_dtype));
  IoSet ios;
  LORA_TRY(build_ioset(p, n_io, io, ios));
  if (n < 0) return fail(LORA_E_ARG, "n < 0");
  if (n == 0) return LORA_OK;
  if (!ids) return fail(LORA_E_ARG, "null ids");
  DevPlanShape sh;
  DevPlanWs w;
  LORA_TRY(devplan_shape(p, ios, n, sh, w));
  if (!ws || ws_bytes < w.bytes)
    return fail(LORA_E_ARG, "workspace of %zu bytes, this call needs %zu (lora_bgmv_planned_workspace_size)",
                ws_bytes, w.bytes);
  if ((uintptr_t)ws & 255u) return fail(LORA_E_ARG, "workspace not 256-byte aligned");
  LORA_TRY(check_pool(p));
  return hip_status(launch_devplan_apply(p->types(y_dtype), p->view(), ios, ids, sh, w,
                                         reinterpret_cast<char*>(ws), (hipStream_t)stream),
                    "bgmv_apply_planned");
}

lora_status lora_dplan_create(lora_pool* p, int32_t max_tokens, int32_t n_io, const lora_io* io,
                              lora_dplan** out) {
  clear_error();
  if (!p || !out) return fail(LORA_E_ARG, "null argument");
  *out = nullptr;
  if (max_tokens <= 0) return fail(LORA_E_ARG, "max_tokens must be positive");
  if (n_io < 1 || n_io > LORA_MAX_IO || !io) return fail(LORA_E_ARG, "n_io must be in [1, %d]", LORA_MAX_IO);
  IoSet ios;
  memset(&ios, 0, sizeof(ios));
  ios.n_io = n_io;
  for (int k = 0; k < n_io; ++k) {
    LORA_TRY(check_slice(p, io[k].slice));
    ios.io[k] = p->io(io[k].slice, nullptr, nullptr);
  }
  DevPlanShape sh;
  DevPlanWs w;
  LORA_TRY(devplan_shape(p, ios, max_tokens, sh, w));
  lora_dplan* d = new (std::nothrow) lora_dplan();
  if (!d) return fail(LORA_E_NOMEM, "out of host memory");
  d->pool = p;
  d->max_tokens = max_tokens;
  d->n_io = n_io;
  for (int k = 0; k < n_io; ++k) {
    d->d_in[k] = ios.io[k].d_in;
    d->d_out[k] = ios.io[k].d_out;
  }
  d->sh = sh;
  d->w = w;
  if (!p->host_only) {
    const hipError_t e = hipMalloc((void**)&d->ws, w.bytes);
    if (e != hipSuccess) {
      delete d;
      return fail(LORA_E_NOMEM, "device plan workspace of %zu bytes: %s", w.bytes, hipGetErrorString(e));
    }
  }
  *out = d;
  return LORA_OK;
}

lora_status lora_dplan_destroy(lora_dplan* d) {
  clear_error();
  if (!d) return LORA_OK;
  if (d->ws) {
    (void)hipDeviceSynchronize();  // launches may still read the plan
    (void)hipFree(d->ws);
  }
  delete d;
  return LORA_OK;
}

lora_status lora_dplan_build(lora_dplan* d, int32_t n_io, const lora_io* io, const int32_t* ids,
                             int32_t n, void* stream) {
  clear_error();
  if (!d) return fail(LORA_E_ARG, "null device plan");
  lora_pool* p = d->pool;
  if (n < 0 || n > d->max_tokens) return fail(LORA_E_ARG, "n %d outside [0, %d]", n, d->max_tokens);
  if (n_io != d->n_io || !io) return fail(LORA_E_ARG, "%d slices, the plan was created for %d", n_io, d->n_io);
  DevPlanShape sh = d->sh;
  for (int k = 0; k < n_io; ++k) {
    LORA_TRY(check_slice(p, io[k].slice));
    if (p->d_in[(size_t)io[k].slice] != d->d_in[k] || p->d_out[(size_t)io[k].slice] != d->d_out[k])
      return fail(LORA_E_ARG, "io %d: slice %d does not have the shape the plan was created for", k, io[k].slice);
    sh.slice[k] = io[k].slice;
  }
  if (n > 0 && !ids) return fail(LORA_E_ARG, "null ids");
  LORA_TRY(check_pool(p));
  sh.n = n;
  d->built = false;
  if (n > 0) {
    const hipError_t e = launch_devplan(p->view(), ids, sh, d->w, d->ws, (hipStream_t)stream);
    if (e != hipSuccess) return fail(LORA_E_HIP, "dplan_build launch: %s", hipGetErrorString(e));
  }
  d->sh = sh;
  d->built = true;
  d->generation = p->generation;
  return LORA_OK;
}

lora_status lora_dplan_apply(lora_pool* p, const lora_dplan* d, int32_t n_io, const lora_io* io,
                             int32_t y_dtype, void* stream) {
  clear_error();
  if (!p || !d) return fail(LORA_E_ARG, "null argument");
  if (d->pool != p) return fail(LORA_E_ARG, "device plan belongs to another pool");
  if (!d->built) return fail(LORA_E_STATE, "device plan not built");
  if (d->generation != p->generation)
    return fail(LORA_E_STATE, "residency changed since the device plan was built");
  LORA_TRY(check_ydt(p, y_dtype));
  IoSet ios;
  LORA_TRY(build_ioset(p, n_io, io, ios));
  if (n_io != d->n_io) return fail(LORA_E_ARG, "%d slices, the plan was created for %d", n_io, d->n_io);
  for (int k = 0; k < n_io; ++k)
    if (ios.io[k].d_in != d->d_in[k] || ios.io[k].d_out != d->d_out[k])
      return fail(LORA_E_ARG, "io %d: slice %d does not have the shape the plan was created for", k,
                  ios.io[k].slice);
  if (d->sh.n == 0) return LORA_OK;
  LORA_TRY(check_pool(p));
  return hip_status(launch_devplan_mfma(p->types(y_dtype), p->view(), ios, d->sh, d->w, d->ws,
                                        (hipStream_t)stream),
                    "dplan_apply");
}

lora_status lora_sgmv_shrink(lora_pool* p, const lora_plan* pl, int32_t slice, const void* x,
                             float* v, int32_t v_ld, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  if (!p) return fail(LORA_E_ARG, "null pool");
  LORA_TRY(check_plan(p, pl));
  LORA_TRY(check_slice(p, slice));
  if (pl->n_tokens == 0) return LORA_OK;
  if (!x || !v) return fail(LORA_E_ARG, "null device pointer");
  if (!aligned16(x)) return fail(LORA_E_ARG, "x not 16-byte aligned");
  if (v_ld < p->max_rank) return fail(LORA_E_ARG, "v_ld %d < max_rank %d", v_ld, p->max_rank);
  const IoDesc io = p->io(slice, x, nullptr);
  const PlanLayout* lay = nullptr;
  LORA_TRY(find_layout(pl, single_io(io), ws, ws_bytes, true, &lay));
  LORA_TRY(check_pool(p));
  return hip_status(launch_sgmv_shrink(p->types(p->act), p->view(), pl->view(lay, ws), io, v, v_ld,
                                       (hipStream_t)stream),
                    "sgmv_shrink");
}

lora_status lora_sgmv_expand(lora_pool* p, const lora_plan* pl, int32_t slice, const float* v,
                             int32_t v_ld, void* y, int32_t y_dtype, void* stream) {
  clear_error();
  LORA_TRY(check_pool(p));
  LORA_TRY(check_plan(p, pl));
  LORA_TRY(check_slice(p, slice));
  LORA_TRY(check_ydt(p, y_dtype));
  if (pl->n_tokens == 0) return LORA_OK;
  if (!v || !y) return fail(LORA_E_ARG, "null device pointer");
  if (!aligned16(y)) return fail(LORA_E_ARG, "y not 16-byte aligned");
  if (v_ld < p->max_rank) return fail(LORA_E_ARG, "v_ld %d < max_rank %d", v_ld, p->max_rank);
  const IoDesc io = p->io(slice, nullptr, y);
  const PlanLayout* lay = nullptr;
  LORA_TRY(find_layout(pl, single_io(io), nullptr, 0, false, &lay));
  return hip_status(launch_sgmv_expand(p->types(y_dtype), p->view(), pl->view(lay, nullptr), io, v, v_ld,
                                       (hipStream_t)stream),
                    "sgmv_expand");
}

lora_status lora_apply(lora_pool* p, const lora_plan* pl, int32_t n_io, const lora_io* io,
                       int32_t y_dtype, void* ws, size_t ws_bytes, void* stream) {
  clear_error();
  if (!p) return fail(LORA_E_ARG, "null pool");
  LORA_TRY(check_plan(p, pl));
  LORA_TRY(check_ydt(p, y_dtype));
  IoSet ios;
  LORA_TRY(build_ioset(p, n_io, io, ios));
  if (pl->n_tokens == 0) return LORA_OK;
  const PlanLayout* lay = nullptr;
  LORA_TRY(find_layout(pl, ios, ws, ws_bytes, true, &lay));
  LORA_TRY(check_pool(p));
  return hip_status(launch_apply(p->types(y_dtype), p->view(), pl->view(lay, ws), ios,
                                 (hipStream_t)stream),
                    "apply");
}

lora_status lora_debug_resolve(lora_pool* p, int32_t slice, const int32_t* ids, int32_t n,
                               int64_t* a_off, int64_t* b_off, void* stream) {
  clear_error();
  LORA_TRY(check_pool(p));
  LORA_TRY(check_slice(p, slice));
  if (n < 0) return fail(LORA_E_ARG, "n < 0");
  if (n == 0) return LORA_OK;
  if (!ids || !a_off || !b_off) return fail(LORA_E_ARG, "null device pointer");
  return hip_status(launch_debug_resolve(p->view(), p->io(slice, nullptr, nullptr), p->max_rank,
                                         p->elt, ids, n, a_off, b_off, (hipStream_t)stream),
                    "debug_resolve");
}

lora_status lora_debug_gather(lora_pool* p, int32_t slice, int32_t adapter, void* A, void* B,
                              void* stream) {
  clear_error();
  LORA_TRY(check_pool(p));
  LORA_TRY(check_slice(p, slice));
  if (adapter < 0 || adapter >= p->max_adapters) return fail(LORA_E_ARG, "adapter %d out of range", adapter);
  const Slot& sl = p->slot(slice, adapter);
  if (!sl.rank) return fail(LORA_E_NOT_RESIDENT, "adapter %d slice %d is not resident", adapter, slice);
  if (!A || !B) return fail(LORA_E_ARG, "null device pointer");
  return hip_status(launch_debug_gather(p->elt, p->view(), p->io(slice, nullptr, nullptr), adapter,
                                        sl.rank, A, B, (hipStream_t)stream),
                    "debug_gather");
}

lora_status lora_debug_decode(int32_t dtype, const void* src, int64_t n, float* dst, void* stream) {
  clear_error();
  if (dtype < LORA_F32 || dtype > LORA_FP8_E4M3) return fail(LORA_E_ARG, "bad dtype %d", dtype);
  if (n < 0 || (n * elt_bytes(dtype)) % 16) return fail(LORA_E_ARG, "n * element bytes must be a multiple of 16");
  if (n == 0) return LORA_OK;
  if (!src || !dst) return fail(LORA_E_ARG, "null device pointer");
  if (!aligned16(src) || !aligned16(dst)) return fail(LORA_E_ARG, "buffers not 16-byte aligned");
  return hip_status(launch_debug_decode(dtype, src, n, dst, (hipStream_t)stream), "debug_decode");
}

lora_status lora_debug_block_timeline(void* host, size_t bytes) {
  clear_error();
  if (!host && bytes) return fail(LORA_E_ARG, "null host buffer");
  if (bytes % (kTimelineWords * sizeof(uint64_t)))
    return fail(LORA_E_ARG, "bytes must be a multiple of one %zu-byte record",
                kTimelineWords * sizeof(uint64_t));
  const hipError_t e = read_block_timeline(host, bytes);
  if (e == hipErrorNotSupported)
    return fail(LORA_E_UNSUPPORTED, "library built without LORA_BLOCK_TIMELINE");
  return hip_status(e, "block timeline");
}

}  // extern "C"
