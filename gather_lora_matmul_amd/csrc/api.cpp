// Compute entry points of the C ABI: argument and state checks, then one
// stream-ordered launch (or two, for plans that mix MFMA tiles and short
// items in the split API).  Nothing here blocks the host.
#include <algorithm>
#include <cstring>

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
  if (y_dtype != p->dtype && y_dtype != LORA_F32)
    return fail(LORA_E_ARG, "y dtype %d must be the pool dtype or LORA_F32", y_dtype);
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

lora_status build_ioset(const lora_pool* p, int32_t n_io, const lora_io* io, IoSet& ios) {
  if (n_io < 1 || n_io > LORA_MAX_IO || !io) return fail(LORA_E_ARG, "n_io must be in [1, %d]", LORA_MAX_IO);
  memset(&ios, 0, sizeof(ios));
  ios.n_io = n_io;
  for (int k = 0; k < n_io; ++k) {
    lora_status st = check_slice(p, io[k].slice);
    if (st) return st;
    if (!io[k].x_dev || !io[k].y_dev) return fail(LORA_E_ARG, "io %d: null x or y", k);
    if (!aligned16(io[k].x_dev) || !aligned16(io[k].y_dev)) return fail(LORA_E_ARG, "io %d: x/y not 16-byte aligned", k);
    ios.io[k] = p->io(io[k].slice, io[k].x_dev, io[k].y_dev);
    ios.max_d_in = std::max(ios.max_d_in, ios.io[k].d_in);
    ios.max_d_out = std::max(ios.max_d_out, ios.io[k].d_out);
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

}  // namespace

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
  return hip_status(launch_bgmv_shrink(p->dtype, p->view(), p->io(slice, x, nullptr), ids, n, v,
                                       v_ld, (hipStream_t)stream),
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
  return hip_status(launch_bgmv_expand(p->dtype, y_dtype, p->view(), p->io(slice, nullptr, y), v,
                                       v_ld, ids, n, tok_scale, (hipStream_t)stream),
                    "bgmv_expand");
}

lora_status lora_bgmv_apply(lora_pool* p, int32_t n_io, const lora_io* io, const int32_t* ids,
                            int32_t n, int32_t y_dtype, void* stream) {
  clear_error();
  LORA_TRY(check_pool(p));
  LORA_TRY(check_ydt(p, y_dtype));
  IoSet ios;
  LORA_TRY(build_ioset(p, n_io, io, ios));
  if (n < 0) return fail(LORA_E_ARG, "n < 0");
  if (n == 0) return LORA_OK;
  if (!ids) return fail(LORA_E_ARG, "null ids");
  return hip_status(launch_bgmv_apply(p->dtype, y_dtype, p->view(), ios, ids, n, (hipStream_t)stream),
                    "bgmv_apply");
}

lora_status lora_sgmv_shrink(lora_pool* p, const lora_plan* pl, int32_t slice, const void* x,
                             float* v, int32_t v_ld, void* stream) {
  clear_error();
  LORA_TRY(check_pool(p));
  LORA_TRY(check_plan(p, pl));
  LORA_TRY(check_slice(p, slice));
  if (pl->n_tokens == 0) return LORA_OK;
  if (!x || !v) return fail(LORA_E_ARG, "null device pointer");
  if (!aligned16(x)) return fail(LORA_E_ARG, "x not 16-byte aligned");
  if (v_ld < p->max_rank) return fail(LORA_E_ARG, "v_ld %d < max_rank %d", v_ld, p->max_rank);
  const IoDesc io = p->io(slice, x, nullptr);
  const PlanLayout* lay = nullptr;
  if (pl->n_mfma > 0) LORA_TRY(plan_layout(pl, single_io(io), (hipStream_t)stream, &lay));
  return hip_status(launch_sgmv_shrink(p->dtype, p->view(), pl->view(lay), io, v, v_ld, (hipStream_t)stream),
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
  if (pl->n_mfma > 0) LORA_TRY(plan_layout(pl, single_io(io), (hipStream_t)stream, &lay));
  return hip_status(launch_sgmv_expand(p->dtype, y_dtype, p->view(), pl->view(lay), io, v, v_ld,
                                       (hipStream_t)stream),
                    "sgmv_expand");
}

lora_status lora_apply(lora_pool* p, const lora_plan* pl, int32_t n_io, const lora_io* io,
                       int32_t y_dtype, void* stream) {
  clear_error();
  LORA_TRY(check_pool(p));
  LORA_TRY(check_plan(p, pl));
  LORA_TRY(check_ydt(p, y_dtype));
  IoSet ios;
  LORA_TRY(build_ioset(p, n_io, io, ios));
  if (pl->n_tokens == 0) return LORA_OK;
  const PlanLayout* lay = nullptr;
  if (pl->n_mfma > 0) LORA_TRY(plan_layout(pl, ios, (hipStream_t)stream, &lay));
  return hip_status(launch_apply(p->dtype, y_dtype, p->view(), pl->view(lay), ios, (hipStream_t)stream),
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

}  // extern "C"
