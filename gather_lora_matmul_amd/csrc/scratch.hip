// Allocation-free planned apply: lora_apply with its partial-tile workspace in
// a static device array instead of a caller buffer, for callers that cannot
// allocate device memory (code under stream capture, tight serving loops,
// harnesses that forbid allocation).
//
// The array lives in this file's code object, one copy per GPU, held until the
// process ends.  Host code never passes its name to a kernel (on the host the
// name is a stand-in, not a device address): the device address of each GPU's
// copy is looked up once, with that GPU current, when a pool is created on it
// (or at the entry point's first call on that GPU), and only that address is
// used afterwards.
#include <mutex>

#include "runtime.h"

namespace lora {

constexpr size_t kScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// Device address of `device`'s scratch array; `device` must be current.
lora_status scratch_init(int device) {
  if (device < 0 || device >= kMaxDevices) return fail(LORA_E_ARG, "device %d out of range", device);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[device]) return LORA_OK;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p)
    return fail(LORA_E_HIP, "scratch address on device %d: %s", device, hipGetErrorString(e));
  g_scratch_ptr[device] = p;
  return LORA_OK;
}

static void* scratch_ptr(int device) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  return (device >= 0 && device < kMaxDevices) ? g_scratch_ptr[device] : nullptr;
}

}  // namespace lora

using namespace lora;

extern "C" lora_status lora_apply_noalloc(lora_pool* p, const lora_plan* pl, int32_t n_io,
                                          const lora_io* io, int32_t y_dtype, void* stream) {
  clear_error();
  if (!p) return fail(LORA_E_ARG, "null pool");
  if (pl && pl->built && pl->n_mfma > 0 && n_io >= 1 && n_io <= LORA_MAX_IO && io) {
    // a launch shape whose partial tiles do not fit is refused with the sizes
    size_t need = 0;
    if (lora_workspace_size(pl, n_io, io, &need) == LORA_OK && need > kScratchBytes)
      return fail(LORA_E_ARG, "launch needs %zu bytes of partial tiles, the static scratch holds %zu",
                  need, kScratchBytes);
    clear_error();
  }
  if (p->host_only) return fail(LORA_E_STATE, "host-only pool cannot run kernels");
  void* ws = scratch_ptr(p->device);
  if (!ws) {
    // first call on this GPU without a pool created there: look the address up
    // now, which needs the pool's device to be current
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || cur != p->device)
      return fail(LORA_E_STATE, "static scratch of device %d not set up (make it current)", p->device);
    const lora_status st = scratch_init(p->device);
    if (st) return st;
    ws = scratch_ptr(p->device);
  }
  return lora_apply(p, pl, n_io, io, y_dtype, ws, kScratchBytes, stream);
}
