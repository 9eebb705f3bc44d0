// Decode with adapter ids on the device, grouped on the device: one
// workgroup builds the plan (devplan.h) into the caller's workspace, then the
// planned MFMA kernels run from it -- tokens sharing an adapter read its
// pages once, and the largest adapters spread over many compute units.
#include "devplan.h"

namespace lora {

namespace {

// Workgroup barrier for LDS traffic only: every exchange between the
// planner's threads goes through LDS (global memory is only read as input and
// written as output), so the barrier need not wait for global stores to land.
__device__ __forceinline__ void dp_barrier() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14));  // lgkmcnt(0) only
  asm volatile("s_barrier" ::: "memory");
}

struct DpDeviceCtx {
  template <class F>
  __device__ __forceinline__ void par(int n, F&& f) {
    for (int i = threadIdx.x; i < n; i += kDpThreads) f(i);
  }
  __device__ __forceinline__ void sync() { dp_barrier(); }
  __device__ __forceinline__ bool leader() const { return threadIdx.x == 0; }
  // a[0, n) -> its inclusive prefix sums (n <= kDpThreads): a scan within each
  // wave by lane shifts, then every wave adds the totals of the waves before it
  __device__ __forceinline__ void scan(int32_t* a, int32_t* wtot, int n) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    int v = t < n ? a[t] : 0;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int u = __shfl_up(v, d, 64);
      if (lane >= d) v += u;
    }
    if (lane == 63) wtot[w] = v;
    dp_barrier();
    int add = 0;
#pragma unroll
    for (int q = 0; q < kDpThreads / 64; ++q) add += q < w ? wtot[q] : 0;
    if (t < n) a[t] = v + add;
    dp_barrier();
  }
};

__global__ __launch_bounds__(kDpThreads) void k_devplan(PoolView pv, DevPlanShape sh,
                                                        const int32_t* __restrict__ ids,
                                                        DevPlanOut o) {
  __shared__ DevPlanLds s;
  DpDeviceCtx cx;
  devplan_run(cx, pv, sh, ids, o, s);
}

}  // namespace

hipError_t launch_devplan(const PoolView& pv, const int32_t* ids, const DevPlanShape& sh,
                          const DevPlanWs& w, char* ws, hipStream_t s) {
  hipLaunchKernelGGL(k_devplan, dim3(1), dim3(kDpThreads), 0, s, pv, sh, ids, devplan_out(ws, w));
  return hipGetLastError();
}

hipError_t launch_devplan_mfma(const Types& ty, const PoolView& pv, const IoSet& ios,
                               const DevPlanShape& sh, const DevPlanWs& w, char* ws, hipStream_t s) {
  const DevPlanOut o = devplan_out(ws, w);
  PlanView pl;
  pl.items = o.items;
  pl.perm = o.perm;
  pl.bs_shrink = reinterpret_cast<const RangePos*>(o.bs);
  pl.bs_expand = reinterpret_cast<const RangePos*>(o.be);
  pl.part_fl = reinterpret_cast<const int2*>(o.fl);
  pl.c_off = o.c_off;
  pl.c_ent = o.c_ent;
  pl.part = reinterpret_cast<float*>(ws + w.part);
  pl.n_tiles_dev = o.counts;
  pl.pool = nullptr;
  // the host knows only a bound on the tiles; no short items
  pl.n_items = sh.n;
  pl.n_tokens = sh.n;
  pl.n_mfma = sh.n;
  pl.G = sh.G;
  return launch_apply(ty, pv, pl, ios, s);
}

hipError_t launch_devplan_apply(const Types& ty, const PoolView& pv, const IoSet& ios,
                                const int32_t* ids, const DevPlanShape& sh, const DevPlanWs& w,
                                char* ws, hipStream_t s) {
  const hipError_t e = launch_devplan(pv, ids, sh, w, ws, s);
  if (e != hipSuccess) return e;
  return launch_devplan_mfma(ty, pv, ios, sh, w, ws, s);
}

}  // namespace lora
