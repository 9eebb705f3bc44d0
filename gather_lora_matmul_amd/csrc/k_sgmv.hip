// Planned (SGMV) kernels: segments of tokens that share an adapter (multi-LoRA
// serving article, SGMV section).  Short items (<= 4 tokens of one adapter) run
// on the vector ALUs and read each adapter row once for all their tokens;
// long groups run as 64-token bf16/fp16 MFMA tiles (kmfma.h).
#include "kmfma.h"
#include "kvalu.h"

namespace lora {

constexpr int kSgNT = 256;

__device__ __forceinline__ void item_tokens(const PlanView& pl, const PlanItem& it,
                                            int (&tok)[kShortG]) {
#pragma unroll
  for (int g = 0; g < kShortG; ++g) tok[g] = g < it.count ? pl.perm[it.start + g] : -1;
}

__device__ __forceinline__ int split_rows(int d_out, int nsplit) {
  return (((d_out + nsplit - 1) / nsplit) + 63) & ~63;
}

// ---- shrink -------------------------------------------------------------------
// Block = (item, group of rank rows).  v rows are indexed by original token.
template <typename T, int U>
__global__ __launch_bounds__(kSgNT) void k_sgmv_shrink(PoolView pv, PlanView pl, IoDesc io,
                                                       float* __restrict__ v, int v_ld,
                                                       int ngroups, int rpg) {
  __shared__ float part[(kSgNT / 64) * kShortG * kMaxR];
  __shared__ float vsh[kShortG * kMaxR];
  int it, grp;
  xcd_unit_split(blockIdx.x, ngroups, it, grp);
  if (it >= pl.n_items) return;
  const PlanItem item = pl.items[it];
  if (item.kind == 1) {
    if (grp == 0) mfma_shrink_tile<T, kSgNT>(pv, pl, item, io, v, v_ld);
    return;
  }
  int tok[kShortG];
  item_tokens(pl, item, tok);
  DevEntry e;
  e.rank = 0;
  if (item.adapter >= 0) e = pv.entries[io.slice * pv.max_adapters + item.adapter];
  const int k_lo = grp * rpg;
  const int k_end = min(k_lo + rpg, v_ld);
  if (k_lo >= k_end) return;
  const int k_hi = max(k_lo, min(e.rank, k_end));
  if (k_lo < k_hi) {
    const char* xr[kShortG];
#pragma unroll
    for (int g = 0; g < kShortG; ++g)
      xr[g] = tok[g] >= 0 ? reinterpret_cast<const char*>(io.x) + (int64_t)tok[g] * io.d_in * sizeof(T)
                          : nullptr;
    valu_shrink<T, kSgNT, U, kShortG, 8>(pv, e, io.d_in, io.npa, xr, k_lo, k_hi, k_hi, part, vsh,
                                         kMaxR);
  }
  const int nk = k_end - k_lo;
  for (int idx = threadIdx.x; idx < kShortG * nk; idx += kSgNT) {
    const int g = idx / nk;
    const int k = k_lo + (idx - g * nk);
    if (tok[g] >= 0) v[(int64_t)tok[g] * v_ld + k] = k < k_hi ? vsh[g * kMaxR + k] : 0.f;
  }
}

// ---- expand -------------------------------------------------------------------
// Block = (item, range of output rows).
template <typename T, typename TY>
__global__ __launch_bounds__(kSgNT) void k_sgmv_expand(PoolView pv, PlanView pl, IoDesc io,
                                                       const float* __restrict__ v, int v_ld,
                                                       int nsplit) {
  __shared__ float vsh[kShortG * kMaxR];
  int it, q;
  xcd_unit_split(blockIdx.x, nsplit, it, q);
  if (it >= pl.n_items) return;
  const PlanItem item = pl.items[it];
  if (item.adapter < 0) return;
  const DevEntry e = pv.entries[io.slice * pv.max_adapters + item.adapter];
  if (e.rank <= 0) return;
  const int rps = split_rows(io.d_out, nsplit);
  const int m_lo = q * rps;
  const int m_hi = min(io.d_out, m_lo + rps);
  if (m_lo >= m_hi) return;
  if (item.kind == 1) {
    mfma_expand_tile<T, TY, kSgNT>(pv, pl, item, e, io, v, v_ld, m_lo, m_hi);
    return;
  }
  int tok[kShortG];
  item_tokens(pl, item, tok);
  for (int idx = threadIdx.x; idx < kShortG * e.rs; idx += kSgNT) {
    const int g = idx / e.rs;
    const int k = idx - g * e.rs;
    vsh[g * kMaxR + k] = (tok[g] >= 0 && k < e.rank) ? v[(int64_t)tok[g] * v_ld + k] : 0.f;
  }
  __syncthreads();
  char* yr[kShortG];
  float sg[kShortG];
#pragma unroll
  for (int g = 0; g < kShortG; ++g) {
    yr[g] = tok[g] >= 0 ? reinterpret_cast<char*>(io.y) + (int64_t)tok[g] * io.d_out * sizeof(TY) : nullptr;
    sg[g] = e.scale;
  }
  valu_expand_any<T, TY, kSgNT, kShortG>(pv, e, vsh, kMaxR, sg, yr, m_lo, m_hi);
}

// ---- fused apply ----------------------------------------------------------------
// Block = ((item, slice) unit, output-row split).  The shrink result never leaves
// the block: LDS for short items, LDS for MFMA tiles.
template <typename T, typename TY, int U>
__global__ __launch_bounds__(kSgNT) void k_apply(PoolView pv, PlanView pl, IoSet ios, int nsplit) {
  __shared__ float part[(kSgNT / 64) * kShortG * kMaxR];
  __shared__ float vsh[kShortG * kMaxR];
  int unit, q;
  xcd_unit_split(blockIdx.x, nsplit, unit, q);
  if (unit >= pl.n_items * ios.n_io) return;
  const int it = unit / ios.n_io;
  const int io_i = unit - it * ios.n_io;
  const PlanItem item = pl.items[it];
  if (item.adapter < 0) return;
  const IoDesc io = ios.io[io_i];
  const DevEntry e = pv.entries[io.slice * pv.max_adapters + item.adapter];
  if (e.rank <= 0) return;
  const int rps = split_rows(io.d_out, nsplit);
  const int m_lo = q * rps;
  const int m_hi = min(io.d_out, m_lo + rps);
  if (m_lo >= m_hi) return;
  if (item.kind == 1) {
    mfma_apply_tile<T, TY, kSgNT>(pv, pl, item, e, io, m_lo, m_hi);
    return;
  }
  int tok[kShortG];
  item_tokens(pl, item, tok);
  const char* xr[kShortG];
  char* yr[kShortG];
  float sg[kShortG];
#pragma unroll
  for (int g = 0; g < kShortG; ++g) {
    xr[g] = tok[g] >= 0 ? reinterpret_cast<const char*>(io.x) + (int64_t)tok[g] * io.d_in * sizeof(T) : nullptr;
    yr[g] = tok[g] >= 0 ? reinterpret_cast<char*>(io.y) + (int64_t)tok[g] * io.d_out * sizeof(TY) : nullptr;
    sg[g] = e.scale;
  }
  valu_shrink<T, kSgNT, U, kShortG, 8>(pv, e, io.d_in, io.npa, xr, 0, e.rank, e.rs, part, vsh, kMaxR);
  valu_expand_any<T, TY, kSgNT, kShortG>(pv, e, vsh, kMaxR, sg, yr, m_lo, m_hi);
}

// ---- launchers ------------------------------------------------------------------
namespace {

inline int sg_u(int d_in, int E) { return d_in / E > kSgNT ? 2 : 1; }

template <typename T>
hipError_t shrink_t(const PoolView& pv, const PlanView& pl, const IoDesc& io, float* v, int v_ld,
                    hipStream_t s) {
  constexpr int E = ET<T>::E;
  int rpg = 16;
  while (rpg > 4 && (long)pl.n_items * ((v_ld + rpg - 1) / rpg) < 512) rpg /= 2;
  const int ngroups = (v_ld + rpg - 1) / rpg;
  const dim3 grid(xcd_grid(pl.n_items, ngroups));
  if (sg_u(io.d_in, E) == 1)
    hipLaunchKernelGGL((k_sgmv_shrink<T, 1>), grid, dim3(kSgNT), 0, s, pv, pl, io, v, v_ld, ngroups, rpg);
  else
    hipLaunchKernelGGL((k_sgmv_shrink<T, 2>), grid, dim3(kSgNT), 0, s, pv, pl, io, v, v_ld, ngroups, rpg);
  return hipGetLastError();
}

inline int pick_nsplit(int units, int d_out) {
  int nsplit = 1;
  while ((long)units * nsplit < 1024 && d_out / (nsplit * 2) >= 1024) nsplit *= 2;
  return nsplit;
}

template <typename T, typename TY>
hipError_t expand_t(const PoolView& pv, const PlanView& pl, const IoDesc& io, const float* v,
                    int v_ld, hipStream_t s) {
  const int nsplit = pick_nsplit(pl.n_items, io.d_out);
  const dim3 grid(xcd_grid(pl.n_items, nsplit));
  hipLaunchKernelGGL((k_sgmv_expand<T, TY>), grid, dim3(kSgNT), 0, s, pv, pl, io, v, v_ld, nsplit);
  return hipGetLastError();
}

template <typename T, typename TY>
hipError_t apply_t(const PoolView& pv, const PlanView& pl, const IoSet& ios, hipStream_t s) {
  constexpr int E = ET<T>::E;
  const int units = pl.n_items * ios.n_io;
  const int nsplit = pick_nsplit(units, ios.max_d_out);
  const dim3 grid(xcd_grid(units, nsplit));
  if (sg_u(ios.max_d_in, E) == 1)
    hipLaunchKernelGGL((k_apply<T, TY, 1>), grid, dim3(kSgNT), 0, s, pv, pl, ios, nsplit);
  else
    hipLaunchKernelGGL((k_apply<T, TY, 2>), grid, dim3(kSgNT), 0, s, pv, pl, ios, nsplit);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sgmv_shrink(int dtype, const PoolView& pv, const PlanView& pl, const IoDesc& io,
                              float* v, int32_t v_ld, hipStream_t s) {
  if (pl.n_items == 0) return hipSuccess;
  switch (dtype) {
    case LORA_F32: return shrink_t<float>(pv, pl, io, v, v_ld, s);
    case LORA_F16: return shrink_t<f16_t>(pv, pl, io, v, v_ld, s);
    default: return shrink_t<bf16_t>(pv, pl, io, v, v_ld, s);
  }
}

hipError_t launch_sgmv_expand(int dtype, int y_dtype, const PoolView& pv, const PlanView& pl,
                              const IoDesc& io, const float* v, int32_t v_ld, hipStream_t s) {
  if (pl.n_items == 0) return hipSuccess;
  const bool yf = (y_dtype == LORA_F32);
  switch (dtype) {
    case LORA_F32: return expand_t<float, float>(pv, pl, io, v, v_ld, s);
    case LORA_F16:
      return yf ? expand_t<f16_t, float>(pv, pl, io, v, v_ld, s) : expand_t<f16_t, f16_t>(pv, pl, io, v, v_ld, s);
    default:
      return yf ? expand_t<bf16_t, float>(pv, pl, io, v, v_ld, s)
                : expand_t<bf16_t, bf16_t>(pv, pl, io, v, v_ld, s);
  }
}

hipError_t launch_apply(int dtype, int y_dtype, const PoolView& pv, const PlanView& pl,
                        const IoSet& ios, hipStream_t s) {
  if (pl.n_items == 0) return hipSuccess;
  const bool yf = (y_dtype == LORA_F32);
  switch (dtype) {
    case LORA_F32: return apply_t<float, float>(pv, pl, ios, s);
    case LORA_F16:
      return yf ? apply_t<f16_t, float>(pv, pl, ios, s) : apply_t<f16_t, f16_t>(pv, pl, ios, s);
    default:
      return yf ? apply_t<bf16_t, float>(pv, pl, ios, s) : apply_t<bf16_t, bf16_t>(pv, pl, ios, s);
  }
}

}  // namespace lora
