// Decode-form kernels (one token per request, adapter ids on the device):
// the BGMV operation of the S-LoRA paper explainer (section "BGMVカーネル"),
// y_i += s_a B_a (A_a x_i) with a different adapter -- and possibly a different
// rank -- per token, every adapter row gathered through the page table of the
// unified pool (section "Unified Paging").
#include "kvalu.h"

namespace lora {

// ---- split API: shrink -------------------------------------------------------
// Block = (token i, group of `rpg` rank rows); groups of one token share an XCD
// so that x_i is read from HBM once.  Writes v[i][k] for the group's k < v_ld.
template <typename T, int NT, int U>
__global__ __launch_bounds__(NT) void k_bgmv_shrink(PoolView pv, IoDesc io,
                                                    const int32_t* __restrict__ ids, int n,
                                                    float* __restrict__ v, int v_ld, int ngroups,
                                                    int rpg) {
  __shared__ float part[(NT / 64) * kMaxR];
  __shared__ float vsh[kMaxR];
  int i, grp;
  xcd_unit_split(blockIdx.x, ngroups, i, grp);
  if (i >= n) return;
  const int a = ids[i];
  DevEntry e;
  e.rank = 0;
  if (a >= 0) e = pv.entries[io.slice * pv.max_adapters + a];
  const int k_lo = grp * rpg;
  const int k_end = min(k_lo + rpg, v_ld);
  const int k_hi = max(k_lo, min(e.rank, k_end));
  if (k_lo < k_hi) {
    const char* xr[1] = {reinterpret_cast<const char*>(io.x) + (int64_t)i * io.d_in * sizeof(T)};
    valu_shrink<T, NT, U, 1, 16>(pv, e, io.d_in, io.npa, xr, k_lo, k_hi, k_hi, part, vsh, kMaxR);
  }
  for (int k = k_lo + (int)threadIdx.x; k < k_end; k += NT)
    v[(int64_t)i * v_ld + k] = k < k_hi ? vsh[k] : 0.f;
}

// ---- split API: expand --------------------------------------------------------
// Block = (token i, range of `rps` output rows); v_i staged in LDS.
template <typename T, typename TY, int NT>
__global__ __launch_bounds__(NT) void k_bgmv_expand(PoolView pv, IoDesc io,
                                                    const float* __restrict__ v, int v_ld,
                                                    const int32_t* __restrict__ ids, int n,
                                                    const float* __restrict__ tok_scale,
                                                    int nsplit, int rps) {
  __shared__ float vsh[kMaxR];
  int i, q;
  xcd_unit_split(blockIdx.x, nsplit, i, q);
  if (i >= n) return;
  const int a = ids[i];
  if (a < 0) return;
  const DevEntry e = pv.entries[io.slice * pv.max_adapters + a];
  if (e.rank <= 0) return;
  const int m_lo = q * rps;
  const int m_hi = min(io.d_out, m_lo + rps);
  if (m_lo >= m_hi) return;
  for (int k = threadIdx.x; k < e.rs; k += NT) vsh[k] = k < e.rank ? v[(int64_t)i * v_ld + k] : 0.f;
  __syncthreads();
  const float s = tok_scale ? tok_scale[i] : e.scale;
  char* yr[1] = {reinterpret_cast<char*>(io.y) + (int64_t)i * io.d_out * sizeof(TY)};
  valu_expand_any<T, TY, NT, 1>(pv, e, vsh, kMaxR, &s, yr, m_lo, m_hi);
}

// ---- fused apply, several slices in one launch --------------------------------
// Block = ((token, slice) unit, output-row split).  Each block computes the
// whole shrink of its unit into LDS, then expands its row range.  The splits
// of a unit share an XCD, so the repeated shrink reads hit that XCD's L2.
template <typename T, typename TY, int NT, int U>
__global__ __launch_bounds__(NT) void k_bgmv_apply(PoolView pv, IoSet ios,
                                                   const int32_t* __restrict__ ids, int n,
                                                   int nsplit, int rps) {
  __shared__ float part[(NT / 64) * kMaxR];
  __shared__ float vsh[kMaxR];
  int unit, q;
  xcd_unit_split(blockIdx.x, nsplit, unit, q);
  if (unit >= n * ios.n_io) return;
  const int i = unit / ios.n_io;
  const int io_i = unit - i * ios.n_io;
  const IoDesc io = ios.io[io_i];
  const int a = ids[i];
  if (a < 0) return;
  const DevEntry e = pv.entries[io.slice * pv.max_adapters + a];
  if (e.rank <= 0) return;
  const int m_lo = q * rps;
  const int m_hi = min(io.d_out, m_lo + rps);
  if (m_lo >= m_hi) return;
  const char* xr[1] = {reinterpret_cast<const char*>(io.x) + (int64_t)i * io.d_in * sizeof(T)};
  valu_shrink<T, NT, U, 1, 16>(pv, e, io.d_in, io.npa, xr, 0, e.rank, e.rs, part, vsh, kMaxR);
  char* yr[1] = {reinterpret_cast<char*>(io.y) + (int64_t)i * io.d_out * sizeof(TY)};
  const float s = e.scale;
  valu_expand_any<T, TY, NT, 1>(pv, e, vsh, kMaxR, &s, yr, m_lo, m_hi);
}

// ---- launchers ----------------------------------------------------------------
namespace {

constexpr int kExpandNT = 256;

// Column chunks per thread for a shrink over d_in with NT threads.
inline int pick_u(int d_in, int E, int NT) {
  const int C = d_in / E;
  return C > NT ? 2 : 1;
}

template <typename T>
hipError_t shrink_t(const PoolView& pv, const IoDesc& io, const int32_t* ids, int n, float* v,
                    int v_ld, hipStream_t s) {
  constexpr int E = ET<T>::E;
  const int C = io.d_in / E;
  // rank rows per block: enough blocks to cover the chip, at most 16
  int rpg = 16;
  while (rpg > 4 && (long)n * ((v_ld + rpg - 1) / rpg) < 512) rpg /= 2;
  const int ngroups = (v_ld + rpg - 1) / rpg;
  const dim3 grid(xcd_grid(n, ngroups));
  if (C >= 512) {
    if (pick_u(io.d_in, E, 512) == 1)
      hipLaunchKernelGGL((k_bgmv_shrink<T, 512, 1>), grid, dim3(512), 0, s, pv, io, ids, n, v,
                         v_ld, ngroups, rpg);
    else
      hipLaunchKernelGGL((k_bgmv_shrink<T, 512, 2>), grid, dim3(512), 0, s, pv, io, ids, n, v,
                         v_ld, ngroups, rpg);
  } else {
    hipLaunchKernelGGL((k_bgmv_shrink<T, 256, 1>), grid, dim3(256), 0, s, pv, io, ids, n, v,
                       v_ld, ngroups, rpg);
  }
  return hipGetLastError();
}

inline void pick_split(int units, int d_out, int min_rows, int& nsplit, int& rps) {
  nsplit = 1;
  while ((long)units * nsplit < 1024 && d_out / (nsplit * 2) >= min_rows) nsplit *= 2;
  rps = (d_out + nsplit - 1) / nsplit;
}

template <typename T, typename TY>
hipError_t expand_t(const PoolView& pv, const IoDesc& io, const float* v, int v_ld,
                    const int32_t* ids, int n, const float* tok_scale, hipStream_t s) {
  int nsplit, rps;
  pick_split(n, io.d_out, 512, nsplit, rps);
  const dim3 grid(xcd_grid(n, nsplit));
  hipLaunchKernelGGL((k_bgmv_expand<T, TY, kExpandNT>), grid, dim3(kExpandNT), 0, s, pv, io, v,
                     v_ld, ids, n, tok_scale, nsplit, rps);
  return hipGetLastError();
}

template <typename T, typename TY>
hipError_t apply_t(const PoolView& pv, const IoSet& ios, const int32_t* ids, int n,
                   hipStream_t s) {
  constexpr int E = ET<T>::E;
  const int units = n * ios.n_io;
  int nsplit, rps;
  pick_split(units, ios.max_d_out, 2048, nsplit, rps);
  const dim3 grid(xcd_grid(units, nsplit));
  const int C = ios.max_d_in / E;
  if (C >= 512) {
    if (pick_u(ios.max_d_in, E, 512) == 1)
      hipLaunchKernelGGL((k_bgmv_apply<T, TY, 512, 1>), grid, dim3(512), 0, s, pv, ios, ids, n,
                         nsplit, rps);
    else
      hipLaunchKernelGGL((k_bgmv_apply<T, TY, 512, 2>), grid, dim3(512), 0, s, pv, ios, ids, n,
                         nsplit, rps);
  } else {
    hipLaunchKernelGGL((k_bgmv_apply<T, TY, 256, 1>), grid, dim3(256), 0, s, pv, ios, ids, n,
                       nsplit, rps);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bgmv_shrink(int dtype, const PoolView& pv, const IoDesc& io,
                              const int32_t* ids, int32_t n, float* v, int32_t v_ld,
                              hipStream_t s) {
  switch (dtype) {
    case LORA_F32: return shrink_t<float>(pv, io, ids, n, v, v_ld, s);
    case LORA_F16: return shrink_t<f16_t>(pv, io, ids, n, v, v_ld, s);
    default: return shrink_t<bf16_t>(pv, io, ids, n, v, v_ld, s);
  }
}

hipError_t launch_bgmv_expand(int dtype, int y_dtype, const PoolView& pv, const IoDesc& io,
                              const float* v, int32_t v_ld, const int32_t* ids, int32_t n,
                              const float* tok_scale, hipStream_t s) {
  const bool yf = (y_dtype == LORA_F32);
  switch (dtype) {
    case LORA_F32: return expand_t<float, float>(pv, io, v, v_ld, ids, n, tok_scale, s);
    case LORA_F16:
      return yf ? expand_t<f16_t, float>(pv, io, v, v_ld, ids, n, tok_scale, s)
                : expand_t<f16_t, f16_t>(pv, io, v, v_ld, ids, n, tok_scale, s);
    default:
      return yf ? expand_t<bf16_t, float>(pv, io, v, v_ld, ids, n, tok_scale, s)
                : expand_t<bf16_t, bf16_t>(pv, io, v, v_ld, ids, n, tok_scale, s);
  }
}

hipError_t launch_bgmv_apply(int dtype, int y_dtype, const PoolView& pv, const IoSet& ios,
                             const int32_t* ids, int32_t n, hipStream_t s) {
  const bool yf = (y_dtype == LORA_F32);
  switch (dtype) {
    case LORA_F32: return apply_t<float, float>(pv, ios, ids, n, s);
    case LORA_F16:
      return yf ? apply_t<f16_t, float>(pv, ios, ids, n, s) : apply_t<f16_t, f16_t>(pv, ios, ids, n, s);
    default:
      return yf ? apply_t<bf16_t, float>(pv, ios, ids, n, s)
                : apply_t<bf16_t, bf16_t>(pv, ios, ids, n, s);
  }
}

}  // namespace lora
