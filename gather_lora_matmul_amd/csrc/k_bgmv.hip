// Decode-form kernels (one token per request, adapter ids on the device):
// the BGMV operation of the S-LoRA paper explainer (section "BGMVカーネル"),
// y_i += s_a B_a (A_a x_i) with a different adapter -- and possibly a different
// rank -- per token, every adapter row gathered through the page table of the
// unified pool (section "Unified Paging").
#include <algorithm>
#include <cstdlib>

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
// whole shrink of its unit into LDS, then expands its row range.  The first
// pass of B rows (and y) is loaded before the shrink so both phases' loads are
// in flight together.  The splits of a unit share an XCD, so the repeated
// shrink reads hit that XCD's L2.  MAXN: largest B-row chunk count given a
// prefetching body in this variant (bigger rows take the plain path).
template <typename T, typename TY, int NT, int U, int NCH>
__device__ __forceinline__ void bgmv_fused_body(const PoolView& pv, const DevEntry& e,
                                                const IoDesc& io, int i, int m_lo, int m_hi,
                                                float* part, float* vsh) {
  constexpr int kKB = U == 1 ? 16 : 8;  // A rows per batch (16-byte loads per thread: kKB * U)
  const char* xr[1] = {reinterpret_cast<const char*>(io.x) + (int64_t)i * io.d_in * sizeof(T)};
  char* yrow = reinterpret_cast<char*>(io.y) + (int64_t)i * io.d_out * sizeof(TY);
  const float s = e.scale;
  if constexpr (NCH > 0) {
    ExpandPrefetch<T, TY, NT, NCH> pf;
    const int m0 = m_lo + (int)threadIdx.x;
    pf.load(pv, e, yrow, m0, m_hi);
    valu_shrink<T, NT, U, 1, kKB>(pv, e, io.d_in, io.npa, xr, 0, e.rank, e.rs, part, vsh, kMaxR);
    pf.finish(vsh, s, yrow, m0, m_hi);
    char* yr[1] = {yrow};
    valu_expand<T, TY, NT, NCH, 1>(pv, e, vsh, kMaxR, &s, yr, m_lo + NT * ExpandPrefetch<T, TY, NT, NCH>::RU,
                                   m_hi);
  } else {
    valu_shrink<T, NT, U, 1, kKB>(pv, e, io.d_in, io.npa, xr, 0, e.rank, e.rs, part, vsh, kMaxR);
    char* yr[1] = {yrow};
    valu_expand<T, TY, NT, 0, 1>(pv, e, vsh, kMaxR, &s, yr, m_lo, m_hi);
  }
}

// Fast body when A rows fit one page and one column pass covers d_in: every
// page id is read first (B rows: one vector load per row; A rows: scalar
// loads), then x, the first 16 A rows and the first pass of B rows and y are
// all issued together, so a block waits for one dependent lookup and one data
// round trip before its first arithmetic.
template <typename T, typename TY, int NT, int U, int NCH>
__device__ __forceinline__ void bgmv_fused_fast(const PoolView& pv, const DevEntry& e,
                                                const IoDesc& io, int i, int m_lo, int m_hi,
                                                float* part, float* vsh) {
  constexpr int E = ET<T>::E;
  constexpr int ELT = ET<T>::bytes;
  constexpr int NW = NT / 64;
  constexpr int KB = 16;
  constexpr int RU = rows_per_pass(NCH);
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int C = io.d_in / E;
  const int r = e.rank;
  const int mlast = m_hi - 1;
  const char* xrow = reinterpret_cast<const char*>(io.x) + (int64_t)i * io.d_in * ELT;
  char* yrow = reinterpret_cast<char*>(io.y) + (int64_t)i * io.d_out * sizeof(TY);
  // (1) page ids: B rows (vector loads), the first 16 A rows (scalar loads);
  //     indices are clamped, so every load below is unconditional
  int64_t bo[RU];
#pragma unroll
  for (int ru = 0; ru < RU; ++ru) bo[ru] = b_offset(pv, e, ELT, min(m_lo + t + ru * NT, mlast));
  int64_t ab[KB];
#pragma unroll
  for (int kk = 0; kk < KB; ++kk) ab[kk] = a_row_uniform(pv, e, ELT, min(kk, r - 1));
  int cc[U];
  bool cv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    cv[u] = t + NT * u < C;
    cc[u] = cv[u] ? t + NT * u : C - 1;
  }
  // (2) all data of the first pass
  uint4 xr[U];
#pragma unroll
  for (int u = 0; u < U; ++u) xr[u] = ld16(xrow + (int64_t)cc[u] * 16);
  uint4 a[KB][U];
#pragma unroll
  for (int kk = 0; kk < KB; ++kk)
#pragma unroll
    for (int u = 0; u < U; ++u) a[kk][u] = ld16(pv.pages + ab[kk] + (int64_t)cc[u] * 16);
  uint4 b[RU][NCH];
  float yv[RU];
#pragma unroll
  for (int ru = 0; ru < RU; ++ru) {
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) b[ru][ch] = ld16(pv.pages + bo[ru] + ch * 16);
    yv[ru] = load_y<TY>(yrow, min(m_lo + t + ru * NT, mlast));
  }
  // (3) shrink: first 16 rank rows, then the rest of the rank
#pragma unroll
  for (int u = 0; u < U; ++u) xr[u] = keep16(xr[u], cv[u]);
#pragma unroll
  for (int kk = 0; kk < KB; ++kk) {
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) acc = dot16<T>(a[kk][u], xr[u], acc);
    const float sum = wave_sum(acc);
    if (lane == 0 && kk < r) part[w * kMaxR + kk] = sum;
  }
  for (int k0 = KB; k0 < r; k0 += KB) {
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) ab[kk] = a_row_uniform(pv, e, ELT, min(k0 + kk, r - 1));
#pragma unroll
    for (int kk = 0; kk < KB; ++kk)
#pragma unroll
      for (int u = 0; u < U; ++u) a[kk][u] = ld16(pv.pages + ab[kk] + (int64_t)cc[u] * 16);
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) {
      float acc = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) acc = dot16<T>(a[kk][u], xr[u], acc);
      const float sum = wave_sum(acc);
      if (lane == 0 && k0 + kk < r) part[w * kMaxR + k0 + kk] = sum;
    }
  }
  __syncthreads();
  for (int k = t; k < e.rs; k += NT) {
    float sum = 0.f;
    if (k < r) {
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) sum += part[ww * kMaxR + k];
    }
    vsh[k] = sum;
  }
  __syncthreads();
  // (4) expand the prefetched rows, then any remaining ones
  const float s = e.scale;
#pragma unroll
  for (int ru = 0; ru < RU; ++ru) {
    const int m = m_lo + t + ru * NT;
    float acc = 0.f;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) acc = dot16v<T>(b[ru][ch], vsh + ch * E, acc);
    if (m < m_hi) store_y<TY>(yrow, m, __builtin_fmaf(s, acc, yv[ru]));
  }
  char* yr[1] = {yrow};
  valu_expand<T, TY, NT, NCH, 1>(pv, e, vsh, kMaxR, &s, yr, m_lo + NT * RU, m_hi);
}

template <typename T, typename TY, int NT, int U, int MAXN>
__global__ __launch_bounds__(NT) void k_bgmv_apply(PoolView pv, IoSet ios,
                                                   const int32_t* __restrict__ ids, int n,
                                                   int nsplit, int rps) {
  __shared__ float part[(NT / 64) * kMaxR];
  __shared__ float vsh[kMaxR];
  int unit, q;
  xcd_unit_split(blockIdx.x, nsplit, unit, q);
  if (unit >= n * ios.n_io) return;
  // slice-major: the launcher puts the costliest slices first, so their units
  // are dispatched first and the cheaper ones fill the compute units that free up
  const int io_i = unit / n;
  const int i = unit - io_i * n;
  const IoDesc io = ios.io[io_i];
  const int a = ids[i];
  if (a < 0) return;
  const DevEntry e = pv.entries[io.slice * pv.max_adapters + a];
  if (e.rank <= 0) return;
  const int m_lo = q * rps;
  const int m_hi = min(io.d_out, m_lo + rps);
  if (m_lo >= m_hi) return;
  const int nch = e.rs / ET<T>::E;
  const bool fast = io.npa == 1 && io.d_in / ET<T>::E <= NT * U;
#define LORA_FUSED_CASE(N)                                                                   \
  if (N <= MAXN && nch == N) {                                                               \
    if (fast)                                                                                \
      bgmv_fused_fast<T, TY, NT, U, (N <= MAXN ? N : 1)>(pv, e, io, i, m_lo, m_hi, part, vsh); \
    else                                                                                     \
      bgmv_fused_body<T, TY, NT, U, (N <= MAXN ? N : 0)>(pv, e, io, i, m_lo, m_hi, part, vsh); \
    return;                                                                                  \
  }
  LORA_FUSED_CASE(1)
  LORA_FUSED_CASE(2)
  LORA_FUSED_CASE(4)
  LORA_FUSED_CASE(8)
  LORA_FUSED_CASE(16)
#undef LORA_FUSED_CASE
  bgmv_fused_body<T, TY, NT, U, 0>(pv, e, io, i, m_lo, m_hi, part, vsh);
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

template <typename T, typename TY, int NT, int U>
void apply_launch(const PoolView& pv, const IoSet& ios, const int32_t* ids, int n, dim3 grid,
                  int nsplit, int rps, hipStream_t s) {
  // variant by the pool's longest B row, so short-row pools get lean kernels
  if (pv.max_nch <= 2)
    hipLaunchKernelGGL((k_bgmv_apply<T, TY, NT, U, 2>), grid, dim3(NT), 0, s, pv, ios, ids, n, nsplit, rps);
  else if (pv.max_nch <= 4)
    hipLaunchKernelGGL((k_bgmv_apply<T, TY, NT, U, 4>), grid, dim3(NT), 0, s, pv, ios, ids, n, nsplit, rps);
  else
    hipLaunchKernelGGL((k_bgmv_apply<T, TY, NT, U, 8>), grid, dim3(NT), 0, s, pv, ios, ids, n, nsplit, rps);
}

template <typename T, typename TY>
hipError_t apply_t(const PoolView& pv, const IoSet& ios_in, const int32_t* ids, int n,
                   hipStream_t s) {
  constexpr int E = ET<T>::E;
  // slices by decreasing bytes per token unit (d_in + d_out): blocks are
  // dispatched in unit order, so the longest units start first
  IoSet ios = ios_in;
  std::stable_sort(ios.io, ios.io + ios.n_io, [](const IoDesc& a, const IoDesc& b) {
    return a.d_in + a.d_out > b.d_in + b.d_out;
  });
  const int units = n * ios.n_io;
  // Splitting a unit repeats its whole shrink, which costs more than it
  // gains (measured, also when only the units with the largest B are split);
  // split only when there are fewer units than CUs.
  int nsplit = 1;
  while ((long)units * nsplit < 256 && ios.max_d_out / (nsplit * 2) >= 512) nsplit *= 2;
  const int rps = (((ios.max_d_out + nsplit - 1) / nsplit) + 63) & ~63;
  const dim3 grid(xcd_grid(units, nsplit));
  const int C = ios.max_d_in / E;
  if (C >= 512) {
    if (pick_u(ios.max_d_in, E, 512) == 1)
      apply_launch<T, TY, 512, 1>(pv, ios, ids, n, grid, nsplit, rps, s);
    else
      apply_launch<T, TY, 512, 2>(pv, ios, ids, n, grid, nsplit, rps, s);
  } else {
    apply_launch<T, TY, 256, 1>(pv, ios, ids, n, grid, nsplit, rps, s);
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
