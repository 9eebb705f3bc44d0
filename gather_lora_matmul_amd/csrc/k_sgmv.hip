// Planned (SGMV) kernels: segments of tokens that share an adapter (multi-LoRA
// serving article, SGMV section).  MFMA tiles (up to 64 tokens of one adapter,
// kmfma.h) and short items (up to 4 tokens, vector ALUs, kvalu.h) are separate
// kernel instantiations, each with its own register budget; a plan's items are
// sorted MFMA tiles first, and each entry point launches one kernel per kind
// present.
#include <algorithm>

#include "kmfma.h"
#include "kvalu.h"

namespace lora {

constexpr int kSgNT = 256;
constexpr int kShortLds = ((kSgNT / 64) * kShortG * kMaxR + kShortG * kMaxR) * 4;

__device__ __forceinline__ void item_tokens(const PlanView& pl, const PlanItem& it,
                                            int (&tok)[kShortG]) {
#pragma unroll
  for (int g = 0; g < kShortG; ++g) tok[g] = g < it.count ? pl.perm[it.start + g] : -1;
}

__device__ __forceinline__ int split_rows(int d_out, int nsplit) {
  return (((d_out + nsplit - 1) / nsplit) + 63) & ~63;
}

// ---- shrink -------------------------------------------------------------------
// Short items: block = (item, group of rank rows).  MFMA tiles: block = (tile,
// 32-token half).  v rows are indexed by original token.
template <typename T, typename X, int U>
__global__ __launch_bounds__(kSgNT) void k_sgmv_shrink_short(PoolView pv, PlanView pl, IoDesc io,
                                                             float* __restrict__ v, int v_ld,
                                                             int first, int count, int ngroups,
                                                             int rpg) {
  __shared__ __attribute__((aligned(16))) char lds[kShortLds];
  float* part = reinterpret_cast<float*>(lds);
  float* vsh = part + (kSgNT / 64) * kShortG * kMaxR;
  int it, grp;
  xcd_unit_split(blockIdx.x, ngroups, it, grp);
  if (it >= count) return;
  const PlanItem item = pl.items[first + it];
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
      xr[g] = tok[g] >= 0 ? reinterpret_cast<const char*>(io.x) + (int64_t)tok[g] * io.d_in * sizeof(X)
                          : nullptr;
    valu_shrink<T, X, kSgNT, U, kShortG, 8>(pv, e, io.d_in, io.npa, xr, k_lo, k_hi, k_hi, part, vsh,
                                            kMaxR, kQRow);
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
__global__ __launch_bounds__(kSgNT, 2) void k_sgmv_expand_short(PoolView pv, PlanView pl, IoDesc io,
                                                                const float* __restrict__ v, int v_ld,
                                                                int first, int count, int nsplit) {
  __shared__ float vsh[kShortG * kMaxR];
  int it, q;
  xcd_unit_split(blockIdx.x, nsplit, it, q);
  if (it >= count) return;
  const PlanItem item = pl.items[first + it];
  if (item.adapter < 0) return;
  const DevEntry e = pv.entries[io.slice * pv.max_adapters + item.adapter];
  if (e.rank <= 0) return;
  const int rps = split_rows(io.d_out, nsplit);
  const int m_lo = q * rps;
  const int m_hi = min(io.d_out, m_lo + rps);
  if (m_lo >= m_hi) return;
  int tok[kShortG];
  item_tokens(pl, item, tok);
  for (int idx = threadIdx.x; idx < kShortG * e.rs; idx += kSgNT) {
    const int g = idx / e.rs;
    const int k = idx - g * e.rs;
    float vk = (tok[g] >= 0 && k < e.rank) ? v[(int64_t)tok[g] * v_ld + k] : 0.f;
    // quantised pages: v[k] * b_scale[k], ready for the codes of B
    if constexpr (is_quant<T>()) vk = k < e.rank ? vk * q_scale(pv, e.q_off + e.rank + k) : 0.f;
    vsh[g * kMaxR + k] = vk;
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
// the block (LDS).
template <typename T, typename X, typename TY, int U>
__global__ __launch_bounds__(kSgNT, 2) void k_apply_short(PoolView pv, PlanView pl, IoSet ios,
                                                          int first, int count, int nsplit) {
  __shared__ __attribute__((aligned(16))) char lds[kShortLds];
  float* part = reinterpret_cast<float*>(lds);
  float* vsh = part + (kSgNT / 64) * kShortG * kMaxR;
  int unit, q;
  xcd_unit_split(blockIdx.x, nsplit, unit, q);
  if (unit >= count * ios.n_io) return;
  const int it = unit / ios.n_io;
  const int io_i = unit - it * ios.n_io;
  const PlanItem item = pl.items[first + it];
  if (item.adapter < 0) return;
  const IoDesc io = ios.io[io_i];
  const DevEntry e = pv.entries[io.slice * pv.max_adapters + item.adapter];
  if (e.rank <= 0) return;
  const int rps = split_rows(io.d_out, nsplit);
  const int m_lo = q * rps;
  const int m_hi = min(io.d_out, m_lo + rps);
  if (m_lo >= m_hi) return;
  int tok[kShortG];
  item_tokens(pl, item, tok);
  const char* xr[kShortG];
  char* yr[kShortG];
  float sg[kShortG];
#pragma unroll
  for (int g = 0; g < kShortG; ++g) {
    xr[g] = tok[g] >= 0 ? reinterpret_cast<const char*>(io.x) + (int64_t)tok[g] * io.d_in * sizeof(X) : nullptr;
    yr[g] = tok[g] >= 0 ? reinterpret_cast<char*>(io.y) + (int64_t)tok[g] * io.d_out * sizeof(TY) : nullptr;
    sg[g] = e.scale;
  }
  valu_shrink<T, X, kSgNT, U, kShortG, 8>(pv, e, io.d_in, io.npa, xr, 0, e.rank, e.rs, part, vsh,
                                          kMaxR, kQRowCol);
  valu_expand_any<T, TY, kSgNT, kShortG>(pv, e, vsh, kMaxR, sg, yr, m_lo, m_hi);
}

// ---- MFMA tiles: persistent kernels (one block range per block) -----------------
template <typename T>
__global__ __launch_bounds__(kMT, 2) void k_sgmv_shrink_tiles(PoolView pv, PlanView pl, IoDesc io,
                                                              float* __restrict__ v, int v_ld) {
  __shared__ __attribute__((aligned(16))) char misc[kMiscB];
  __shared__ __attribute__((aligned(16))) char ba[kBufB];
  __shared__ __attribute__((aligned(16))) char bb[kBufB];
  __shared__ __attribute__((aligned(16))) char bc[kBufB];
  const int L = logical_block(blockIdx.x, pl.G);
  shrink_range<T>(pv, pl, [&](int) -> const IoDesc& { return io; }, L, v, v_ld, LdsBufs{misc, ba, bb, bc});
}

// Split API: v rows of the tiles whose shrink several blocks shared (block = tile).
__global__ __launch_bounds__(kMT) void k_sgmv_shrink_reduce(PoolView pv, PlanView pl, IoDesc io,
                                                            float* __restrict__ v, int v_ld) {
  __shared__ int toks[kTileM];
  const int tile = blockIdx.x;
  const PlanItem item = pl.items[tile];
  const int rank = pv.entries[io.slice * pv.max_adapters + item.adapter].rank;
  shrink_reduce_tile(pl, io, tile, rank, v, v_ld, toks);
}

template <typename T, typename TY>
__global__ __launch_bounds__(kMT, 2) void k_sgmv_expand_tiles(PoolView pv, PlanView pl, IoDesc io,
                                                              const float* __restrict__ v, int v_ld) {
  __shared__ __attribute__((aligned(16))) char misc[kOffApg];
  __shared__ __attribute__((aligned(16))) char ba[kVpB];
  __shared__ __attribute__((aligned(16))) char bb[kVpB];
  __shared__ __attribute__((aligned(16))) char bc[kDsB];
  const int L = logical_block(blockIdx.x, pl.G);
  expand_range<T, TY, false>(pv, pl, [&](int) -> const IoDesc& { return io; }, L, v, v_ld,
                            LdsBufs{misc, ba, bb, bc});
}

// Fused apply on MFMA tiles: two launches on one stream.  The first runs every
// block's shrink range (over the launch slices in order) and keeps each
// contribution as a partial tile; the second runs the expand ranges, V of a
// tile being the sum of its partial tiles (block order).  v itself is never
// materialized.
template <typename T>
__global__ __launch_bounds__(kMT, 2) void k_apply_shrink_tiles(PoolView pv, PlanView pl, IoSet ios) {
  __shared__ __attribute__((aligned(16))) char misc[kMiscB];
  __shared__ __attribute__((aligned(16))) char ba[kBufB];
  __shared__ __attribute__((aligned(16))) char bb[kBufB];
  __shared__ __attribute__((aligned(16))) char bc[kBufB];
  const int L = logical_block(blockIdx.x, pl.G);
  const LdsBufs lb{misc, ba, bb, bc};
  // the expand launch that follows claims its pool through this counter
  if (pl.pool && blockIdx.x == 0 && threadIdx.x == 0)
    reinterpret_cast<int*>(pl.part)[4 * (int64_t)pl.pool[2]] = 0;
  shrink_range<T>(pv, pl, [&](int j) -> const IoDesc& { return ios.io[j]; }, L, nullptr, 0, lb);
}

template <typename T, typename TY>
__global__ __launch_bounds__(kMT, 2) void k_apply_expand_tiles(PoolView pv, PlanView pl, IoSet ios) {
  __shared__ __attribute__((aligned(16))) char misc[kOffApg];
  __shared__ __attribute__((aligned(16))) char ba[kVpB];
  __shared__ __attribute__((aligned(16))) char bb[kVpB];
  __shared__ __attribute__((aligned(16))) char bc[kDsB];
  const int L = logical_block(blockIdx.x, pl.G);
  const LdsBufs lb{misc, ba, bb, bc};
  expand_range<T, TY, true>(pv, pl, [&](int j) -> const IoDesc& { return ios.io[j]; }, L, nullptr, 0,
                            lb);
}

// ---- launchers ------------------------------------------------------------------
namespace {

inline int sg_u(int d_in, int E) { return d_in / E > kSgNT ? 2 : 1; }

// Output-row splits: grow until the grid reaches `target` blocks, keeping at
// least `min_rows` rows per block.
inline int pick_nsplit(int units, int d_out, int target, int min_rows) {
  int nsplit = 1;
  while ((long)units * nsplit < target && d_out / (nsplit * 2) >= min_rows) nsplit *= 2;
  return nsplit;
}

template <typename T, typename X>
hipError_t shrink_t(const PoolView& pv, const PlanView& pl, const IoDesc& io, float* v, int v_ld,
                    hipStream_t s) {
  constexpr int E = ET<T>::E;
  const int n_short = pl.n_items - pl.n_mfma;
  if constexpr (ET<T>::bytes == 2) {
    if (pl.n_mfma > 0) {
      hipLaunchKernelGGL((k_sgmv_shrink_tiles<T>), dim3(pl.G), dim3(kMT), 0, s, pv, pl, io, v, v_ld);
      hipLaunchKernelGGL(k_sgmv_shrink_reduce, dim3(pl.n_mfma), dim3(kMT), 0, s, pv, pl, io, v, v_ld);
    }
  }
  if (n_short > 0) {
    int rpg = 16;
    while (rpg > 4 && (long)n_short * ((v_ld + rpg - 1) / rpg) < 512) rpg /= 2;
    const int ngroups = (v_ld + rpg - 1) / rpg;
    const dim3 grid(xcd_grid(n_short, ngroups));
    if (sg_u(io.d_in, E) == 1)
      hipLaunchKernelGGL((k_sgmv_shrink_short<T, X, 1>), grid, dim3(kSgNT), 0, s, pv, pl, io, v, v_ld,
                         pl.n_mfma, n_short, ngroups, rpg);
    else
      hipLaunchKernelGGL((k_sgmv_shrink_short<T, X, 2>), grid, dim3(kSgNT), 0, s, pv, pl, io, v, v_ld,
                         pl.n_mfma, n_short, ngroups, rpg);
  }
  return hipGetLastError();
}

template <typename T, typename TY>
hipError_t expand_t(const PoolView& pv, const PlanView& pl, const IoDesc& io, const float* v,
                    int v_ld, hipStream_t s) {
  const int n_short = pl.n_items - pl.n_mfma;
  if constexpr (ET<T>::bytes == 2) {
    if (pl.n_mfma > 0)
      hipLaunchKernelGGL((k_sgmv_expand_tiles<T, TY>), dim3(pl.G), dim3(kMT), 0, s, pv, pl, io, v,
                         v_ld);
  }
  if (n_short > 0) {
    const int nsplit = pick_nsplit(n_short, io.d_out, 1024, 1024);
    hipLaunchKernelGGL((k_sgmv_expand_short<T, TY>), dim3(xcd_grid(n_short, nsplit)), dim3(kSgNT), 0,
                       s, pv, pl, io, v, v_ld, pl.n_mfma, n_short, nsplit);
  }
  return hipGetLastError();
}

template <typename T, typename X, typename TY>
hipError_t apply_t(const PoolView& pv, const PlanView& pl, const IoSet& ios, hipStream_t s) {
  constexpr int E = ET<T>::E;
  const int n_short = pl.n_items - pl.n_mfma;
  if constexpr (ET<T>::bytes == 2) {
    if (pl.n_mfma > 0) {
      hipLaunchKernelGGL((k_apply_shrink_tiles<T>), dim3(pl.G), dim3(kMT), 0, s, pv, pl, ios);
      hipLaunchKernelGGL((k_apply_expand_tiles<T, TY>), dim3(pl.G), dim3(kMT), 0, s, pv, pl, ios);
    }
  }
  if (n_short > 0) {
    const int units = n_short * ios.n_io;
    const int nsplit = pick_nsplit(units, ios.max_d_out, 512, 2048);
    const dim3 grid(xcd_grid(units, nsplit));
    if (sg_u(ios.max_d_in, E) == 1)
      hipLaunchKernelGGL((k_apply_short<T, X, TY, 1>), grid, dim3(kSgNT), 0, s, pv, pl, ios, pl.n_mfma,
                         n_short, nsplit);
    else
      hipLaunchKernelGGL((k_apply_short<T, X, TY, 2>), grid, dim3(kSgNT), 0, s, pv, pl, ios, pl.n_mfma,
                         n_short, nsplit);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sgmv_shrink(const Types& ty, const PoolView& pv, const PlanView& pl,
                              const IoDesc& io, float* v, int32_t v_ld, hipStream_t s) {
  if (pl.n_items == 0) return hipSuccess;
  switch (ty.w) {
    case LORA_F32: return shrink_t<float, float>(pv, pl, io, v, v_ld, s);
    case LORA_F16: return shrink_t<f16_t, f16_t>(pv, pl, io, v, v_ld, s);
    case LORA_BF16: return shrink_t<bf16_t, bf16_t>(pv, pl, io, v, v_ld, s);
    default:
      return ty.x == LORA_F16 ? shrink_t<fp8_t, f16_t>(pv, pl, io, v, v_ld, s)
                              : shrink_t<fp8_t, bf16_t>(pv, pl, io, v, v_ld, s);
  }
}

hipError_t launch_sgmv_expand(const Types& ty, const PoolView& pv, const PlanView& pl,
                              const IoDesc& io, const float* v, int32_t v_ld, hipStream_t s) {
  if (pl.n_items == 0) return hipSuccess;
  const bool yf = (ty.y == LORA_F32);
  switch (ty.w) {
    case LORA_F32: return expand_t<float, float>(pv, pl, io, v, v_ld, s);
    case LORA_F16:
      return yf ? expand_t<f16_t, float>(pv, pl, io, v, v_ld, s) : expand_t<f16_t, f16_t>(pv, pl, io, v, v_ld, s);
    case LORA_BF16:
      return yf ? expand_t<bf16_t, float>(pv, pl, io, v, v_ld, s)
                : expand_t<bf16_t, bf16_t>(pv, pl, io, v, v_ld, s);
    default:
      if (yf) return expand_t<fp8_t, float>(pv, pl, io, v, v_ld, s);
      return ty.y == LORA_F16 ? expand_t<fp8_t, f16_t>(pv, pl, io, v, v_ld, s)
                              : expand_t<fp8_t, bf16_t>(pv, pl, io, v, v_ld, s);
  }
}

hipError_t launch_apply(const Types& ty, const PoolView& pv, const PlanView& pl, const IoSet& ios,
                        hipStream_t s) {
  if (pl.n_items == 0) return hipSuccess;
  const bool yf = (ty.y == LORA_F32);
  switch (ty.w) {
    case LORA_F32: return apply_t<float, float, float>(pv, pl, ios, s);
    case LORA_F16:
      return yf ? apply_t<f16_t, f16_t, float>(pv, pl, ios, s) : apply_t<f16_t, f16_t, f16_t>(pv, pl, ios, s);
    case LORA_BF16:
      return yf ? apply_t<bf16_t, bf16_t, float>(pv, pl, ios, s)
                : apply_t<bf16_t, bf16_t, bf16_t>(pv, pl, ios, s);
    default:
      if (ty.x == LORA_F16)
        return yf ? apply_t<fp8_t, f16_t, float>(pv, pl, ios, s)
                  : apply_t<fp8_t, f16_t, f16_t>(pv, pl, ios, s);
      return yf ? apply_t<fp8_t, bf16_t, float>(pv, pl, ios, s)
                : apply_t<fp8_t, bf16_t, bf16_t>(pv, pl, ios, s);
  }
}

}  // namespace lora
