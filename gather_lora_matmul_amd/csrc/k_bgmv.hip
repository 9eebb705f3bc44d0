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
template <typename T, typename X, int NT, int U>
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
  if (adapter_in_table(pv, a)) e = pv.entries[io.slice * pv.max_adapters + a];
  const int k_lo = grp * rpg;
  const int k_end = min(k_lo + rpg, v_ld);
  const int k_hi = max(k_lo, min(e.rank, k_end));
  if (k_lo < k_hi) {
    const char* xr[1] = {reinterpret_cast<const char*>(io.x) + (int64_t)i * io.d_in * sizeof(X)};
    valu_shrink<T, X, NT, U, 1, 16>(pv, e, io.d_in, io.npa, xr, k_lo, k_hi, k_hi, part, vsh, kMaxR,
                                    kQRow);
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
  if (!adapter_in_table(pv, a)) return;
  const DevEntry e = pv.entries[io.slice * pv.max_adapters + a];
  if (e.rank <= 0) return;
  const int m_lo = q * rps;
  const int m_hi = min(io.d_out, m_lo + rps);
  if (m_lo >= m_hi) return;
  for (int k = threadIdx.x; k < e.rs; k += NT) {
    float vk = k < e.rank ? v[(int64_t)i * v_ld + k] : 0.f;
    if constexpr (is_quant<T>()) vk = k < e.rank ? vk * q_scale(pv, e.q_off + e.rank + k) : 0.f;
    vsh[k] = vk;
  }
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
template <typename T, typename X, typename TY, int NT, int U, int NCH>
__device__ __forceinline__ void bgmv_fused_body(const PoolView& pv, const DevEntry& e,
                                                const IoDesc& io, int i, int m_lo, int m_hi,
                                                float* part, float* vsh) {
  constexpr int kKB = U == 1 ? 16 : 8;  // A rows per batch (16-byte loads per thread: kKB * U)
  const char* xr[1] = {reinterpret_cast<const char*>(io.x) + (int64_t)i * io.d_in * sizeof(X)};
  char* yrow = reinterpret_cast<char*>(io.y) + (int64_t)i * io.d_out * sizeof(TY);
  const float s = e.scale;
  if constexpr (NCH > 0) {
    ExpandPrefetch<T, TY, NT, NCH> pf;
    const int m0 = m_lo + (int)threadIdx.x;
    pf.load(pv, e, yrow, m0, m_hi);
    valu_shrink<T, X, NT, U, 1, kKB>(pv, e, io.d_in, io.npa, xr, 0, e.rank, e.rs, part, vsh, kMaxR,
                                     kQRowCol);
    pf.finish(vsh, s, yrow, m0, m_hi);
    char* yr[1] = {yrow};
    valu_expand<T, TY, NT, NCH, 1>(pv, e, vsh, kMaxR, &s, yr, m_lo + NT * ExpandPrefetch<T, TY, NT, NCH>::RU,
                                   m_hi);
  } else {
    valu_shrink<T, X, NT, U, 1, kKB>(pv, e, io.d_in, io.npa, xr, 0, e.rank, e.rs, part, vsh, kMaxR,
                                     kQRowCol);
    char* yr[1] = {yrow};
    valu_expand<T, TY, NT, 0, 1>(pv, e, vsh, kMaxR, &s, yr, m_lo, m_hi);
  }
}

// Fast body when A rows fit one page and one column pass covers d_in: every
// page id is read first (B rows: one vector load per row; A rows: scalar
// loads), then x, the first 16 A rows and the first pass of B rows and y are
// all issued together, so a block waits for one dependent lookup and one data
// round trip before its first arithmetic.
// x of token i as this thread's column chunks (the registers the fast body
// dots every A row against).
template <typename T, typename X, int NT, int U>
__device__ __forceinline__ void load_x_regs(const IoDesc& io, int i,
                                            uint4 (&xr)[U][x_chunks<T, X>()]) {
  constexpr int XC = x_chunks<T, X>();
  const int C = io.d_in / ET<T>::E;
  const char* xrow = reinterpret_cast<const char*>(io.x) + (int64_t)i * io.d_in * (int)sizeof(X);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = min((int)threadIdx.x + NT * u, C - 1);
#pragma unroll
    for (int q = 0; q < XC; ++q) xr[u][q] = ld16(xrow + ((int64_t)c * XC + q) * 16);
  }
}

// LOADX: load x into xr along with the first pass; otherwise xr already holds
// this token's x (slices sharing one x).
template <typename T, typename X, typename TY, int NT, int U, int NCH, bool LOADX = true>
__device__ __forceinline__ void bgmv_fused_fast(const PoolView& pv, const DevEntry& e,
                                                const IoDesc& io, int i, int m_lo, int m_hi,
                                                float* part, float* vsh,
                                                uint4 (&xr)[U][x_chunks<T, X>()]) {
  constexpr int E = ET<T>::E;
  constexpr int ELT = ET<T>::bytes;
  constexpr int XC = x_chunks<T, X>();
  constexpr int NW = NT / 64;
  constexpr int KB = 16;
  constexpr int RU = rows_per_pass(NCH);
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int C = io.d_in / E;
  const int r = e.rank;
  const int mlast = m_hi - 1;
  const char* xrow = reinterpret_cast<const char*>(io.x) + (int64_t)i * io.d_in * (int)sizeof(X);
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
  if constexpr (LOADX) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < XC; ++q) xr[u][q] = ld16(xrow + ((int64_t)cc[u] * XC + q) * 16);
  }
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
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int q = 0; q < XC; ++q) xr[u][q] = keep16(xr[u][q], cv[u]);
#pragma unroll
  for (int kk = 0; kk < KB; ++kk) {
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) acc = dotwx<T, X>(a[kk][u], xr[u], acc);
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
      for (int u = 0; u < U; ++u) acc = dotwx<T, X>(a[kk][u], xr[u], acc);
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
      // quantised pages: v[k] * b_scale[k], ready for the codes of B
      if constexpr (is_quant<T>())
        sum *= q_scale(pv, e.q_off + k) * q_scale(pv, e.q_off + r + k);
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

// One (slice, token) unit, output rows [q * rps, (q + 1) * rps): the whole
// shrink of the token into LDS, then the expand of those rows.  Returns at
// once (block-uniform) for skipped tokens and empty row ranges.
template <typename T, typename X, typename TY, int NT, int U, int MAXN>
__device__ __forceinline__ void fused_unit(const PoolView& pv, const IoSet& ios,
                                           const int32_t* __restrict__ ids, int n, int unit,
                                           int q, int rps, float* part, float* vsh) {
  const int io_i = unit / n;
  const int i = unit - io_i * n;
  const IoDesc io = ios.io[io_i];
  const int a = ids[i];
  if (!adapter_in_table(pv, a)) return;
  const DevEntry e = pv.entries[io.slice * pv.max_adapters + a];
  if (e.rank <= 0) return;
  const int m_lo = q * rps;
  const int m_hi = min(io.d_out, m_lo + rps);
  if (m_lo >= m_hi) return;
  const int nch = e.rs / ET<T>::E;
  const bool fast = io.npa == 1 && io.d_in / ET<T>::E <= NT * U;
  uint4 xr[U][x_chunks<T, X>()];
#define LORA_FUSED_CASE(N)                                                                   \
  if (N <= MAXN && nch == N) {                                                               \
    if (fast)                                                                                \
      bgmv_fused_fast<T, X, TY, NT, U, (N <= MAXN ? N : 1)>(pv, e, io, i, m_lo, m_hi, part, vsh, xr); \
    else                                                                                     \
      bgmv_fused_body<T, X, TY, NT, U, (N <= MAXN ? N : 0)>(pv, e, io, i, m_lo, m_hi, part, vsh); \
    return;                                                                                  \
  }
  LORA_FUSED_CASE(1)
  LORA_FUSED_CASE(2)
  LORA_FUSED_CASE(4)
  LORA_FUSED_CASE(8)
  LORA_FUSED_CASE(16)
#undef LORA_FUSED_CASE
  bgmv_fused_body<T, X, TY, NT, U, 0>(pv, e, io, i, m_lo, m_hi, part, vsh);
}

#ifdef LORA_BLOCK_TIMELINE
// Profiling builds: per block of the last fused launch, {start, end} on the
// 100 MHz constant clock, the hardware wave id register of wave 0, and the
// block's unit: {slice, rank (0: skipped), token, row split}.
__device__ unsigned long long block_timeline[kTimelineBlocks * kTimelineWords];
#endif

// ---- longest units first ---------------------------------------------------------
// When the adapters differ in rank, (slice, token) units differ in cost by up
// to 16x, and the order in which blocks are dispatched sets the step time: a
// costly unit dispatched late ends the launch.  With `lpt` set (one unit per
// block, at most kLptMax units), block b runs the unit at position b of the
// batch ordered by decreasing weight bytes r * (d_in + d_out), ties by unit
// index.  Every block ranks the units itself in LDS (the ranks from the
// adapter table, units^2 / NT comparisons): no pre-pass launch, no scratch.
constexpr int kLptMax = 1024;
constexpr int kLptUnitBits = 10;
constexpr unsigned kLptCostMax = (1u << (32 - kLptUnitBits)) - 1;

// Unit at position p of the cost order; all threads call it, the result is
// uniform.  key: kLptMax words, cnt: NT + 1 words, es/ew: LORA_MAX_IO words.
template <int NT>
__device__ __forceinline__ int unit_by_cost(const PoolView& pv, const IoSet& ios,
                                            const int32_t* __restrict__ ids, int n, int p,
                                            unsigned* key, int* cnt, int* es, int* ew) {
  const int units = n * ios.n_io;
  const int t = threadIdx.x;
  if (t == 0) {
    for (int j = 0; j < ios.n_io; ++j) {  // uniform index into the argument block
      es[j] = ios.io[j].slice;
      ew[j] = (ios.io[j].d_in + ios.io[j].d_out + 1023) >> 10;
    }
  }
  __syncthreads();
  const int u4 = (units + 3) & ~3;
  for (int u = t; u < u4; u += NT) {
    unsigned k = 0xFFFFFFFFu;  // padding ranks after every unit
    if (u < units) {
      const int j = u / n;
      const int a = ids[u - j * n];
      unsigned c = 0;
      if (adapter_in_table(pv, a))
        c = (unsigned)pv.entries[es[j] * pv.max_adapters + a].rank * (unsigned)ew[j];
      k = ((kLptCostMax - min(c, kLptCostMax)) << kLptUnitBits) | (unsigned)u;
    }
    key[u] = k;
  }
  __syncthreads();
  // R threads per candidate unit, each counting the keys below its key in one
  // part of the list
  const int upad = (units + 63) & ~63;
  const int R = upad <= NT ? NT / upad : 1;
  const int g = t / upad;
  const int per = ((u4 / 4 + R - 1) / R) * 4;
  int found = -1;
  for (int u = t - g * upad; u < units && g < R; u += NT) {
    const unsigned ku = key[u];
    const int k_end = min(u4, (g + 1) * per);
    int below = 0;
    for (int k = g * per; k < k_end; k += 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(key + k);
      below += (v.x < ku) + (v.y < ku) + (v.z < ku) + (v.w < ku);
    }
    if (R == 1) {
      if (below == p) found = u;
    } else {
      cnt[t] = below;
    }
  }
  if (R > 1) {
    __syncthreads();
    if (t < units && t < upad) {
      int below = 0;
      for (int gg = 0; gg < R; ++gg) below += cnt[gg * upad + t];
      if (below == p) found = t;
    }
  }
  if (found >= 0) cnt[NT] = found;  // keys are distinct: one writer
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(cnt[NT]);
}

// Block = ((slice, token) unit, output-row split).
template <typename T, typename X, typename TY, int NT, int U, int MAXN>
__global__ __launch_bounds__(NT) void k_bgmv_apply(PoolView pv, IoSet ios,
                                                   const int32_t* __restrict__ ids, int n,
                                                   int nsplit, int rps, int lpt) {
  __shared__ float part[(NT / 64) * kMaxR];
  __shared__ float vsh[kMaxR];
  __shared__ __align__(16) unsigned key[kLptMax];
  __shared__ int cnt[NT + 1];
  __shared__ int es[LORA_MAX_IO], ew[LORA_MAX_IO];
#ifdef LORA_BLOCK_TIMELINE
  const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
#endif
  int unit, q;
  if (lpt) {
    q = 0;
    unit = blockIdx.x < n * ios.n_io
               ? unit_by_cost<NT>(pv, ios, ids, n, blockIdx.x, key, cnt, es, ew)
               : n * ios.n_io;
  } else {
    // slice-major: the launcher puts the costliest slices first, so their units
    // are dispatched first and the cheaper ones fill the compute units that free up
    xcd_unit_split(blockIdx.x, nsplit, unit, q);
  }
  if (unit < n * ios.n_io) fused_unit<T, X, TY, NT, U, MAXN>(pv, ios, ids, n, unit, q, rps, part, vsh);
#ifdef LORA_BLOCK_TIMELINE
  __syncthreads();
  if (threadIdx.x == 0 && blockIdx.x < kTimelineBlocks) {
    unsigned long long* r = block_timeline + (size_t)blockIdx.x * kTimelineWords;
    int slice = -1, rank = 0, tok = -1;
    if (unit < n * ios.n_io) {
      const int io_i = unit / n;
      tok = unit - io_i * n;
      slice = ios.io[io_i].slice;
      const int a = ids[tok];
      if (adapter_in_table(pv, a)) rank = pv.entries[slice * pv.max_adapters + a].rank;
    }
    r[0] = t0;
    r[1] = __builtin_amdgcn_s_memrealtime();
    r[2] = __builtin_amdgcn_s_getreg((31 << 11) | 4);  // HW_ID: CU, SH, SE of this wave
    r[3] = (unsigned long long)(unsigned)slice;
    r[4] = rank;
    r[5] = (unsigned long long)(unsigned)tok;
    r[6] = q;
    r[7] = 1;
  }
#endif
}

// Slices that share one x: block = (group of slices, token).  x of the token
// is loaded into registers once; every member slice's A rows are dotted
// against those registers, then that slice's rows are expanded.  Per slice the
// arithmetic is the one of k_bgmv_apply, so the results are the same bits.
template <typename T, typename X, typename TY, int NT, int U, int MAXN>
__global__ __launch_bounds__(NT) void k_bgmv_apply_grouped(PoolView pv, IoSet ios,
                                                           const int32_t* __restrict__ ids, int n) {
  __shared__ float part[(NT / 64) * kMaxR];
  __shared__ float vsh[kMaxR];
  int unit, q;
  xcd_unit_split(blockIdx.x, 1, unit, q);
  if (unit >= n * ios.n_groups) return;
  const int g = unit / n;
  const int i = unit - g * n;
  const int a = ids[i];
  if (!adapter_in_table(pv, a)) return;
  const int m0 = ios.grp_start[g], m1 = ios.grp_start[g + 1];
  const IoDesc io0 = ios.io[m0];
  const bool fast = io0.npa == 1 && io0.d_in / ET<T>::E <= NT * U;
  uint4 xr[U][x_chunks<T, X>()];
  if (fast) load_x_regs<T, X, NT, U>(io0, i, xr);
  for (int m = m0; m < m1; ++m) {
    const IoDesc io = ios.io[m];
    const DevEntry e = pv.entries[io.slice * pv.max_adapters + a];
    if (e.rank <= 0) continue;
    const int nch = e.rs / ET<T>::E;
    bool done = false;
#define LORA_GROUP_CASE(N)                                                                    \
    if (!done && N <= MAXN && nch == N) {                                                    \
      if (fast)                                                                              \
        bgmv_fused_fast<T, X, TY, NT, U, (N <= MAXN ? N : 1), false>(pv, e, io, i, 0, io.d_out, \
                                                                     part, vsh, xr);         \
      else                                                                                   \
        bgmv_fused_body<T, X, TY, NT, U, (N <= MAXN ? N : 0)>(pv, e, io, i, 0, io.d_out, part, vsh); \
      done = true;                                                                           \
    }
    LORA_GROUP_CASE(1)
    LORA_GROUP_CASE(2)
    LORA_GROUP_CASE(4)
    LORA_GROUP_CASE(8)
    LORA_GROUP_CASE(16)
#undef LORA_GROUP_CASE
    if (!done) bgmv_fused_body<T, X, TY, NT, U, 0>(pv, e, io, i, 0, io.d_out, part, vsh);
    __syncthreads();  // part and vsh are reused by the next member
  }
}

// ---- launchers ----------------------------------------------------------------
namespace {

constexpr int kExpandNT = 256;

// Column chunks per thread for a shrink over d_in with NT threads.
inline int pick_u(int d_in, int E, int NT) {
  const int C = d_in / E;
  return C > NT ? 2 : 1;
}

template <typename T, typename X>
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
      hipLaunchKernelGGL((k_bgmv_shrink<T, X, 512, 1>), grid, dim3(512), 0, s, pv, io, ids, n, v,
                         v_ld, ngroups, rpg);
    else
      hipLaunchKernelGGL((k_bgmv_shrink<T, X, 512, 2>), grid, dim3(512), 0, s, pv, io, ids, n, v,
                         v_ld, ngroups, rpg);
  } else {
    hipLaunchKernelGGL((k_bgmv_shrink<T, X, 256, 1>), grid, dim3(256), 0, s, pv, io, ids, n, v,
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

template <typename T, typename X, typename TY, int NT, int U>
void apply_grouped_launch(const PoolView& pv, const IoSet& ios, const int32_t* ids, int n,
                          hipStream_t s) {
  constexpr int kMaxN = (is_quant<T>() && NT == 512) ? 4 : 8;
  const dim3 grid(xcd_grid(n * ios.n_groups, 1));
  if (pv.max_nch <= 2)
    hipLaunchKernelGGL((k_bgmv_apply_grouped<T, X, TY, NT, U, 2>), grid, dim3(NT), 0, s, pv, ios, ids, n);
  else if (pv.max_nch <= 4 || kMaxN == 4)
    hipLaunchKernelGGL((k_bgmv_apply_grouped<T, X, TY, NT, U, 4>), grid, dim3(NT), 0, s, pv, ios, ids, n);
  else
    hipLaunchKernelGGL((k_bgmv_apply_grouped<T, X, TY, NT, U, kMaxN>), grid, dim3(NT), 0, s, pv, ios, ids, n);
}

// Blocks of `kernel` (NT threads) resident per compute unit, looked up once
// per kernel; 1 if the query fails.
inline int resident_blocks(const void* kernel, int nt) {
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kernel, nt, 0) != hipSuccess) {
    (void)hipGetLastError();
    return 1;
  }
  return nb > 0 ? nb : 1;
}

// Splitting a unit repeats its whole shrink, which costs more than it gains
// (measured, also when only the units with the largest B are split); split
// only while the split units still run in one round of resident blocks: a
// second, partly filled round costs more than the slots one round leaves idle
// (Llama-7B q/k/v at 64 tokens, 192 units: 20.0 us with two-way splits, 15.1
// us without).  Kernels with two resident blocks per compute unit (the
// 256-thread FP8 variants) split a batch of one block per compute unit in two.
template <typename T, typename X, typename TY, int NT, int U, int MAXN>
void apply_launch_v(const PoolView& pv, const IoSet& ios, const int32_t* ids, int n,
                    hipStream_t s) {
  auto kern = k_bgmv_apply<T, X, TY, NT, U, MAXN>;
  static const int nb = resident_blocks(reinterpret_cast<const void*>(kern), NT);
  const long slots = (long)pv.n_cu * nb;
  const int units = n * ios.n_io;
  int nsplit = 1;
  while ((long)units * nsplit * 2 <= slots && ios.max_d_out / (nsplit * 2) >= 512) nsplit *= 2;
  const int rps = (((ios.max_d_out + nsplit - 1) / nsplit) + 63) & ~63;
  // longest units first when ranks differ and the units take more than one round
  const int lpt = pv.mixed_ranks && nsplit == 1 && units > slots && units <= kLptMax ? 1 : 0;
  hipLaunchKernelGGL(kern, dim3(xcd_grid(units, nsplit)), dim3(NT), 0, s, pv, ios, ids, n, nsplit,
                     rps, lpt);
}

template <typename T, typename X, typename TY, int NT, int U>
void apply_launch(const PoolView& pv, const IoSet& ios, const int32_t* ids, int n,
                  hipStream_t s) {
  // variant by the pool's longest B row, so short-row pools get lean kernels
  // (FP8 rows of 8 chunks at 512 threads take the loop body: an FP8 chunk
  // unpacks to twice the values of a 16-bit one)
  constexpr int kMaxN = (is_quant<T>() && NT == 512) ? 4 : 8;
  if (pv.max_nch <= 2)
    apply_launch_v<T, X, TY, NT, U, 2>(pv, ios, ids, n, s);
  else if (pv.max_nch <= 4 || kMaxN == 4)
    apply_launch_v<T, X, TY, NT, U, 4>(pv, ios, ids, n, s);
  else
    apply_launch_v<T, X, TY, NT, U, kMaxN>(pv, ios, ids, n, s);
}

template <typename T, typename X, typename TY>
hipError_t apply_t(const PoolView& pv, const IoSet& ios_in, const int32_t* ids, int n,
                   hipStream_t s) {
  constexpr int E = ET<T>::E;
  // Slices sharing x: one block per (group, token) reads x once into
  // registers for all of them -- when that still gives every compute unit a
  // block.  A smaller batch keeps one block per (slice, token): a token's
  // blocks run on one XCD, so its x comes from HBM once and from L2 after
  // (measured on the Llama-7B q/k/v shapes: per-slice blocks 1.5x faster at 64
  // tokens, both within 3% from 256 tokens on).
  if (ios_in.n_groups > 0 && (long)n * ios_in.n_groups >= pv.n_cu) {
    const int C = ios_in.max_d_in / E;
    if (C >= 512) apply_grouped_launch<T, X, TY, 512, 1>(pv, ios_in, ids, n, s);
    else apply_grouped_launch<T, X, TY, 256, 1>(pv, ios_in, ids, n, s);
    return hipGetLastError();
  }
  // slices by decreasing bytes per token unit (d_in + d_out): blocks are
  // dispatched in unit order, so the longest units start first
  IoSet ios = ios_in;
  std::stable_sort(ios.io, ios.io + ios.n_io, [](const IoDesc& a, const IoDesc& b) {
    return a.d_in + a.d_out > b.d_in + b.d_out;
  });
  const int C = ios.max_d_in / E;
  if (C >= 512) {
    // FP8: one column chunk per thread (a wider row loops over the columns)
    if (is_quant<T>() || pick_u(ios.max_d_in, E, 512) == 1)
      apply_launch<T, X, TY, 512, 1>(pv, ios, ids, n, s);
    else
      apply_launch<T, X, TY, 512, is_quant<T>() ? 1 : 2>(pv, ios, ids, n, s);
  } else {
    apply_launch<T, X, TY, 256, 1>(pv, ios, ids, n, s);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bgmv_shrink(const Types& ty, const PoolView& pv, const IoDesc& io,
                              const int32_t* ids, int32_t n, float* v, int32_t v_ld,
                              hipStream_t s) {
  switch (ty.w) {
    case LORA_F32: return shrink_t<float, float>(pv, io, ids, n, v, v_ld, s);
    case LORA_F16: return shrink_t<f16_t, f16_t>(pv, io, ids, n, v, v_ld, s);
    case LORA_BF16: return shrink_t<bf16_t, bf16_t>(pv, io, ids, n, v, v_ld, s);
    default:
      return ty.x == LORA_F16 ? shrink_t<fp8_t, f16_t>(pv, io, ids, n, v, v_ld, s)
                              : shrink_t<fp8_t, bf16_t>(pv, io, ids, n, v, v_ld, s);
  }
}

hipError_t launch_bgmv_expand(const Types& ty, const PoolView& pv, const IoDesc& io,
                              const float* v, int32_t v_ld, const int32_t* ids, int32_t n,
                              const float* tok_scale, hipStream_t s) {
  const bool yf = (ty.y == LORA_F32);
  switch (ty.w) {
    case LORA_F32: return expand_t<float, float>(pv, io, v, v_ld, ids, n, tok_scale, s);
    case LORA_F16:
      return yf ? expand_t<f16_t, float>(pv, io, v, v_ld, ids, n, tok_scale, s)
                : expand_t<f16_t, f16_t>(pv, io, v, v_ld, ids, n, tok_scale, s);
    case LORA_BF16:
      return yf ? expand_t<bf16_t, float>(pv, io, v, v_ld, ids, n, tok_scale, s)
                : expand_t<bf16_t, bf16_t>(pv, io, v, v_ld, ids, n, tok_scale, s);
    default:
      if (yf) return expand_t<fp8_t, float>(pv, io, v, v_ld, ids, n, tok_scale, s);
      return ty.y == LORA_F16 ? expand_t<fp8_t, f16_t>(pv, io, v, v_ld, ids, n, tok_scale, s)
                              : expand_t<fp8_t, bf16_t>(pv, io, v, v_ld, ids, n, tok_scale, s);
  }
}

hipError_t launch_bgmv_apply(const Types& ty, const PoolView& pv, const IoSet& ios,
                             const int32_t* ids, int32_t n, hipStream_t s) {
  const bool yf = (ty.y == LORA_F32);
  switch (ty.w) {
    case LORA_F32: return apply_t<float, float, float>(pv, ios, ids, n, s);
    case LORA_F16:
      return yf ? apply_t<f16_t, f16_t, float>(pv, ios, ids, n, s)
                : apply_t<f16_t, f16_t, f16_t>(pv, ios, ids, n, s);
    case LORA_BF16:
      return yf ? apply_t<bf16_t, bf16_t, float>(pv, ios, ids, n, s)
                : apply_t<bf16_t, bf16_t, bf16_t>(pv, ios, ids, n, s);
    default:
      if (ty.x == LORA_F16)
        return yf ? apply_t<fp8_t, f16_t, float>(pv, ios, ids, n, s)
                  : apply_t<fp8_t, f16_t, f16_t>(pv, ios, ids, n, s);
      return yf ? apply_t<fp8_t, bf16_t, float>(pv, ios, ids, n, s)
                : apply_t<fp8_t, bf16_t, bf16_t>(pv, ios, ids, n, s);
  }
}

hipError_t read_block_timeline(void* host, size_t bytes) {
#ifdef LORA_BLOCK_TIMELINE
  if (bytes > sizeof(block_timeline)) bytes = sizeof(block_timeline);
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(block_timeline), bytes, 0, hipMemcpyDeviceToHost);
#else
  (void)host;
  (void)bytes;
  return hipErrorNotSupported;
#endif
}

}  // namespace lora
