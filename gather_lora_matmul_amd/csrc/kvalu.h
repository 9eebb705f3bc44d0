// Block-level shrink and expand on the vector ALUs, for 1..G tokens that share
// one adapter.  Used by the decode (BGMV) kernels with G = 1 and by the short
// SGMV items with G = kShortG.
//
// Shrink: every thread owns 16-byte column chunks of d_in; it keeps the chunks
// of x in registers and streams the matching chunks of KB adapter rows (all
// loads of a batch are issued before any use), then each wave reduces its
// partial dot products with DPP and the waves combine through LDS in a fixed
// order.  Expand: every thread owns B rows (r_s contiguous elements, i.e.
// NCH 16-byte chunks), reads v from LDS and does one read-modify-write of y per
// token with a single rounding.
//
// Loads in these loops are unconditional: indices past the rank, the row range
// or d_in are clamped to the last valid one and the loaded value is masked to
// zero afterwards.  A load under a condition becomes a branch with a wait for
// it behind, which serialises the round trips; unconditional loads issue back
// to back, so one round trip to memory covers a whole batch.
#pragma once

#include "kcommon.h"

namespace lora {

__device__ __forceinline__ uint4 keep16(uint4 v, bool keep) {
  return keep ? v : make_uint4(0, 0, 0, 0);
}

// Scale modes of a quantised shrink (ignored for 16/32-bit pages): the sum
// over the codes of A row k is multiplied by a_scale[k] (the true v[k]), or by
// a_scale[k] * b_scale[k] when the expand that follows reads codes of B.
constexpr int kQNone = 0, kQRow = 1, kQRowCol = 2;

// vsh[g*VS + k] = sum_j A[k][j] * x_g[j] for k in [k_lo, k_hi); zero for k in
// [k_hi, k_zero).  T: page type, X: activation type of x.  xrow[g] == nullptr
// marks an unused token slot (xrow[0] must be valid).  part: LDS scratch of
// (NT/64) * G * kMaxR floats.  Must be called by the whole block with
// block-uniform arguments (it contains barriers).
template <typename T, typename X, int NT, int U, int G, int KB>
__device__ __forceinline__ void valu_shrink(const PoolView& pv, const DevEntry& e, int d_in,
                                            int npa, const char* const* xrow, int k_lo,
                                            int k_hi, int k_zero, float* part, float* vsh,
                                            int VS, int qmode = kQNone) {
  constexpr int E = ET<T>::E;
  constexpr int ELT = ET<T>::bytes;
  constexpr int XC = x_chunks<T, X>();
  constexpr int NW = NT / 64;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int C = d_in / E;
  const char* xs[G];
  bool xv[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    xv[g] = xrow[g] != nullptr;
    xs[g] = xv[g] ? xrow[g] : xrow[0];
  }
  for (int k0 = k_lo; k0 < k_hi; k0 += KB) {
    float acc[G][KB];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) acc[g][kk] = 0.f;
    for (int cb = 0; cb < C; cb += NT * U) {
      int cc[U];
      bool cv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = cb + t + NT * u;
        cv[u] = c < C;
        cc[u] = cv[u] ? c : C - 1;
      }
      uint4 a[KB][U];
      if (npa == 1) {
        int64_t rowb[KB];
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) rowb[kk] = a_row_uniform(pv, e, ELT, min(k0 + kk, k_hi - 1));
#pragma unroll
        for (int kk = 0; kk < KB; ++kk)
#pragma unroll
          for (int u = 0; u < U; ++u) a[kk][u] = ld16(pv.pages + rowb[kk] + (int64_t)cc[u] * 16);
      } else {
#pragma unroll
        for (int kk = 0; kk < KB; ++kk)
#pragma unroll
          for (int u = 0; u < U; ++u)
            a[kk][u] = ld16(pv.pages + a_offset(pv, e, npa, ELT, min(k0 + kk, k_hi - 1), cc[u] * E));
      }
      uint4 xr[G][U][XC];
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int q = 0; q < XC; ++q) xr[g][u][q] = ld16(xs[g] + ((int64_t)cc[u] * XC + q) * 16);
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int q = 0; q < XC; ++q) xr[g][u][q] = keep16(xr[g][u][q], xv[g] && cv[u]);
#pragma unroll
      for (int kk = 0; kk < KB; ++kk)
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int u = 0; u < U; ++u) acc[g][kk] = dotwx<T, X>(a[kk][u], xr[g][u], acc[g][kk]);
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) {
        const float s = wave_sum(acc[g][kk]);
        if (lane == 0 && k0 + kk < k_hi) part[(w * G + g) * kMaxR + (k0 + kk - k_lo)] = s;
      }
  }
  __syncthreads();
  const int nk = k_hi - k_lo;
  for (int idx = t; idx < G * nk; idx += NT) {
    const int g = idx / nk;
    const int kk = idx - g * nk;
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) s += part[(ww * G + g) * kMaxR + kk];
    if constexpr (is_quant<T>()) {
      if (qmode != kQNone) {
        float f = q_scale(pv, e.q_off + k_lo + kk);
        if (qmode == kQRowCol) f *= q_scale(pv, e.q_off + e.rank + k_lo + kk);
        s *= f;
      }
    }
    vsh[g * VS + k_lo + kk] = s;
  }
  const int nz = k_zero - k_hi;
  for (int idx = t; idx < G * nz; idx += NT) {
    const int g = idx / nz;
    vsh[g * VS + k_hi + (idx - g * nz)] = 0.f;
  }
  __syncthreads();
}

// Rows of B each thread keeps in flight per pass: about 16 loads (NCH B chunks
// and G y values per row).
__host__ __device__ constexpr int rows_per_pass(int nch, int g = 1) {
  return nch + g - 1 >= 16 ? 1 : 16 / (nch + g - 1);
}

// The first expand pass of a single token, issued before its shrink finishes:
// B rows do not depend on v, so their loads (and the y reads) overlap the
// shrink's loads and reduction.  Rows m0 + ru*NT, ru < RU.
template <typename T, typename TY, int NT, int NCH>
struct ExpandPrefetch {
  static constexpr int RU = rows_per_pass(NCH);
  uint4 b[RU][NCH];
  float yv[RU];
  __device__ __forceinline__ void load(const PoolView& pv, const DevEntry& e, const char* yrow,
                                       int m0, int m_hi) {
    int64_t off[RU];
#pragma unroll
    for (int ru = 0; ru < RU; ++ru) off[ru] = b_offset(pv, e, ET<T>::bytes, min(m0 + ru * NT, m_hi - 1));
#pragma unroll
    for (int ru = 0; ru < RU; ++ru) {
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) b[ru][ch] = ld16(pv.pages + off[ru] + ch * 16);
      yv[ru] = load_y<TY>(yrow, min(m0 + ru * NT, m_hi - 1));
    }
  }
  __device__ __forceinline__ void finish(const float* vsh, float s, char* yrow, int m0, int m_hi) {
    constexpr int E = ET<T>::E;
#pragma unroll
    for (int ru = 0; ru < RU; ++ru) {
      const int m = m0 + ru * NT;
      if (m < m_hi) {
        float acc = 0.f;
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) acc = dot16v<T>(b[ru][ch], vsh + ch * E, acc);
        store_y<TY>(yrow, m, __builtin_fmaf(s, acc, yv[ru]));
      }
    }
  }
};

// y_g[m] += s_g * sum_k B[m][k] vsh[g*VS + k] for m in [m_lo, m_hi).
// NCH = r_s / E (compile time) or 0 for a runtime loop over the chunks.
template <typename T, typename TY, int NT, int NCH, int G>
__device__ __forceinline__ void valu_expand(const PoolView& pv, const DevEntry& e,
                                            const float* vsh, int VS, const float* sg,
                                            char* const* yrow, int m_lo, int m_hi) {
  constexpr int E = ET<T>::E;
  constexpr int ELT = ET<T>::bytes;
  const int t = threadIdx.x;
  if constexpr (NCH > 0) {
    constexpr int RU = rows_per_pass(NCH, G);
    if (m_lo >= m_hi) return;
    const int mlast = m_hi - 1;
    const char* ys[G];
#pragma unroll
    for (int g = 0; g < G; ++g) ys[g] = yrow[g] ? yrow[g] : yrow[0];
    for (int mb = m_lo + t; mb < m_hi; mb += NT * RU) {
      // keep the v reads (LDS) inside the loop: hoisted out, G tokens x r_s
      // values would all sit in registers
      asm volatile("" ::: "memory");
      int64_t off[RU];
#pragma unroll
      for (int ru = 0; ru < RU; ++ru) off[ru] = b_offset(pv, e, ELT, min(mb + ru * NT, mlast));
      uint4 b[RU][NCH];
      float yv[RU][G];
#pragma unroll
      for (int ru = 0; ru < RU; ++ru) {
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) b[ru][ch] = ld16(pv.pages + off[ru] + ch * 16);
#pragma unroll
        for (int g = 0; g < G; ++g) yv[ru][g] = load_y<TY>(ys[g], min(mb + ru * NT, mlast));
      }
      float acc[RU][G];
#pragma unroll
      for (int ru = 0; ru < RU; ++ru)
#pragma unroll
        for (int g = 0; g < G; ++g) acc[ru][g] = 0.f;
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        asm volatile("" ::: "memory");  // v values of one chunk live at a time
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int ru = 0; ru < RU; ++ru) acc[ru][g] = dot16v<T>(b[ru][ch], vsh + g * VS + ch * E, acc[ru][g]);
      }
#pragma unroll
      for (int ru = 0; ru < RU; ++ru) {
        const int m = mb + ru * NT;
        if (m < m_hi) {
#pragma unroll
          for (int g = 0; g < G; ++g)
            if (yrow[g]) store_y<TY>(yrow[g], m, __builtin_fmaf(sg[g], acc[ru][g], yv[ru][g]));
        }
      }
    }
  } else {
    const int nch = e.rs / E;
    for (int m = m_lo + t; m < m_hi; m += NT) {
      const char* p = pv.pages + b_offset(pv, e, ELT, m);
      float acc[G];
#pragma unroll
      for (int g = 0; g < G; ++g) acc[g] = 0.f;
      for (int ch = 0; ch < nch; ++ch) {
        const uint4 b = ld16(p + ch * 16);
#pragma unroll
        for (int g = 0; g < G; ++g) acc[g] = dot16v<T>(b, vsh + g * VS + ch * E, acc[g]);
      }
#pragma unroll
      for (int g = 0; g < G; ++g)
        if (yrow[g]) store_y<TY>(yrow[g], m, __builtin_fmaf(sg[g], acc[g], load_y<TY>(yrow[g], m)));
    }
  }
}

// Dispatch on the number of 16-byte chunks in a stored B row.
template <typename T, typename TY, int NT, int G>
__device__ __forceinline__ void valu_expand_any(const PoolView& pv, const DevEntry& e,
                                                const float* vsh, int VS, const float* sg,
                                                char* const* yrow, int m_lo, int m_hi) {
  constexpr int E = ET<T>::E;
  // multi-token items keep the unrolled bodies small (v of G tokens per chunk)
  // and instantiate only the short-row bodies they use
  const int nch = e.rs / E;
#define LORA_NCH_CASE(N) \
  case N:                \
    valu_expand<T, TY, NT, N, G>(pv, e, vsh, VS, sg, yrow, m_lo, m_hi); \
    break;
  if constexpr (G > 1 && is_quant<T>()) {
    // an FP8 chunk unpacks to 16 values: the same rank span as 2 chunks of
    // 16-bit pages, so half the unrolled chunk counts keep the registers
    switch (nch) {
      LORA_NCH_CASE(1)
      LORA_NCH_CASE(2)
      default:
        valu_expand<T, TY, NT, 0, G>(pv, e, vsh, VS, sg, yrow, m_lo, m_hi);
    }
  } else if constexpr (G > 1 || is_quant<T>()) {
    switch (nch) {
      LORA_NCH_CASE(1)
      LORA_NCH_CASE(2)
      LORA_NCH_CASE(3)
      LORA_NCH_CASE(4)
      default:
        valu_expand<T, TY, NT, 0, G>(pv, e, vsh, VS, sg, yrow, m_lo, m_hi);
    }
  } else {
    switch (nch) {
      LORA_NCH_CASE(1)
      LORA_NCH_CASE(2)
      LORA_NCH_CASE(3)
      LORA_NCH_CASE(4)
      LORA_NCH_CASE(6)
      LORA_NCH_CASE(8)
      default:
        valu_expand<T, TY, NT, 0, G>(pv, e, vsh, VS, sg, yrow, m_lo, m_hi);
    }
  }
#undef LORA_NCH_CASE
}

}  // namespace lora
