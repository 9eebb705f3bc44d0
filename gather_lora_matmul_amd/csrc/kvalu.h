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
#pragma once

#include "kcommon.h"

namespace lora {

// vsh[g*VS + k] = sum_j A[k][j] * x_g[j] for k in [k_lo, k_hi); zero for k in
// [k_hi, k_zero).  xrow[g] == nullptr marks an unused token slot.
// part: LDS scratch of (NT/64) * G * kMaxR floats.  Must be called by the whole
// block with block-uniform arguments (it contains barriers).
template <typename T, int NT, int U, int G, int KB>
__device__ __forceinline__ void valu_shrink(const PoolView& pv, const DevEntry& e, int d_in,
                                            int npa, const char* const* xrow, int k_lo,
                                            int k_hi, int k_zero, float* part, float* vsh,
                                            int VS) {
  constexpr int E = ET<T>::E;
  constexpr int ELT = ET<T>::bytes;
  constexpr int NW = NT / 64;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int C = d_in / E;
  for (int k0 = k_lo; k0 < k_hi; k0 += KB) {
    float acc[G][KB];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) acc[g][kk] = 0.f;
    for (int cb = 0; cb < C; cb += NT * U) {
      uint4 a[KB][U];
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) {
        const int k = k0 + kk;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = cb + t + NT * u;
          if (k < k_hi && c < C)
            a[kk][u] = ld16(pv.pages + a_offset(pv, e, npa, ELT, k, c * E));
          else
            a[kk][u] = make_uint4(0, 0, 0, 0);
        }
      }
      uint4 xr[G][U];
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int c = cb + t + NT * u;
          xr[g][u] = (xrow[g] != nullptr && c < C) ? ld16(xrow[g] + (int64_t)c * 16)
                                                   : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
      for (int kk = 0; kk < KB; ++kk)
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int u = 0; u < U; ++u) acc[g][kk] = dot16<T>(a[kk][u], xr[g][u], acc[g][kk]);
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
    vsh[g * VS + k_lo + kk] = s;
  }
  const int nz = k_zero - k_hi;
  for (int idx = t; idx < G * nz; idx += NT) {
    const int g = idx / nz;
    vsh[g * VS + k_hi + (idx - g * nz)] = 0.f;
  }
  __syncthreads();
}

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
    constexpr int RU = NCH >= 8 ? 1 : (NCH >= 4 ? 2 : (NCH >= 2 ? 4 : 8));
    for (int mb = m_lo + t; mb < m_hi; mb += NT * RU) {
      uint4 b[RU][NCH];
      float yv[RU][G];
#pragma unroll
      for (int ru = 0; ru < RU; ++ru) {
        const int m = mb + ru * NT;
        if (m < m_hi) {
          const char* p = pv.pages + b_offset(pv, e, ELT, m);
#pragma unroll
          for (int ch = 0; ch < NCH; ++ch) b[ru][ch] = ld16(p + ch * 16);
#pragma unroll
          for (int g = 0; g < G; ++g) yv[ru][g] = yrow[g] ? load_y<TY>(yrow[g], m) : 0.f;
        }
      }
#pragma unroll
      for (int ru = 0; ru < RU; ++ru) {
        const int m = mb + ru * NT;
        if (m < m_hi) {
#pragma unroll
          for (int g = 0; g < G; ++g) {
            if (!yrow[g]) continue;
            float acc = 0.f;
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) acc = dot16v<T>(b[ru][ch], vsh + g * VS + ch * E, acc);
            store_y<TY>(yrow[g], m, __builtin_fmaf(sg[g], acc, yv[ru][g]));
          }
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
  switch (e.rs / E) {
#define LORA_NCH_CASE(N) \
  case N:                \
    valu_expand<T, TY, NT, N, G>(pv, e, vsh, VS, sg, yrow, m_lo, m_hi); \
    break;
    LORA_NCH_CASE(1)
    LORA_NCH_CASE(2)
    LORA_NCH_CASE(3)
    LORA_NCH_CASE(4)
    LORA_NCH_CASE(5)
    LORA_NCH_CASE(6)
    LORA_NCH_CASE(7)
    LORA_NCH_CASE(8)
    LORA_NCH_CASE(10)
    LORA_NCH_CASE(12)
    LORA_NCH_CASE(16)
#undef LORA_NCH_CASE
    default:
      valu_expand<T, TY, NT, 0, G>(pv, e, vsh, VS, sg, yrow, m_lo, m_hi);
  }
}

}  // namespace lora
