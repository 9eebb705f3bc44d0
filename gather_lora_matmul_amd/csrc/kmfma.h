// 64-token MFMA tiles for groups of tokens that share one adapter (the long
// SGMV segments of the multi-LoRA serving article, SGMV section).
//
// Block = 4 waves; wave w owns token slots [16w, 16w + 16) of the tile.
//
// Shrink  V[t][n] = sum_j X[t][j] A[n][j]          (M = tokens, N = rank, K = d_in)
//   v_mfma_f32_16x16x32_{bf16,f16}: the X operand comes straight from HBM (each
//   lane reads 16 contiguous elements of its token row per 64-column chunk), the
//   A^T operand from an LDS copy of the chunk's rank rows, staged by the whole
//   block one chunk ahead.  N = rank padded to 16; rows >= rank are zero.
// Expand  Y^T[m][t] += s * sum_k B[m][k] V[t][k]   (M = output rows, N = tokens,
//   K = rank).  B rows are read from their pages in natural [d_out][r_s]
//   layout, which is exactly the MFMA A-operand layout (8 contiguous k per
//   lane), and V is split into hi + lo 16-bit parts so that the fp32 shrink
//   result enters the 16-bit MFMA with ~2^-16 relative error.  Each lane ends
//   with 4 consecutive outputs of one token: one read-modify-write of y.
//
// The same k-to-lane assignment is used for both operands of every MFMA, so the
// hardware's internal k order does not matter; only the row/column placement
// of the operands and of the accumulator (A row = lane % 16, B column =
// lane % 16, accumulator column = lane % 16, rows 4 * (lane / 16) + i) is used.
#pragma once

#include "kcommon.h"

namespace lora {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <typename T>
struct MfmaOp;
template <>
struct MfmaOp<bf16_t> {
  typedef bf16x8_t vec;
  static __device__ __forceinline__ f32x4_t mma(const vec a, const vec b, const f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // split f into hi + lo with hi = RNE(f) and lo = RNE(f - hi)
  static __device__ __forceinline__ void split(float f, uint16_t& hi, uint16_t& lo) {
    hi = f32_to_bf16_rne(f);
    const float fh = __uint_as_float((uint32_t)hi << 16);
    lo = f32_to_bf16_rne(f - fh);
  }
};
template <>
struct MfmaOp<f16_t> {
  typedef f16x8_t vec;
  static __device__ __forceinline__ f32x4_t mma(const vec a, const vec b, const f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ void split(float f, uint16_t& hi, uint16_t& lo) {
    const _Float16 h = (_Float16)f;
    hi = __builtin_bit_cast(uint16_t, h);
    lo = __builtin_bit_cast(uint16_t, (_Float16)(f - (float)h));
  }
};
template <>
struct MfmaOp<float> {  // fp32 pools never form MFMA tiles (the planner keeps them short)
  typedef bf16x8_t vec;
  static __device__ __forceinline__ f32x4_t mma(const vec, const vec, const f32x4_t c) { return c; }
  static __device__ __forceinline__ void split(float, uint16_t& hi, uint16_t& lo) { hi = lo = 0; }
};

constexpr int kKC = 64;            // shrink K chunk (columns of d_in)
constexpr int kAsStride = kKC + 8; // LDS row stride of the staged A chunk (elements)
constexpr int kVsStride = kMaxR + 4;  // LDS row stride of V (floats)
constexpr int kMfmaLds = kMaxR * kAsStride * 2 + kTileM * kVsStride * 4;

template <typename V>
__device__ __forceinline__ V as_vec(const uint4 u) {
  return __builtin_bit_cast(V, u);
}

// ---- shrink of one tile: acc[nb] for the wave's 16 tokens --------------------
// tok: this lane's token (slot 16w + lane % 16), or -1.
template <typename T>
__device__ __forceinline__ void mfma_shrink_core(const PoolView& pv, const DevEntry& e,
                                                 const IoDesc& io, int tok, char* lds,
                                                 f32x4_t (&acc)[kMaxR / 16]) {
  typedef typename MfmaOp<T>::vec vec;
  constexpr int ELT = 2;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int g = lane >> 4;
  const int r = e.rank;
  const int NB = (r + 15) >> 4;
  const int d_in = io.d_in;
  uint16_t* As = reinterpret_cast<uint16_t*>(lds);
#pragma unroll
  for (int nb = 0; nb < kMaxR / 16; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // staging assignment: chunk row n = idx / 8, 16-byte piece p = idx % 8 (8 pieces per 64 cols)
  const int nstage = NB * 16 * 8;  // pieces per chunk
  const char* xrow = tok >= 0 ? reinterpret_cast<const char*>(io.x) + (int64_t)tok * d_in * ELT : nullptr;
  uint4 ast[4];   // up to 4 staged pieces per thread (NB * 128 <= 1024 = 4 * 256)
  uint4 xnext[2];
  auto load_chunk = [&](int kc) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = t + 256 * u;
      const int n = idx >> 3;
      const int col = kc + ((idx & 7) << 3);
      if (idx < nstage && n < r && col < d_in)
        ast[u] = ld16(pv.pages + a_offset(pv, e, io.npa, ELT, n, col));
      else
        ast[u] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int col = kc + 16 * g + 8 * s;
      xnext[s] = (xrow && col < d_in) ? ld16(xrow + (int64_t)col * ELT) : make_uint4(0, 0, 0, 0);
    }
  };
  load_chunk(0);
  for (int kc = 0; kc < d_in; kc += kKC) {
    __syncthreads();  // the previous chunk's LDS reads are done
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = t + 256 * u;
      if (idx < nstage)
        *reinterpret_cast<uint4*>(As + (idx >> 3) * kAsStride + ((idx & 7) << 3)) = ast[u];
    }
    const uint4 x0 = xnext[0], x1 = xnext[1];
    __syncthreads();
    if (kc + kKC < d_in) load_chunk(kc + kKC);  // in flight during the MFMAs
#pragma unroll
    for (int nb = 0; nb < kMaxR / 16; ++nb) {
      if (nb < NB) {
        const uint16_t* brow = As + (nb * 16 + (lane & 15)) * kAsStride + 16 * g;
        const uint4 b0 = *reinterpret_cast<const uint4*>(brow);
        const uint4 b1 = *reinterpret_cast<const uint4*>(brow + 8);
        acc[nb] = MfmaOp<T>::mma(as_vec<vec>(x0), as_vec<vec>(b0), acc[nb]);
        acc[nb] = MfmaOp<T>::mma(as_vec<vec>(x1), as_vec<vec>(b1), acc[nb]);
      }
    }
  }
}

// ---- split-API shrink of one MFMA tile: v rows of the tile's tokens ----------
template <typename T, int NT>
__device__ __forceinline__ void mfma_shrink_tile(const PoolView& pv, const PlanView& pl,
                                                 const PlanItem& item, const IoDesc& io,
                                                 float* v, int v_ld) {
  __shared__ __attribute__((aligned(16))) char lds[kMaxR * kAsStride * 2];
  const DevEntry e = pv.entries[io.slice * pv.max_adapters + item.adapter];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int slot = 16 * w + (lane & 15);
  const int tok = slot < item.count ? pl.perm[item.start + slot] : -1;
  if (e.rank <= 0) {
    // not resident: zero rows
    for (int idx = t; idx < item.count * v_ld; idx += NT) {
      const int s = idx / v_ld;
      v[(int64_t)pl.perm[item.start + s] * v_ld + (idx - s * v_ld)] = 0.f;
    }
    return;
  }
  f32x4_t acc[kMaxR / 16];
  mfma_shrink_core<T>(pv, e, io, tok, lds, acc);
  const int NB = (e.rank + 15) >> 4;
  const int g = lane >> 4;
  // accumulator: column n = nb*16 + lane%16, rows (slots) 16w + 4g + i
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = 16 * w + 4 * g + i;
    if (s < item.count) {
      const int tk = pl.perm[item.start + s];
      float* vr = v + (int64_t)tk * v_ld;
#pragma unroll
      for (int nb = 0; nb < kMaxR / 16; ++nb) {
        const int n = nb * 16 + (lane & 15);
        if (nb < NB && n < v_ld) vr[n] = n < e.rank ? acc[nb][i] : 0.f;
      }
      for (int n = NB * 16 + (lane & 15); n < v_ld; n += 16) vr[n] = 0.f;
    }
  }
}

// ---- expand core: y rows of the wave's 16 tokens, output rows [m_lo, m_hi) -----
// vhi/vlo: this lane's V^T operands for the rank steps (column = slot lane%16,
// k = 32 s + 8 g + j).
template <typename T, typename TY>
__device__ __forceinline__ void mfma_expand_core(const PoolView& pv, const DevEntry& e,
                                                 const IoDesc& io, const uint4 (&vhi)[kMaxR / 32],
                                                 const uint4 (&vlo)[kMaxR / 32], int tok_out,
                                                 int m_lo, int m_hi) {
  typedef typename MfmaOp<T>::vec vec;
  constexpr int ELT = 2;
  constexpr int MB = 4;  // m-blocks in flight per iteration
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int nK = (e.rs + 31) >> 5;
  const float s = e.scale;
  char* yrow = tok_out >= 0 ? reinterpret_cast<char*>(io.y) + (int64_t)tok_out * io.d_out * sizeof(TY)
                            : nullptr;
  for (int mb0 = m_lo; mb0 < m_hi; mb0 += 16 * MB) {
    uint4 bop[MB][kMaxR / 32];
    float yv[MB][4];
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      const int m = mb0 + 16 * b + (lane & 15);  // operand row of this lane
      const bool mv = m < m_hi;
      const char* brow = mv ? pv.pages + b_offset(pv, e, ELT, m) : nullptr;
#pragma unroll
      for (int ks = 0; ks < kMaxR / 32; ++ks) {
        const int k = 32 * ks + 8 * g;
        bop[b][ks] = (ks < nK && mv && k < e.rs) ? ld16(brow + k * ELT) : make_uint4(0, 0, 0, 0);
      }
      const int mo = mb0 + 16 * b + 4 * g;  // first output row of this lane
#pragma unroll
      for (int i = 0; i < 4; ++i) yv[b][i] = (yrow && mo < m_hi) ? load_y<TY>(yrow, mo + i) : 0.f;
    }
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kMaxR / 32; ++ks) {
        if (ks < nK) {
          acc = MfmaOp<T>::mma(as_vec<vec>(bop[b][ks]), as_vec<vec>(vhi[ks]), acc);
          acc = MfmaOp<T>::mma(as_vec<vec>(bop[b][ks]), as_vec<vec>(vlo[ks]), acc);
        }
      }
      const int mo = mb0 + 16 * b + 4 * g;
      if (yrow && mo < m_hi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) store_y<TY>(yrow, mo + i, __builtin_fmaf(s, acc[i], yv[b][i]));
      }
    }
  }
}

// Pack 8 fp32 values of V (k = k0 .. k0+7, zero at k >= r) into hi/lo operands.
template <typename T>
__device__ __forceinline__ void pack_v(const float* f, uint4& hi, uint4& lo) {
  uint16_t h[8], l[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) MfmaOp<T>::split(f[j], h[j], l[j]);
  hi = make_uint4(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16),
                  h[4] | ((uint32_t)h[5] << 16), h[6] | ((uint32_t)h[7] << 16));
  lo = make_uint4(l[0] | ((uint32_t)l[1] << 16), l[2] | ((uint32_t)l[3] << 16),
                  l[4] | ((uint32_t)l[5] << 16), l[6] | ((uint32_t)l[7] << 16));
}

// ---- split-API expand of one MFMA tile (V from global v) -----------------------
template <typename T, typename TY, int NT>
__device__ __forceinline__ void mfma_expand_tile(const PoolView& pv, const PlanView& pl,
                                                 const PlanItem& item, const DevEntry& e,
                                                 const IoDesc& io, const float* v, int v_ld,
                                                 int m_lo, int m_hi) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  if (16 * w >= item.count) return;  // wave without tokens (no barriers below)
  const int g = lane >> 4;
  const int slot = 16 * w + (lane & 15);
  const int tok = slot < item.count ? pl.perm[item.start + slot] : -1;
  uint4 vhi[kMaxR / 32], vlo[kMaxR / 32];
  const int nK = (e.rs + 31) >> 5;
#pragma unroll
  for (int ks = 0; ks < kMaxR / 32; ++ks) {
    float f[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = 32 * ks + 8 * g + j;
      f[j] = (ks < nK && tok >= 0 && k < e.rank) ? v[(int64_t)tok * v_ld + k] : 0.f;
    }
    pack_v<T>(f, vhi[ks], vlo[ks]);
  }
  // output: accumulator column = slot lane%16 -> the same token as the operand
  mfma_expand_core<T, TY>(pv, e, io, vhi, vlo, tok, m_lo, m_hi);
}

// ---- fused tile: shrink into LDS, then expand ---------------------------------
template <typename T, typename TY, int NT>
__device__ __forceinline__ void mfma_apply_tile(const PoolView& pv, const PlanView& pl,
                                                const PlanItem& item, const DevEntry& e,
                                                const IoDesc& io, int m_lo, int m_hi) {
  __shared__ __attribute__((aligned(16))) char lds[kMfmaLds];
  float* Vs = reinterpret_cast<float*>(lds + kMaxR * kAsStride * 2);
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int g = lane >> 4;
  const int slot = 16 * w + (lane & 15);
  const int tok = slot < item.count ? pl.perm[item.start + slot] : -1;
  f32x4_t acc[kMaxR / 16];
  mfma_shrink_core<T>(pv, e, io, tok, lds, acc);
  const int NB = (e.rank + 15) >> 4;
#pragma unroll
  for (int nb = 0; nb < kMaxR / 16; ++nb)
    if (nb < NB)
#pragma unroll
      for (int i = 0; i < 4; ++i) Vs[(16 * w + 4 * g + i) * kVsStride + nb * 16 + (lane & 15)] = acc[nb][i];
  __syncthreads();
  if (16 * w >= item.count) return;
  uint4 vhi[kMaxR / 32], vlo[kMaxR / 32];
  const int nK = (e.rs + 31) >> 5;
#pragma unroll
  for (int ks = 0; ks < kMaxR / 32; ++ks) {
    float f[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = 32 * ks + 8 * g + j;
      f[j] = (ks < nK && k < e.rank) ? Vs[slot * kVsStride + k] : 0.f;
    }
    pack_v<T>(f, vhi[ks], vlo[ks]);
  }
  mfma_expand_core<T, TY>(pv, e, io, vhi, vlo, tok, m_lo, m_hi);
}

}  // namespace lora
