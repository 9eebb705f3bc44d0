// MFMA tiles for groups of tokens that share one adapter (the long SGMV
// segments of the multi-LoRA serving article, SGMV section).
//
// A tile is up to 64 token slots of one group, processed by one block of four
// waves, with v_mfma_f32_16x16x32_{bf16,f16}.
//
// Shrink  V[t][n] = sum_j X[t][j] A[n][j]         (M = tokens, N = rank, K = d_in)
//   The four waves split K into quarters; each wave streams the X rows of all
//   the tile's tokens and the A rows of its quarter straight from HBM into
//   registers (double buffered, one 32-column step ahead), then the four
//   partial tiles are summed in LDS in a fixed order.  N = rank padded to 16.
// Expand  Y^T[m][t] += s * sum_k B[m][k] V[t][k]  (M = output rows, N = tokens,
//   K = rank).  B rows are read from their pages in natural [d_out][r_s] layout,
//   which is exactly the MFMA A-operand layout (8 contiguous k per lane).  V is
//   split into hi + lo 16-bit parts (packed in LDS) so that the fp32 shrink
//   result enters the 16-bit MFMA with ~2^-16 relative error.  Each lane ends
//   with 4 consecutive outputs of one token: one 8-byte read-modify-write of y.
//   The waves take interleaved 16-row m-blocks, two per step, and load the next
//   step's B rows and y before computing the current one.
//
// The same k-to-lane assignment is used for both operands of every MFMA, so the
// hardware's internal k order does not matter; only the row/column placement
// of the operands and of the accumulator (A row = lane % 16, B column =
// lane % 16, accumulator column = lane % 16, rows 4 * (lane / 16) + i) is used.
// All global loads are unconditional (clamped indices, masked values).
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
  // hi = RNE(f), lo = RNE(f - hi)
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

constexpr int kVsStride = kMaxR + 4;          // LDS row stride of V (floats) = 528 bytes
constexpr int kVsBytes = kTileM * kVsStride * 4;

template <typename V>
__device__ __forceinline__ V as_vec(const uint4 u) {
  return __builtin_bit_cast(V, u);
}
__device__ __forceinline__ uint4 keep16m(uint4 v, bool keep) {
  return keep ? v : make_uint4(0, 0, 0, 0);
}

// Token of every slot of the tile, -1 past the item's count (LDS).
__device__ __forceinline__ void load_tile_tokens(const PlanView& pl, const PlanItem& item,
                                                 int* toks) {
  if (threadIdx.x < kTileM)
    toks[threadIdx.x] = (int)threadIdx.x < item.count ? pl.perm[item.start + threadIdx.x] : -1;
}

// ---- shrink: V tile (fp32) into LDS Vs[slot][n], n < 16*NB ------------------
// MBT: 16-token blocks in the tile (4 for 64 slots, 2 for 32 slots starting at
// slot `slot0`).  Requires blockDim = 256 and toks[] visible to the block.
template <typename T, int NB, int MBT>
__device__ __forceinline__ void mfma_shrink_lds(const PoolView& pv, const DevEntry& e,
                                                const IoDesc& io, const int* toks, int slot0,
                                                float* Vs) {
  typedef typename MfmaOp<T>::vec vec;
  constexpr int ELT = 2;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int d_in = io.d_in;
  const int r = e.rank;
  // this lane's X rows (one per 16-token block) and A rows (one per 16-rank block)
  const int tok0 = toks[slot0];
  const char* xrow[MBT];
  bool xok[MBT];
#pragma unroll
  for (int mb = 0; mb < MBT; ++mb) {
    const int tk = toks[slot0 + mb * 16 + r16];
    xok[mb] = tk >= 0;
    xrow[mb] = reinterpret_cast<const char*>(io.x) + (int64_t)(tk >= 0 ? tk : tok0) * d_in * ELT;
  }
  int64_t arow[NB];
  bool aok[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int n = nb * 16 + r16;
    aok[nb] = n < r;
    arow[nb] = io.npa == 1 ? a_offset(pv, e, 1, ELT, min(n, r - 1), 0) : 0;
  }
  // K split into four contiguous ranges of 32-column steps
  const int nsteps = (d_in + 31) >> 5;
  const int per = (nsteps + 3) >> 2;
  const int s_beg = w * per;
  const int s_end = min(nsteps, s_beg + per);
  f32x4_t acc[MBT][NB];
#pragma unroll
  for (int mb = 0; mb < MBT; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint4 xc[MBT], ac[NB], xn[MBT], an[NB];
  auto load_step = [&](int s, uint4 (&xo)[MBT], uint4 (&ao)[NB]) {
    const int col = 32 * s + 8 * g;
    const bool cok = col < d_in;
    const int colc = cok ? col : d_in - 8;
#pragma unroll
    for (int mb = 0; mb < MBT; ++mb) xo[mb] = ld16(xrow[mb] + (int64_t)colc * ELT);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int64_t off = io.npa == 1 ? arow[nb] + (int64_t)colc * ELT
                                      : a_offset(pv, e, io.npa, ELT, min(nb * 16 + r16, r - 1), colc);
      ao[nb] = ld16(pv.pages + off);
    }
#pragma unroll
    for (int mb = 0; mb < MBT; ++mb) xo[mb] = keep16m(xo[mb], cok && xok[mb]);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) ao[nb] = keep16m(ao[nb], cok && aok[nb]);
  };
  if (s_beg < s_end) {
    // double buffered while the registers allow (ranks up to 64)
    constexpr bool kDouble = NB <= 4;
    load_step(s_beg, xc, ac);
    for (int s = s_beg; s < s_end; ++s) {
      if constexpr (kDouble) load_step(min(s + 1, s_end - 1), xn, an);  // next step in flight
#pragma unroll
      for (int mb = 0; mb < MBT; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[mb][nb] = MfmaOp<T>::mma(as_vec<vec>(xc[mb]), as_vec<vec>(ac[nb]), acc[mb][nb]);
      if constexpr (kDouble) {
#pragma unroll
        for (int mb = 0; mb < MBT; ++mb) xc[mb] = xn[mb];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) ac[nb] = an[nb];
      } else if (s + 1 < s_end) {
        load_step(s + 1, xc, ac);
      }
    }
  }
  // fixed-order sum of the four partial tiles: wave 0 stores, waves 1..3 add
  for (int ww = 0; ww < 4; ++ww) {
    if (w == ww) {
#pragma unroll
      for (int mb = 0; mb < MBT; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float* p = Vs + (slot0 + mb * 16 + 4 * g + i) * kVsStride + nb * 16 + r16;
            *p = ww == 0 ? acc[mb][nb][i] : *p + acc[mb][nb][i];
          }
    }
    __syncthreads();
  }
}

// ---- V (fp32 in LDS) -> packed hi/lo 16-bit operands, in place ---------------
// Row `slot` becomes hi[0..32*NK) followed by lo[0..32*NK) (k >= rank: zero).
template <typename T, int NK>
__device__ __forceinline__ void pack_v_lds(float* Vs, int rank) {
  constexpr int KW = 32 * NK;
  constexpr int PER = kTileM * KW / 256;  // values per thread
  const int t = threadIdx.x;
  uint16_t hi[PER], lo[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int idx = t + 256 * j;
    const int slot = idx / KW;
    const int k = idx - slot * KW;
    const float f = k < rank ? Vs[slot * kVsStride + k] : 0.f;
    MfmaOp<T>::split(f, hi[j], lo[j]);
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int idx = t + 256 * j;
    const int slot = idx / KW;
    const int k = idx - slot * KW;
    uint16_t* row = reinterpret_cast<uint16_t*>(Vs + slot * kVsStride);
    row[k] = hi[j];
    row[KW + k] = lo[j];
  }
  __syncthreads();
}

// 4 consecutive y elements of one row: load / store (8 bytes for 16-bit, 16 for fp32)
template <typename TY>
struct Y4 {
  typedef uint2 raw;
  static __device__ __forceinline__ uint2 load_raw(const char* row, int m) {
    return *reinterpret_cast<const uint2*>(row + (int64_t)m * 2);
  }
  static __device__ __forceinline__ void unpack(const uint2 u, float (&v)[4]) {
    v[0] = bits_to_f<TY>(u.x & 0xffffu);
    v[1] = bits_to_f<TY>(u.x >> 16);
    v[2] = bits_to_f<TY>(u.y & 0xffffu);
    v[3] = bits_to_f<TY>(u.y >> 16);
  }
  static __device__ __forceinline__ void store(char* row, int m, const float (&v)[4]) {
    *reinterpret_cast<uint2*>(row + (int64_t)m * 2) =
        make_uint2(f_to_bits<TY>(v[0]) | (f_to_bits<TY>(v[1]) << 16),
                   f_to_bits<TY>(v[2]) | (f_to_bits<TY>(v[3]) << 16));
  }
};
template <>
struct Y4<float> {
  typedef uint4 raw;
  static __device__ __forceinline__ uint4 load_raw(const char* row, int m) {
    return *reinterpret_cast<const uint4*>(row + (int64_t)m * 4);
  }
  static __device__ __forceinline__ void unpack(const uint4 u, float (&v)[4]) {
    v[0] = __uint_as_float(u.x);
    v[1] = __uint_as_float(u.y);
    v[2] = __uint_as_float(u.z);
    v[3] = __uint_as_float(u.w);
  }
  static __device__ __forceinline__ void store(char* row, int m, const float (&v)[4]) {
    *reinterpret_cast<float4*>(row + (int64_t)m * 4) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

// ---- expand from packed V in LDS: rows [m_lo, m_hi) for all the tile's tokens --
// m_lo is a multiple of 64 and m_hi of 8.
template <typename T, typename TY, int NK>
__device__ __forceinline__ void mfma_expand_lds(const PoolView& pv, const DevEntry& e,
                                                const IoDesc& io, const int* toks, int count,
                                                const float* Vs, int m_lo, int m_hi) {
  typedef typename MfmaOp<T>::vec vec;
  constexpr int ELT = 2;
  constexpr int KW = 32 * NK;
  constexpr int MB = 2;  // m-blocks per step per wave
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int ntb = (count + 15) >> 4;  // token blocks with at least one token
  const float s = e.scale;
  const int rs = e.rs;
  // this lane's output tokens (accumulator column = slot tb*16 + r16)
  const int tok0 = toks[0];
  char* yrow[4];
  bool yok[4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    const int tk = toks[tb * 16 + r16];
    yok[tb] = tk >= 0;
    yrow[tb] = reinterpret_cast<char*>(io.y) + (int64_t)(tk >= 0 ? tk : tok0) * io.d_out * sizeof(TY);
  }
  // V^T operands: column = slot, k = 32 ks + 8 g + j
  const uint16_t* vrow[4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb)
    vrow[tb] = reinterpret_cast<const uint16_t*>(Vs + (tb * 16 + r16) * kVsStride);
  const int nmb = (m_hi - m_lo + 15) >> 4;
  const int mlast = m_hi - 1;
  const bool wave_pages = e.rpp >= 16;
  const int q_last = mlast / e.rpp;
  typedef typename Y4<TY>::raw yraw;
  auto load_blk = [&](int b, uint4 (&bo)[NK], yraw (&yv)[4]) {
    const int mb0 = __builtin_amdgcn_readfirstlane(m_lo + 16 * min(b, nmb - 1));
    const int m = min(mb0 + r16, mlast);
    const int64_t off = wave_pages ? b_offset_wave(pv, e, ELT, m, mb0, q_last) : b_offset(pv, e, ELT, m);
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const int k = 32 * ks + 8 * g;
      bo[ks] = keep16m(ld16(pv.pages + off + (int64_t)min(k, rs - 8) * ELT), k < rs);
    }
    const int mo = min(mb0 + 4 * g, m_hi - 4);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) yv[tb] = Y4<TY>::load_raw(yrow[tb], mo);
  };
  uint4 bc[MB][NK], bn[MB][NK];
  yraw yc[MB][4], yn[MB][4];
  // wave w handles m-blocks w + 4 * (MB * j + u), u < MB
#pragma unroll
  for (int u = 0; u < MB; ++u) load_blk(w + 4 * u, bc[u], yc[u]);
  for (int b0 = w; b0 < nmb; b0 += 4 * MB) {
    asm volatile("" ::: "memory");  // V operands are re-read from LDS every step
#pragma unroll
    for (int u = 0; u < MB; ++u) load_blk(b0 + 4 * (MB + u), bn[u], yn[u]);
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      const int b = b0 + 4 * u;
      f32x4_t acc[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) acc[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        asm volatile("" ::: "memory");  // one rank step of V operands live at a time
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          if (tb < ntb) {
            const uint4 vh = *reinterpret_cast<const uint4*>(vrow[tb] + 32 * ks + 8 * g);
            const uint4 vl = *reinterpret_cast<const uint4*>(vrow[tb] + KW + 32 * ks + 8 * g);
            acc[tb] = MfmaOp<T>::mma(as_vec<vec>(bc[u][ks]), as_vec<vec>(vh), acc[tb]);
            acc[tb] = MfmaOp<T>::mma(as_vec<vec>(bc[u][ks]), as_vec<vec>(vl), acc[tb]);
          }
        }
      }
      const int mo = m_lo + 16 * b + 4 * g;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        if (tb < ntb && b < nmb && mo < m_hi && yok[tb]) {
          float yv[4], out[4];
          Y4<TY>::unpack(yc[u][tb], yv);
#pragma unroll
          for (int i = 0; i < 4; ++i) out[i] = __builtin_fmaf(s, acc[tb][i], yv[i]);
          Y4<TY>::store(yrow[tb], mo, out);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < MB; ++u) {
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) bc[u][ks] = bn[u][ks];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) yc[u][tb] = yn[u][tb];
    }
  }
}

// ---- dispatch helpers (rank-dependent template arguments) -------------------
template <typename T, int MBT>
__device__ __forceinline__ void mfma_shrink_any(const PoolView& pv, const DevEntry& e,
                                                const IoDesc& io, const int* toks, int slot0,
                                                float* Vs) {
  switch ((e.rank + 15) >> 4) {
    case 1: mfma_shrink_lds<T, 1, MBT>(pv, e, io, toks, slot0, Vs); break;
    case 2: mfma_shrink_lds<T, 2, MBT>(pv, e, io, toks, slot0, Vs); break;
    case 3: mfma_shrink_lds<T, 3, MBT>(pv, e, io, toks, slot0, Vs); break;
    case 4: mfma_shrink_lds<T, 4, MBT>(pv, e, io, toks, slot0, Vs); break;
    case 5: mfma_shrink_lds<T, 5, MBT>(pv, e, io, toks, slot0, Vs); break;
    case 6: mfma_shrink_lds<T, 6, MBT>(pv, e, io, toks, slot0, Vs); break;
    case 7: mfma_shrink_lds<T, 7, MBT>(pv, e, io, toks, slot0, Vs); break;
    default: mfma_shrink_lds<T, 8, MBT>(pv, e, io, toks, slot0, Vs); break;
  }
}

template <typename T, typename TY>
__device__ __forceinline__ void mfma_pack_expand_any(const PoolView& pv, const DevEntry& e,
                                                     const IoDesc& io, const int* toks, int count,
                                                     float* Vs, int m_lo, int m_hi) {
  switch ((e.rs + 31) >> 5) {
    case 1:
      pack_v_lds<T, 1>(Vs, e.rank);
      mfma_expand_lds<T, TY, 1>(pv, e, io, toks, count, Vs, m_lo, m_hi);
      break;
    case 2:
      pack_v_lds<T, 2>(Vs, e.rank);
      mfma_expand_lds<T, TY, 2>(pv, e, io, toks, count, Vs, m_lo, m_hi);
      break;
    case 3:
      pack_v_lds<T, 3>(Vs, e.rank);
      mfma_expand_lds<T, TY, 3>(pv, e, io, toks, count, Vs, m_lo, m_hi);
      break;
    default:
      pack_v_lds<T, 4>(Vs, e.rank);
      mfma_expand_lds<T, TY, 4>(pv, e, io, toks, count, Vs, m_lo, m_hi);
      break;
  }
}

// ---- the three entry shapes ----------------------------------------------------
// Split-API shrink of half a tile (32 slots from slot0): v rows of its tokens.
template <typename T>
__device__ __forceinline__ void mfma_shrink_tile(const PoolView& pv, const PlanView& pl,
                                                 const PlanItem& item, const IoDesc& io,
                                                 int half, float* v, int v_ld, char* lds) {
  int* toks = reinterpret_cast<int*>(lds);
  float* Vs = reinterpret_cast<float*>(lds + 256);
  const DevEntry e = pv.entries[io.slice * pv.max_adapters + item.adapter];
  load_tile_tokens(pl, item, toks);
  __syncthreads();
  const int slot0 = 32 * half;
  if (slot0 >= item.count) return;
  const int t = threadIdx.x;
  if (e.rank <= 0) {
    for (int idx = t; idx < 32 * v_ld; idx += 256) {
      const int sl = slot0 + idx / v_ld;
      if (toks[sl] >= 0) v[(int64_t)toks[sl] * v_ld + idx % v_ld] = 0.f;
    }
    return;
  }
  mfma_shrink_any<T, 2>(pv, e, io, toks, slot0, Vs);
  const int rp = (e.rank + 15) & ~15;
  for (int idx = t; idx < 32 * v_ld; idx += 256) {
    const int sl = slot0 + idx / v_ld;
    const int n = idx % v_ld;
    const int tk = toks[sl];
    if (tk >= 0) v[(int64_t)tk * v_ld + n] = (n < e.rank && n < rp) ? Vs[sl * kVsStride + n] : 0.f;
  }
}

// Split-API expand of one tile over output rows [m_lo, m_hi): V from global v.
template <typename T, typename TY>
__device__ __forceinline__ void mfma_expand_tile(const PoolView& pv, const PlanView& pl,
                                                 const PlanItem& item, const DevEntry& e,
                                                 const IoDesc& io, const float* v, int v_ld,
                                                 int m_lo, int m_hi, char* lds) {
  int* toks = reinterpret_cast<int*>(lds);
  float* Vs = reinterpret_cast<float*>(lds + 256);
  load_tile_tokens(pl, item, toks);
  __syncthreads();
  const int KW = ((e.rs + 31) >> 5) * 32;
  for (int idx = threadIdx.x; idx < kTileM * KW; idx += 256) {
    const int sl = idx / KW;
    const int k = idx - sl * KW;
    const int tk = toks[sl];
    Vs[sl * kVsStride + k] = (tk >= 0 && k < e.rank) ? v[(int64_t)tk * v_ld + k] : 0.f;
  }
  __syncthreads();
  mfma_pack_expand_any<T, TY>(pv, e, io, toks, item.count, Vs, m_lo, m_hi);
}

// Fused tile: shrink into LDS, then expand rows [m_lo, m_hi).
template <typename T, typename TY>
__device__ __forceinline__ void mfma_apply_tile(const PoolView& pv, const PlanView& pl,
                                                const PlanItem& item, const DevEntry& e,
                                                const IoDesc& io, int m_lo, int m_hi, char* lds) {
  int* toks = reinterpret_cast<int*>(lds);
  float* Vs = reinterpret_cast<float*>(lds + 256);
  load_tile_tokens(pl, item, toks);
  __syncthreads();
  mfma_shrink_any<T, 4>(pv, e, io, toks, 0, Vs);
  mfma_pack_expand_any<T, TY>(pv, e, io, toks, item.count, Vs, m_lo, m_hi);
}

constexpr int kMfmaLds = 256 + kVsBytes;

}  // namespace lora
