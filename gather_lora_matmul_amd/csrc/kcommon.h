// Device helpers shared by the gfx950 kernels: element decode/encode, 16-byte
// gathers through the page table, DPP wave reductions and XCD-aware block
// mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lora_internal.h"

namespace lora {

constexpr int kMaxR = LORA_MAX_RANK;

// Storage tags.  fp32 is plain float.
struct f16_t {
  uint16_t b;
};
struct bf16_t {
  uint16_t b;
};
// OCP FP8 E4M3 adapter codes (quantised pools; per-row scales in the table)
struct fp8_t {
  uint8_t b;
};

template <typename T>
struct ET;
template <>
struct ET<float> {
  static constexpr int E = 4;  // elements per 16 bytes
  static constexpr int bytes = 4;
};
template <>
struct ET<f16_t> {
  static constexpr int E = 8;
  static constexpr int bytes = 2;
};
template <>
struct ET<bf16_t> {
  static constexpr int E = 8;
  static constexpr int bytes = 2;
};
template <>
struct ET<fp8_t> {
  static constexpr int E = 16;
  static constexpr int bytes = 1;
};
template <typename T>
constexpr bool is_quant() {
  return ET<T>::bytes == 1;
}
// 16-byte chunks of x (activation type X) that cover the columns of one
// 16-byte chunk of a weight row (type T): 2 for FP8 codes with 16-bit x.
template <typename T, typename X>
constexpr int x_chunks() {
  return ET<X>::bytes / ET<T>::bytes;
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// ---- 16-byte chunk -> E floats ---------------------------------------------
template <typename T>
__device__ __forceinline__ void unpack16(const uint4 u, float* f);

template <>
__device__ __forceinline__ void unpack16<float>(const uint4 u, float* f) {
  f[0] = __uint_as_float(u.x);
  f[1] = __uint_as_float(u.y);
  f[2] = __uint_as_float(u.z);
  f[3] = __uint_as_float(u.w);
}
template <>
__device__ __forceinline__ void unpack16<bf16_t>(const uint4 u, float* f) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void unpack16<f16_t>(const uint4 u, float* f) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    half2_t h = __builtin_bit_cast(half2_t, w[i]);
    f[2 * i] = (float)h.x;
    f[2 * i + 1] = (float)h.y;
  }
}

// 16 FP8 E4M3 codes -> floats with the hardware conversion (two codes per
// instruction; NaN codes stay NaN, subnormals are exact).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
template <>
__device__ __forceinline__ void unpack16<fp8_t>(const uint4 u, float* f) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
    const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
    f[4 * i] = lo.x;
    f[4 * i + 1] = lo.y;
    f[4 * i + 2] = hi.x;
    f[4 * i + 3] = hi.y;
  }
}

// acc + sum_e a[e] * x[e] over the E_T columns of one 16-byte weight chunk, x
// given as x_chunks<T, X>() 16-byte chunks of activations, ascending e.
template <typename T, typename X>
__device__ __forceinline__ float dotwx(const uint4 a, const uint4* x, float acc) {
  constexpr int E = ET<T>::E;
  constexpr int XC = x_chunks<T, X>();
  float fa[E], fx[E];
  unpack16<T>(a, fa);
#pragma unroll
  for (int q = 0; q < XC; ++q) unpack16<X>(x[q], fx + q * ET<X>::E);
#pragma unroll
  for (int e = 0; e < E; ++e) acc = __builtin_fmaf(fa[e], fx[e], acc);
  return acc;
}

// acc + sum_e a[e] * b[e] over one 16-byte chunk pair, ascending e.
template <typename T>
__device__ __forceinline__ float dot16(const uint4 a, const uint4 b, float acc) {
  constexpr int E = ET<T>::E;
  float fa[E], fb[E];
  unpack16<T>(a, fa);
  unpack16<T>(b, fb);
#pragma unroll
  for (int e = 0; e < E; ++e) acc = __builtin_fmaf(fa[e], fb[e], acc);
  return acc;
}
// acc + sum_e a[e] * v[e] with v already fp32 (LDS).
template <typename T>
__device__ __forceinline__ float dot16v(const uint4 a, const float* v, float acc) {
  constexpr int E = ET<T>::E;
  float fa[E];
  unpack16<T>(a, fa);
#pragma unroll
  for (int e = 0; e < E; ++e) acc = __builtin_fmaf(fa[e], v[e], acc);
  return acc;
}

// ---- scalar y access -------------------------------------------------------
// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

template <typename TY>
__device__ __forceinline__ float load_y(const void* base, int64_t idx);
template <>
__device__ __forceinline__ float load_y<float>(const void* base, int64_t idx) {
  return reinterpret_cast<const float*>(base)[idx];
}
template <>
__device__ __forceinline__ float load_y<bf16_t>(const void* base, int64_t idx) {
  return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(base)[idx] << 16);
}
template <>
__device__ __forceinline__ float load_y<f16_t>(const void* base, int64_t idx) {
  _Float16 h = __builtin_bit_cast(_Float16, reinterpret_cast<const uint16_t*>(base)[idx]);
  return (float)h;
}

template <typename TY>
__device__ __forceinline__ void store_y(void* base, int64_t idx, float v);
template <>
__device__ __forceinline__ void store_y<float>(void* base, int64_t idx, float v) {
  reinterpret_cast<float*>(base)[idx] = v;
}
template <>
__device__ __forceinline__ void store_y<bf16_t>(void* base, int64_t idx, float v) {
  reinterpret_cast<uint16_t*>(base)[idx] = f32_to_bf16_rne(v);
}
template <>
__device__ __forceinline__ void store_y<f16_t>(void* base, int64_t idx, float v) {
  reinterpret_cast<uint16_t*>(base)[idx] = __builtin_bit_cast(uint16_t, (_Float16)v);
}

// 16-bit storage <-> float without going through memory
template <typename TY>
__device__ __forceinline__ float bits_to_f(uint32_t h);
template <>
__device__ __forceinline__ float bits_to_f<bf16_t>(uint32_t h) {
  return __uint_as_float(h << 16);
}
template <>
__device__ __forceinline__ float bits_to_f<f16_t>(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
template <typename TY>
__device__ __forceinline__ uint32_t f_to_bits(float f);
template <>
__device__ __forceinline__ uint32_t f_to_bits<bf16_t>(float f) {
  return f32_to_bf16_rne(f);
}
template <>
__device__ __forceinline__ uint32_t f_to_bits<f16_t>(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
// Two fp32 -> two 16-bit values (RNE) packed lo | hi << 16: one conversion
// instruction for bf16.
template <typename TY>
__device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <>
__device__ __forceinline__ uint32_t pack2<bf16_t>(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
template <>
__device__ __forceinline__ uint32_t pack2<f16_t>(float lo, float hi) {
  const f16x2_t v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// ---- page-table resolution ---------------------------------------------------
// A device id names an adapter iff it lies in [0, max_adapters); negative ids
// (no adapter) and ids past the table are both skipped, so a bad id never
// indexes past the adapter table.
__device__ __forceinline__ bool adapter_in_table(const PoolView& pv, int a) {
  return (unsigned)a < (unsigned)pv.max_adapters;
}

// Load of a wave-uniform index of a read-only table through the scalar cache:
// the pointer is cast to the constant address space, so the load is an s_load
// tracked by its own counter and never waits behind outstanding vector loads.
__device__ __forceinline__ int32_t ld_uniform(const int32_t* p, int idx) {
  typedef const __attribute__((address_space(4))) int32_t* cptr;
  return ((cptr)p)[idx];
}

// Quantised adapters: the per-rank scales follow the page ids in the same
// table, as float bits: a_scale[k] at q_off + k, b_scale[k] at q_off + rank + k.
__device__ __forceinline__ float q_scale(const PoolView& pv, int idx) {
  return __int_as_float(pv.page_ids[idx]);
}

// Byte offset (from the pool base) of element j of A row k.
__device__ __forceinline__ int64_t a_offset(const PoolView& pv, const DevEntry& e, int npa,
                                            int elt, int k, int j) {
  const int c = (npa == 1) ? 0 : j / pv.P;
  const int pg = pv.page_ids[e.a_off + k * npa + c];
  return ((int64_t)pg * pv.P + (j - c * pv.P)) * elt;
}
// Byte offset of the page holding A row k when a row fits one page (npa == 1);
// k must be wave-uniform.
__device__ __forceinline__ int64_t a_row_uniform(const PoolView& pv, const DevEntry& e, int elt,
                                                 int k) {
  return (int64_t)ld_uniform(pv.page_ids, e.a_off + k) * pv.P * elt;
}
// Byte offset of B row m (r_s elements, 16-byte aligned).
__device__ __forceinline__ int64_t b_offset(const PoolView& pv, const DevEntry& e, int elt,
                                            int m) {
  int q = (int)((float)m * e.inv_rpp);
  int rem = m - q * e.rpp;
  if (rem < 0) {
    --q;
    rem += e.rpp;
  } else if (rem >= e.rpp) {
    ++q;
    rem -= e.rpp;
  }
  const int pg = pv.page_ids[e.b_off + q];
  return ((int64_t)pg * pv.P + (int64_t)rem * e.rs) * elt;
}

// Byte offset of B row m for a lane of a wave whose rows all lie in
// [m0, m0 + 16), m0 wave-uniform (the MFMA expand's 16-row groups): with
// rpp >= 16 (the planner only makes tiles of such layouts) those rows touch at
// most two pages, whose ids are read with scalar loads (q_last bounds the page
// list).
__device__ __forceinline__ int64_t b_offset_wave(const PoolView& pv, const DevEntry& e, int elt,
                                                 int m, int m0, int q_last) {
  int q0 = (int)((float)m0 * e.inv_rpp);
  int rem0 = m0 - q0 * e.rpp;
  if (rem0 < 0) --q0;
  else if (rem0 >= e.rpp) ++q0;
  const int pg0 = ld_uniform(pv.page_ids, e.b_off + q0);
  const int pg1 = ld_uniform(pv.page_ids, e.b_off + min(q0 + 1, q_last));
  int rem = m - q0 * e.rpp;
  const bool second = rem >= e.rpp;
  rem = second ? rem - e.rpp : rem;
  return ((int64_t)(second ? pg1 : pg0) * pv.P + (int64_t)rem * e.rs) * elt;
}

// ---- wave reductions (DPP inside rows of 16, then 4 readlanes) --------------
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over the 64 lanes, returned in every lane (wave-uniform).  The order of
// additions is fixed, so the result is run-to-run deterministic.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0x141>(v);  // row_half_mirror
  v += dpp_mov<0x140>(v);  // row_mirror: every lane holds its row-of-16 sum
  const int iv = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(iv, 48));
  return (r0 + r1) + (r2 + r3);
}

// ---- XCD-aware block mapping ------------------------------------------------
// Workgroups are dealt round-robin to the 8 XCDs (block b -> XCD b % 8).  All
// `nsplit` blocks of one work unit should share an XCD so that what they both
// read (the shrink operands) is served from that XCD's L2.  Unit u goes to XCD
// u % 8; its split q gets block ((u / 8) * nsplit + q) * 8 + u % 8.
__device__ __forceinline__ void xcd_unit_split(int b, int nsplit, int& unit, int& split) {
  const int xcd = b & 7;
  const int j = b >> 3;
  split = j % nsplit;
  unit = (j / nsplit) * 8 + xcd;
}
inline int xcd_grid(int units, int nsplit) { return ((units + 7) / 8) * nsplit * 8; }

}  // namespace lora
