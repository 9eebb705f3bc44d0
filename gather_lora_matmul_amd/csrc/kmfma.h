// MFMA tiles for groups of tokens that share one adapter (the long SGMV
// segments of the multi-LoRA serving article, SGMV section).
//
// A tile is up to 64 token slots of one group; blocks of four waves run
// v_mfma_f32_16x16x32_{bf16,f16}.  The kernels are persistent: for each launch
// shape the host splits the launch's work sequence (the tiles of launch slice
// 0, then of slice 1, ...; stages or chunks weighted by the bytes they move)
// into one contiguous range per block (layout.h), so every block moves about
// the same number of bytes and no block waits for a second wave of the grid.
//
// Shrink  V^T[n][t] = sum_j A[n][j] X[t][j]   (M = rank, N = tokens, K = d_in)
//   Stages of 64 columns: the X rows of the tile's tokens and the A rows of
//   the adapter go from global memory straight into LDS (16-byte loads, eight
//   lanes per 128-byte row segment) through a three-buffer ring, two stages
//   in flight while one is computed; wave w owns tokens [16w, 16w + 16) and
//   all rank blocks.  A range may cover only part of a tile's stages (split
//   K); each such contribution is a partial tile.  Split API: a block that
//   covers a whole tile writes v, a reduce kernel sums the partials of the
//   others in block order; fused apply: the expand sums them while loading V.
// Expand  Y^T[m][t] += s * sum_k B[m][k] V[t][k]  (M = output rows, N = tokens,
//   K = rank), in chunks of 64 rows: wave w computes rows [16w, 16w + 16) of
//   the chunk for all tokens; B rows are read from their pages in natural
//   [d_out][r_s] layout (the MFMA A-operand layout); V is split into hi + lo
//   16-bit parts in LDS so the fp32 shrink result enters the 16-bit MFMA with
//   ~2^-16 relative error.  The accumulators go through LDS so that y is read,
//   updated and written with coalesced 16-byte accesses; y and B of the chunk
//   two ahead are in flight while a chunk is computed.
//
// The same k-to-lane assignment is used for both operands of every MFMA, so the
// hardware's internal k order does not matter; only the row/column placement
// of the operands and of the accumulator (A row = lane % 16, B column =
// lane % 16, accumulator column = lane % 16, rows 4 * (lane / 16) + i) is used.
// Global loads inside the pipelines are unconditional per lane (clamped
// indices, masked values); only block-uniform conditions skip work.
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

template <typename V>
__device__ __forceinline__ V as_vec(const uint4 u) {
  return __builtin_bit_cast(V, u);
}
__device__ __forceinline__ uint4 keep16m(uint4 v, bool keep) {
  return keep ? v : make_uint4(0, 0, 0, 0);
}

// ---- LDS layout -------------------------------------------------------------------
// Four separate LDS arrays per block (separate arrays let the compiler see that
// reading one buffer does not alias the global -> LDS loads in flight to the
// others): `misc` (tile tokens, flags, A page ids) and three work buffers a, b,
// c: the shrink's stage ring, or the expand's packed V (hi in a, lo in b) and
// accumulator staging (c).
constexpr int kMT = 256;                       // threads per block
constexpr int kKC = 64;                        // shrink stage: columns of X and A
constexpr int kRowB = kKC * 2;                 // staged row: 128 bytes (swizzled units)
constexpr int kStageB = (kTileM + kMaxR) * kRowB;  // X rows, then A rows
constexpr int kDsRow = 64 + 4;                 // accumulator staging row (floats)
constexpr int kOffToks = 0;                    // misc: int[64]
constexpr int kOffMisc = 256;                  // misc: int[4]
constexpr int kOffApg = 512;                   // misc: int[kMaxR][npa]: A page ids of the tile
constexpr int kMiscB = kOffApg + kMaxR * kMaxNpa * 4;
constexpr int kVpB = kTileM * kMaxR * 2;      // packed V (uint16): hi or lo
constexpr int kDsB = kTileM * kDsRow * 4;
constexpr int kBufB = kStageB;
static_assert(kVpB <= kBufB && kDsB <= kBufB, "expand buffers must fit the work buffers");
static_assert(kMiscB + 3 * kBufB <= 80 * 1024, "two blocks per CU must fit the LDS");

struct LdsBufs {
  char* misc;
  char* a;
  char* b;
  char* c;
};

// Packed V (hi or lo parts, uint16): element (slot, k) sits at
// ((k / 8) * kTileM + slot) * 8 + k % 8, k-group major, so the 16 lanes of an
// MFMA operand read (16 slots, one 8-element k group) cover 256 contiguous
// bytes; with slot-major rows the same read spreads over 16 rows and takes
// twice the LDS cycles (bank conflicts).
__device__ __forceinline__ int vp_index(int slot, int k) { return ((k >> 3) * kTileM + slot) * 8 + (k & 7); }

// s_waitcnt immediate that waits for vmcnt <= n only (expcnt and lgkmcnt at
// their maxima; vmcnt is split over bits 3:0 and 15:14).
constexpr int wait_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// Block barrier for LDS traffic only: the wave's LDS accesses are complete
// (lgkmcnt 0) and global loads in flight stay in flight.  __syncthreads also
// waits for every outstanding global load of the wave, which would drain the
// prefetch pipelines at every step.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14));  // lgkmcnt(0) only
  asm volatile("s_barrier" ::: "memory");
}

// ---- block ranges -----------------------------------------------------------------
// Block L's range is [pos[L], pos[L + 1]) of the launch's work sequence (the
// tiles of launch slice 0, then of slice 1, ...).  L is block-uniform: the
// table entries are scalar loads.
__device__ __forceinline__ RangePos load_pos(const RangePos* tab, int L) {
  typedef const __attribute__((address_space(4))) int32_t* cptr;
  const cptr p = (cptr)(tab + L);
  return RangePos{p[0], p[1], p[2], 0};
}
__device__ __forceinline__ bool pos_before(int j, int t, int k, const RangePos& b) {
  return j < b.j || (j == b.j && (t < b.tile || (t == b.tile && k < b.k)));
}
// fn(j, tile, k0, k1, first, last) for every piece of block L's range, in
// order: units [k0, k1) of `tile` in launch slice j (units(j) per tile),
// first / last: the piece is the range's first / last one.
template <typename Units, typename Fn>
__device__ __forceinline__ void for_each_piece(const RangePos* tab, int L, int n_tiles,
                                               Units&& units, Fn&& fn) {
  const RangePos a = load_pos(tab, L);
  const RangePos b = load_pos(tab, L + 1);
  int j = a.j, t = a.tile, k = a.k;
  bool first = true;
  while (pos_before(j, t, k, b)) {
    const bool ends_here = j == b.j && t == b.tile;
    const int k1 = ends_here ? b.k : units(j);
    int nj = j, nt = t + 1;
    if (nt == n_tiles) {
      nt = 0;
      ++nj;
    }
    fn(j, t, k, k1, first, ends_here || !pos_before(nj, nt, 0, b));
    first = false;
    j = nj;
    t = nt;
    k = 0;
  }
}
// Blocks are dealt round-robin to the 8 XCDs; logical blocks [x*G/8, (x+1)*G/8)
// run on XCD x, so neighbouring ranges (the same adapters) share an L2.
__device__ __forceinline__ int logical_block(int b, int G) { return (b & 7) * (G >> 3) + (b >> 3); }

__device__ __forceinline__ void load_tile_tokens(const PlanView& pl, const PlanItem& item,
                                                 int* toks) {
  if (threadIdx.x < kTileM)
    toks[threadIdx.x] = (int)threadIdx.x < item.count ? pl.perm[item.start + threadIdx.x] : -1;
}

// ---- shrink ---------------------------------------------------------------------
// One 16-byte global -> LDS load per lane: lane L's bytes land at lds + 16 L
// (lds wave-uniform).  The data never passes through VGPRs.  Written as inline
// asm so that the compiler does not track these LDS writes: it would otherwise
// wait for every such load in flight before any LDS read it cannot prove
// disjoint, draining the stage ring.  The callers wait for the loads
// themselves (s_waitcnt vmcnt + barrier) before reading the stage; loads
// return in order, so the compiler's own vmcnt waits stay correct (only more
// conservative).  The asm has no register outputs.
__device__ __forceinline__ void load_lds16(const void* g, void* lds) {
  const uint32_t la = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(la), "v"(g) : "memory", "m0");
}

// Staged rows are 128 bytes (64 columns) with the eight 16-byte units of row r
// stored in the order u ^ (r & 7): the 16 rows an MFMA operand read touches
// then fall on 16 different bank groups.
__device__ __forceinline__ int stage_unit(int row, int u) { return row * 8 + (u ^ (row & 7)); }

// acc[nb] (wave w, tokens [16w, 16w+16)) += the tile's stages [s0, s1).
// A stage is X[64 slots][64 cols] and A[16*NB rank rows][64 cols], loaded into
// one of two LDS buffers while the other is computed.
template <typename T, int NB>
__device__ __forceinline__ void shrink_stages(const PoolView& pv, const DevEntry& e,
                                              const IoDesc& io, const int* toks, int count,
                                              int s0, int s1, const LdsBufs& lb, f32x4_t (&acc)[NB]) {
  typedef typename MfmaOp<T>::vec vec;
  constexpr int NAQ = (NB + 1) / 2;  // A loads per wave per stage (8 rows each)
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int ntb = (count + 15) >> 4;
  const int d_in = io.d_in;
  const int rank = e.rank;
  // lane L of a load covers row 8 i + L / 8 of the load's 8 rows and the
  // 16-byte unit that lands at position L % 8 of that row
  const int lrow = lane >> 3;
  const int c8 = 8 * ((lane & 7) ^ lrow);  // column within the stage
  // X: load i = w + 4 q (q < 2) covers slots [8 i, 8 i + 8) (slots past the
  // count repeat the last token: cache hits, never stored)
  const char* xrow[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int slot = 8 * (w + 4 * q) + lrow;
    xrow[q] = reinterpret_cast<const char*>(io.x) + (int64_t)toks[min(slot, count - 1)] * d_in * 2;
  }
  // A: load i = w + 4 q (q < NAQ) covers rank rows [8 i, 8 i + 8); rows past the
  // rank repeat the last one (finite; no MFMA result column past the rank is kept)
  const int* apg = reinterpret_cast<const int*>(lb.misc + kOffApg);
  const int npa = io.npa;
  const int P = pv.P;
  const float invP = 1.0f / (float)P;
  int arow[NAQ];
#pragma unroll
  for (int q = 0; q < NAQ; ++q) arow[q] = min(8 * (w + 4 * q) + lrow, rank - 1);
  // Every wave issues the same 2 + NAQ loads per stage (none is skipped), so a
  // wait with a fixed count separates the stages.
  constexpr int LPS = 2 + NAQ;
  auto issue = [&](int s, char* b) {
    const int colc = min(kKC * s + c8, d_in - 8);
    int c = (int)((float)colc * invP);  // page chunk: float quotient, corrected
    int ofs = colc - c * P;
    c = ofs < 0 ? c - 1 : (ofs >= P ? c + 1 : c);
    ofs = colc - c * P;
#pragma unroll
    for (int q = 0; q < 2; ++q) load_lds16(xrow[q] + (int64_t)colc * 2, b + (w + 4 * q) * 1024);
#pragma unroll
    for (int q = 0; q < NAQ; ++q)
      load_lds16(pv.pages + ((int64_t)apg[arow[q] * npa + c] * P + ofs) * 2,
                 b + kTileM * kRowB + (w + 4 * q) * 1024);
  };
  auto compute = [&](int s, const char* b) {
    if (w < ntb) {
      const int row = 16 * w + r16;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        // X columns past d_in (last stage only) are zero; A there is finite
        const bool cok = kKC * s + 32 * ks + 8 * g < d_in;
        const uint4 xo = keep16m(*reinterpret_cast<const uint4*>(b + 16 * stage_unit(row, 4 * ks + g)), cok);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int ar = 16 * nb + r16;
          const uint4 ao =
              *reinterpret_cast<const uint4*>(b + kTileM * kRowB + 16 * stage_unit(ar, 4 * ks + g));
          acc[nb] = MfmaOp<T>::mma(as_vec<vec>(ao), as_vec<vec>(xo), acc[nb]);
        }
      }
    }
  };
  // Three-buffer ring: stages s + 1 and s + 2 are in flight while stage s is
  // computed.  Each step waits for the wave's own loads of stage s (stage s + 1,
  // if there is one, stays outstanding); the barrier then makes every wave's
  // loads of stage s visible and frees the buffer of stage s - 1 for stage
  // s + 2.  No stage past s1 - 1 is issued, so no load is in flight when the
  // range ends.  (The conditions are block-uniform.)
  auto step = [&](int s, const char* cur, char* nxt2) {
    if (s + 1 < s1) __builtin_amdgcn_s_waitcnt(wait_vm(LPS));
    else __builtin_amdgcn_s_waitcnt(wait_vm(0));
    lds_barrier();
    if (s + 2 < s1) issue(s + 2, nxt2);
    compute(s, cur);
  };
  issue(s0, lb.a);
  if (s0 + 1 < s1) issue(s0 + 1, lb.b);
  for (int s = s0; s < s1; s += 3) {
    step(s, lb.a, lb.c);
    if (s + 1 < s1) step(s + 1, lb.b, lb.a);
    if (s + 2 < s1) step(s + 2, lb.c, lb.b);
  }
  lds_barrier();  // every wave is done with the stage buffers
}

// ---- shrink outputs ---------------------------------------------------------------
// A block's contribution to a tile is a partial tile in the MFMA lane layout:
// float4 unit (nb * ntb + w) * 64 + lane holds ranks 16 nb + 4 g + [0, 4) of
// slot 16 w + r16 (ntb = token blocks of the tile), at the contribution's
// float4 offset in the plan's partial-tile workspace.
__device__ __forceinline__ float4* part_at(const PlanView& pl, int32_t off) {
  return reinterpret_cast<float4*>(pl.part) + off;
}
// Tiles per launch slice: the plan's count, or, for a plan built on the
// device, the count the planner wrote.
__device__ __forceinline__ int plan_tiles(const PlanView& pl) {
  return pl.n_tiles_dev ? *pl.n_tiles_dev : pl.n_mfma;
}
// Contributions [c_off[0], c_off[1]) of tile i in launch slice j (T tiles).
__device__ __forceinline__ const int32_t* contrib_range(const PlanView& pl, int T, int j, int i) {
  return pl.c_off + (int64_t)j * (T + 1) + i;
}
// Unit u of a partial tile with ntb token blocks -> (slot, first rank)
__device__ __forceinline__ int unit_slot(int u, int ntb) { return 16 * ((u >> 6) % ntb) + (u & 15); }
__device__ __forceinline__ int unit_rank(int u, int ntb) { return 16 * ((u >> 6) / ntb) + 4 * ((u & 63) >> 4); }

// v[token][n .. n + 4) of a tile slot (split API rows; n >= rank -> 0).
__device__ __forceinline__ void v_store4(float* v, int v_ld, int tok, int n, int rank, float4 a4) {
  float* row = v + (int64_t)tok * v_ld;
  const float a[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (n + i < v_ld) row[n + i] = n + i < rank ? a[i] : 0.f;
}
// v columns [w0, v_ld) of the tile's tokens are zero.
__device__ __forceinline__ void v_zero_tail(float* v, int v_ld, const int* toks, int count, int w0) {
  const int nz = v_ld - w0;
  if (nz <= 0) return;
  for (int idx = threadIdx.x; idx < count * nz; idx += kMT) {
    const int slot = idx / nz;
    v[(int64_t)toks[slot] * v_ld + w0 + (idx - slot * nz)] = 0.f;
  }
}

// One piece of the block's shrink range: stages [k0, k1) of nst of a tile.
// Split API (v != null): a block that covers the whole tile writes v; others
// write their partial tile (at float4 offset part_off), summed by the reduce
// kernel.  Fused (v == null): every contribution is a partial tile, summed
// when the expand loads V.
template <typename T, int NB>
__device__ __forceinline__ void shrink_tile(const PoolView& pv, const PlanView& pl,
                                            const DevEntry& e, const IoDesc& io, int count,
                                            int k0, int k1, int nst, int32_t part_off, float* v,
                                            int v_ld, const LdsBufs& lb) {
  const int* toks = reinterpret_cast<const int*>(lb.misc + kOffToks);
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int ntb = (count + 15) >> 4;
  f32x4_t acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  shrink_stages<T, NB>(pv, e, io, toks, count, k0, k1, lb, acc);
  const int slot = 16 * w + r16;
  if (v && k0 == 0 && k1 == nst) {
    if (w < ntb && slot < count) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        v_store4(v, v_ld, toks[slot], 16 * nb + 4 * g, e.rank,
                 make_float4(acc[nb][0], acc[nb][1], acc[nb][2], acc[nb][3]));
    }
    v_zero_tail(v, v_ld, toks, count, 16 * NB);
  } else {
    float4* part = part_at(pl, part_off);
    if (w < ntb) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        part[(nb * ntb + w) * 64 + lane] = make_float4(acc[nb][0], acc[nb][1], acc[nb][2], acc[nb][3]);
    }
  }
  lds_barrier();  // the tile's tokens in LDS are free (the stores stay in flight)
}

// The block's shrink range over the launch slices ios[0 .. n_io).  The
// partial tiles of its first and last piece sit at part_fl[L]; a piece in
// between covers a whole tile, the tile's only contribution.
template <typename T, typename IoOf>
__device__ __forceinline__ void shrink_range(const PoolView& pv, const PlanView& pl, IoOf&& io_of,
                                             int L, float* v, int v_ld, const LdsBufs& lb) {
  typedef const __attribute__((address_space(4))) int32_t* cptr;
  const cptr fl = (cptr)(pl.part_fl + L);
  const int32_t part_first = fl[0], part_last = fl[1];
  int* toks = reinterpret_cast<int*>(lb.misc + kOffToks);
  const int ntl = plan_tiles(pl);
  for_each_piece(pl.bs_shrink, L, ntl, [&](int j) { return (io_of(j).d_in + kKC - 1) / kKC; },
                 [&](int j, int i, int k0, int k1, bool first, bool last) {
    const IoDesc io = io_of(j);
    const int nst = (io.d_in + kKC - 1) / kKC;
    const PlanItem item = pl.items[i];
    const DevEntry e = pv.entries[io.slice * pv.max_adapters + item.adapter];
    // (device-built plans: an adapter not resident in this slice has no work
    // here, and the expand skips the same piece)
    if (e.rank <= 0) return;
    const int32_t part_off = first ? part_first : last ? part_last : pl.c_ent[*contrib_range(pl, ntl, j, i)];
    load_tile_tokens(pl, item, toks);
    {  // A page ids of the tile's rank rows (rows past the rank repeat the last)
      int* apg = reinterpret_cast<int*>(lb.misc + kOffApg);
      const int rp = (e.rank + 15) & ~15;
      for (int idx = threadIdx.x; idx < rp * io.npa; idx += kMT) {
        const int n = idx / io.npa;
        const int c = idx - n * io.npa;
        apg[idx] = pv.page_ids[e.a_off + min(n, e.rank - 1) * io.npa + c];
      }
    }
    __syncthreads();
    switch ((e.rank + 15) >> 4) {
      case 1: shrink_tile<T, 1>(pv, pl, e, io, item.count, k0, k1, nst, part_off, v, v_ld, lb); break;
      case 2: shrink_tile<T, 2>(pv, pl, e, io, item.count, k0, k1, nst, part_off, v, v_ld, lb); break;
      case 3: shrink_tile<T, 3>(pv, pl, e, io, item.count, k0, k1, nst, part_off, v, v_ld, lb); break;
      case 4: shrink_tile<T, 4>(pv, pl, e, io, item.count, k0, k1, nst, part_off, v, v_ld, lb); break;
      case 5: shrink_tile<T, 5>(pv, pl, e, io, item.count, k0, k1, nst, part_off, v, v_ld, lb); break;
      case 6: shrink_tile<T, 6>(pv, pl, e, io, item.count, k0, k1, nst, part_off, v, v_ld, lb); break;
      case 7: shrink_tile<T, 7>(pv, pl, e, io, item.count, k0, k1, nst, part_off, v, v_ld, lb); break;
      default: shrink_tile<T, 8>(pv, pl, e, io, item.count, k0, k1, nst, part_off, v, v_ld, lb); break;
    }
  });
}

// Split API: v rows of a tile that several blocks shared: the sum of their
// partial tiles in block order (the first one, then += the others).
__device__ __forceinline__ void shrink_reduce_tile(const PlanView& pl, const IoDesc& io, int tile,
                                                   int rank, float* v, int v_ld, int* toks) {
  const int32_t* off = contrib_range(pl, pl.n_mfma, 0, tile);
  const int c0 = off[0], c1 = off[1];
  if (c1 - c0 <= 1) return;  // a single block covered the tile and wrote v
  const PlanItem item = pl.items[tile];
  load_tile_tokens(pl, item, toks);
  __syncthreads();
  const int ntb = (item.count + 15) >> 4;
  const int nu = ((rank + 15) >> 4) * ntb * 64;
  for (int u = threadIdx.x; u < nu; u += kMT) {
    const int sl = unit_slot(u, ntb);
    if (sl >= item.count) continue;
    float4 sum = part_at(pl, pl.c_ent[c0])[u];
    for (int c = c0 + 1; c < c1; ++c) {
      const float4 q = part_at(pl, pl.c_ent[c])[u];
      sum.x += q.x;
      sum.y += q.y;
      sum.z += q.z;
      sum.w += q.w;
    }
    v_store4(v, v_ld, toks[sl], unit_rank(u, ntb), rank, sum);
  }
  v_zero_tail(v, v_ld, toks, item.count, (rank + 15) & ~15);
}

// ---- expand ---------------------------------------------------------------------
// 16-byte y pieces: PPR per 64-row chunk row, YP per thread.
template <typename TY>
struct YPiece {
  static constexpr int EPP = 8;  // elements per piece
  static __device__ __forceinline__ uint4 fma(uint4 y, const float* a, float s) {
    const uint32_t w[4] = {y.x, y.y, y.z, y.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __builtin_fmaf(s, a[2 * i], bits_to_f<TY>(w[i] & 0xffffu));
      const float hi = __builtin_fmaf(s, a[2 * i + 1], bits_to_f<TY>(w[i] >> 16));
      o[i] = pack2<TY>(lo, hi);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
  }
};
template <>
struct YPiece<float> {
  static constexpr int EPP = 4;
  static __device__ __forceinline__ uint4 fma(uint4 y, const float* a, float s) {
    return make_uint4(__float_as_uint(__builtin_fmaf(s, a[0], __uint_as_float(y.x))),
                      __float_as_uint(__builtin_fmaf(s, a[1], __uint_as_float(y.y))),
                      __float_as_uint(__builtin_fmaf(s, a[2], __uint_as_float(y.z))),
                      __float_as_uint(__builtin_fmaf(s, a[3], __uint_as_float(y.w))));
  }
};

// Split API: V rows of the tile (fp32, the caller's v by token) -> hi and lo
// 16-bit parts in LDS.  All of a thread's loads are issued before any is used.
template <typename T, int NK>
__device__ __forceinline__ void load_v_tile(const float* v, int v_ld, const int* toks, int count,
                                            int rank, uint16_t* Vh, uint16_t* Vl) {
  constexpr int KW = 32 * NK;
  constexpr int PER = kTileM * KW / kMT;  // 8, 16, 24 or 32
  static_assert(kTileM == 64, "packed V index: 64 slots x 8 elements per k group");
  // thread element p is packed position p (vp_index order): slot (p / 8) % 64,
  // k = 8 (p / 512) + p % 8
  for (int q0 = 0; q0 < PER; q0 += 8) {
    float f[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int p = threadIdx.x + kMT * (q0 + q);
      const int slot = (p >> 3) & (kTileM - 1);
      const int k = ((p >> 9) << 3) | (p & 7);
      f[q] = v[(int64_t)toks[min(slot, count - 1)] * v_ld + min(k, rank - 1)];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int p = threadIdx.x + kMT * (q0 + q);
      const int slot = (p >> 3) & (kTileM - 1);
      const int k = ((p >> 9) << 3) | (p & 7);
      uint16_t hi, lo;
      MfmaOp<T>::split((slot < count && k < rank) ? f[q] : 0.f, hi, lo);
      Vh[p] = hi;
      Vl[p] = lo;
    }
  }
}

// Chunks [c0, c1) (64 output rows each) of one tile.  `load_v` packs the
// tile's V into LDS (Vh, Vl); it runs while the loads of the first two chunks
// are in flight, so their latencies overlap.
template <typename T, typename TY, int NK, typename LoadV>
__device__ __forceinline__ void expand_chunks(const PoolView& pv, const DevEntry& e,
                                              const IoDesc& io, const int* toks, int count,
                                              int c0, int c1, const uint16_t* Vh,
                                              const uint16_t* Vl, float* D, LoadV&& load_v) {
  typedef typename MfmaOp<T>::vec vec;
  constexpr int EPP = YPiece<TY>::EPP;
  constexpr int PPR = 64 / EPP;              // pieces per token row of a chunk
  constexpr int YP = kTileM * PPR / kMT;     // pieces per thread
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int ntb = (count + 15) >> 4;
  const int d_out = io.d_out;
  const int rs = e.rs;
  const float s = e.scale;
  // this thread's y pieces
  char* yrow[YP];
  bool yok[YP];
  int yslot[YP], ymo[YP];
#pragma unroll
  for (int j = 0; j < YP; ++j) {
    const int q = t + kMT * j;
    yslot[j] = q / PPR;
    ymo[j] = (q % PPR) * EPP;
    yok[j] = yslot[j] < count;
    yrow[j] = reinterpret_cast<char*>(io.y) +
              (int64_t)toks[min(yslot[j], count - 1)] * d_out * (int)sizeof(TY);
  }
  const int q_last = (d_out - 1) / e.rpp;
  auto loadB = [&](int c, uint4 (&bo)[NK]) {
    // rpp >= 16 (planner): the wave's 16 rows lie on at most two pages, whose
    // ids are scalar loads
    const int mb0 = __builtin_amdgcn_readfirstlane(min(64 * c + 16 * w, d_out - 1));
    const int m = min(mb0 + r16, d_out - 1);
    const int64_t off = b_offset_wave(pv, e, 2, m, mb0, q_last);
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
      bo[ks] = ld16(pv.pages + off + (int64_t)min(32 * ks + 8 * g, rs - 8) * 2);
  };
  bool kok[NK];  // B columns past the stored row length are masked at use
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) kok[ks] = 32 * ks + 8 * g < rs;
  auto loadY = [&](int c, uint4 (&yv)[YP]) {
#pragma unroll
    for (int j = 0; j < YP; ++j) {
      const int m = min(64 * c + ymo[j], d_out - EPP);
      yv[j] = ld16(yrow[j] + (int64_t)m * (int)sizeof(TY));
    }
  };
  // Three register sets rotate by unrolling (a register copy of a load in
  // flight would wait for it): chunk c uses set (c - c0) % 3, and the loads of
  // chunk c + 2 are issued before chunk c is computed.  Prefetches are never
  // skipped (register loads under a branch compile to a wait right behind
  // them): past c1 they repeat the last chunk.
  auto process = [&](int c, const uint4 (&bc)[NK], const uint4 (&yc)[YP]) {
    f32x4_t acc[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) acc[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      if (tb < ntb) {
        const int vo = vp_index(16 * tb + r16, 8 * g);  // + 4 k groups per k step
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
          const uint4 vh = *reinterpret_cast<const uint4*>(Vh + vo + 32 * kTileM * ks);
          const uint4 vl = *reinterpret_cast<const uint4*>(Vl + vo + 32 * kTileM * ks);
          const vec bk = as_vec<vec>(keep16m(bc[ks], kok[ks]));
          acc[tb] = MfmaOp<T>::mma(bk, as_vec<vec>(vh), acc[tb]);
          acc[tb] = MfmaOp<T>::mma(bk, as_vec<vec>(vl), acc[tb]);
        }
      }
    }
    lds_barrier();  // D is free: every wave is done with the previous chunk's RMW
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
      if (tb < ntb)
        *reinterpret_cast<float4*>(D + (16 * tb + r16) * kDsRow + 16 * w + 4 * g) =
            make_float4(acc[tb][0], acc[tb][1], acc[tb][2], acc[tb][3]);
    lds_barrier();
#pragma unroll
    for (int j = 0; j < YP; ++j) {
      const int m = 64 * c + ymo[j];
      if (yok[j] && m < d_out) {
        float a[EPP];
        const float* dr = D + yslot[j] * kDsRow + ymo[j];
#pragma unroll
        for (int i = 0; i < EPP; i += 4) {
          const float4 q = *reinterpret_cast<const float4*>(dr + i);
          a[i] = q.x;
          a[i + 1] = q.y;
          a[i + 2] = q.z;
          a[i + 3] = q.w;
        }
        *reinterpret_cast<uint4*>(yrow[j] + (int64_t)m * (int)sizeof(TY)) = YPiece<TY>::fma(yc[j], a, s);
      }
    }
  };
  uint4 b0[NK], b1[NK], b2[NK], y0[YP], y1[YP], y2[YP];
  loadB(c0, b0);
  loadY(c0, y0);
  __builtin_amdgcn_sched_barrier(0);  // keep the prologue in loop order
  loadB(min(c0 + 1, c1 - 1), b1);
  loadY(min(c0 + 1, c1 - 1), y1);
  __builtin_amdgcn_sched_barrier(0);
  load_v();
  lds_barrier();  // V is in LDS
  for (int c = c0; c < c1; c += 3) {
    loadB(min(c + 2, c1 - 1), b2);
    loadY(min(c + 2, c1 - 1), y2);
    process(c, b0, y0);
    loadB(min(c + 3, c1 - 1), b0);
    loadY(min(c + 3, c1 - 1), y0);
    if (c + 1 < c1) process(c + 1, b1, y1);
    loadB(min(c + 4, c1 - 1), b1);
    loadY(min(c + 4, c1 - 1), y1);
    if (c + 2 < c1) process(c + 2, b2, y2);
  }
}

// Tiles of at most 16 tokens (one token block; decode groups): steps of JB
// chunks (64 JB output rows), wave w computing rows [16 JB w, 16 JB (w + 1))
// of the step as JB 16-row MFMA blocks (JB = 4 up to rank 64, 2 above).  A
// step moves JB chunks' B rows while y (<= 16 tokens) stays small, so each
// round trip carries JB times the bytes of a 64-row chunk; B and y of the next
// step are in flight while a step is computed.  Rows past the range's last
// chunk (or d_out) are not written.
template <typename T, typename TY, int NK, typename LoadV>
__device__ __forceinline__ void expand_chunks_wide(const PoolView& pv, const DevEntry& e,
                                                   const IoDesc& io, const int* toks, int count,
                                                   int c0, int c1, const uint16_t* Vh,
                                                   const uint16_t* Vl, float* D, LoadV&& load_v) {
  constexpr int JB = NK <= 2 ? 4 : 2;      // 16-row blocks per wave and step
  typedef typename MfmaOp<T>::vec vec;
  constexpr int EPP = YPiece<TY>::EPP;
  constexpr int WR = 64 * JB;              // output rows per step
  constexpr int PPR = WR / EPP;            // pieces per token row of a step
  constexpr int YP = 16 * PPR / kMT;       // pieces per thread
  constexpr int DROW = WR + 4;             // accumulator staging row (floats)
  static_assert(16 * DROW * 4 <= kDsB, "wide accumulator staging must fit D");
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int d_out = io.d_out;
  const int m_end = min(64 * c1, d_out);   // rows of this range end here
  const int rs = e.rs;
  const float s = e.scale;
  char* yrow[YP];
  bool yok[YP];
  int yslot[YP], ymo[YP];
#pragma unroll
  for (int j = 0; j < YP; ++j) {
    const int q = t + kMT * j;
    yslot[j] = q / PPR;
    ymo[j] = (q % PPR) * EPP;
    yok[j] = yslot[j] < count;
    yrow[j] = reinterpret_cast<char*>(io.y) +
              (int64_t)toks[min(yslot[j], count - 1)] * d_out * (int)sizeof(TY);
  }
  const int q_last = (d_out - 1) / e.rpp;
  auto loadB = [&](int c, uint4 (&bo)[JB][NK]) {
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) {
      const int mb0 = __builtin_amdgcn_readfirstlane(min(64 * c + 16 * JB * w + 16 * jb, d_out - 1));
      const int m = min(mb0 + r16, d_out - 1);
      const int64_t off = b_offset_wave(pv, e, 2, m, mb0, q_last);
#pragma unroll
      for (int ks = 0; ks < NK; ++ks)
        bo[jb][ks] = ld16(pv.pages + off + (int64_t)min(32 * ks + 8 * g, rs - 8) * 2);
    }
  };
  bool kok[NK];
#pragma unroll
  for (int ks = 0; ks < NK; ++ks) kok[ks] = 32 * ks + 8 * g < rs;
  auto loadY = [&](int c, uint4 (&yv)[YP]) {
#pragma unroll
    for (int j = 0; j < YP; ++j) {
      const int m = min(64 * c + ymo[j], d_out - EPP);
      yv[j] = ld16(yrow[j] + (int64_t)m * (int)sizeof(TY));
    }
  };
  auto process = [&](int c, const uint4 (&bc)[JB][NK], const uint4 (&yc)[YP]) {
    const int vo = vp_index(r16, 8 * g);  // + 4 k groups per k step
    f32x4_t acc[JB];
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) acc[jb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NK; ++ks) {
      const uint4 vh = *reinterpret_cast<const uint4*>(Vh + vo + 32 * kTileM * ks);
      const uint4 vl = *reinterpret_cast<const uint4*>(Vl + vo + 32 * kTileM * ks);
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
        const vec bk = as_vec<vec>(keep16m(bc[jb][ks], kok[ks]));
        acc[jb] = MfmaOp<T>::mma(bk, as_vec<vec>(vh), acc[jb]);
        acc[jb] = MfmaOp<T>::mma(bk, as_vec<vec>(vl), acc[jb]);
      }
    }
    lds_barrier();  // D is free: every wave is done with the previous step's RMW
#pragma unroll
    for (int jb = 0; jb < JB; ++jb)
      *reinterpret_cast<float4*>(D + r16 * DROW + 16 * JB * w + 16 * jb + 4 * g) =
          make_float4(acc[jb][0], acc[jb][1], acc[jb][2], acc[jb][3]);
    lds_barrier();
#pragma unroll
    for (int j = 0; j < YP; ++j) {
      const int m = 64 * c + ymo[j];
      if (yok[j] && m < m_end) {
        float a[EPP];
        const float* dr = D + yslot[j] * DROW + ymo[j];
#pragma unroll
        for (int i = 0; i < EPP; i += 4) {
          const float4 q = *reinterpret_cast<const float4*>(dr + i);
          a[i] = q.x;
          a[i + 1] = q.y;
          a[i + 2] = q.z;
          a[i + 3] = q.w;
        }
        *reinterpret_cast<uint4*>(yrow[j] + (int64_t)m * (int)sizeof(TY)) = YPiece<TY>::fma(yc[j], a, s);
      }
    }
  };
  // Two register sets alternate by unrolling; prefetches past the range
  // repeat its last step (clamped, never skipped).
  const int cl = c0 + JB * ((c1 - c0 - 1) / JB);  // first chunk of the last step
  uint4 b0[JB][NK], b1[JB][NK], y0[YP], y1[YP];
  loadB(c0, b0);
  loadY(c0, y0);
  __builtin_amdgcn_sched_barrier(0);
  load_v();
  lds_barrier();  // V is in LDS
  for (int c = c0; c < c1; c += 2 * JB) {
    loadB(min(c + JB, cl), b1);
    loadY(min(c + JB, cl), y1);
    process(c, b0, y0);
    loadB(min(c + 2 * JB, cl), b0);
    loadY(min(c + 2 * JB, cl), y0);
    if (c + JB < c1) process(c + JB, b1, y1);
  }
}

// Fused: V of a tile from its contributors' partial tiles (summed in block
// order, as the split API's reduce does) -> hi and lo parts in LDS.  Columns
// [16 * ceil(rank / 16), 32 * NK) and slots past the count are zero.  A tile
// has at most 2 NK rank blocks of 4 token blocks, so each thread owns at most
// UPT = 2 NK float4 units of a partial tile; the loads of CG contributors are
// issued together (clamped to the last contributor, whose repeats are not
// added).
template <typename T, int NK>
__device__ __forceinline__ void load_v_parts(const PlanView& pl, int c0, int c1, int count,
                                             int rank, uint16_t* Vh, uint16_t* Vl) {
  constexpr int KW = 32 * NK;
  constexpr int UPT = 2 * NK;
  constexpr int CG = UPT >= 8 ? 1 : 8 / UPT;
  const int ntb = (count + 15) >> 4;
  const int nu = ((rank + 15) >> 4) * ntb * 64;  // <= UPT * kMT
  float4 sum[UPT];
  for (int c = c0; c < c1; c += CG) {
    float4 q[CG][UPT];
#pragma unroll
    for (int g = 0; g < CG; ++g) {
      const float4* src = part_at(pl, pl.c_ent[min(c + g, c1 - 1)]);
#pragma unroll
      for (int i = 0; i < UPT; ++i) q[g][i] = src[min((int)threadIdx.x + kMT * i, nu - 1)];
    }
#pragma unroll
    for (int g = 0; g < CG; ++g) {
      if (c + g >= c1) break;
#pragma unroll
      for (int i = 0; i < UPT; ++i) {
        if (c + g == c0) {
          sum[i] = q[g][i];
        } else {
          sum[i].x += q[g][i].x;
          sum[i].y += q[g][i].y;
          sum[i].z += q[g][i].z;
          sum[i].w += q[g][i].w;
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int u = threadIdx.x + kMT * i;
    if (u < nu) {
      const int sl = unit_slot(u, ntb);
      const int n = unit_rank(u, ntb);
      const float a[4] = {sum[i].x, sum[i].y, sum[i].z, sum[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float f = (sl < count && n + e < rank) ? a[e] : 0.f;
        uint16_t hi, lo;
        MfmaOp<T>::split(f, hi, lo);
        Vh[vp_index(sl, n + e)] = hi;
        Vl[vp_index(sl, n + e)] = lo;
      }
    }
  }
  // zero: columns [16 * ceil(rank / 16), KW) of the computed slots (slots past
  // 16 * ntb are never read: tb < ntb only)
  const int w0 = (rank + 15) & ~15;
  for (int idx = threadIdx.x; idx < 16 * ntb * (KW - w0); idx += kMT) {
    const int sl = idx / (KW - w0);
    const int k = w0 + idx - sl * (KW - w0);
    Vh[vp_index(sl, k)] = 0;
    Vl[vp_index(sl, k)] = 0;
  }
}

// The block's expand range over the launch slices ios[0 .. n_io).  Split
// API: V from the caller's v (rows by token).  Fused (kFused, v unused): V of
// a tile from its partial tiles, written by the shrink launch that precedes
// this one on the stream.
template <typename T, typename TY, bool kFused, typename IoOf>
__device__ __forceinline__ void expand_range(const PoolView& pv, const PlanView& pl, IoOf&& io_of,
                                             int L, const float* v, int v_ld, const LdsBufs& lb) {
  int* toks = reinterpret_cast<int*>(lb.misc + kOffToks);
  uint16_t* Vh = reinterpret_cast<uint16_t*>(lb.a);
  uint16_t* Vl = reinterpret_cast<uint16_t*>(lb.b);
  float* Ds = reinterpret_cast<float*>(lb.c);
  const int ntl = plan_tiles(pl);
  // chunks [c0, c1) of tile i in launch slice j
  auto piece = [&](int j, int i, int c0, int c1) {
    const IoDesc io = io_of(j);
    const PlanItem item = pl.items[i];
    const DevEntry e = pv.entries[io.slice * pv.max_adapters + item.adapter];
    if (e.rank <= 0) return;  // not resident in this slice: y untouched
    load_tile_tokens(pl, item, toks);
    const int32_t* off = contrib_range(pl, ntl, j, i);
    const int cb0 = off[0], cb1 = off[1];
    __syncthreads();
    switch ((e.rs + 31) >> 5) {
      case 1: {
        auto load_v = [&] {
          if constexpr (kFused) load_v_parts<T, 1>(pl, cb0, cb1, item.count, e.rank, Vh, Vl);
          else load_v_tile<T, 1>(v, v_ld, toks, item.count, e.rank, Vh, Vl);
        };
        if (item.count <= 16)
          expand_chunks_wide<T, TY, 1>(pv, e, io, toks, item.count, c0, c1, Vh, Vl, Ds, load_v);
        else
          expand_chunks<T, TY, 1>(pv, e, io, toks, item.count, c0, c1, Vh, Vl, Ds, load_v);
        break;
      }
      case 2: {
        auto load_v = [&] {
          if constexpr (kFused) load_v_parts<T, 2>(pl, cb0, cb1, item.count, e.rank, Vh, Vl);
          else load_v_tile<T, 2>(v, v_ld, toks, item.count, e.rank, Vh, Vl);
        };
        if (item.count <= 16)
          expand_chunks_wide<T, TY, 2>(pv, e, io, toks, item.count, c0, c1, Vh, Vl, Ds, load_v);
        else
          expand_chunks<T, TY, 2>(pv, e, io, toks, item.count, c0, c1, Vh, Vl, Ds, load_v);
        break;
      }
      case 3: {
        auto load_v = [&] {
          if constexpr (kFused) load_v_parts<T, 3>(pl, cb0, cb1, item.count, e.rank, Vh, Vl);
          else load_v_tile<T, 3>(v, v_ld, toks, item.count, e.rank, Vh, Vl);
        };
        if (sizeof(TY) == 2 && item.count <= 16)  // (fp32 y: registers for the narrow steps only)
          expand_chunks_wide<T, TY, 3>(pv, e, io, toks, item.count, c0, c1, Vh, Vl, Ds, load_v);
        else
          expand_chunks<T, TY, 3>(pv, e, io, toks, item.count, c0, c1, Vh, Vl, Ds, load_v);
        break;
      }
      default: {
        auto load_v = [&] {
          if constexpr (kFused) load_v_parts<T, 4>(pl, cb0, cb1, item.count, e.rank, Vh, Vl);
          else load_v_tile<T, 4>(v, v_ld, toks, item.count, e.rank, Vh, Vl);
        };
        if (sizeof(TY) == 2 && item.count <= 16)  // (fp32 y: registers for the narrow steps only)
          expand_chunks_wide<T, TY, 4>(pv, e, io, toks, item.count, c0, c1, Vh, Vl, Ds, load_v);
        else
          expand_chunks<T, TY, 4>(pv, e, io, toks, item.count, c0, c1, Vh, Vl, Ds, load_v);
        break;
      }
    }
    lds_barrier();  // tokens and V are free (the y stores stay in flight)
  };
  // One loop and one call of `piece` (a second inlined copy of its body costs
  // registers and spills): first the block's static range, then, in fused
  // launches with a pool, claims of `batch` pool chunks until a claim starts
  // past the pool's end (every block gets there; nothing waits).
  const RangePos b = load_pos(pl.bs_expand, L + 1);
  RangePos a = load_pos(pl.bs_expand, L);
  bool pooled = false;
  int g = 0, g1 = 0;  // pool chunks still to do in the current claim
  __shared__ int claim;
  for (;;) {
    int j, i, c0, c1;
    if (!pooled && pos_before(a.j, a.tile, a.k, b)) {
      j = a.j;
      i = a.tile;
      c0 = a.k;
      c1 = (a.j == b.j && a.tile == b.tile) ? b.k : (io_of(a.j).d_out + 63) / 64;
      a.k = 0;
      if (++a.tile == ntl) {
        a.tile = 0;
        ++a.j;
      }
    } else {
      if (!kFused || !pl.pool) break;
      pooled = true;
      const RangePos p0 = load_pos(pl.bs_expand, pl.G);  // the pool's first tile
      const int nch = (io_of(p0.j).d_out + 63) / 64;
      if (g >= g1) {
        const int pool_units = pl.pool[0], batch = pl.pool[1];
        if (threadIdx.x == 0)
          claim = atomicAdd(reinterpret_cast<int*>(pl.part) + 4 * (int64_t)pl.pool[2], batch);
        __syncthreads();
        g = claim;
        __syncthreads();
        if (g >= pool_units) break;
        g1 = min(g + batch, pool_units);
      }
      const int t = g / nch;
      j = p0.j;
      i = p0.tile + t;
      c0 = g - t * nch;
      c1 = min(nch, c0 + (g1 - g));
      g += c1 - c0;
    }
    piece(j, i, c0, c1);
  }
}

}  // namespace lora
