// Internal declarations shared by the host runtime (pool, plan, entry points)
// and the HIP kernels.  Nothing here is part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/lora_mi355x.h"

namespace lora {

// One (slice, adapter) row of the device adapter table: 32 bytes, read with a
// single scalar load by every kernel.
struct DevEntry {
  int32_t rank;    // 0: adapter not resident in this slice
  int32_t rs;      // stored B row length (rank rounded up to 16 bytes)
  float scale;     // stored per-adapter scale
  int32_t rpp;     // B rows per page = floor(P / rs)
  int32_t a_off;   // index of the adapter's first A page id in the page-id list
  int32_t b_off;   // index of its first B page id
  float inv_rpp;   // 1.0f / rpp (quotient estimate, corrected exactly)
  int32_t q_off;   // quantised pools: index of the adapter's scales in the
                   // page-id list (rank a_scale words, then rank b_scale words)
};
static_assert(sizeof(DevEntry) == 32, "DevEntry must stay 32 bytes");

// Pool view handed to kernels.
struct PoolView {
  const char* pages;          // pool base
  const DevEntry* entries;    // [n_slices][max_adapters]
  const int32_t* page_ids;    // concatenated page lists
  int32_t P;                  // elements per page
  int32_t max_adapters;
  int32_t max_nch;            // 16-byte chunks in the longest stored B row of the pool
  int32_t n_cu;               // compute units of the pool's device
  int32_t mixed_ranks;        // 1: the resident adapters of this table differ in rank
};

// Per-slice input/output of one launch.
struct IoDesc {
  const void* x;
  void* y;
  int32_t slice;
  int32_t d_in;
  int32_t d_out;
  int32_t npa;                // pages per A row = ceil(d_in / P)
};

struct IoSet {
  IoDesc io[LORA_MAX_IO];
  int32_t n_io;
  int32_t max_d_out;
  int32_t max_d_in;
  // Slices that share one x (lora_io.x_group): 0 = none; otherwise io is
  // ordered by group and group g holds io[grp_start[g] .. grp_start[g + 1]).
  int32_t n_groups;
  int32_t grp_start[LORA_MAX_IO + 1];
};

// One unit of planned SGMV work: `count` tokens (perm[start .. start+count))
// that all use `adapter` (-1: tokens with no adapter, only v rows are zeroed).
struct PlanItem {
  int32_t adapter;
  int32_t start;
  int32_t count;
  int32_t kind;   // 0: VALU short item (count <= 4), 1: MFMA tile (count <= 64)
};

constexpr int kShortG = 4;   // tokens per short item
constexpr int kTileM = 64;   // tokens per MFMA tile
constexpr int kMaxNpa = 8;            // MFMA tiles: pages per A row, at most

// Cost weights of one MFMA tile of `count` tokens whose adapter has rank
// `rmax` (largest over the slices; stored B rows of `rs` elements), for the
// persistent kernels' block ranges, and the size of one of its partial tiles.
// Used by the host planner and by the device planner alike.
struct TileCost {
  int32_t ws;  // one shrink stage (64 columns of d_in), units of ~8 ns
  int32_t we;  // one expand chunk (64 rows of d_out), units of ~4 ns
  int32_t tu;  // float4 units of a partial tile
};
// Set-up of one tile piece of a block range, in the weight units of TileCost
// (measured: ~5 us for a shrink piece -- tokens, A page ids, pipeline fill --
// and ~6 us for an expand piece -- tokens, V from the partial tiles, fill).
constexpr int64_t kPieceSetupShrink = 600;
constexpr int64_t kPieceSetupExpand = 1800;
__host__ __device__ inline TileCost tile_cost(int count, int rmax, int rs) {
  const int rp = (rmax + 15) / 16 * 16;
  const int tb = (count + 15) / 16;  // 16-token blocks
  // a stage costs about one memory round trip whatever it moves: a large
  // fixed part plus half the 128-byte rows it loads
  const int ws = 64 + (16 * tb + rp) / 2;
  // an expand chunk, from per-chunk times measured on MI355X: tiles of more
  // than 16 tokens take 64-row steps, ~141 + 60 NK + 2 count; tiles of at
  // most 16 tokens take wide steps (4 or 2 chunks, B of several chunks per
  // round trip), ~51 + 51 NK + count per chunk (NK = 32-column k steps of the
  // stored B row)
  const int nk = (rs + 31) / 32;
  const int we = count <= 16 ? 51 + 51 * nk + count : 141 + 60 * nk + 2 * count;
  return TileCost{ws, we, (rp / 16) * tb * 64};
}

// Element types of one call: pages (w), activations x (x) and y (y), as
// lora_dtype codes.  x equals w except on FP8 pools (16-bit x).
struct Types {
  int w, x, y;
};

// ---- kernel launchers (defined in the .hip files) -------------------------
hipError_t launch_fill_pages(char* pages, int64_t page_bytes, const int32_t* ids_dev,
                             int64_t n, uint32_t pattern, int elt, hipStream_t s);
hipError_t launch_fill_all(char* pages, int64_t bytes, uint32_t pattern, int elt,
                           hipStream_t s);
hipError_t launch_scatter_pages(char* pages, int64_t page_bytes, const char* staging,
                                const int32_t* ids_dev, int64_t n, hipStream_t s);

hipError_t launch_bgmv_shrink(const Types& ty, const PoolView& pv, const IoDesc& io,
                              const int32_t* ids, int32_t n, float* v, int32_t v_ld,
                              hipStream_t s);
hipError_t launch_bgmv_expand(const Types& ty, const PoolView& pv, const IoDesc& io,
                              const float* v, int32_t v_ld, const int32_t* ids, int32_t n,
                              const float* tok_scale, hipStream_t s);
hipError_t launch_bgmv_apply(const Types& ty, const PoolView& pv, const IoSet& ios,
                             const int32_t* ids, int32_t n, hipStream_t s);
// Profiling builds (LORA_BLOCK_TIMELINE): per-block records of the last fused
// decode launch, kTimelineWords 64-bit words per block for the first
// kTimelineBlocks blocks; hipErrorNotSupported in other builds.
constexpr int kTimelineBlocks = 65536;
constexpr int kTimelineWords = 8;
hipError_t read_block_timeline(void* host, size_t bytes);

// Position in a launch's sequence of MFMA work for the persistent kernels:
// the tiles of launch slice 0, then those of slice 1, ...; unit k of a tile is
// a shrink stage (64 columns of d_in) or an expand chunk (64 rows of d_out).
// A position is normalized (k < units of the tile, tile < n_mfma, j < n_io) or
// is the end {n_io, 0, 0}; block L's range is [pos[L], pos[L + 1]).
struct RangePos {
  int32_t j;
  int32_t tile;
  int32_t k;
  int32_t pad;
};

// Items [0, n_mfma) are MFMA tiles, [n_mfma, n_items) short items.  The range
// tables and the split-K contributions belong to one launch shape (the stage
// and chunk counts of the launch's slices); a plan keeps a few such layouts.
struct PlanView {
  const PlanItem* items;
  const int32_t* perm;
  const RangePos* bs_shrink;   // [G + 1]
  const RangePos* bs_expand;   // [G + 1]
  // Split-K shrink: float4 offsets (into part) of block L's partial tiles for
  // the first and the last piece of its range.  A piece between them covers a
  // whole tile, whose only contribution is c_ent[c_off[j][tile]].
  const int2* part_fl;         // [G]
  // contributions to tile i of launch slice j, in block order: the partial
  // tiles at float4 offsets c_ent[c_off[j][i] .. c_off[j][i + 1])
  const int32_t* c_off;        // [n_io][n_mfma + 1]
  const int32_t* c_ent;
  float* part;                 // partial tiles
  // Plans built on the device: the tile count as the planner wrote it (the
  // host knows only a bound, in n_mfma); null for host-built plans.
  const int32_t* n_tiles_dev;
  // Expand pool of a fused launch (null: none): {units, batch, float4 offset
  // of the claim counter in part, 0}; the chunks from bs_expand[G] to the end
  // of the sequence are claimed by blocks that finished their range.
  const int32_t* pool;
  int32_t n_items;
  int32_t n_tokens;
  int32_t n_mfma;
  int32_t G;                   // persistent grid (blocks)
};

hipError_t launch_sgmv_shrink(const Types& ty, const PoolView& pv, const PlanView& pl,
                              const IoDesc& io, float* v, int32_t v_ld, hipStream_t s);
hipError_t launch_sgmv_expand(const Types& ty, const PoolView& pv, const PlanView& pl,
                              const IoDesc& io, const float* v, int32_t v_ld, hipStream_t s);
hipError_t launch_apply(const Types& ty, const PoolView& pv, const PlanView& pl,
                        const IoSet& ios, hipStream_t s);
// Decode n stored elements of `dtype` to fp32 with the kernels' decoder
// (n * element bytes a multiple of 16).
hipError_t launch_debug_decode(int dtype, const void* src, int64_t n, float* dst, hipStream_t s);

hipError_t launch_debug_resolve(const PoolView& pv, const IoDesc& io, int32_t max_rank,
                                int elt, const int32_t* ids, int32_t n, int64_t* a_off,
                                int64_t* b_off, hipStream_t s);
hipError_t launch_debug_gather(int elt, const PoolView& pv, const IoDesc& io, int32_t adapter,
                               int32_t rank, void* A, void* B, hipStream_t s);

}  // namespace lora
