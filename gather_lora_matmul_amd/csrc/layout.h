// Block ranges and split-K contributions of the persistent MFMA kernels for
// one launch shape (host side, plain C++; no HIP dependency).
//
// A launch's work sequence is the MFMA tiles of launch slice 0, then those of
// slice 1, ...; tile t of slice j has n[j] units (shrink stages or expand
// chunks) of weight w[t] each.  The sequence is split into G contiguous ranges
// of equal weight, one per block of the persistent grid.
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

namespace lora {

// A position {j, tile, k} in the sequence, as 4 int32 (the device RangePos).
// Positions are normalized: k < n[j], tile < T, j < J, or the end {J, 0, 0}.
constexpr int kPosInts = 4;

// Block L's range is [pos[L], pos[L + 1]); out: (G + 1) positions.  ov == 0:
// pos[L] is the first unit whose cumulative start weight is at least
// total * L / G.  ov > 0: a block also pays ov for every tile piece it touches
// (its per-tile set-up); ranges are cut greedily under the smallest per-block
// cap that G blocks cover, so blocks that touch more tiles get fewer units
// (sequences of more than kMaxPiecesOv tiles fall back to ov == 0).
constexpr int64_t kMaxPiecesOv = 16384;
// seq_end >= 0: only the tiles before sequence index seq_end (j T + t) are
// cut, and the ranges end at the position {seq_end / T, seq_end % T, 0}.
void balance_ranges(const std::vector<int32_t>& w, const std::vector<int32_t>& n, int G, int64_t ov,
                    int32_t* out, int seq_end = -1);
// Block L's range starts at the first unit whose start is at or past
// total * L / G, where every tile adds its set-up ov before its unit 0 (unit 0
// of a tile spans the set-up and its own weight; total counts all units and
// set-ups).  Every boundary is independent of the others (the device planner
// cuts its ranges this way); with ov == 0 it is balance_ranges' plain split.
void spread_ranges(const std::vector<int32_t>& w, const std::vector<int32_t>& n, int G, int64_t ov,
                   int32_t* out);

// The int32 image of a launch shape's layout, copied to the device as is:
//   [o_bs]  shrink ranges, (G + 1) positions (stage units, weights ws)
//   [o_be]  expand ranges, (G + 1) positions (chunk units, weights we)
//   [o_fl]  per block: float4 offsets of the partial tiles of the first and
//           the last piece of its shrink range (a piece between them covers a
//           whole tile, the tile's only contribution)
//   [o_pool] the expand pool: {units, batch, float4 offset of its claim
//           counter, 0} (units 0: no pool).  With a pool the expand ranges end
//           at the pool's start, a tile boundary of the last launch slice; the
//           pool's chunks (every chunk from there to the end of the sequence)
//           are claimed by blocks that finished their range, `batch` chunks a
//           claim, through a counter the shrink launch clears
//   [o_off] per (j, tile): first contribution index, J * (T + 1) entries
//   [o_ent] contributions in (j, tile, block) order: float4 offset of each
//           partial tile (tile t's partials hold tu[t] float4 units)
struct LayoutHost {
  std::vector<int32_t> buf;
  size_t o_bs = 0, o_be = 0, o_fl = 0, o_pool = 0, o_off = 0, o_ent = 0;
  int64_t part_units = 0;  // float4 units of all partial tiles (and the pool counter)
  bool pool = false;
};

// ov_s, ov_e: per-piece set-up cost of the shrink and expand ranges (in the
// units of ws, we).  False if the partial tiles would exceed 2^31 float4 units.
// spread: cut the ranges with spread_ranges instead of balance_ranges.
// pool_frac > 0 (two or more launch slices, not spread): leave about that
// fraction of the expand weight, whole tiles at the end of the last slice, to
// the pool.
bool layout_host(const std::vector<int32_t>& ws, const std::vector<int32_t>& we,
                 const std::vector<int32_t>& tu, const std::vector<int32_t>& nst,
                 const std::vector<int32_t>& nch, int G, int64_t ov_s, int64_t ov_e,
                 LayoutHost& h, bool spread = false, double pool_frac = 0.0);

}  // namespace lora
