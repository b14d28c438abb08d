// moe_tiles.hpp -- tile spaces of the slot-blocked MoE GEMMs (Phases 1 and 3).
//
// Block b's slots past its extent (one past its last routed slot) are padding,
// so the block contributes ceil(extent / W) slot tiles of W slots, each times
// `other` tiles along the GEMM's other dimension.  start[b] (b = 0..N-1) is the
// index of block b's first tile and start[N] the total, built on the device
// before the GEMM (launch_tile_ranges), followed by each tile's block
// (start[N + 1 + t]).  The GEMM's grid covers every tile a
// full block could have; workgroups past the total exit at once.  Being the
// highest ids, those are spread over all XCDs, and the live ids are handed to
// the XCDs evenly (in contiguous ranges or round robin, see block_tile):
// skipped tiles never leave one XCD idle while another still holds its full
// share.
#pragma once
#include "gemm_v2.hpp"

namespace mx {

struct BlockTiles {
  int b;       // block
  int local;   // tile index inside the block's range
  int slots;   // slot tiles of the block
};

// Maps a workgroup id to its tile; false: no tile (exit).  Two orders:
//   rr = 0: each XCD takes a contiguous range of tiles, so consecutive blocks
//     of one expert meet in one XCD's L2 -- the better order while an
//     expert's weights are small next to the 4 MB L2;
//   rr = 1: ids as the hardware hands them out, round robin over the XCDs,
//     so all XCDs work on the same blocks at once and stream one expert's
//     weights together through the infinity cache -- the better order for
//     weights many times the L2, which no single XCD can keep.  With a
//     block's tile count a multiple of 8, each XCD still holds a compact
//     group of tiles.  The blocks whose slot tiles are all live come first
//     (launch_tile_ranges), so that a round's tiles are whole blocks of one
//     expert, not the tail of one block and the head of the next.
// ext: the blocks' extents; W: slots per slot tile.
__device__ __forceinline__ bool block_tile(const int32_t* __restrict__ start, const int32_t* __restrict__ ext, int W,
                                           int N, int wg, int rr, BlockTiles& t) {
  const int total = start[N];
  const int t8 = (total + 7) & ~7;   // the XCD remap needs a multiple of 8 ids
  if (wg >= t8) return false;
  const int id = rr ? wg : v2::xcd_remap(wg, t8);
  if (id >= total) return false;
  const int b = start[N + 1 + id];   // the tile -> block map after the starts
  t.b = b;
  t.local = id - start[b];
  t.slots = (ext[b] + W - 1) / W;
  return true;
}

// The last round of a GEMM's tiles cut along K (Phase 3, moe_phase3.hip).
// The tiles take equal times and run in rounds of `conc` workgroups (those
// resident at once), conc / 8 per XCD; XCD x runs the workgroup ids equal to
// x mod 8 in order and holds nx of the live tiles, and its last
// nx mod (conc / 8) tiles would run while most of its CUs idle.  Each of
// those is cut into S parts of whole stage pairs, S <= kCutMaxParts, at least
// kCutMinPairs pairs a part, S * tail <= conc / 8; the parts after the first
// are numbered XCD by XCD (base), tile by tile, part by part.  A part pays a
// tile's fixed costs (the ring's fill, its store) and the parts are added up
// afterwards, so the cut pays only on long contractions: measured on Phase 3,
// 6% faster with 448 stages a tile (2I = 28672), slower with 44 (2I = 2816).
constexpr int kCutMaxParts = 4;
constexpr int kCutMinPairs = 16;
struct TailCut {
  int nx;     // live tiles of the XCD
  int tail;   // its last `tail` tiles are cut (0: none)
  int S;      // parts of a cut tile
  int base;   // number of the XCD's first later part
};
__host__ __device__ inline TailCut tail_cut_one(int total, int x, int rr, int conc, int npairs) {
  int nx;
  if (rr) {   // ids as dispatched
    nx = total > x ? (total - x + 7) / 8 : 0;
  } else {    // block_tile's contiguous ranges of t8 / 8 ids
    const int per = ((total + 7) & ~7) / 8;
    nx = total - x * per < per ? total - x * per : per;
    nx = nx > 0 ? nx : 0;
  }
  TailCut c{nx, 0, 1, 0};
  const int cx = conc / 8;
  const int r = cx > 0 ? nx % cx : 0;
  if (r == 0) return c;
  int S = cx / r;
  S = S < kCutMaxParts ? S : kCutMaxParts;
  S = S < npairs / kCutMinPairs ? S : npairs / kCutMinPairs;
  if (S > 1) {
    c.tail = r;
    c.S = S;
  }
  return c;
}

}  // namespace mx
