// moe_tiles.hpp -- tile spaces of the slot-blocked MoE GEMMs (Phases 1 and 3).
//
// Block b's slots past its extent (one past its last routed slot) are padding,
// so the block contributes ceil(extent / W) slot tiles of W slots, each times
// `other` tiles along the GEMM's other dimension.  start[b] (b = 0..N) is the
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
//     group of tiles.
__device__ __forceinline__ bool block_tile(const int32_t* __restrict__ start, int N, int other, int wg, int rr,
                                           BlockTiles& t) {
  const int total = start[N];
  const int t8 = (total + 7) & ~7;   // the XCD remap needs a multiple of 8 ids
  if (wg >= t8) return false;
  const int id = rr ? wg : v2::xcd_remap(wg, t8);
  if (id >= total) return false;
  const int b = start[N + 1 + id];   // the tile -> block map after the starts
  t.b = b;
  t.local = id - start[b];
  t.slots = (start[b + 1] - start[b]) / other;
  return true;
}

}  // namespace mx
