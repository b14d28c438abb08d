// moe_phase1_128.hip -- Phase 1 at 128 x 128 tiles (I = 128, or H not a multiple of 128 on the
// bf16-value loop) and the tile-shape dispatch.
#include "moe_phase1.hpp"

namespace mx {

template hipError_t phase1_launch<128, 128, false>(Phase1Args, int, int, hipStream_t);
template hipError_t phase1_launch<128, 128, true>(Phase1Args, int, int, hipStream_t);
template hipError_t phase1_fused_launch<128, 128>(Phase1Args, int, int, hipStream_t);
extern template hipError_t phase1_launch<256, 256, false>(Phase1Args, int, int, hipStream_t);
extern template hipError_t phase1_launch<256, 128, false>(Phase1Args, int, int, hipStream_t);


// Tile shape: 256 along a dimension when it is at least 256, else 128.  The
// block size B is a power of two >= 128, so every tile lies inside one block.
// A contraction H of 2048 or less takes 128 x 128 tiles, two workgroups per
// CU, so one's fp8 -> bf16 conversions and loads overlap the other's MFMAs
// (measured 4% faster at H = 2048 and 1536; 12% slower at H = 4096, where
// 256 x 256 tiles' longer loop amortises its start and end).
// H not a multiple of 128 (a ragged last K stage, scale rows not in whole
// pairs): the v2 loop on bf16 values, 128 x 128.
hipError_t launch_phase1(const Phase1Args& p, int fg, int fw, hipStream_t st) {
  if (p.H % 128 != 0) return phase1_launch<128, 128, true>(p, fg, fw, st);
  if (p.H <= 2048) return phase1_launch<128, 128, false>(p, fg, fw, st);
  if (p.I >= 256 && p.B >= 256) return phase1_launch<256, 256, false>(p, fg, fw, st);
  if (p.I >= 256) return phase1_launch<256, 128, false>(p, fg, fw, st);
  return phase1_launch<128, 128, false>(p, fg, fw, st);
}

// Where Phase 1 runs with its epilogue in the same kernel (phase1_fused_kernel):
// H % 128 == 0 (the ring loop), no caller checkpoints, H <= 2048 (128 x 128
// tiles, two workgroups per CU) and I <= 512.  Measured against the two
// kernels (Phase 1 + epilogue): 6% faster with I = 256 (H = 1536, B = 128),
// even with I = 1408 (H = 2048), and 7% / 17% slower on H = 4096, I = 14336 at
// 128 x 128 / 256 x 256 tiles: the epilogue's loads and stores do not overlap
// the other workgroup's MFMAs, and the product itself needs both workgroups
// to hide its latency, so the element-wise work adds to the product's time.
bool phase1_fusable(const Phase1Args& p) {
  return p.H % 128 == 0 && p.H <= 2048 && p.I <= 512 && !p.ga_ckpt && !p.in_ckpt && !p.sc_ckpt;
}

hipError_t launch_phase1_fused(const Phase1Args& p, int fg, int fw, hipStream_t st) {
  if (!phase1_fusable(p)) return hipErrorInvalidValue;
  return phase1_fused_launch<128, 128>(p, fg, fw, st);
}

}  // namespace mx
