// moe_phase1_epi.hip -- the stand-alone Phase-1 epilogue kernel: the SwiGLU (or
// GeGLU) backward on the product dS that Phase 1 left in HBM (the arithmetic is
// in moe_phase1_epi.hpp).  Taken where the fused Phase-1 kernel is not: caller
// checkpoints, H not a multiple of 128.
#include "moe_phase1_epi.hpp"

namespace mx {

// One workgroup per chunk of TI rows i x TS slots.  Chunk order: the 128 / TI
// row chunks that share a slot's 128-byte run of dgu_row codes and its scale
// words are consecutive, and consecutive chunks run on one XCD, so those lines
// fill up in one L2 instead of reaching HBM in pieces from several.
template <int FG, bool ON_I, int TS, bool CK, bool GEGLU>
__global__ void __launch_bounds__(kEpiThreads) phase1_epi_kernel(Phase1Args p) {
  constexpr int TI = kEpiElems / TS;
  __shared__ __attribute__((aligned(16))) uint8_t lds[EpiLds<TS>::BYTES];
  constexpr int GI = 128 / TI;
  const int tiles_i = int((p.I + TI - 1) / TI), tiles_s = int(p.B / TS);
  const int per_b = tiles_i * tiles_s;
  const int id = v2::xcd_remap(blockIdx.x, gridDim.x);
  const int b = id / per_b;
  int tile_i, tile_s;
  v2::grouped_tile<GI>(id - b * per_b, tiles_i, tiles_s, tile_i, tile_s);
  const int64_t ti0 = int64_t(tile_i) * TI, s0 = int64_t(tile_s) * TS;
  if (!p.flag[b]) {
    epi_empty_chunk<TS>(p, b, ti0, s0);
    return;
  }
  epi_chunk<FG, ON_I ? 1 : 0, TS, CK, GEGLU, false>(p, b, ti0, 32, s0, lds);
}

template <int TS, bool CK, bool GEGLU>
static hipError_t epi_launch(const Phase1Args& p, int fg, hipStream_t st) {
  constexpr int TI = kEpiElems / TS;
  const int64_t grid = int64_t(p.N) * ((p.I + TI - 1) / TI) * (p.B / TS);
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  const bool on_i = p.affinity_on_i != 0;
  if (fg == kE4M3) {
    if (on_i) phase1_epi_kernel<kE4M3, true, TS, CK, GEGLU><<<unsigned(grid), kEpiThreads, 0, st>>>(p);
    else phase1_epi_kernel<kE4M3, false, TS, CK, GEGLU><<<unsigned(grid), kEpiThreads, 0, st>>>(p);
  } else {
    if (on_i) phase1_epi_kernel<kE5M2, true, TS, CK, GEGLU><<<unsigned(grid), kEpiThreads, 0, st>>>(p);
    else phase1_epi_kernel<kE5M2, false, TS, CK, GEGLU><<<unsigned(grid), kEpiThreads, 0, st>>>(p);
  }
  return hipGetLastError();
}
template <int TS, bool GEGLU>
static hipError_t epi_launch(const Phase1Args& p, int fg, hipStream_t st) {
  if (p.ga_ckpt || p.in_ckpt || p.sc_ckpt) return epi_launch<TS, true, GEGLU>(p, fg, st);
  return epi_launch<TS, false, GEGLU>(p, fg, st);
}
template <int TS>
static hipError_t epi_launch(const Phase1Args& p, int fg, hipStream_t st) {
  if (p.geglu) return epi_launch<TS, true>(p, fg, st);
  return epi_launch<TS, false>(p, fg, st);
}

// Block size B: a power of two >= 128 (chunks of 256 slots, or of the whole block at 128).
hipError_t launch_phase1_epi(const Phase1Args& p, int fg, hipStream_t st) {
  if (p.B % 256 == 0) return epi_launch<256>(p, fg, st);
  if (p.B == 128) return epi_launch<128>(p, fg, st);
  return hipErrorInvalidValue;
}

}  // namespace mx
