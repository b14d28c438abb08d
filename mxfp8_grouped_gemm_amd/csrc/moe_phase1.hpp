// moe_phase1.hpp -- Phase 1 of the MoE backward, its product (P1, "Blockwise
// MM Backward MXFP8 Kernel API Reference": Phase 1; P3, sonic-moe
// functional/backward.py: _down_projection_backward_act, the product with the
// down projection).  The kernel template and its launcher; the tile shapes are
// instantiated in moe_phase1_*.hip so they compile in parallel.  The SwiGLU
// backward that consumes the product is in moe_phase1_epi.hip.
//
// Per block b of expert e (tile rows = intermediate index i, tile columns =
// block slot p, contraction over H; the operands' exact MX values reduced with
// bf16 MFMAs, whose fp32 accumulation is exact enough that requantising the
// epilogue's results makes the same rounding decisions as an exact sum would):
//   dS[b][i][p] = sum_h deq(W_down[e])[i][h] * deq(dY[tok_p])[h]   (fp32; dY rows
//                 are quantised along H once and gathered here by token id)
// Only tiles holding a slot before the block's extent (one past its last routed
// slot) run (moe_tiles.hpp); dS stays unwritten past it, and the epilogue
// treats padding slots as zeros.
#pragma once
#include "gemm_v2.hpp"
#include "gemm_v3.hpp"
#include "gemm_v4.hpp"
#include "kernels.hpp"
#include "moe_phase1_epi.hpp"
#include "moe_tiles.hpp"
#include "mx_device.hpp"

namespace mx {

using v2::v16f;
using v2::KMapPlain;

// The product of one tile on the ring loop (H % 128 == 0): A = W_down[e] code
// rows m0 .., B = Q_H(dY) code rows gathered by token (tok_of(r) < 0: zeros).
// The pair-slot ring (v4) for 256 x 256 tiles, measured 3% faster there than
// the four-slot ring (v3), which the smaller tiles keep.
template <int BM, int BN>
constexpr int phase1_ring_smem() {
  return BM == 256 && BN == 256 ? v4::smem_bytes(BM, BN) : v3::smem_bytes(BM, BN);
}
template <int BM, int BN, int FG, int FW, class TokOf>
__device__ __forceinline__ void phase1_ring_product(const Phase1Args& p, int64_t e, int64_t m0, const TokOf& tok_of,
                                                    uint8_t* smem, v2::v16f (&acc)[BM / 64][BN / 64]) {
  v3::ScaleDma<BM, BN> sd;
  const int64_t I_ = p.I;
  v3::setup_scales_map(
      sd, p.wd_scales + e * p.I * (p.H / 32), p.I, p.I * (p.H / 32),
      [&](int r) -> int64_t { return m0 + r < I_ ? m0 + r : -1; }, p.dy_scales, p.T, p.T * (p.H / 32), tok_of);
  if constexpr (BM == 256 && BN == 256) {
    v4::Op<BM> A;
    v4::Op<BN> B;
    v4::setup_rows(A, p.wd_codes + e * p.I * p.H, m0, p.I, p.H);
    v4::setup_gather(B, p.dy_codes, p.T, p.H, tok_of);
    v4::mainloop<BM, BN, v3::kFp8Bf16, FW, FG>(A, B, &sd, int(p.H / v4::PK), v4::KMapPlain{}, smem, acc);
  } else {
    v3::Op<BM> A;
    v3::Op<BN> B;
    v3::setup_rows(A, p.wd_codes + e * p.I * p.H, m0, p.I, p.H);
    v3::setup_gather(B, p.dy_codes, p.T, p.H, tok_of);
    v3::mainloop<BM, BN, v3::kFp8Bf16, FW, FG>(A, B, &sd, int(p.H / v3::SK), v3::KMapPlain{}, smem, acc);
  }
}

// ---------------------------------------------------------------------------
// One 256-thread workgroup per tile; the tile's fp32 result goes straight to
// dS: lane (r, h) of a fragment holds slot column r and 16 of its 32 rows, so
// each store instruction writes two 128-byte row segments (with the
// nontemporal hint: whole lines, read back once by the epilogue).
template <int BM, int BN, int FG, int FW, bool GENERIC>
__global__ void __launch_bounds__(v2::kThreads) phase1_kernel(Phase1Args p) {
  // GENERIC: H not a multiple of 128 (v2 loop on the bf16 values); otherwise a
  // ring on the codes (fp8 in memory and LDS, exact bf16 on the MFMA)
  constexpr int SMEM = GENERIC ? 2 * (BM + BN) * v2::BK : phase1_ring_smem<BM, BN>();
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  constexpr int FM = BM / 64, FN = BN / 64;
  // live tiles only: block b's slot tiles up to its extent, times the I tiles
  BlockTiles bt;
  if (!block_tile(p.tile_start, p.flag, BN, int(p.N), blockIdx.x, p.rr_tiles, bt)) return;
  const int b = bt.b;
  int tm, tn;
  v2::grouped_tile<8>(bt.local, p.tiles_m, bt.slots, tm, tn);
  const int64_t m0 = int64_t(tm) * BM, n0 = int64_t(tn) * BN;   // m: i, n: slot within block
  const int64_t sbase = int64_t(b) * p.B;
  const int64_t e = p.b2e[b];
  const int wave = threadIdx.x >> 6;

  const int32_t* st = p.slot_tok + sbase;
  const int64_t B_ = p.B;
  auto tok_of = [&](int r) -> int64_t { const int64_t s = n0 + r; return s < B_ ? int64_t(st[s]) : -1; };
  v16f acc[FM][FN];
  if constexpr (GENERIC) {
    // A: dequantised W_down[e] rows i; B: dequantised dY rows gathered by token
    const uint8_t* wd = reinterpret_cast<const uint8_t*>(p.wd_deq + e * p.I * p.H);
    const uint8_t* dyd = reinterpret_cast<const uint8_t*>(p.dy_deq);
    v2::Operand<BM, FM> A;
    v2::Operand<BN, FN> B;
    v2::setup_rows(A, wd, nullptr, m0, p.I, 2 * p.H, 0, (wave >> 1) * (BM / 2));
    v2::setup_gather(B, dyd, nullptr, p.T, 2 * p.H, 0, (wave & 1) * (BN / 2), tok_of);
    v2::mainloop<BM, BN, v2::kBf16, 0, 0, true>(A, B, int((2 * p.H + v2::BK - 1) / v2::BK), KMapPlain{2 * p.H},
                                                 smem, acc);
  } else {
    phase1_ring_product<BM, BN, FG, FW>(p, e, m0, tok_of, smem, acc);
  }
  // dS[b][i][slot]; I % 32 == 0, so a fragment row lies inside [0, I) or outside it
  float* ds = p.ds + int64_t(b) * p.I * p.B;
  v2::static_for<FM>([&](auto FI) {
    const int64_t i0 = m0 + (wave >> 1) * (BM / 2) + 32 * int(FI);   // the fragment row's first row
    if (i0 < p.I) {
      v2::static_for<16>([&](auto Q) {
        float* row = ds + (m0 + v2::acc_row<BM, BN>(FI, Q)) * p.B + n0;
        v2::static_for<FN>([&](auto FJ) { store_nt(row + v2::acc_col<BM, BN>(FJ), acc[FI][FJ][int(Q)]); });
      });
    }
  });
}

// ---------------------------------------------------------------------------
template <int BM, int BN, bool G, int FG, int FW>
inline void phase1_go(const Phase1Args& p, unsigned blocks, hipStream_t st) {
  phase1_kernel<BM, BN, FG, FW, G><<<blocks, v2::kThreads, 0, st>>>(p);
}

template <int BM, int BN, bool G>
hipError_t phase1_launch(Phase1Args p, int fg, int fw, hipStream_t st) {
  p.tiles_m = int((p.I + BM - 1) / BM);
  p.tiles_n = int((p.B + BN - 1) / BN);
  const int64_t blocks = (int64_t(p.tiles_m) * p.tiles_n * p.N + 7) & ~int64_t(7);   // every tile, rounded to 8
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  const unsigned grid = unsigned(blocks);
  hipError_t e = launch_tile_ranges(p.flag, p.N, BN, p.tiles_m, p.tile_start, st, nullptr, 0, 0, p.rr_tiles,
                                    int(p.B));
  if (e != hipSuccess) return e;
  if (G) {   // the bf16 values carry no format
    phase1_go<BM, BN, G, kE4M3, kE4M3>(p, grid, st);
  } else if (fg == kE4M3) {
    if (fw == kE4M3) phase1_go<BM, BN, G, kE4M3, kE4M3>(p, grid, st);
    else phase1_go<BM, BN, G, kE4M3, kE5M2>(p, grid, st);
  } else {
    if (fw == kE4M3) phase1_go<BM, BN, G, kE5M2, kE4M3>(p, grid, st);
    else phase1_go<BM, BN, G, kE5M2, kE5M2>(p, grid, st);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Phase 1 with its epilogue fused (H % 128 == 0, no caller checkpoints): the
// tile's product stays on chip.  After the ring, the tile is cut into the
// epilogue's chunks of TI = 8192 / BN rows x BN slots, each made of fragment
// rows of the accumulators: with TI = 64 (BN = 128) chunk c is fragment row c
// of both wave rows (tile rows 32c and BM/2 + 32c, + 32), with TI = 32 chunk k
// is fragment row k / 2 of wave row k % 2.  So the fragments of the early
// chunks are dead once stored, which leaves registers to the epilogue's loads.
// For each chunk the waves holding it store their fragments into LDS (the
// ring's bytes, free once the loop is done), and the whole workgroup runs the
// epilogue on it (epi_chunk), which gives the same bits as the stand-alone
// kernel reading dS from HBM.  The grid covers every tile of every block:
// tiles past a block's extent skip the product (all padding, dS = 0) but still
// write the padding's codes and scales; blocks without tokens write their zero
// intermediate operand.  Tile order as in phase1_kernel, over all tiles.
template <int BM, int BN, int FG, int FW, bool GEGLU>
__global__ void __launch_bounds__(v2::kThreads) phase1_fused_kernel(Phase1Args p) {
  constexpr int SMEM = phase1_ring_smem<BM, BN>();
  static_assert(SMEM >= EpiLds<BN>::BYTES, "the epilogue's chunk fits the ring's LDS");
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  constexpr int FM = BM / 64, FN = BN / 64;
  constexpr int TI = kEpiElems / BN, NCH = BM / TI;
  static_assert(TI == 32 || TI == 64, "chunks of one or two fragment rows");
  constexpr int DSW = EpiLds<BN>::DSW;
  const int per_b = p.tiles_m * p.tiles_n;
  const int total = int(p.N) * per_b;
  const int t8 = (total + 7) & ~7;   // the grid
  const int id = p.rr_tiles ? int(blockIdx.x) : v2::xcd_remap(blockIdx.x, t8);
  if (id >= total) return;
  const int b = id / per_b;
  int tm, tn;
  v2::grouped_tile<8>(id - b * per_b, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = int64_t(tm) * BM, n0 = int64_t(tn) * BN;   // m: i, n: slot within block
  // chunk C: first row group and the stride to the second
  auto chunk_row0 = [&](int c) -> int64_t {
    return TI == 64 ? m0 + 32 * c : m0 + (c & 1) * (BM / 2) + 32 * (c >> 1);
  };
  constexpr int64_t GSTRIDE = BM / 2;
  const int ext = p.flag[b];
  if (ext == 0) {
    // the zero intermediate operand of the tile's rows, in the stand-alone layout of chunks
    v2::static_for<BM / TI>([&](auto C) { epi_empty_chunk<BN>(p, b, m0 + int(C) * TI, n0); });
    return;
  }
  // the first chunk's checkpoint values: loaded ahead of the product where the
  // ring leaves registers for them (128 x 128), else right after it
  constexpr bool EARLY = BM * BN <= 128 * 128;
  EpiGU pre[2];
  if (EARLY) epi_load_gu<BN>(p, b, chunk_row0(0), GSTRIDE, n0, pre[0]);
  v16f acc[FM][FN];
  if (n0 < ext) {
    const int32_t* st = p.slot_tok + int64_t(b) * p.B;
    const int64_t B_ = p.B;
    auto tok_of = [&](int r) -> int64_t { const int64_t s = n0 + r; return s < B_ ? int64_t(st[s]) : -1; };
    phase1_ring_product<BM, BN, FG, FW>(p, p.b2e[b], m0, tok_of, smem, acc);
  } else {
    v2::static_for<FM>([&](auto FI) {
      v2::static_for<FN>([&](auto FJ) {
        v2::static_for<16>([&](auto Q) { acc[FI][FJ][int(Q)] = 0.f; });
      });
    });
  }
  if (!EARLY) epi_load_gu<BN>(p, b, chunk_row0(0), GSTRIDE, n0, pre[0]);
  __syncthreads();   // every wave is done reading the ring
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, r = lane & 31, wm = wave >> 1;
  float* dsl = reinterpret_cast<float*>(smem);
  v2::static_for<NCH>([&](auto C) {
    constexpr int c = C;
    constexpr int FI = TI == 64 ? c : c >> 1;
    // lane (r, h) of fragment (FI, FJ) holds rows 8 (q >> 2) + 4 h + (q & 3) of
    // its 32, slot column (wave & 1) * BN / 2 + 32 FJ + r
    if (TI == 64 || wm == (c & 1)) {
      const int g = TI == 64 ? wm : 0;   // the chunk's row group this wave holds
      v2::static_for<16>([&](auto Q) {
        float* row = dsl + (32 * g + 8 * (int(Q) >> 2) + 4 * h + (int(Q) & 3)) * DSW + (wave & 1) * (BN / 2) + r;
        v2::static_for<FN>([&](auto FJ) { row[32 * int(FJ)] = acc[FI][FJ][int(Q)]; });
      });
    }
    if constexpr (c + 1 < NCH) epi_load_gu<BN>(p, b, chunk_row0(c + 1), GSTRIDE, n0, pre[(c + 1) & 1]);
    __syncthreads();
    epi_chunk<FG, 2, BN, false, GEGLU, true>(p, b, chunk_row0(c), GSTRIDE, n0, smem, &pre[c & 1]);
    __syncthreads();   // pass 2 is done with the staging before the next chunk's dS
  });
}

template <int BM, int BN, int FG, int FW>
inline void phase1_fused_go(const Phase1Args& p, unsigned blocks, hipStream_t st) {
  if (p.geglu) phase1_fused_kernel<BM, BN, FG, FW, true><<<blocks, v2::kThreads, 0, st>>>(p);
  else phase1_fused_kernel<BM, BN, FG, FW, false><<<blocks, v2::kThreads, 0, st>>>(p);
}

template <int BM, int BN>
hipError_t phase1_fused_launch(Phase1Args p, int fg, int fw, hipStream_t st) {
  p.tiles_m = int((p.I + BM - 1) / BM);
  p.tiles_n = int(p.B / BN);
  const int64_t blocks = (int64_t(p.tiles_m) * p.tiles_n * p.N + 7) & ~int64_t(7);
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  const unsigned grid = unsigned(blocks);
  if (fg == kE4M3) {
    if (fw == kE4M3) phase1_fused_go<BM, BN, kE4M3, kE4M3>(p, grid, st);
    else phase1_fused_go<BM, BN, kE4M3, kE5M2>(p, grid, st);
  } else {
    if (fw == kE4M3) phase1_fused_go<BM, BN, kE5M2, kE4M3>(p, grid, st);
    else phase1_fused_go<BM, BN, kE5M2, kE5M2>(p, grid, st);
  }
  return hipGetLastError();
}

}  // namespace mx
