// moe_phase3.hip -- Phase 3 of the MoE backward (P1, "Blockwise MM Backward
// MXFP8 Kernel API Reference": Phase 3; P3, sonic-moe functional/backward.py:
// _up_projection_backward_act, the input-gradient product).
//
// Per block b (tile rows = slot p, columns = hidden index h, contraction over 2I):
//   dX_slot[p][h] = sum_{j,i} deq(dGU)[p][j][i] * deq(W_gate_up[e])[h][j][i]
//   stored per slot in fp32; the finalisation sums each token's slots (they
//   sit in different blocks) in expert order, so dX is deterministic.
#include "gemm_v2.hpp"
#include "gemm_v3.hpp"
#include "kernels.hpp"
#include "moe_tiles.hpp"
#include "mx_device.hpp"

namespace mx {

using v2::v16f;
using v2::KMapPlain;

// ---------------------------------------------------------------------------
// Phase 3 tiles: block b, rows = slots m0.., columns = hidden index n0..
// Live tiles only (moe_tiles.hpp): block b's slot tiles up to its extent, times
// the H tiles.  b < 0: no tile.
struct P3Pos {
  int b;
  int64_t m0, n0;
};
template <int BM, int BN>
__device__ __forceinline__ P3Pos p3_pos(const Phase3Args& p, int wg) {
  BlockTiles bt;
  if (!block_tile(p.tile_start, int(p.N), p.tiles_n, wg, p.rr_tiles, bt)) return P3Pos{-1, 0, 0};
  int tm, tn;
  v2::grouped_tile<8>(bt.local, bt.slots, p.tiles_n, tm, tn);
  return P3Pos{bt.b, int64_t(tm) * BM, int64_t(tn) * BN};
}

// dX rows of one tile.  Every slot of the tile stores its row: a padding
// slot's dGU row is zeros, so its row is zeros too, and the finalisation
// reads only routed slots' rows.  (Storing only routed rows made every store
// wait for a load of the slot's token.)  Tiles lie inside one block (BM <= B).
template <int BM, int BN>
__device__ __forceinline__ void p3_store(const Phase3Args& p, const P3Pos& tp, const v16f (&acc)[BM / 64][BN / 64]) {
  const int64_t sbase = int64_t(tp.b) * p.B;
  v2::static_for<BM / 64>([&](auto FI) {
    v2::static_for<16>([&](auto Q) {
      const int64_t s = tp.m0 + v2::acc_row<BM, BN>(FI, Q);
      float* dst = p.dx_slot + (sbase + s) * p.H;
      v2::static_for<BN / 64>([&](auto FJ) {
        const int64_t hh = tp.n0 + v2::acc_col<BM, BN>(FJ);
        if (hh < p.H) dst[hh] = acc[FI][FJ][int(Q)];
      });
    });
  });
}

// The same rows through LDS (the ring's, free after the main loop), in passes
// of R rows padded by 16 bytes: every thread then stores 16-byte runs, so each
// store instruction writes whole row segments (BN * 4 bytes) instead of
// 128-byte pieces of 2 rows.  Nontemporal stores: the rows ([P, H] fp32, the
// largest output) are read once, by the finalisation, after the other phases;
// measured 24% faster on the fine workload (H = 1536, 2I = 512), 10% with
// 2I = 2816, 1% with 2I = 28672.
template <int BM, int BN, int SMEM>
__device__ __forceinline__ void p3_store_staged(const Phase3Args& p, const P3Pos& tp,
                                                const v16f (&acc)[BM / 64][BN / 64], uint8_t* smem) {
  constexpr int RB = BN * 4 + 16;                       // bytes per staged row
  constexpr int R = (SMEM / RB) >= BM ? BM : BM / 2;    // rows per pass
  static_assert(R * RB <= SMEM && BM % R == 0 && (BM / 2) % 32 == 0, "staging passes");
  const int64_t sbase = int64_t(tp.b) * p.B;
  const int wave = threadIdx.x >> 6;
  constexpr int CPR = BN * 4 / 16;                      // 16-byte runs per row
  v2::static_for<BM / R>([&](auto PASS) {
    __syncthreads();                                    // the ring, or the previous pass, is done
    // pass PASS holds tile rows [PASS * R, PASS * R + R): R == BM, or the waves
    // whose half of the rows (wave >> 1) is PASS
    if (R == BM || (wave >> 1) == int(PASS)) {
      v2::static_for<BM / 64>([&](auto FI) {
        v2::static_for<16>([&](auto Q) {
          const int r = v2::acc_row<BM, BN>(FI, Q) - int(PASS) * R;
          v2::static_for<BN / 64>([&](auto FJ) {
            *reinterpret_cast<float*>(smem + r * RB + v2::acc_col<BM, BN>(FJ) * 4) = acc[FI][FJ][int(Q)];
          });
        });
      });
    }
    __syncthreads();
#pragma unroll 4
    for (int k = threadIdx.x; k < R * CPR; k += v2::kThreads) {
      const int r = k / CPR, ch = k % CPR;
      const int64_t s = tp.m0 + int(PASS) * R + r, hh = tp.n0 + ch * 4;
      if (hh < p.H)
        store_nt(p.dx_slot + (sbase + s) * p.H + hh, *reinterpret_cast<const uint4*>(smem + r * RB + ch * 16));
    }
  });
}

// 2I not a multiple of 128 bytes: one tile per workgroup on the v2 loop.
template <int BM, int BN, int FG, int FW>
__global__ void __launch_bounds__(v2::kThreads) phase3_generic(Phase3Args p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (BM + BN) * v2::BK];
  constexpr int FM = BM / 64, FN = BN / 64;
  const P3Pos tp = p3_pos<BM, BN>(p, blockIdx.x);
  if (tp.b < 0) return;
  const int64_t e = p.b2e[tp.b];
  const int wave = threadIdx.x >> 6;
  const int64_t sbase = int64_t(tp.b) * p.B, twoI = 2 * p.I;
  v2::Operand<BM, FM> A;
  v2::Operand<BN, FN> B;
  v2::setup_rows(A, p.dgu_row_codes + sbase * twoI, p.dgu_row_scales + sbase * (twoI / 32), tp.m0, p.B, twoI,
                 twoI / 32, (wave >> 1) * (BM / 2));
  v2::setup_rows(B, p.wgu_codes + e * p.H * twoI, p.wgu_scales + e * p.H * (twoI / 32), tp.n0, p.H, twoI,
                 twoI / 32, (wave & 1) * (BN / 2));
  v16f acc[FM][FN];
  v2::mainloop<BM, BN, v2::kFp8, FG, FW, true>(A, B, int((twoI + v2::BK - 1) / v2::BK), KMapPlain{twoI}, smem,
                                                acc);
  p3_store<BM, BN>(p, tp, acc);
}

// Aligned: one tile per workgroup on the four-slot ring loop (its deeper
// look-ahead measured 4% faster here than the pair-slot ring).
template <int BM, int BN, int FG, int FW>
__global__ void __launch_bounds__(v2::kThreads) phase3_ring(Phase3Args p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[v3::smem_bytes(BM, BN)];
  constexpr int FM = BM / 64, FN = BN / 64;
  const P3Pos tp = p3_pos<BM, BN>(p, blockIdx.x);
  if (tp.b < 0) return;
  const int64_t e = p.b2e[tp.b];
  const int64_t sbase = int64_t(tp.b) * p.B, twoI = 2 * p.I;
  v3::Op<BM> A;
  v3::Op<BN> B;
  v3::ScaleDma<BM, BN> sd;
  const int64_t P = p.N * p.B;
  // dGU stage-major over all P slots (the tile's rows stop at its block's end);
  // W_gate_up row-major, as the caller holds it
  v3::setup_rows_sm(A, p.dgu_row_codes, sbase + tp.m0, sbase + p.B, P, twoI);
  v3::setup_rows(B, p.wgu_codes + e * p.H * twoI, tp.n0, p.H, twoI);
  // pair-major scales: dGU along I over all P slots; W_gate_up re-laid per expert
  v3::setup_scales(sd, p.dgu_row_scales, sbase + tp.m0, P, P * (twoI / 32), p.wgu_scales + e * p.H * (twoI / 32),
                   tp.n0, p.H, p.H * (twoI / 32));
  v16f acc[FM][FN];
  v3::mainloop<BM, BN, v3::kFp8, FG, FW>(A, B, &sd, int(twoI / v3::SK), v3::KMapPlain{}, smem, acc);
  p3_store_staged<BM, BN, sizeof(smem)>(p, tp, acc, smem);
}

template <int BM, int BN>
static hipError_t phase3_launch(Phase3Args p, int fg, int fw, bool generic, hipStream_t st) {
  p.tiles_m = int((p.B + BM - 1) / BM);
  p.tiles_n = int((p.H + BN - 1) / BN);
  const int64_t total = (int64_t(p.tiles_m) * p.tiles_n * p.N + 7) & ~int64_t(7);   // every tile, rounded to 8
  if (total > INT32_MAX) return hipErrorInvalidValue;
  hipError_t e = launch_tile_ranges(p.flag, p.N, BM, p.tiles_n, p.tile_start, st);
  if (e != hipSuccess) return e;
  if (generic) {
    const unsigned grid = unsigned(total);
    if (fg == 0 && fw == 0) phase3_generic<BM, BN, 0, 0><<<grid, v2::kThreads, 0, st>>>(p);
    else if (fg == 0) phase3_generic<BM, BN, 0, 1><<<grid, v2::kThreads, 0, st>>>(p);
    else if (fw == 0) phase3_generic<BM, BN, 1, 0><<<grid, v2::kThreads, 0, st>>>(p);
    else phase3_generic<BM, BN, 1, 1><<<grid, v2::kThreads, 0, st>>>(p);
  } else {
    const unsigned grid = unsigned(total);
    if (fg == 0 && fw == 0) phase3_ring<BM, BN, 0, 0><<<grid, v2::kThreads, 0, st>>>(p);
    else if (fg == 0) phase3_ring<BM, BN, 0, 1><<<grid, v2::kThreads, 0, st>>>(p);
    else if (fw == 0) phase3_ring<BM, BN, 1, 0><<<grid, v2::kThreads, 0, st>>>(p);
    else phase3_ring<BM, BN, 1, 1><<<grid, v2::kThreads, 0, st>>>(p);
  }
  return hipGetLastError();
}

// Tile shape: 256 x 256 when the block and H allow, else 128 x 256; 2I not a
// multiple of 128 bytes (unaligned scale rows / ragged last K stage): the v2
// loop at 128 x 256.  A short contraction (2I < 1024: a few ring stages per
// tile) also takes 128 x 256 tiles: with the rows stored through LDS, they
// measured 5% faster at 2I = 512 than 128 x 128 tiles at two per CU.
static bool phase3_wide(const Phase3Args& p) {
  return (2 * p.I) % v2::BK == 0 && 2 * p.I >= 1024 && p.B >= 256 && p.H >= 256;
}
hipError_t launch_phase3(const Phase3Args& p, int fg, int fw, hipStream_t st) {
  if (phase3_wide(p)) return phase3_launch<256, 256>(p, fg, fw, false, st);
  return phase3_launch<128, 256>(p, fg, fw, (2 * p.I) % v2::BK != 0, st);
}

int64_t phase3_max_tiles(const Phase3Args& p) {
  const int64_t bm = phase3_wide(p) ? 256 : 128, bn = 256;
  return p.N * ((p.B + bm - 1) / bm) * ((p.H + bn - 1) / bn);
}

}  // namespace mx
