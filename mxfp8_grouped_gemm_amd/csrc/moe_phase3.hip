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
  if (!block_tile(p.tile_start, p.flag, BM, int(p.N), wg, p.rr_tiles, bt)) return P3Pos{-1, 0, 0};
  int tm, tn;
  v2::grouped_tile<8>(bt.local, bt.slots, p.tiles_n, tm, tn);
  return P3Pos{bt.b, int64_t(tm) * BM, int64_t(tn) * BN};
}

// ---------------------------------------------------------------------------
// The last round of tiles, cut along K (moe_tiles.hpp, TailCut; the cut of each
// XCD is computed with the tile ranges).  A cut tile's own workgroup runs its
// first part and stores its rows to dx_slot as usual; extra workgroups after
// the main grid (ids x mod 8 again: the same XCD, after its last round has
// started) run the other parts and store their fp32 tiles to the parts
// buffer; p3_fixup_kernel then adds those into dx_slot in part order, so the
// result stays the same from run to run.
constexpr int kP3MaxExtra = 256;   // extra workgroups (and part tiles) at most

__device__ __forceinline__ const TailCut* p3_cuts(const Phase3Args& p) {
  return reinterpret_cast<const TailCut*>(p.parts);
}
__device__ __forceinline__ float* p3_part_tiles(const Phase3Args& p) {
  return reinterpret_cast<float*>(p.parts + 256);
}

// What workgroup wg runs: a whole tile, the first part of a cut tile (its own
// id), or another part (ids from grid_main on), and where that part goes.
struct P3Work {
  P3Pos tp;        // tp.b < 0: nothing
  int pair0, npairs;
  int part_slot;   // >= 0: the fp32 tile goes to part tile part_slot
};
template <int BM, int BN>
__device__ __forceinline__ P3Work p3_work(const Phase3Args& p, int wg) {
  P3Work w{P3Pos{-1, 0, 0}, 0, p.npairs, -1};
  const bool extra = wg >= p.grid_main;
  if (p.conc <= 0) {
    if (!extra) w.tp = p3_pos<BM, BN>(p, wg);
    return w;
  }
  const int e = extra ? wg - p.grid_main : wg;
  const int x = e % 8, q = e / 8;
  const TailCut c = p3_cuts(p)[x];
  int main_wg = wg, part = 0;
  bool cut;
  if (extra) {
    if (q >= c.tail * (c.S - 1)) return w;   // also every extra id when nothing is cut
    const int i = q / (c.S - 1);
    part = 1 + q % (c.S - 1);
    main_wg = 8 * (c.nx - c.tail + i) + x;
    w.part_slot = c.base + q;
    cut = true;
  } else {
    cut = q >= c.nx - c.tail && q < c.nx;   // tail == 0: never
  }
  w.tp = p3_pos<BM, BN>(p, main_wg);
  if (cut) {
    w.pair0 = part * p.npairs / c.S;
    w.npairs = (part + 1) * p.npairs / c.S - w.pair0;
  }
  return w;
}

// stage s of a part that starts at stage s0
struct P3KMap {
  int s0;
  __device__ __forceinline__ uint32_t operator()(int s) const { return uint32_t(s + s0) * v3::SK; }
};

// A part's fp32 tile, row-major BM x BN (lanes of a fragment row write 128
// consecutive bytes).
template <int BM, int BN>
__device__ __forceinline__ void p3_store_part(float* dst, const v16f (&acc)[BM / 64][BN / 64]) {
  v2::static_for<BM / 64>([&](auto FI) {
    v2::static_for<16>([&](auto Q) {
      float* row = dst + v2::acc_row<BM, BN>(FI, Q) * BN;
      v2::static_for<BN / 64>([&](auto FJ) { row[v2::acc_col<BM, BN>(FJ)] = acc[FI][FJ][int(Q)]; });
    });
  });
}

// dx_slot += the other parts of each cut tile, in part order.  One workgroup
// per 16 rows of a cut tile: ids x + 8 (i * BM / 16 + slab) for tile i of XCD
// x; a thread takes one 4-column group of 4 rows, all of its loads issued
// before the sums.
template <int BM, int BN>
__global__ void __launch_bounds__(256) p3_fixup_kernel(Phase3Args p) {
  constexpr int NSL = BM / 16, CG = BN / 4;   // slabs per tile, 4-column groups per row
  static_assert(CG * 4 == 256, "a thread per 4-column group and row of 4");
  const int x = blockIdx.x % 8, rest = blockIdx.x / 8, i = rest / NSL, slab = rest % NSL;
  const TailCut c = p3_cuts(p)[x];
  if (i >= c.tail) return;
  const P3Pos tp = p3_pos<BM, BN>(p, 8 * (c.nx - c.tail + i) + x);
  if (tp.b < 0) return;
  const int col = (threadIdx.x % CG) * 4, r0 = slab * 16 + threadIdx.x / CG;
  if (tp.n0 + col >= p.H) return;   // H % 32 == 0: a group is all inside or all outside
  const float* part = p3_part_tiles(p) + int64_t(c.base + i * (c.S - 1)) * (BM * BN);
  float* out = p.dx_slot + (int64_t(tp.b) * p.B + tp.m0) * p.H + tp.n0 + col;
  float4 v[4], q[kCutMaxParts - 1][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = r0 + 4 * j;
    v[j] = *reinterpret_cast<const float4*>(out + int64_t(r) * p.H);
#pragma unroll
    for (int k = 0; k < kCutMaxParts - 1; ++k)
      q[k][j] = k < c.S - 1 ? *reinterpret_cast<const float4*>(part + int64_t(k) * (BM * BN) + r * BN + col)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int k = 0; k < kCutMaxParts - 1; ++k) {
      if (k < c.S - 1) {
        v[j].x += q[k][j].x;
        v[j].y += q[k][j].y;
        v[j].z += q[k][j].z;
        v[j].w += q[k][j].w;
      }
    }
    *reinterpret_cast<float4*>(out + int64_t(r0 + 4 * j) * p.H) = v[j];
  }
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
    // a thread keeps one 16-byte column run and walks the rows RPP apart
    constexpr int RPP = v2::kThreads / CPR;   // rows per pass
    static_assert(v2::kThreads % CPR == 0 && R % RPP == 0, "passes of whole rows");
    const int ch = threadIdx.x % CPR, r0 = threadIdx.x / CPR;
    const int64_t hh = tp.n0 + ch * 4;
    if (hh < p.H) {
      float* dst = p.dx_slot + (sbase + tp.m0 + int(PASS) * R + r0) * p.H + hh;
      const uint8_t* src = smem + r0 * RB + ch * 16;
#pragma unroll 8
      for (int q = 0; q < R / RPP; ++q)
        store_nt(dst + int64_t(q) * RPP * p.H, *reinterpret_cast<const uint4*>(src + q * (RPP * RB)));
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
  const P3Work w = p3_work<BM, BN>(p, blockIdx.x);
  const P3Pos& tp = w.tp;
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
  v3::mainloop<BM, BN, v3::kFp8, FG, FW>(A, B, &sd, 2 * w.npairs, P3KMap{2 * w.pair0}, smem, acc);
  if (w.part_slot >= 0)
    p3_store_part<BM, BN>(p3_part_tiles(p) + int64_t(w.part_slot) * (BM * BN), acc);
  else
    p3_store_staged<BM, BN, sizeof(smem)>(p, tp, acc, smem);
}

template <int BM, int BN>
static hipError_t phase3_launch(Phase3Args p, int fg, int fw, bool generic, hipStream_t st) {
  // the ring's LDS keeps these tiles at one workgroup per CU, so the CU count
  // is the number resident at once (TailCut)
  static_assert(2 * v3::smem_bytes(BM, BN) > 160 * 1024, "one workgroup per CU");
  p.tiles_m = int((p.B + BM - 1) / BM);
  p.tiles_n = int((p.H + BN - 1) / BN);
  const int64_t total = (int64_t(p.tiles_m) * p.tiles_n * p.N + 7) & ~int64_t(7);   // every tile, rounded to 8
  if (total + kP3MaxExtra > INT32_MAX) return hipErrorInvalidValue;
  p.grid_main = int(total);
  p.npairs = int(2 * p.I / 128);
  // the cut needs the ring, the parts buffer, whole XCDs of CUs (at most
  // kP3MaxExtra: the extra workgroups and part tiles) and at least two parts'
  // worth of stage pairs
  const bool cut = !generic && p.parts && phase3_parts_bytes(p) > 0 && p.conc >= 8 && p.conc % 8 == 0 &&
                   p.conc <= kP3MaxExtra && p.npairs >= 2 * kCutMinPairs;
  if (!cut) p.conc = 0;
  hipError_t e = launch_tile_ranges(p.flag, p.N, BM, p.tiles_n, p.tile_start, st,
                                    cut ? reinterpret_cast<TailCut*>(p.parts) : nullptr, p.conc, p.npairs,
                                    p.rr_tiles, int(p.B));
  if (e != hipSuccess) return e;
  if (generic) {
    const unsigned grid = unsigned(total);
    if (fg == 0 && fw == 0) phase3_generic<BM, BN, 0, 0><<<grid, v2::kThreads, 0, st>>>(p);
    else if (fg == 0) phase3_generic<BM, BN, 0, 1><<<grid, v2::kThreads, 0, st>>>(p);
    else if (fw == 0) phase3_generic<BM, BN, 1, 0><<<grid, v2::kThreads, 0, st>>>(p);
    else phase3_generic<BM, BN, 1, 1><<<grid, v2::kThreads, 0, st>>>(p);
  } else {
    const unsigned grid = unsigned(total + p.conc);   // p.conc extra workgroups for the cut parts
    if (fg == 0 && fw == 0) phase3_ring<BM, BN, 0, 0><<<grid, v2::kThreads, 0, st>>>(p);
    else if (fg == 0) phase3_ring<BM, BN, 0, 1><<<grid, v2::kThreads, 0, st>>>(p);
    else if (fw == 0) phase3_ring<BM, BN, 1, 0><<<grid, v2::kThreads, 0, st>>>(p);
    else phase3_ring<BM, BN, 1, 1><<<grid, v2::kThreads, 0, st>>>(p);
    if (p.conc) p3_fixup_kernel<BM, BN><<<unsigned(p.conc * (BM / 16)), 256, 0, st>>>(p);
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

// The parts buffer: the 8 XCDs' cuts (256 bytes), then the later parts' tiles:
// fewer than the extra workgroups, and at most kCutMaxParts - 1 per tile.
// Empty where nothing can be cut (the v2 loop, or too few stage pairs).
int64_t phase3_parts_bytes(const Phase3Args& p) {
  if ((2 * p.I) % v2::BK != 0 || 2 * p.I / 128 < 2 * kCutMinPairs) return 0;
  const int64_t bm = phase3_wide(p) ? 256 : 128, bn = 256;
  int64_t tiles = (kCutMaxParts - 1) * phase3_max_tiles(p);
  tiles = tiles < kP3MaxExtra ? tiles : kP3MaxExtra;
  return 256 + tiles * bm * bn * 4;
}

}  // namespace mx
