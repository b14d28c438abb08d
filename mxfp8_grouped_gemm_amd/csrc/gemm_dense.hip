// gemm_dense.hip -- MXFP8 NT GEMM with a bf16 store, for
//   * the dense backward (P2, "Matmul MXFP8 Backward Kernel API Reference"):
//       dX [M,K] = dY [M,N] . W^T [K,N]^T      (contraction over N)
//       dW [N,K] = dY^T [N,M] . X^T [K,M]^T    (contraction over M)
//   * the MoE weight gradients (P1 Phases 2 and 4), one group per expert,
//     whose contraction runs over the expert's blocks of token slots:
//       dW_gate_up[e] [H,2I] = X_tok [H,P] . dGU_tok [2I,P]^T
//       dW_down[e]    [I,H]  = inter_tok [I,P] . gy_tok [H,P]^T
//     where the K columns of expert e are the slots of the blocks
//     list[off[e] .. off[e+1]) (B slots each).
#include <type_traits>
#include <utility>

#include "gemm_v2.hpp"
#include "gemm_v3.hpp"
#include "gemm_v4.hpp"
#include "kernels.hpp"
#include "mx_device.hpp"

namespace mx {

// K column of stage s.  Grouped: the block list is read through the constant
// address space (a scalar load: the main loop only waits on vector loads for
// its DMA), and block sizes are powers of two >= 128 (shift = log2(blk/128)).
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
struct KMapGrouped {
  const int32_t* list;   // null: plain K range [0, K)
  int b0, blk, shift;
  int64_t K;
  __device__ __forceinline__ void operator()(int s, uint32_t& kc, int& kv) const {
    if (list) {
      const int blkid = ((const_i32_ptr)(uintptr_t)list)[b0 + (s >> shift)];
      kc = uint32_t(blkid) * uint32_t(blk) + uint32_t(s & ((1 << shift) - 1)) * v2::BK;
      kv = v2::BK;
    } else {
      const int64_t q = int64_t(s) * v2::BK;
      kc = uint32_t(q);
      const int64_t rem = K - q;
      kv = rem < v2::BK ? int(rem) : v2::BK;
    }
  }
};

// Output tile store.  The launcher swaps the operands, so a tile is C^T: tile
// row m is an output column and tile column n an output row.  A lane's
// registers 4k..4k+3 are four consecutive tile rows, i.e. four adjacent output
// columns: one 8-byte store.  M and N are multiples of 32, so such a group is
// wholly inside or outside the output.
template <int BM, int BN>
__device__ __forceinline__ void store_tile(const GemmStoreArgs& p, int g, int64_t m0, int64_t n0,
                                           const v2::v16f (&acc)[BM / 64][BN / 64]) {
  uint16_t* out = p.out + int64_t(g) * p.out_gstride;
  v2::static_for<BM / 64>([&](auto I) {
    v2::static_for<BN / 64>([&](auto J) {
      const int64_t orow = n0 + v2::acc_col<BM, BN>(J);
      if (orow < p.N) {
        uint16_t* dst = out + orow * p.ldo + m0;
        v2::static_for<4>([&](auto K) {
          const int ocol = v2::acc_row<BM, BN>(I, 4 * K);
          if (m0 + ocol < p.M) {
            float v0 = acc[I][J][4 * K], v1 = acc[I][J][4 * K + 1];
            float v2 = acc[I][J][4 * K + 2], v3 = acc[I][J][4 * K + 3];
            if (p.accumulate) {   // add the output's old values, then round once
              const uint2 o = *reinterpret_cast<const uint2*>(dst + ocol);
              v0 += bf16_to_f32(uint16_t(o.x)); v1 += bf16_to_f32(uint16_t(o.x >> 16));
              v2 += bf16_to_f32(uint16_t(o.y)); v3 += bf16_to_f32(uint16_t(o.y >> 16));
            }
            store_nt(dst + ocol, make_uint2(bf16x2_pack(v0, v1), bf16x2_pack(v2, v3)));
          }
        });
      }
    });
  });
}

// The same store through LDS (the ring's, free once the main loop is done):
// the tile's bf16 values are written to LDS as output rows padded by 16 bytes
// (so a fragment's 32 rows fall on different banks), then every thread stores
// 16-byte runs, and each store instruction writes whole row segments of the
// output (two rows of 512 bytes for a 256-wide tile) instead of 16-byte
// pieces of 32 rows.  Not for accumulation, which adds the old value to the
// fp32 result before its one rounding.  The outputs (weight gradients) are
// stored with the nontemporal hint, as in store_tile: measured 15% faster on
// Phase 2 with 0.2-1.6 MB experts, 2% with 117 MB ones.  (On 16-byte pieces
// of lines that other stores complete, as in the epilogue and the quantisers,
// the hint made those kernels 2-5x slower.)
template <int BM, int BN, int SMEM>
__device__ __forceinline__ void store_tile_staged(const GemmStoreArgs& p, int g, int64_t m0, int64_t n0,
                                                  const v2::v16f (&acc)[BM / 64][BN / 64], uint8_t* smem) {
  constexpr int RB = BM * 2 + 16;   // bytes per staged row
  static_assert(BN * RB <= SMEM, "the staged tile fits in the ring's LDS");
  __syncthreads();                  // every wave is done with the ring
  v2::static_for<BM / 64>([&](auto I) {
    v2::static_for<BN / 64>([&](auto J) {
      const int r = v2::acc_col<BM, BN>(J);
      v2::static_for<4>([&](auto K) {
        const int c = v2::acc_row<BM, BN>(I, 4 * K);
        *reinterpret_cast<uint2*>(smem + r * RB + c * 2) =
            make_uint2(bf16x2_pack(acc[I][J][4 * K], acc[I][J][4 * K + 1]),
                       bf16x2_pack(acc[I][J][4 * K + 2], acc[I][J][4 * K + 3]));
      });
    });
  });
  __syncthreads();
  // a thread keeps one 16-byte column run and walks the rows RPP apart, so its
  // addresses advance by constants; whole tiles skip the row test
  constexpr int CPR = BM * 2 / 16;           // 16-byte runs per row
  constexpr int RPP = v2::kThreads / CPR;    // rows per pass
  static_assert(v2::kThreads % CPR == 0 && BN % RPP == 0, "passes of whole rows");
  const int ch = threadIdx.x % CPR, r0 = threadIdx.x / CPR;
  const int64_t ocol = m0 + ch * 8;
  if (ocol >= p.M) return;
  uint16_t* dst = p.out + int64_t(g) * p.out_gstride + (n0 + r0) * p.ldo + ocol;
  const uint8_t* src = smem + r0 * RB + ch * 16;
  const int64_t step = int64_t(RPP) * p.ldo;
  if (n0 + BN <= p.N) {
#pragma unroll
    for (int q = 0; q < BN / RPP; ++q)
      store_nt(dst + q * step, *reinterpret_cast<const uint4*>(src + q * (RPP * RB)));
  } else {
    const int64_t nr = p.N - n0;   // rows of the tile inside the output
#pragma unroll 4
    for (int q = 0; q < BN / RPP; ++q)
      if (r0 + q * RPP < nr) store_nt(dst + q * step, *reinterpret_cast<const uint4*>(src + q * (RPP * RB)));
  }
}

// Workgroup id -> (group, first row, first column).  Hardware hands out
// workgroup ids round robin over the 8 XCDs, so ids are remapped to give each
// XCD a contiguous range, walked GM tile-rows at a time (co-resident tiles
// share operand rows in that XCD's L2).  With several groups (experts, whose
// contraction lengths differ) and a tile count per group divisible by 8, each
// XCD takes a contiguous eighth of every group instead, so no XCD is left
// holding the longest group alone; for one group the two maps coincide.
struct TilePos {
  int g;
  int64_t m0, n0;
};
//
// Several groups whose tile count P is not a multiple of 8 (e.g. 12 or 6 tiles
// per expert): XCD x takes, of group g, the contiguous tiles
// [floor(s P / 8), floor((s + 1) P / 8)) with s = (x - g) mod 8, so each XCD
// still holds an eighth of every group, and which XCDs take the larger
// shares rotates from group to group (over 8 groups every XCD takes exactly
// P tiles).  The launcher then gives every XCD room for ceil(G / 8) * P
// workgroups; those past its last tile exit (g = -1).  With contiguous
// ranges instead, the XCDs holding the most loaded experts ran up to three
// times longer than the others on skewed routing.
template <int BM, int BN>
__device__ __forceinline__ TilePos tile_pos(const GemmStoreArgs& p, int tile, int groups) {
  const int per_group = p.tiles_m * p.tiles_n;
  int id;
  if (per_group % 8 == 0) {
    const int share = per_group / 8, j = tile / 8;   // j-th workgroup on XCD tile % 8
    const int gg = j / share;
    id = gg * per_group + (tile % 8) * share + (j - gg * share);
  } else if (groups > 1) {
    const int x = tile % 8, j = tile / 8;
    const int q = j / per_group;
    int r = j - q * per_group;
    int g = -1, t = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int sl = (x - k + 64) & 7;
      const int lo = sl * per_group / 8, c = (sl + 1) * per_group / 8 - lo;
      if (g < 0) {
        if (r < c) {
          g = 8 * q + k;
          t = lo + r;
        } else {
          r -= c;
        }
      }
    }
    if (g < 0 || g >= groups) return TilePos{-1, 0, 0};
    id = g * per_group + t;
  } else {
    id = v2::xcd_remap(tile, p.total);
  }
  const int g = id / per_group;
  int tm, tn;
  v2::grouped_tile<8>(id - g * per_group, p.tiles_m, p.tiles_n, tm, tn);
  return TilePos{g, int64_t(tm) * BM, int64_t(tn) * BN};
}

// Unaligned shapes (ragged K or scale rows not 4-byte aligned): one tile per
// workgroup on the two-stage loop.
template <int BM, int BN, int FA, int FB>
__global__ void __launch_bounds__(v2::kThreads) gemm_store_generic(GemmStoreArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (BM + BN) * v2::BK];
  constexpr int FM = BM / 64, FN = BN / 64;
  const TilePos tp = tile_pos<BM, BN>(p, blockIdx.x, p.groups);
  if (tp.g < 0) return;
  const int wave = threadIdx.x >> 6;
  v2::Operand<BM, FM> A;
  v2::Operand<BN, FN> B;
  v2::setup_rows(A, p.a_codes, p.a_scales, tp.m0, p.M, p.lda, p.lda / 32, (wave >> 1) * (BM / 2));
  v2::setup_rows(B, p.b_codes, p.b_scales, tp.n0, p.N, p.ldb, p.ldb / 32, (wave & 1) * (BN / 2));
  KMapGrouped km{p.blk_list, 0, p.blk, 31 - __builtin_clz(unsigned(p.blk / v2::BK) | 1u), p.K};
  int nstages;
  if (p.blk_list) {
    km.b0 = p.blk_off[tp.g];
    nstages = int((int64_t(p.blk_off[tp.g + 1] - km.b0) * p.blk) / v2::BK);
  } else {
    nstages = int((p.K + v2::BK - 1) / v2::BK);
  }
  v2::v16f acc[FM][FN];
  v2::mainloop<BM, BN, v2::kFp8, FA, FB, true>(A, B, nstages, km, smem, acc);
  store_tile<BM, BN>(p, tp.g, tp.m0, tp.n0, acc);
}

// Aligned shapes: one tile per workgroup on a ring loop, the pair-slot ring
// (v4) when PAIR, else the four-slot ring (v3).
// LIST: K runs over each group's block list (MoE Phases 2 and 4).
template <int BM, int BN, int FA, int FB, bool LIST, bool PAIR>
__global__ void __launch_bounds__(v2::kThreads) gemm_store_ring(GemmStoreArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[PAIR ? v4::smem_bytes(BM, BN) : v3::smem_bytes(BM, BN)];
  constexpr int FM = BM / 64, FN = BN / 64;
  const TilePos tp = tile_pos<BM, BN>(p, blockIdx.x, p.groups);
  if (tp.g < 0) return;
  v3::ScaleDma<BM, BN> sd;
  v3::setup_scales(sd, p.a_scales, tp.m0, p.M, p.M * p.lda / 32, p.b_scales, tp.n0, p.N, p.N * p.ldb / 32);
  // K bytes of the tile's group: its blocks, the last one cut at its extent
  int64_t kbytes = p.K;
  int b0 = 0;
  if constexpr (LIST) {
    b0 = p.blk_off[tp.g];
    const int b1 = p.blk_off[tp.g + 1];
    kbytes = int64_t(b1 - b0) * p.blk;
    if (p.blk_ext && b1 > b0) kbytes -= p.blk - ((p.blk_ext[p.blk_list[b1 - 1]] + 127) & ~127);
  }
  v2::v16f acc[FM][FN];
  if constexpr (PAIR) {
    v4::Op<BM> A;
    v4::Op<BN> B;
    v4::setup_rows(A, p.a_codes, tp.m0, p.M, p.lda);
    v4::setup_rows(B, p.b_codes, tp.n0, p.N, p.ldb);
    const int npairs = int(kbytes / v4::PK);
    if constexpr (LIST) {
      const v4::KMapList km{p.blk_list, b0, p.blk, 31 - __builtin_clz(unsigned(p.blk / v4::PK))};
      v4::mainloop<BM, BN, v3::kFp8, FA, FB>(A, B, &sd, npairs, km, smem, acc);
    } else {
      v4::mainloop<BM, BN, v3::kFp8, FA, FB>(A, B, &sd, npairs, v4::KMapPlain{}, smem, acc);
    }
  } else {
    v3::Op<BM> A;
    v3::Op<BN> B;
    if (p.stage_major) {
      v3::setup_rows_sm(A, p.a_codes, tp.m0, p.M, p.M, p.lda);
      v3::setup_rows_sm(B, p.b_codes, tp.n0, p.N, p.N, p.ldb);
    } else {
      v3::setup_rows(A, p.a_codes, tp.m0, p.M, p.lda);
      v3::setup_rows(B, p.b_codes, tp.n0, p.N, p.ldb);
    }
    const int nstages = int(kbytes / v3::SK);
    if constexpr (LIST) {
      const v3::KMapList km{p.blk_list, b0, p.blk, 31 - __builtin_clz(unsigned(p.blk / v3::SK))};
      v3::mainloop<BM, BN, v3::kFp8, FA, FB>(A, B, &sd, nstages, km, smem, acc);
    } else {
      v3::mainloop<BM, BN, v3::kFp8, FA, FB>(A, B, &sd, nstages, v3::KMapPlain{}, smem, acc);
    }
  }
  if (p.accumulate) store_tile<BM, BN>(p, tp.g, tp.m0, tp.n0, acc);
  else store_tile_staged<BM, BN, sizeof(smem)>(p, tp.g, tp.m0, tp.n0, acc, smem);
}

template <int BM, int BN>
static void launch_generic(const GemmStoreArgs& p, int fa, int fb, unsigned grid, hipStream_t st) {
  if (fa == 0 && fb == 0) gemm_store_generic<BM, BN, 0, 0><<<grid, v2::kThreads, 0, st>>>(p);
  else if (fa == 0) gemm_store_generic<BM, BN, 0, 1><<<grid, v2::kThreads, 0, st>>>(p);
  else if (fb == 0) gemm_store_generic<BM, BN, 1, 0><<<grid, v2::kThreads, 0, st>>>(p);
  else gemm_store_generic<BM, BN, 1, 1><<<grid, v2::kThreads, 0, st>>>(p);
}

template <int BM, int BN, bool LIST, bool PAIR>
static void launch_ring(const GemmStoreArgs& p, int fa, int fb, unsigned grid, hipStream_t st) {
  if (fa == 0 && fb == 0) gemm_store_ring<BM, BN, 0, 0, LIST, PAIR><<<grid, v2::kThreads, 0, st>>>(p);
  else if (fa == 0) gemm_store_ring<BM, BN, 0, 1, LIST, PAIR><<<grid, v2::kThreads, 0, st>>>(p);
  else if (fb == 0) gemm_store_ring<BM, BN, 1, 0, LIST, PAIR><<<grid, v2::kThreads, 0, st>>>(p);
  else gemm_store_ring<BM, BN, 1, 1, LIST, PAIR><<<grid, v2::kThreads, 0, st>>>(p);
}

hipError_t launch_gemm_store(GemmStoreArgs p, int groups, int fa, int fb, hipStream_t st) {
  if (p.M <= 0 || p.N <= 0 || groups <= 0) return hipSuccess;
  // compute C^T = B . A^T so that the store is along the output's rows (see store_tile)
  std::swap(p.a_codes, p.b_codes);
  std::swap(p.a_scales, p.b_scales);
  std::swap(p.lda, p.ldb);
  std::swap(p.M, p.N);
  std::swap(fa, fb);
  // every stage full and scale rows 4-byte aligned -> the ring; otherwise the v2 loop
  const bool generic = (p.lda % v2::BK) || (p.ldb % v2::BK) || (!p.blk_list && (p.K % v2::BK)) ||
                       (p.blk_list && (p.blk % v2::BK));
  // stage-major operands: only the four-slot ring reads them
  if (p.stage_major && (generic || p.pair)) return hipErrorInvalidValue;
  // larger tiles once there are enough of them to fill the chip
  const bool big = !generic && p.M >= 256 && p.N >= 256 &&
                   ((p.M + 255) / 256) * ((p.N + 255) / 256) * int64_t(groups) >= 200;
  const int BM = big ? 256 : 128, BN = big ? 256 : 128;
  p.tiles_m = int((p.M + BM - 1) / BM);
  p.tiles_n = int((p.N + BN - 1) / BN);
  const int64_t per_group = int64_t(p.tiles_m) * p.tiles_n;
  const int64_t total = per_group * groups;
  if (total > INT32_MAX) return hipErrorInvalidValue;
  p.total = int(total);
  p.groups = groups;
  // rotating eighths (tile_pos): room for ceil(G / 8) * P workgroups per XCD
  const int64_t launched = (per_group % 8 && groups > 1) ? 8 * ((groups + 7) / 8) * per_group : total;
  if (launched > INT32_MAX) return hipErrorInvalidValue;
  if (generic) {
    launch_generic<128, 128>(p, fa, fb, unsigned(launched), st);
    return hipGetLastError();
  }
  const unsigned grid = unsigned(launched);
  if (big) {
    if (p.blk_list) {
      if (p.pair) launch_ring<256, 256, true, true>(p, fa, fb, grid, st);
      else launch_ring<256, 256, true, false>(p, fa, fb, grid, st);
    } else {
      if (p.pair) launch_ring<256, 256, false, true>(p, fa, fb, grid, st);
      else launch_ring<256, 256, false, false>(p, fa, fb, grid, st);
    }
  } else {
    if (p.blk_list) launch_ring<128, 128, true, false>(p, fa, fb, grid, st);
    else launch_ring<128, 128, false, false>(p, fa, fb, grid, st);
  }
  return hipGetLastError();
}

}  // namespace mx
