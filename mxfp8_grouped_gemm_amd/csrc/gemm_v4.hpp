// gemm_v4.hpp -- MX GEMM main loop for gfx950: a ring of two LDS pair slots.
//
// C[m][n] = sum_k A[m][k] * B[n][k] for operands whose code rows are 128-byte
// aligned and whose K is a multiple of 128 bytes, in two element modes:
//   kFp8    : fp8 codes + E8M0 scales on v_mfma_scale_f32_32x32x64_f8f6f4;
//   kFp8Bf16: fp8 codes + E8M0 scales moved like kFp8, converted in registers
//             to their exact bf16 values (v_cvt_scalef32_pk_bf16_fp8/bf8: a
//             code times a power of two has at most 4 significant bits) and
//             reduced on the bf16 MFMA, whose accumulation is exact enough
//             that results requantised afterwards round as an exact sum would.
//
// A stage is 64 bytes of K (one 64-element fp8 MFMA step, four 16-element bf16
// steps); a pair is two consecutive stages, 128 bytes of K, which is what one
// scale word per row covers (four E8M0 groups).  LDS holds two pair slots of
// (BM + BN) rows x 128 bytes, then two scale slots of one 4-byte word per row,
// loaded from pair-major scale arrays (see ScaleDma).
//
// Why 128-byte rows: a DMA instruction then moves 8 rows x 128 bytes, whole
// cache lines, where the four-slot ring of 64-byte stages (gemm_v3.hpp) moves
// 16 rows x 64 bytes, two requests per line.  The price is look-ahead: that
// ring issues each stage three stages before its use, this one a pair one pair
// (two stages) before.  Measured with row-major operands: 6% faster on the
// dense 8192^3 GEMM and 3% on Phase 1 and Phase 2, whose operand tiles are
// reused from L2; 4% slower on Phase 3 and 2% on Phase 4, which stream more
// of their operands from HBM and need the deeper look-ahead.  Operands the
// library writes itself are stage-major (gemm_v3.hpp, Op), which gives the
// four-slot ring whole lines too; with them it beats this ring by 5-9% (dense
// from bf16, Phase 2).  This ring keeps the products of row-major operands
// the caller holds: Phase 1 (W_down and the dY rows it gathers) and the dense
// GEMMs on pre-quantised operands.
//
// Loads are issued with inline asm (s_mov_b32 m0 + buffer_load_dword{,x4} ...
// lds) because the compiler's wait-count pass treats every LDS read after an
// LDS DMA builtin as possibly aliased and waits for all outstanding loads,
// which would serialise the ring.  The asm loads are invisible to that pass;
// the loop waits on them explicitly (vmcnt) and they only ever write LDS.
// The asm sets m0 itself; m0 is reserved (not allocatable), and code built on
// this core has no other m0 users, so no compiler value lives there across it.
//
// Pair step u (pair u in slot u % 2; stage 2u's fragments already in
// registers, set 0):
//   stage 2u: the DMA of pair u+1 into the other slot (its previous pair was
//     finished by every wave at the last barrier), stage 2u+1's fragment reads
//     into set 1, and stage 2u's MFMAs, interleaved in fenced regions;
//   stage 2u+1: half its MFMAs; wait until pair u+1 has landed and barrier;
//     the other half interleaved with the reads of stage 2u+2's fragments
//     (set 0, pair u+1) and scale words.
// Every step is straight-line code, so the compiler keeps this order.
#pragma once
#include "gemm_v3.hpp"

namespace mx {
namespace v4 {

using v2::Buf;
using v2::v16f;
using v2::v8bf;
using v2::v8i;
using v2::kFp8;
using v2::kFp8Bf16;

using v3::SK;
using v3::kThreads;
using v3::kOOB;
using v3::v4i;
using v3::waitcnt;
using v3::ScaleDma;
using v3::setup_scales_map;
using v3::setup_scales;
using v3::mma;
#if defined(__HIP_DEVICE_COMPILE__)
using v3::rsrc;
using v3::dma16;
using v3::dma4;
#endif
using v3::lds_addr;

constexpr int PK = 128;         // bytes of K per pair (two stages)
constexpr int NP = 2;           // pair slots in LDS

// LDS bytes of a tile's ring.
__host__ __device__ constexpr int code_slot(int BM, int BN) { return (BM + BN) * PK; }
__host__ __device__ constexpr int scale_chunks(int BM, int BN) { return 4 * ((BM + BN + 255) / 256); }
__host__ __device__ constexpr int scale_slot(int BM, int BN) { return scale_chunks(BM, BN) * 256; }
__host__ __device__ constexpr int smem_bytes(int BM, int BN) { return NP * (code_slot(BM, BN) + scale_slot(BM, BN)); }

// One operand's code rows: buffer and this lane's DMA offsets.  Instruction j
// of wave w fills rows w*ROWS/4 + 8j .. +8 of a pair slot; lane l fills row
// +(l >> 3), physical chunk l & 7, fetching the logical chunk stored there.
template <int ROWS>
struct Op {
  Buf codes;
  uint32_t off[ROWS / 32];
};

template <int ROWS>
__device__ __forceinline__ int dma_row(int j) {
  return (threadIdx.x >> 6) * (ROWS / 4) + 8 * j + ((threadIdx.x & 63) >> 3);
}
// Physical 16-byte chunk of logical chunk c (0..3: the pair's first stage,
// 4..7 its second) in row `row` is c ^ swz(row).  LDS serves 16 lanes of a
// 16-byte read per clock; a fragment read has lanes r = 0..31 on rows r, all
// on one logical chunk, and rows 2 apart are 256 bytes apart, so XOR with
// bits 1-3 of the row puts any 16 consecutive rows on 16 distinct 16-byte
// bank groups.  Rows 32 apart share a swizzle, so a wave's fragments sit at
// constant offsets from each other.
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

template <int ROWS>
__device__ __forceinline__ void setup_rows(Op<ROWS>& op, const uint8_t* codes, int64_t row0, int64_t nrows,
                                           int64_t ld) {
  const int64_t have = nrows - row0 < ROWS ? nrows - row0 : ROWS;
  op.codes = v2::make_rsrc(codes + row0 * ld, uint32_t(have * ld));
#pragma unroll
  for (int j = 0; j < ROWS / 32; ++j) {
    const int r = dma_row<ROWS>(j);
    const int lc = (threadIdx.x & 7) ^ swz(r);
    op.off[j] = r < have ? uint32_t(r * ld + 16 * lc) : kOOB;
  }
}

// Gathered rows: tile row r reads source row rowid(r) (negative: zeros).
template <int ROWS, class RowId>
__device__ __forceinline__ void setup_gather(Op<ROWS>& op, const uint8_t* codes, int64_t src_rows, int64_t ld,
                                             const RowId& rowid) {
  op.codes = v2::make_rsrc(codes, uint32_t(src_rows * ld));
#pragma unroll
  for (int j = 0; j < ROWS / 32; ++j) {
    const int r = dma_row<ROWS>(j);
    const int64_t t = rowid(r);
    const int lc = (threadIdx.x & 7) ^ swz(r);
    op.off[j] = t >= 0 ? uint32_t(t * ld + 16 * lc) : kOOB;
  }
}

// K map over pairs: the byte offset of pair u's first element.  Plain: [0, K).
// Grouped: the K columns of a group are the blocks list[b0 ..] of blk columns
// each (blk a power of two >= 128, so a pair never straddles two blocks).
struct KMapPlain {
  __device__ __forceinline__ uint32_t operator()(int u) const { return uint32_t(u) * PK; }
};
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
struct KMapList {
  const int32_t* list;
  int b0, blk, shift;   // shift = log2(blk / 128)
  __device__ __forceinline__ uint32_t operator()(int u) const {
    const int blkid = ((const_i32_ptr)(uintptr_t)list)[b0 + (u >> shift)];
    return uint32_t(blkid) * uint32_t(blk) + uint32_t(u & ((1 << shift) - 1)) * PK;
  }
};
// One tile's operands: code rows of A and B, their scale rows, the K map and
// the number of pairs (K / 128 bytes).
template <int BM, int BN, class KMap>
struct Tile {
  Op<BM> A;
  Op<BN> B;
  ScaleDma<BM, BN> sd;
  KMap km;
  int npairs;
};

// The ring of one tile.  Pairs past the last one load through descriptors with
// no records, which the hardware answers with zeros without touching memory,
// so every pair step issues the same loads and waits.  The kernels here run
// one tile per workgroup: chaining tiles through the ring in a persistent grid
// was measured slower (the next tile's descriptors spill, and their reloads'
// waits drain the ring at every tile boundary).
template <int BM, int BN, int ELEM, int FA, int FB, class KMap>
struct Ring {
  static constexpr int FM = BM / 64, FN = BN / 64;
  static constexpr int CS = code_slot(BM, BN), SSB = scale_slot(BM, BN);
  static constexpr int NCA = BM / 32, NCI = (BM + BN) / 32;   // code DMA instructions per wave per pair
  static constexpr int NS = ScaleDma<BM, BN>::NS;               // scale DMA instructions per wave per pair
  using T = Tile<BM, BN, KMap>;

  // A stage's work in items:
  //   read items j < NRD   fragment j (A: j < FM, B: j >= FM), and its scale
  //                        word when the stage is a pair's first;
  //   MFMA items k < NMF   (c, i, j) with k = (c * FM + i) * FN + j, c the
  //                        16-element step in kFp8Bf16 mode (0 in kFp8 mode);
  //   DMA items j < NCI    code rows (A: j < NCA), plus scale chunk j (j < NS).
  static constexpr int NC = ELEM == kFp8 ? 1 : 4;   // MFMAs per fragment pair and stage
  static constexpr int NMF = NC * FM * FN;
  static constexpr int NRD = FM + FN;
  static constexpr int NR = NRD;                   // regions of a stage: one fragment read each

  uint8_t* smem;
  const T& x;
  v4i dA, dB, dS[NS];   // descriptors, built once (scalar registers)

  __device__ __forceinline__ static int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
  // K byte of pair u (pair 0's for pairs past the end: any offset is harmless
  // there, and a grouped K map must not read past its list)
  __device__ __forceinline__ uint32_t kc_of(int u) const { return x.km(u < x.npairs ? u : 0); }

  // DMA item J of pair u into pair slot Q from K byte kc.
  template <int J, int Q>
  __device__ __forceinline__ void issue_item(int u, uint32_t kc) const {
#if defined(__HIP_DEVICE_COMPILE__)
    const bool live = u < x.npairs;
    const int wave = wave_id();
    const uint32_t cs = lds_addr(smem) + Q * CS;
    if (J < NCA) {
      v4i ra = dA;
      ra[2] = live ? ra[2] : 0;
      dma16(ra, cs + uint32_t(wave * (BM / 4) + 8 * J) * PK, x.A.off[J], kc);
    } else {
      v4i rb = dB;
      rb[2] = live ? rb[2] : 0;
      dma16(rb, cs + uint32_t(BM + wave * (BN / 4) + 8 * (J - NCA)) * PK, x.B.off[J - NCA], kc);
    }
    if (J < NS) {
      const uint32_t ss = lds_addr(smem) + NP * CS + Q * SSB;
      v4i rs = dS[J < NS ? J : 0];
      rs[2] = live ? rs[2] : 0;
      dma4(rs, ss + uint32_t(wave + 4 * J) * 256, x.sd.off[J], (kc >> 7) * x.sd.pstride[J]);
    }
#endif
  }

  uint4 fa[2][FM][2], fb[2][FN][2];   // fragments of the two stages of a pair
  uint32_t sa[NP][FM], sb[NP][FN];    // scale words, by pair slot (both stages use them)

  // Read item J of stage parity P from pair slot Q into set P.  Lane half h
  // takes 16-byte chunks h and 2 + h of the stage in each row.  The fp8 MFMA
  // reads them as K positions of its 64-element step; in kFp8Bf16 mode the
  // chunks are the operands of four bf16 steps: chunk h's low and high 8 bytes
  // are this lane half's elements of steps 0 and 1, chunk 2 + h's of steps 2
  // and 3.  A and B are permuted alike, so each step still pairs equal K
  // indices, and a chunk lies inside one 32-element scale group (h: the
  // stage's first group, 2 + h: its second).
  template <int P, int J, int Q>
  __device__ __forceinline__ void read_item() {
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int h = lane >> 5, r = lane & 31;
    const uint8_t* cs = smem + Q * CS;
    const uint8_t* ss = smem + NP * CS + Q * SSB;
    if (J < FM) {
      const int row = (wave >> 1) * (BM / 2) + 32 * J + r;
      fa[P][J][0] = *reinterpret_cast<const uint4*>(cs + row * PK + 16 * ((4 * P + h) ^ swz(row)));
      fa[P][J][1] = *reinterpret_cast<const uint4*>(cs + row * PK + 16 * ((4 * P + 2 + h) ^ swz(row)));
      if (P == 0) sa[Q][J] = *reinterpret_cast<const uint32_t*>(ss + (row >> 6) * 256 + (row & 63) * 4);
    } else {
      constexpr int j = J >= FM ? J - FM : 0;
      const int row = (wave & 1) * (BN / 2) + 32 * j + r;
      fb[P][j][0] = *reinterpret_cast<const uint4*>(cs + (BM + row) * PK + 16 * ((4 * P + h) ^ swz(row)));
      fb[P][j][1] = *reinterpret_cast<const uint4*>(cs + (BM + row) * PK + 16 * ((4 * P + 2 + h) ^ swz(row)));
      const int srow = BM + row;
      if (P == 0) sb[Q][j] = *reinterpret_cast<const uint32_t*>(ss + (srow >> 6) * 256 + (srow & 63) * 4);
    }
  }

  // kFp8Bf16 operand of step c (see gemm_v3.hpp: the exact bf16 values of a
  // fragment's codes times the stage's scale byte)
  template <int F, int P, int C>
  __device__ __forceinline__ static v8bf step_operand(const uint4 (&f)[2], uint32_t sw) {
    return v3::Ring<BM, BN, ELEM, FA, FB, v3::KMapPlain>::template step_operand<F, P, C>(f, sw);
  }

  // MFMA item K of the stage of parity P (scale byte within the pair's word)
  // in pair slot Q
  template <int P, int K, int Q>
  __device__ __forceinline__ void mfma_item(v16f (&acc)[FM][FN]) const {
    constexpr int c = K / (FM * FN), i = (K / FN) % FM, j = K % FN;
    if (ELEM == kFp8Bf16) {
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(step_operand<FA, P, c>(fa[P][i], sa[Q][i]),
                                                          step_operand<FB, P, c>(fb[P][j], sb[Q][j]), acc[i][j], 0,
                                                          0, 0);
    } else {
      const int h = (threadIdx.x & 63) >> 5;
      acc[i][j] = mma<FA, FB, 2 * P>(fa[P][i], fb[P][j], acc[i][j], int(sa[Q][i] >> (8 * h)),
                                     int(sb[Q][j] >> (8 * h)));
    }
  }

  // Pair step u in slot Q (see the top of the file).  kc_next holds the K byte
  // of pair u+1, loaded one step earlier; the K byte of pair u+2 is loaded
  // here (a grouped K map reads it with a scalar load), so that load's latency
  // passes behind this step's MFMAs: the wait before the mid-step barrier
  // covers it, and no wait for it stands at the top of the next step.
  uint32_t kc_next;
  template <int Q>
  __device__ __forceinline__ void pair_step(int u, v16f (&acc)[FM][FN]) {
    constexpr int QN = Q ^ 1;
    const uint32_t kc = kc_next;
    kc_next = kc_of(u + 2);
    v2::static_for<NR>([&](auto R) {
      constexpr int r = R;
      constexpr int j0 = r * NCI / NR, j1 = (r + 1) * NCI / NR;
      v2::static_for<j1 - j0>([&](auto J) { issue_item<j0 + J, QN>(u + 1, kc); });
      read_item<1, r, Q>();
      constexpr int k0 = r * NMF / NR, k1 = (r + 1) * NMF / NR;
      v2::static_for<k1 - k0>([&](auto K) { mfma_item<0, k0 + K, Q>(acc); });
      __builtin_amdgcn_sched_barrier(0);
    });
    v2::static_for<NMF / 2>([&](auto K) { mfma_item<1, K, Q>(acc); });
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt(0, 0));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    v2::static_for<NR>([&](auto R) {
      constexpr int r = R;
      read_item<0, r, QN>();
      constexpr int k0 = NMF / 2 + r * (NMF / 2) / NR, k1 = NMF / 2 + (r + 1) * (NMF / 2) / NR;
      v2::static_for<k1 - k0>([&](auto K) { mfma_item<1, k0 + K, Q>(acc); });
      __builtin_amdgcn_sched_barrier(0);
    });
  }

  // The whole tile: pair 0, then every pair step.  Slots alternate, so the
  // steady state runs two pair steps per iteration with compile-time slots.
  __device__ __forceinline__ void run(v16f (&acc)[FM][FN]) {
#if defined(__HIP_DEVICE_COMPILE__)
    dA = rsrc(x.A.codes);
    dB = rsrc(x.B.codes);
#pragma unroll
    for (int j = 0; j < NS; ++j) dS[j] = rsrc(x.sd.buf[j]);
#endif
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
    const int n = x.npairs;
    kc_next = kc_of(1);
    {
      const uint32_t kc = kc_of(0);
      v2::static_for<NCI>([&](auto J) { issue_item<J, 0>(0, kc); });
    }
    __builtin_amdgcn_s_waitcnt(waitcnt(0, 0));
    __builtin_amdgcn_s_barrier();
    v2::static_for<NRD>([&](auto J) { read_item<0, J, 0>(); });
    int u = 0;
    for (; u + 2 <= n; u += 2) {
      pair_step<0>(u, acc);
      pair_step<1>(u + 1, acc);
    }
    if (u < n) pair_step<0>(u, acc);
  }
};

// One tile per workgroup; npairs = K / 128 bytes.
template <int BM, int BN, int ELEM, int FA, int FB, class KMap>
__device__ __forceinline__ void mainloop(const Op<BM>& A, const Op<BN>& B, const ScaleDma<BM, BN>* sd, int npairs,
                                         const KMap& kmap, uint8_t* smem, v16f (&acc)[BM / 64][BN / 64]) {
  const Tile<BM, BN, KMap> tile{A, B, *sd, kmap, npairs};
  Ring<BM, BN, ELEM, FA, FB, KMap> ring{smem, tile};
  ring.run(acc);
  // the look-ahead loads past the end still write (zeros) into the ring: let
  // them land before the caller reuses the LDS
  __builtin_amdgcn_s_waitcnt(waitcnt(0, 15));
}

}  // namespace v4
}  // namespace mx
