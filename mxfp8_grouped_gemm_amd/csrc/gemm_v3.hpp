// gemm_v3.hpp -- MX GEMM main loop for gfx950 with a four-stage LDS ring.
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
// Why a ring: a stage can only start when the slowest of its ~500 cache lines
// has landed, and a few percent of them miss L2.  With one stage in flight the
// loop runs at that miss latency; with three it runs near the stream rate (a
// fifth slot measured no faster).  The stream rate goes by cache lines: a CU
// moves about 66 B/clk of L2-resident whole lines with buffer_load ... lds but
// about 34 B/clk when every row gives half a line, hence the stage-major
// operand layout (see Op).
//
// Stage = 64 bytes of K (one 64-element fp8 MFMA step, two 16-element bf16
// steps).  LDS: NBUF code slots of (BM + BN) rows x 64 B (16-byte chunks
// XOR-swizzled by row so that 16 consecutive rows reading one logical chunk
// hit distinct banks, see swz), then NBUF scale slots holding, for a pair of
// stages, one 4-byte word per row (the pair's four E8M0 groups), loaded from
// pair-major scale arrays (see ScaleDma).
//
// Loads are issued with inline asm (s_mov_b32 m0 + buffer_load_dword{,x4} ...
// lds) because the compiler's wait-count pass treats every LDS read after an
// LDS DMA builtin as possibly aliased and waits for all outstanding loads,
// which would serialise the ring.  The asm loads are invisible to that pass;
// the loop waits on them explicitly (vmcnt) and they only ever write LDS.
// The asm sets m0 itself; m0 is reserved (not allocatable), and code built on
// this core has no other m0 users, so no compiler value lives there across it.
//
// Iteration t (fragments of stage t already in registers F[t & 1]):
//   wait until stage t+1 has landed (loads of t+2 and t+3 may remain), barrier
//     (also: every wave has finished reading stage t's slot);
//   DMA stage t+4 into slot (t+4) % 4 == t % 4 (and the scales of pair
//     (t+4)/2 when t+4 is even);
//   MFMAs of stage t from F[t & 1], interleaved with the reads of stage t+1
//     into F[(t+1) & 1].
// The iteration is straight-line code (no branch for the ring's tail), so the
// compiler keeps this order.
#pragma once
#include "gemm_v2.hpp"
#include "mx_device.hpp"

namespace mx {
namespace v3 {

using v2::Buf;
using v2::v16f;
using v2::v8bf;
using v2::v8i;
using v2::kFp8;
using v2::kFp8Bf16;

constexpr int SK = 64;          // bytes of K per stage
constexpr int NBUF = 4;         // ring depth (stages in LDS)
constexpr int kThreads = 256;
constexpr uint32_t kOOB = 0x80000000u;

typedef int v4i __attribute__((ext_vector_type(4)));

// LDS bytes of a tile's ring.
__host__ __device__ constexpr int code_slot(int BM, int BN) { return (BM + BN) * SK; }
__host__ __device__ constexpr int scale_chunks(int BM, int BN) { return 4 * ((BM + BN + 255) / 256); }
__host__ __device__ constexpr int scale_slot(int BM, int BN) { return scale_chunks(BM, BN) * 256; }
__host__ __device__ constexpr int smem_bytes(int BM, int BN) { return NBUF * (code_slot(BM, BN) + scale_slot(BM, BN)); }

// s_waitcnt immediate: vmcnt(vm) lgkmcnt(lgkm), expcnt left alone.
__host__ __device__ constexpr int waitcnt(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8);
}

#if defined(__HIP_DEVICE_COMPILE__)
__device__ __forceinline__ v4i rsrc(const Buf& b) {
  const uint64_t a = reinterpret_cast<uint64_t>(b.base);
  v4i r;
  r[0] = int(__builtin_amdgcn_readfirstlane(uint32_t(a)));
  r[1] = int(__builtin_amdgcn_readfirstlane(uint32_t(a >> 32) & 0xffffu));   // stride 0
  r[2] = int(__builtin_amdgcn_readfirstlane(b.bytes));
  r[3] = 0x00020000;
  return r;
}
// 16 bytes per lane into LDS at m0 + 16 * lane.
__device__ __forceinline__ void dma16(const v4i& rs, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rs),
                 "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory");
}
// 4 bytes per lane into LDS at m0 + 4 * lane.
__device__ __forceinline__ void dma4(const v4i& rs, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rs),
                 "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory");
}
#endif

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>(p));   // low half of the generic address = LDS offset
}

// One operand's code rows: buffer and this lane's DMA offsets.  Instruction j
// of wave w fills rows w*ROWS/4 + 16j .. +16 of a slot; lane l fills row
// +(l >> 2), physical chunk l & 3, fetching the logical chunk stored there.
// Two code layouts of an operand with R rows contracted over K bytes:
//   row-major    [R][K] (kmul == 1): the lane offsets point at K byte 0 of
//                their rows and a position's K byte kc is the scalar offset;
//   stage-major  panels of 256 rows, each [K/64][rows][64] (see
//                stage_major_off; kmul == the tile's panel's rows): the lane
//                offsets are row * 64 within the panel's first stage, and the
//                scalar offset kc * kmul moves them to stage kc / 64.
// Why stage-major: one DMA instruction then reads 1 KB of consecutive bytes,
// 8 whole 128-byte lines, where 16 rows x 64 bytes of a row-major operand are
// 16 half lines; the texture path's throughput goes by lines, not bytes
// (measured on gfx950 with L2-resident data: ~34 B/clk per CU with 64-byte
// pieces of rows, ~66 B/clk with whole lines).
template <int ROWS>
struct Op {
  Buf codes;
  uint32_t off[ROWS / 64];
  uint32_t kmul;   // scalar offset of K byte kc: kc * kmul
};

template <int ROWS>
__device__ __forceinline__ int dma_row(int j) {
  return (threadIdx.x >> 6) * (ROWS / 4) + 16 * j + ((threadIdx.x & 63) >> 2);
}
// Physical 16-byte chunk of logical chunk c in row `row` is c ^ swz(row).  A
// fragment read has lanes r and 32 + r on row r (chunks h and 2 + h for lane
// half h).  LDS serves a 16-byte read at 256 B per clock, and the swizzle was
// chosen by measurement (rocprofv3 SQ_LDS_BANK_CONFLICT over the exact
// fragment access pattern): XOR with row bits 2-3 reads both chunk pairs in
// 4 clocks per instruction with no conflict cycles, like contiguous data,
// while any swizzle that also depends on row bit 1 or bit 4 costs a 2-way
// conflict (8 clocks).  Rows 32 apart share a swizzle.
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

template <int ROWS>
__device__ __forceinline__ void setup_rows(Op<ROWS>& op, const uint8_t* codes, int64_t row0, int64_t nrows,
                                           int64_t ld) {
  const int64_t have = nrows - row0 < ROWS ? nrows - row0 : ROWS;
  op.codes = v2::make_rsrc(codes + row0 * ld, uint32_t(have * ld));
  op.kmul = 1;
#pragma unroll
  for (int j = 0; j < ROWS / 64; ++j) {
    const int r = dma_row<ROWS>(j);
    const int lc = (threadIdx.x & 3) ^ swz(r);
    op.off[j] = r < have ? uint32_t(r * ld + 16 * lc) : kOOB;
  }
}

// Stage-major codes (see Op) of an operand with R rows and K bytes: the
// tile's rows row0 .. (a multiple of ROWS, so they lie in one panel) of the
// rows below `limit` (<= R; rows from there on load zeros).  The descriptor
// covers the panel from the tile's first row on.
template <int ROWS>
__device__ __forceinline__ void setup_rows_sm(Op<ROWS>& op, const uint8_t* codes, int64_t row0, int64_t limit,
                                              int64_t R, int64_t K) {
  static_assert(kPanelRows % ROWS == 0, "a tile lies in one panel");
  const int64_t have = limit - row0 < ROWS ? limit - row0 : ROWS;
  const int64_t p0 = row0 & ~int64_t(kPanelRows - 1);
  const int64_t rp = R - p0 < kPanelRows ? R - p0 : kPanelRows;
  const int64_t skip = (row0 - p0) * SK;
  op.codes = v2::make_rsrc(codes + p0 * K + skip, uint32_t(rp * K - skip));
  op.kmul = uint32_t(rp);
#pragma unroll
  for (int j = 0; j < ROWS / 64; ++j) {
    const int r = dma_row<ROWS>(j);
    const int lc = (threadIdx.x & 3) ^ swz(r);
    op.off[j] = r < have ? uint32_t(r * SK + 16 * lc) : kOOB;
  }
}

// Gathered rows: tile row r reads source row rowid(r) (negative: zeros).
template <int ROWS, class RowId>
__device__ __forceinline__ void setup_gather(Op<ROWS>& op, const uint8_t* codes, int64_t src_rows, int64_t ld,
                                             const RowId& rowid) {
  op.codes = v2::make_rsrc(codes, uint32_t(src_rows * ld));
  op.kmul = 1;
#pragma unroll
  for (int j = 0; j < ROWS / 64; ++j) {
    const int r = dma_row<ROWS>(j);
    const int64_t t = rowid(r);
    const int lc = (threadIdx.x & 3) ^ swz(r);
    op.off[j] = t >= 0 ? uint32_t(t * ld + 16 * lc) : kOOB;
  }
}

// Scale words of both operands.  Scales of an operand with R rows and K
// contraction elements are stored pair-major, [K/128][R][4]: word (p, r) holds
// the four E8M0 bytes of row r for K elements [128p, 128p + 128), so the words
// of a stage pair for consecutive rows are contiguous.  They are loaded in
// 64-row chunks: chunk c (A rows first, then B rows) by wave c % 4 as its
// instruction c / 4, one 4-byte word per lane at (row0 + row) * 4 plus the
// pair's offset p * R * 4; chunks past the tile's rows load zeros into the
// slot's tail so every wave issues the same number of instructions.
template <int BM, int BN>
struct ScaleDma {
  static constexpr int NS = scale_chunks(BM, BN) / 4;
  Buf buf[NS];
  uint32_t off[NS];       // this lane's row word (or out of range)
  uint32_t pstride[NS];   // bytes per pair (R * 4) of the operand the chunk belongs to
};

// a_scales / b_scales: pair-major scale arrays of the whole operands (a_rows /
// b_rows rows, a_bytes / b_bytes bytes); tile row r of A reads scale row
// a_row(r), of B b_row(r) (negative: zeros).
template <int BM, int BN, class ARow, class BRow>
__device__ __forceinline__ void setup_scales_map(ScaleDma<BM, BN>& sd, const uint8_t* a_scales, int64_t a_rows,
                                                 int64_t a_bytes, const ARow& a_row, const uint8_t* b_scales,
                                                 int64_t b_rows, int64_t b_bytes, const BRow& b_row) {
  // wave-uniform chunk choice: descriptors and strides stay in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const Buf ba = v2::make_rsrc(a_scales, uint32_t(a_bytes));
  const Buf bb = v2::make_rsrc(b_scales, uint32_t(b_bytes));
#pragma unroll
  for (int i = 0; i < ScaleDma<BM, BN>::NS; ++i) {
    const int c = wave + 4 * i;
    if (c < BM / 64) {
      const int64_t r = a_row(64 * c + lane);
      sd.buf[i] = ba;
      sd.off[i] = r >= 0 ? uint32_t(r * 4) : kOOB;
      sd.pstride[i] = uint32_t(a_rows * 4);
    } else if (c < (BM + BN) / 64) {
      const int64_t r = b_row(64 * (c - BM / 64) + lane);
      sd.buf[i] = bb;
      sd.off[i] = r >= 0 ? uint32_t(r * 4) : kOOB;
      sd.pstride[i] = uint32_t(b_rows * 4);
    } else {
      sd.buf[i] = ba;
      sd.off[i] = kOOB;
      sd.pstride[i] = 0;
    }
  }
}

// Both operands as contiguous row ranges: the tile covers rows a_row0.. / b_row0..
template <int BM, int BN>
__device__ __forceinline__ void setup_scales(ScaleDma<BM, BN>& sd, const uint8_t* a_scales, int64_t a_row0,
                                             int64_t a_rows, int64_t a_bytes, const uint8_t* b_scales,
                                             int64_t b_row0, int64_t b_rows, int64_t b_bytes) {
  setup_scales_map(
      sd, a_scales, a_rows, a_bytes, [&](int r) -> int64_t { return a_row0 + r < a_rows ? a_row0 + r : -1; },
      b_scales, b_rows, b_bytes, [&](int r) -> int64_t { return b_row0 + r < b_rows ? b_row0 + r : -1; });
}

// K map with 64-byte stages.  Plain: [0, K).  Grouped: the K columns of a
// group are the blocks list[b0 ..] of blk columns each (blk a power of two >=
// 128, so a scale word never straddles two blocks).
struct KMapPlain {
  __device__ __forceinline__ uint32_t operator()(int s) const { return uint32_t(s) * SK; }
};
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
struct KMapList {
  const int32_t* list;
  int b0, blk, shift;   // shift = log2(blk / 64)
  __device__ __forceinline__ uint32_t operator()(int s) const {
    const int blkid = ((const_i32_ptr)(uintptr_t)list)[b0 + (s >> shift)];
    return uint32_t(blkid) * uint32_t(blk) + uint32_t(s & ((1 << shift) - 1)) * SK;
  }
};

// One scaled fp8 MFMA (32 x 32 x 64); OPS selects the scale byte of the
// operands' words (2 * stage parity; lane half h's word is pre-shifted by h bytes).
template <int FA, int FB, int OPS>
__device__ __forceinline__ v16f mma(const uint4 (&a)[2], const uint4 (&b)[2], const v16f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v2::as_v8i(a[0], a[1]), v2::as_v8i(b[0], b[1]), c, FA, FB,
                                                         OPS, sa, OPS, sb);
}

// One tile's operands: code rows of A and B, their scale rows (fp8 mode), the
// K map and the number of 64-byte stages (even: K is a multiple of 128 bytes).
template <int BM, int BN, class KMap>
struct Tile {
  Op<BM> A;
  Op<BN> B;
  ScaleDma<BM, BN> sd;
  KMap km;
  int nstages;
};

// The ring of one tile: stage t lives in code slot t % NBUF; an even stage's
// scale slot t % NBUF holds its pair's scale words (one 4-byte word per row
// covering K elements [128p, 128p + 128)), which the odd stage reuses from
// registers (loading them for both stages kept the texture addresser busier
// on the address-bound Phases 3 and 4).  Loads are
// issued NBUF stages ahead of use: after the prologue (positions 0 .. NBUF-1),
// step t issues position t + NBUF into stage t's slot once every wave has read
// that slot.  Positions past the last stage load through descriptors with no
// records, which the hardware answers with zeros without touching memory, so
// every step issues the same loads and the wait counts are fixed.
//
// The steady state runs NBUF stages per iteration, so every slot index, and
// with it every LDS address, is a compile-time constant there; the last
// stages (2 to 6; K is a multiple of 128 bytes, so the count is even) run with
// run-time slots.  The kernels here run one tile per workgroup: chaining tiles
// through the ring in a persistent grid was measured slower (at 256 VGPRs the
// next tile's descriptors spill, and the reloads' waits drain the ring at
// every tile boundary).
template <int BM, int BN, int ELEM, int FA, int FB, class KMap>
struct Ring {
  static constexpr int FM = BM / 64, FN = BN / 64;
  static constexpr int CS = code_slot(BM, BN), SSB = scale_slot(BM, BN);
  static constexpr int NCI = (BM + BN) / 64;               // code DMA instructions per wave per stage
  static constexpr int NS = ScaleDma<BM, BN>::NS;          // scale DMA instructions per wave per stage
  // DMA instructions per wave of a position: NCI code rows, plus NS scale
  // chunks at even positions.  Wait counts: a position has landed once at
  // most the loads of the positions issued after it remain, i.e. of the next
  // two (one even, one odd) in a step, of the next three (one even) after the
  // prologue.
  static constexpr int VM_2AFTER = 2 * NCI + NS;
  static constexpr int VM_3AFTER = 3 * NCI + NS;
  using T = Tile<BM, BN, KMap>;

  uint8_t* smem;
  const T& x;
  v4i dA, dB, dS[NS];   // descriptors, built once (scalar registers)

  // A stage's work in items, so a stage can be laid out as regions that each
  // issue one DMA instruction and read one fragment for the next stage ahead
  // of a share of the MFMAs (the MFMA pipe keeps running while those issue):
  //   DMA items j < NCI      code rows (A: j < FM, B: j >= FM), plus scale
  //                          chunk j (j < NS);
  //   read items j < FM + FN fragment j (A: j < FM, B: j >= FM) and its scale word;
  //   MFMA items k < NMF     (c, i, j) with k = (c * FM + i) * FN + j, c the
  //                          16-element step in kFp8Bf16 mode (0 in kFp8 mode).
  static constexpr int NC = ELEM == kFp8 ? 1 : 4;   // MFMAs per fragment pair and stage
  static constexpr int NMF = NC * FM * FN;
  static constexpr int NR = FM + FN;               // regions of a stage (== NCI)
  static_assert(NR == NCI, "one code DMA instruction per region");

  // slot of stage t: S when the caller knows it (S >= 0), else t % NBUF
  template <int S>
  __device__ __forceinline__ static uint32_t slot_of(int t) {
    return S >= 0 ? uint32_t(S) : uint32_t(t) & (NBUF - 1);
  }
  __device__ __forceinline__ static int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

  // K byte of position pos (stage 0's for positions past the end: any offset
  // is harmless there, and a grouped K map must not read past its list)
  __device__ __forceinline__ uint32_t kc_of(int pos) const { return x.km(pos < x.nstages ? pos : 0); }

  // DMA item J of position pos (slot of stage S, see slot_of) from K byte kc.
  template <int J, int S>
  __device__ __forceinline__ void issue_item(int pos, uint32_t kc) const {
#if defined(__HIP_DEVICE_COMPILE__)
    const bool live = pos < x.nstages;
    const int wave = wave_id();
    const uint32_t slot = slot_of<S>(pos);
    const uint32_t cs = lds_addr(smem) + slot * CS;
    if (J < FM) {
      v4i ra = dA;
      ra[2] = live ? ra[2] : 0;
      dma16(ra, cs + uint32_t(wave * (BM / 4) + 16 * J) * SK, x.A.off[J], kc * x.A.kmul);
    } else {
      v4i rb = dB;
      rb[2] = live ? rb[2] : 0;
      dma16(rb, cs + uint32_t(BM + wave * (BN / 4) + 16 * (J - FM)) * SK, x.B.off[J - FM], kc * x.B.kmul);
    }
    // a pair's scale words go with its first (even) stage only: the odd stage
    // takes them from the registers its even stage read them into (read_item)
    if (J < NS && (S >= 0 ? (S & 1) == 0 : (pos & 1) == 0)) {
      const uint32_t ss = lds_addr(smem) + NBUF * CS + slot * SSB;
      v4i rs = dS[J < NS ? J : 0];
      rs[2] = live ? rs[2] : 0;
      dma4(rs, ss + uint32_t(wave + 4 * J) * 256, x.sd.off[J], (kc >> 7) * x.sd.pstride[J]);
    }
#endif
  }
  template <int S>
  __device__ __forceinline__ void issue(int pos) const {
    const uint32_t kc = kc_of(pos);
    v2::static_for<NCI>([&](auto J) { issue_item<J, S>(pos, kc); });
  }

  uint4 fa[2][FM][2], fb[2][FN][2];
  uint32_t sa[2][FM], sb[2][FN];

  // Read item J of stage t (slot S, see slot_of) into set P: fragment J's two
  // 16-byte chunks and its raw scale word (shifted to this lane's group where it
  // is used, so nothing here waits on the reads).
  // Lane half h takes 16-byte chunks h and 2 + h of each row.  The fp8 MFMA
  // reads them as K positions of its 64-element step; in kFp8Bf16 mode the
  // chunks are the operands of four bf16 steps: chunk h's low and high 8 bytes
  // are this lane half's elements of steps 0 and 1, chunk 2 + h's of steps 2
  // and 3.  A and B are permuted alike, so each step still pairs equal K
  // indices, and a chunk lies inside one 32-element scale group (h: the
  // stage's first group, 2 + h: its second).  Rows 32 apart share a swizzle,
  // so a wave's fragments differ by constant offsets.
  template <int P, int J, int S>
  __device__ __forceinline__ void read_item(int t) {
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int h = lane >> 5, r = lane & 31;
    const uint32_t slot = slot_of<S>(t);
    const uint8_t* cs = smem + slot * CS;
    const uint8_t* ss = smem + NBUF * CS + slot * SSB;
    if (J < FM) {
      const int row = (wave >> 1) * (BM / 2) + 32 * J + r;
      fa[P][J][0] = *reinterpret_cast<const uint4*>(cs + row * SK + 16 * (h ^ swz(row)));
      fa[P][J][1] = *reinterpret_cast<const uint4*>(cs + row * SK + 16 * ((2 + h) ^ swz(row)));
      // stage parity P: the odd stage's pair word is its even stage's, in set 0
      if (P == 0) sa[P][J] = *reinterpret_cast<const uint32_t*>(ss + (row >> 6) * 256 + (row & 63) * 4);
      else sa[P][J] = sa[0][J];
    } else {
      constexpr int j = J - FM;
      const int row = (wave & 1) * (BN / 2) + 32 * j + r;
      fb[P][j][0] = *reinterpret_cast<const uint4*>(cs + (BM + row) * SK + 16 * (h ^ swz(row)));
      fb[P][j][1] = *reinterpret_cast<const uint4*>(cs + (BM + row) * SK + 16 * ((2 + h) ^ swz(row)));
      const int srow = BM + row;
      if (P == 0) sb[P][j] = *reinterpret_cast<const uint32_t*>(ss + (srow >> 6) * 256 + (srow & 63) * 4);
      else sb[P][j] = sb[0][j];
    }
  }

  // kFp8Bf16: the exact bf16 values of 8 codes (one 16-element step of a lane)
  // with E8M0 scale byte sc.  The converter takes the exponent field of its
  // fp32 scale operand as the E8M0 byte (2^(sc - 127), byte 0 included: the
  // float 0.0 scales by 2^-127), so the byte shifted into that field is the
  // operand.  Checked exhaustively: every code of both formats times every
  // scale byte 0..254 gives the exact product rounded to bf16.
  template <int F>
  __device__ __forceinline__ static v8bf to_bf16(uint32_t w0, uint32_t w1, uint32_t sc) {
    const float s = __uint_as_float(sc << 23);
    typedef uint32_t u4v __attribute__((ext_vector_type(4)));
    auto cv = [&](uint32_t w, auto HI) -> uint32_t {
      if (F == 0) return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, s, decltype(HI)::value));
      return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, s, decltype(HI)::value));
    };
    return __builtin_bit_cast(v8bf, u4v{cv(w0, std::false_type{}), cv(w0, std::true_type{}), cv(w1, std::false_type{}),
                                        cv(w1, std::true_type{})});
  }
  // operand of step c from a fragment and its scale word (stage parity P picks
  // the pair's group: bytes 2P and 2P + 1)
  template <int F, int P, int C>
  __device__ __forceinline__ static v8bf step_operand(const uint4 (&f)[2], uint32_t sw) {
    const uint4& x = f[C >> 1];
    return to_bf16<F>((C & 1) ? x.z : x.x, (C & 1) ? x.w : x.y, (sw >> (8 * (2 * P + (C >> 1)))) & 0xffu);
  }

  // MFMA item K of the stage in set P (stage parity P = scale byte within the pair)
  template <int P, int K>
  __device__ __forceinline__ void mfma_item(v16f (&acc)[FM][FN]) const {
    constexpr int c = K / (FM * FN), i = (K / FN) % FM, j = K % FN;
    if (ELEM == kFp8Bf16) {
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(step_operand<FA, P, c>(fa[P][i], sa[P][i]),
                                                          step_operand<FB, P, c>(fb[P][j], sb[P][j]), acc[i][j], 0,
                                                          0, 0);
    } else {
      const int h = (threadIdx.x & 63) >> 5;
      acc[i][j] = mma<FA, FB, 2 * P>(fa[P][i], fb[P][j], acc[i][j], int(sa[P][i] >> (8 * h)),
                                     int(sb[P][j] >> (8 * h)));
    }
  }

  // One stage t (fragments in set P == t & 1, slot S, see slot_of).  With READ:
  // wait until stage t+1 has landed (t+2, t+3 may still be in flight) and every
  // wave has finished reading stage t's slot (barrier), then NR regions, region
  // q issuing DMA item q of position t + NBUF and read item q of stage t+1
  // (into set P ^ 1) before its share of stage t's MFMAs.  Each region is
  // fenced, so the memory instructions issue between MFMAs, which keep
  // executing meanwhile.  The K byte comes first: a grouped K map reads it with
  // a scalar load, which the wait below covers (inside the regions its wait
  // would also drain the fragment reads).  Without READ: the tile's last stage.
  template <int P, int S, bool READ>
  __device__ __forceinline__ void step(int t, v16f (&acc)[FM][FN]) {
    constexpr int SN = S >= 0 ? (S + 1) % NBUF : -1;   // slot of stage t + 1
    if (READ) {
      const uint32_t kc = kc_of(t + NBUF);
      __builtin_amdgcn_s_waitcnt(waitcnt(VM_2AFTER, 0));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      v2::static_for<NR>([&](auto Q) {
        constexpr int q = Q;
        issue_item<q, S>(t + NBUF, kc);
        read_item<P ^ 1, q, SN>(t + 1);
        constexpr int k0 = q * NMF / NR, k1 = (q + 1) * NMF / NR;
        v2::static_for<k1 - k0>([&](auto K) { mfma_item<P, k0 + K>(acc); });
        __builtin_amdgcn_sched_barrier(0);
      });
    } else {
      v2::static_for<NMF>([&](auto K) { mfma_item<P, K>(acc); });
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // The whole tile: positions 0 .. NBUF-1, then every stage.
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
    const int n = x.nstages;
    issue<0>(0);
    issue<1>(1);
    issue<2>(2);
    issue<3>(3);
    // stage 0 has landed once at most the three later positions' loads remain
    __builtin_amdgcn_s_waitcnt(waitcnt(VM_3AFTER, 0));
    __builtin_amdgcn_s_barrier();
    v2::static_for<NR>([&](auto J) { read_item<0, J, 0>(0); });
    int t = 0;
    // steady state: positions t + NBUF .. t + 2 NBUF - 1 all inside the tile
    for (; t + 2 * NBUF - 1 < n; t += NBUF) {
      step<0, 0, true>(t, acc);
      step<1, 1, true>(t + 1, acc);
      step<0, 2, true>(t + 2, acc);
      step<1, 3, true>(t + 3, acc);
    }
    // the last stages (n - t is 2, 4 or 6)
    for (; t + 2 < n; t += 2) {
      step<0, -1, true>(t, acc);
      step<1, -1, true>(t + 1, acc);
    }
    step<0, -1, true>(t, acc);
    step<1, -1, false>(t + 1, acc);
  }
};

// One tile per workgroup.
template <int BM, int BN, int ELEM, int FA, int FB, class KMap>
__device__ __forceinline__ void mainloop(const Op<BM>& A, const Op<BN>& B, const ScaleDma<BM, BN>* sd, int nstages,
                                         const KMap& kmap, uint8_t* smem, v16f (&acc)[BM / 64][BN / 64]) {
  const Tile<BM, BN, KMap> tile{A, B, *sd, kmap, nstages};
  Ring<BM, BN, ELEM, FA, FB, KMap> ring{smem, tile};
  ring.run(acc);
  // the look-ahead loads past the end still write (zeros) into the ring: let
  // them land before the caller reuses the LDS
  __builtin_amdgcn_s_waitcnt(waitcnt(0, 15));
}

}  // namespace v3
}  // namespace mx
