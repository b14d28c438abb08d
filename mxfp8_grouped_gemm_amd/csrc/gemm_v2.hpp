// gemm_v2.hpp -- MX GEMM main loop for gfx950 with direct-to-LDS loads.
//
// C[m][n] = sum_k A[m][k] * B[n][k] over K-contiguous operands, in one of two
// element modes:
//   kFp8 : fp8 codes + one E8M0 byte per 32 elements along K, reduced with
//          v_mfma_scale_f32_32x32x64_f8f6f4 (the MX GEMM of P1 / P2);
//   kBf16: bf16 operands (exactly dequantised MX values), reduced with
//          v_mfma_f32_32x32x16_bf16, whose accumulation is fp32-exact -- used
//          where the result is requantised (the Phase-1 epilogue).
//
// Tile: BM x BN (128 or 256), 4 waves as 2 x 2, wave tile (BM/2) x (BN/2) in
// 32x32 fragments.  K advances 128 bytes per stage through two LDS buffers.
// Loads go global -> LDS with buffer_load_dwordx4 ... lds: a wave instruction
// fills 8 rows x 128 B; lane l fills row (l >> 3) of its group, LDS chunk
// (l & 7), and fetches the logical chunk that the XOR swizzle maps there.
// A row outside the operand (or a padding slot) gets an offset beyond the
// buffer's num_records, which the hardware returns as zeros.
//
// Per stage: wait for this stage's DMA + barrier; read every fragment of the
// stage into registers; then issue the next stage's DMA (so the compiler never
// has to wait on it before a read); then the MFMAs, overlapping the DMA.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace mx {
namespace v2 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kFp8 = 0;
constexpr int kBf16 = 1;
constexpr int kFp8Bf16 = 2;   // fp8 codes + scales in memory, exact bf16 values on the MFMA (ring loop only)
constexpr int BK = 128;         // bytes of K per stage
constexpr int kThreads = 256;
constexpr uint32_t kOOB = 0x80000000u;   // offset returned as zeros (>= num_records)

#define MX_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// A buffer: base address and size in bytes; the hardware descriptor is built
// where it is used (device code only).
struct Buf {
  const uint8_t* base;
  uint32_t bytes;
};

__device__ __forceinline__ int lds_off(int r, int c) { return r * BK + ((c ^ ((r >> 1) & 7)) << 4); }

__device__ __forceinline__ Buf make_rsrc(const void* base, uint32_t bytes) {
  return Buf{static_cast<const uint8_t*>(base), bytes};
}

#if defined(__HIP_DEVICE_COMPILE__)
// The descriptor must live in scalar registers: make its fields provably uniform.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t to_rsrc(const Buf& b) {
  const uint64_t a = reinterpret_cast<uint64_t>(b.base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(a >> 32));
  void* base = reinterpret_cast<void*>((uint64_t(hi) << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, __builtin_amdgcn_readfirstlane(b.bytes), 0x00020000);
}
#define MX_RSRC(b) to_rsrc(b)
#endif

// One operand of a tile: the buffer over its codes, this lane's DMA row
// offsets (row * ld + 16 * logical chunk) and, in fp8 mode, the buffer over
// its scales and this lane's fragment scale-row offsets.
template <int ROWS, int F>
struct Operand {
  static constexpr int NI = ROWS / 32;   // DMA instructions per wave per stage (8 rows each, 4 waves)
  Buf codes;
  Buf scales;
  uint32_t off[NI];
  uint32_t soff[F];
};

// Lane's DMA rows: wave w handles rows [w*ROWS/4, (w+1)*ROWS/4); instruction j
// covers rows w*ROWS/4 + 8j .. +8; lane l -> row +(l>>3), physical chunk l&7.
template <int ROWS>
__device__ __forceinline__ int dma_row(int j) {
  return (threadIdx.x >> 6) * (ROWS / 4) + 8 * j + ((threadIdx.x & 63) >> 3);
}
template <int ROWS>
__device__ __forceinline__ int dma_chunk(int j) {
  const int r = dma_row<ROWS>(j);
  return (threadIdx.x & 7) ^ ((r >> 1) & 7);      // logical chunk stored at physical (l & 7)
}

template <bool GENERIC, int ROWS, int F>
__device__ __forceinline__ void dma_stage(const Operand<ROWS, F>& op, uint8_t* lds_tile, uint32_t kcol, int kvalid) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NI = ROWS / 32;
  const int wave = threadIdx.x >> 6;
  const auto rs = MX_RSRC(op.codes);
  kcol = __builtin_amdgcn_readfirstlane(kcol);
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    uint32_t o = op.off[j];
    if (GENERIC && kvalid < BK && dma_chunk<ROWS>(j) * 16 >= kvalid) o = kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, MX_LDS(lds_tile + (wave * (ROWS / 4) + 8 * j) * BK), 16, o, kcol, 0,
                                             0);
  }
#endif
}

// fp8 mode: per fragment, the stage's 4 scale bytes [g0 g1 g2 g3] of its row
// (raw: the consumer shifts them by 8*h so opsel 0 / 2 give g_h / g_{2+h}, the
// groups lane half h supplies for the two 64-element steps -- shifting here
// would force a wait on the loads right after issuing them).
// GENERIC: scale rows may be unaligned or the stage may straddle the end of
// K (byte loads, groups past K read as 0); otherwise one dword per fragment.
template <bool GENERIC, int ROWS, int F>
__device__ __forceinline__ void load_scales(const Operand<ROWS, F>& op, uint32_t kcol, int kvalid,
                                            uint32_t (&reg)[F]) {
#if defined(__HIP_DEVICE_COMPILE__)
  const auto rs = MX_RSRC(op.scales);
  const uint32_t sk = __builtin_amdgcn_readfirstlane(kcol >> 5);
#pragma unroll
  for (int f = 0; f < F; ++f) {
    uint32_t s;
    if (!GENERIC) {
      s = __builtin_amdgcn_raw_buffer_load_b32(rs, op.soff[f], sk, 0);
    } else {
      s = 0;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        if (g * 32 < kvalid)
          s |= uint32_t(__builtin_amdgcn_raw_buffer_load_b8(rs, op.soff[f] + g, sk, 0)) << (8 * g);
    }
    reg[f] = s;
  }
#endif
}

template <int FA, int FB, int OPS>
__device__ __forceinline__ v16f mfma_fp8(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, OPS, sa, OPS, sb);
}

// Read all fragments a lane needs for one stage.
//   fp8 : frag[f][ks] = chunks (4ks + h, 4ks + 2 + h)  (split-16 MX layout)
//   bf16: frag[f][t]  = chunk 2t + h for t = 0..3        (8 bf16, K = 16 per step)
template <int ELEM>
__device__ __forceinline__ void read_frag(const uint8_t* tile, int row, int h, uint4 (&v)[4]) {
  if (ELEM == kFp8) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v[2 * ks] = *reinterpret_cast<const uint4*>(tile + lds_off(row, 4 * ks + h));
      v[2 * ks + 1] = *reinterpret_cast<const uint4*>(tile + lds_off(row, 4 * ks + 2 + h));
    }
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) v[t] = *reinterpret_cast<const uint4*>(tile + lds_off(row, 2 * t + h));
  }
}

__device__ __forceinline__ v8i as_v8i(const uint4& lo, const uint4& hi) {
  v8i r;
  r[0] = int(lo.x); r[1] = int(lo.y); r[2] = int(lo.z); r[3] = int(lo.w);
  r[4] = int(hi.x); r[5] = int(hi.y); r[6] = int(hi.z); r[7] = int(hi.w);
  return r;
}
// K map over one contiguous byte range [0, K): stage s covers bytes s*BK ..,
// the last one possibly ragged.
struct KMapPlain {
  int64_t K;   // bytes
  __device__ __forceinline__ void operator()(int s, uint32_t& kc, int& kv) const {
    kc = uint32_t(int64_t(s) * v2::BK);
    const int64_t rem = K - int64_t(kc);
    kv = rem < v2::BK ? int(rem) : v2::BK;
  }
};

__device__ __forceinline__ v8bf as_v8bf(const uint4& v) {
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(v8bf, u4v{v.x, v.y, v.z, v.w});
}

// The K loop.  kmap(s, kcol, kvalid): byte column of stage s (the same in
// both operands) and how many of its 128 bytes lie inside K.
// GENERIC selects the slower handling of unaligned scale rows / a ragged end
// of K; the common case (every stage full, scale rows 4-byte aligned) has none.
template <int BM, int BN, int ELEM, int FA, int FB, bool GENERIC, class KMap>
__device__ __forceinline__ void mainloop(const Operand<BM, BM / 64>& A, const Operand<BN, BN / 64>& B, int nstages,
                                         const KMap& kmap, uint8_t* smem, v16f (&acc)[BM / 64][BN / 64]) {
  constexpr int FM = BM / 64, FN = BN / 64;
  constexpr int STAGE = (BM + BN) * BK;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, r = lane & 31;
  const int wrow = (wave >> 1) * (BM / 2);
  const int wcol = (wave & 1) * (BN / 2);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
  if (nstages <= 0) return;

  uint32_t sa_next[FM], sb_next[FN];
  uint32_t kc_next = 0;     // K column of the stage after the one being loaded (fetched one stage early)
  int kv_next = BK;
  {
    uint32_t kc;
    int kv;
    kmap(0, kc, kv);
    dma_stage<GENERIC>(A, smem, kc, kv);
    dma_stage<GENERIC>(B, smem + BM * BK, kc, kv);
    if (ELEM == kFp8) {
      load_scales<GENERIC>(A, kc, kv, sa_next);
      load_scales<GENERIC>(B, kc, kv, sb_next);
    }
    if (nstages > 1) kmap(1, kc_next, kv_next);
  }
  for (int s = 0; s < nstages; ++s) {
    uint8_t* cur = smem + (s & 1) * STAGE;
    uint8_t* nxt = smem + ((s + 1) & 1) * STAGE;
    __builtin_amdgcn_s_waitcnt(0x3f70);   // vmcnt(0): this stage's DMA and scale loads have landed
    __syncthreads();
    int sa[FM], sb[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) sa[i] = int(sa_next[i] >> (8 * h));
#pragma unroll
    for (int j = 0; j < FN; ++j) sb[j] = int(sb_next[j] >> (8 * h));
    uint4 af[FM][4], bf[FN][4];
#pragma unroll
    for (int i = 0; i < FM; ++i) read_frag<ELEM>(cur, wrow + i * 32 + r, h, af[i]);
#pragma unroll
    for (int j = 0; j < FN; ++j) read_frag<ELEM>(cur + BM * BK, wcol + j * 32 + r, h, bf[j]);
    __builtin_amdgcn_sched_barrier(0);
    if (s + 1 < nstages) {
      dma_stage<GENERIC>(A, nxt, kc_next, kv_next);
      dma_stage<GENERIC>(B, nxt + BM * BK, kc_next, kv_next);
      if (ELEM == kFp8) {
        load_scales<GENERIC>(A, kc_next, kv_next, sa_next);
        load_scales<GENERIC>(B, kc_next, kv_next, sb_next);
      }
      if (s + 2 < nstages) kmap(s + 2, kc_next, kv_next);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (ELEM == kFp8) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const v8i a = as_v8i(af[i][2 * ks], af[i][2 * ks + 1]);
            const v8i b = as_v8i(bf[j][2 * ks], bf[j][2 * ks + 1]);
            if (ks == 0) acc[i][j] = mfma_fp8<FA, FB, 0>(a, b, acc[i][j], sa[i], sb[j]);
            else acc[i][j] = mfma_fp8<FA, FB, 2>(a, b, acc[i][j], sa[i], sb[j]);
          }
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_v8bf(af[i][t]), as_v8bf(bf[j][t]), acc[i][j],
                                                                0, 0, 0);
    }
  }
}

// Operand set-up for rows [row0, row0 + ROWS) of a row-major operand with
// `nrows` rows of `ld` bytes (codes) and `sld` bytes (scales); the buffers are
// rebased at row0 so offsets stay small.  Rows at or past nrows read as 0.
template <int ROWS, int F>
__device__ __forceinline__ void setup_rows(Operand<ROWS, F>& op, const uint8_t* codes, const uint8_t* scales,
                                           int64_t row0, int64_t nrows, int64_t ld, int64_t sld, int frag_row0) {
  const int64_t have = nrows - row0 < ROWS ? nrows - row0 : ROWS;
  op.codes = make_rsrc(codes + row0 * ld, uint32_t(have * ld));
  if (scales) op.scales = make_rsrc(scales + row0 * sld, uint32_t(have * sld));
#pragma unroll
  for (int j = 0; j < ROWS / 32; ++j) {
    const int r = dma_row<ROWS>(j);
    op.off[j] = r < have ? uint32_t(r * ld + 16 * dma_chunk<ROWS>(j)) : kOOB;
  }
#pragma unroll
  for (int f = 0; f < F; ++f) {
    const int r = frag_row0 + f * 32 + ((threadIdx.x & 63) & 31);
    op.soff[f] = r < have ? uint32_t(r * sld) : kOOB;
  }
}

// Operand set-up for gathered rows: tile row r reads source row rowid(r)
// (negative = padding, read as zeros) of a [src_rows][ld] operand.
template <int ROWS, int F, class RowId>
__device__ __forceinline__ void setup_gather(Operand<ROWS, F>& op, const uint8_t* codes, const uint8_t* scales,
                                             int64_t src_rows, int64_t ld, int64_t sld, int frag_row0,
                                             const RowId& rowid) {
  op.codes = make_rsrc(codes, uint32_t(src_rows * ld));
  if (scales) op.scales = make_rsrc(scales, uint32_t(src_rows * sld));
#pragma unroll
  for (int j = 0; j < ROWS / 32; ++j) {
    const int64_t t = rowid(dma_row<ROWS>(j));
    op.off[j] = t >= 0 ? uint32_t(t * ld + 16 * dma_chunk<ROWS>(j)) : kOOB;
  }
#pragma unroll
  for (int f = 0; f < F; ++f) {
    const int64_t t = rowid(frag_row0 + f * 32 + ((threadIdx.x & 63) & 31));
    op.soff[f] = t >= 0 ? uint32_t(t * sld) : kOOB;
  }
}

// Accumulator register q of fragment (i, j): row / column in the block tile.
template <int BM, int BN>
__device__ __forceinline__ int acc_row(int i, int q) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  return (wave >> 1) * (BM / 2) + i * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
}
template <int BM, int BN>
__device__ __forceinline__ int acc_col(int j) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  return (wave & 1) * (BN / 2) + j * 32 + (lane & 31);
}

// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>): a loop over
// fragments whose index is a compile-time constant however large the body, so
// accumulator fragments are always addressed statically (stay in registers).
template <class F, int... Is>
__device__ __forceinline__ void static_for_(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_(f, std::make_integer_sequence<int, N>{});
}

// Tile order: consecutive workgroups land on different XCDs (round-robin over
// 8), so remap ids to give each XCD a contiguous range, then walk tiles in
// groups of GM tile-rows so that co-resident tiles share operand rows in L2.
__device__ __forceinline__ int xcd_remap(int id, int total) {
  if (total % 8) return id;
  return (id % 8) * (total / 8) + id / 8;
}
template <int GM>
__device__ __forceinline__ void grouped_tile(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int per_group = GM * tiles_n;
  const int g = t / per_group;
  const int first = g * GM;
  const int rows = tiles_m - first < GM ? tiles_m - first : GM;
  const int w = t - g * per_group;
  tm = first + w % rows;
  tn = w / rows;
}

}  // namespace v2
}  // namespace mx
