// gemm_core.hpp -- the MXFP8 scaled-MFMA main loop for gfx950.
//
// C[m][n] = sum_k deq(A)[m][k] * deq(B)[n][k] with both operands stored
// K-contiguous as fp8 codes plus one E8M0 byte per 32 elements along K (the
// MX layout every GEMM of the MoE backward and the dense backward reads; P1:
// "32-element quantization group", P2: the dX / dW contractions).
//
// Hardware mapping (v_mfma_scale_f32_32x32x64_f8f6f4, one 64-wide wave):
//   - lane l = 32*h + r works on row r of a 32-row fragment; of a 64-element
//     K step made of groups G0 = k[0,32) and G1 = k[32,64) it holds
//     G0[16h, 16h+16) in bytes 0-15 and G1[16h, 16h+16) in bytes 16-31, and
//     supplies the scale of group G_h (selected from its register by opsel);
//   - the 32x32 fp32 accumulator: register i of lane l is
//     C[8*(i/4) + 4*h + i%4][r].
// Block tile BM x BN (128 or 256 each), 4 waves as 2 x 2, wave tile
// (BM/2) x (BN/2) in 32x32 fragments.  K is staged 128 bytes (4 groups) at a
// time through double-buffered LDS: global -> registers -> LDS, one barrier
// per stage.  LDS rows are 128 B (8 chunks of 16 B); chunk c of row r lives at
// c ^ ((r >> 1) & 7), so the 16 rows one ds_read_b128 phase touches hit 16
// distinct bank groups.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBK = 128;       // K bytes per stage
constexpr int kThreads = 256;  // 4 waves

__device__ __forceinline__ int lds_off(int r, int c) { return r * kBK + ((c ^ ((r >> 1) & 7)) << 4); }

// Staging of one operand tile: thread t moves 16-byte chunk (t & 7) of rows
// (t >> 3) + 32 * p.  A null row pointer (padding / beyond the matrix) loads
// zeros.
template <int ROWS>
struct Stager {
  static constexpr int P = ROWS / 32;
  const uint8_t* row[P];
  uint4 v[P];
  __device__ __forceinline__ void load(int64_t kcol, int kvalid) {
    const int c = threadIdx.x & 7;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      if (row[p] && c * 16 < kvalid)
        v[p] = *reinterpret_cast<const uint4*>(row[p] + kcol + c * 16);
      else
        v[p] = make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(uint8_t* lds) const {
    const int c = threadIdx.x & 7;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int r = (threadIdx.x >> 3) + 32 * p;
      *reinterpret_cast<uint4*>(lds + lds_off(r, c)) = v[p];
    }
  }
};

// Scale registers of the fragments a lane feeds: one row per fragment.  The
// stage's 4 scale bytes [g0 g1 g2 g3] are shifted right by 8*h so that
// opsel 0 gives g_h (first 64-element step) and opsel 2 gives g_{2+h}.
template <int F, bool ALIGNED>
struct ScaleRegs {
  const uint8_t* row[F];
  int reg[F];
  __device__ __forceinline__ void load(int64_t kcol, int kvalid) {
    const int h = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int f = 0; f < F; ++f) {
      uint32_t s = 0;
      if (row[f]) {
        if (ALIGNED && kvalid == kBK) {
          s = *reinterpret_cast<const uint32_t*>(row[f] + (kcol >> 5));
        } else {
          for (int g = 0; g < 4; ++g)
            if (g * 32 < kvalid) s |= uint32_t(row[f][(kcol >> 5) + g]) << (8 * g);
        }
      }
      reg[f] = int(s >> (8 * h));
    }
  }
};

template <int FA, int FB, int OPS>
__device__ __forceinline__ v16f mfma_mx(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, OPS, sa, OPS, sb);
}

__device__ __forceinline__ v8i frag_from_lds(const uint8_t* tile, int row, int ks, int h) {
  const uint4 lo = *reinterpret_cast<const uint4*>(tile + lds_off(row, ks * 4 + h));
  const uint4 hi = *reinterpret_cast<const uint4*>(tile + lds_off(row, ks * 4 + 2 + h));
  v8i v;
  v[0] = int(lo.x); v[1] = int(lo.y); v[2] = int(lo.z); v[3] = int(lo.w);
  v[4] = int(hi.x); v[5] = int(hi.y); v[6] = int(hi.z); v[7] = int(hi.w);
  return v;
}

// Per-thread state of one tile's main loop.
template <int BM, int BN, bool SALIGN>
struct TileOperands {
  static constexpr int FM = BM / 64;   // 32-row fragments per wave along M
  static constexpr int FN = BN / 64;
  Stager<BM> a;
  Stager<BN> b;
  ScaleRegs<FM, SALIGN> sa;
  ScaleRegs<FN, SALIGN> sb;
};

// The K loop.  kmap(s) gives the byte column of stage s in both operands (the
// same K index space), kvalid(s) how many of its 128 bytes are inside K.
// smem must hold 2 * (BM + BN) * kBK bytes.
template <int BM, int BN, int FA, int FB, bool SALIGN, class KMap>
__device__ __forceinline__ void mx_mainloop(TileOperands<BM, BN, SALIGN>& op, int nstages, const KMap& kmap,
                                            uint8_t* smem, v16f (&acc)[BM / 64][BN / 64]) {
  constexpr int FM = BM / 64, FN = BN / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
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

  uint8_t* buf[2] = {smem, smem + (BM + BN) * kBK};
  {
    int64_t kc;
    int kv;
    kmap(0, kc, kv);
    op.a.load(kc, kv);
    op.b.load(kc, kv);
    op.sa.load(kc, kv);
    op.sb.load(kc, kv);
    op.a.store(buf[0]);
    op.b.store(buf[0] + BM * kBK);
  }
  __syncthreads();
  int sa_cur[FM], sb_cur[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) sa_cur[i] = op.sa.reg[i];
#pragma unroll
  for (int j = 0; j < FN; ++j) sb_cur[j] = op.sb.reg[j];

  for (int s = 0; s < nstages; ++s) {
    const bool more = s + 1 < nstages;
    if (more) {
      int64_t kc;
      int kv;
      kmap(s + 1, kc, kv);
      op.a.load(kc, kv);
      op.b.load(kc, kv);
      op.sa.load(kc, kv);
      op.sb.load(kc, kv);
    }
    const uint8_t* At = buf[s & 1];
    const uint8_t* Bt = At + BM * kBK;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v8i af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = frag_from_lds(At, wrow + i * 32 + r, ks, h);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = frag_from_lds(Bt, wcol + j * 32 + r, ks, h);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if (ks == 0)
            acc[i][j] = mfma_mx<FA, FB, 0>(af[i], bfr[j], acc[i][j], sa_cur[i], sb_cur[j]);
          else
            acc[i][j] = mfma_mx<FA, FB, 2>(af[i], bfr[j], acc[i][j], sa_cur[i], sb_cur[j]);
        }
    }
    if (more) {
      op.a.store(buf[(s + 1) & 1]);
      op.b.store(buf[(s + 1) & 1] + BM * kBK);
#pragma unroll
      for (int i = 0; i < FM; ++i) sa_cur[i] = op.sa.reg[i];
#pragma unroll
      for (int j = 0; j < FN; ++j) sb_cur[j] = op.sb.reg[j];
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Precise variant: the same fp8 tiles and LDS staging, but each fragment is
// converted in registers to bf16 with its E8M0 scale folded in (exact: an
// fp8 code times a power of two has at most 4 significant bits) and reduced
// with v_mfma_f32_32x32x16_bf16, which accumulates at fp32 precision.  The
// scaled fp8 MFMA's internal reduction carries ~1e-5 relative error; that is
// invisible in a bf16 output but flips e5m2 rounding decisions when a result
// is requantised (the Phase-1 epilogue), so Phase 1 uses this loop.
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  return s ? __uint_as_float(s << 23) : __uint_as_float(0x00400000u);   // 2^(s-127)
}

template <int FMT, bool HI>
__device__ __forceinline__ uint32_t cvt_pk_bf16(uint32_t codes, float scale) {
  v2bf r;
  if (FMT == 0)
    r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, scale, HI);
  else
    r = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(codes, scale, HI);
  return __builtin_bit_cast(uint32_t, r);
}

// 16 codes (one uint4) -> two bf16 vectors of 8 (codes 0-7, 8-15), times scale.
template <int FMT>
__device__ __forceinline__ void cvt16(const uint4& c, float scale, v8bf& lo, v8bf& hi) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  uint32_t o[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o[2 * k] = cvt_pk_bf16<FMT, false>(w[k], scale);
    o[2 * k + 1] = cvt_pk_bf16<FMT, true>(w[k], scale);
  }
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  lo = __builtin_bit_cast(v8bf, u4v{o[0], o[1], o[2], o[3]});
  hi = __builtin_bit_cast(v8bf, u4v{o[4], o[5], o[6], o[7]});
}

// Raw per-row stage scales (4 bytes: the stage's 4 groups) for the precise loop.
template <int F, bool ALIGNED>
struct RawScales {
  const uint8_t* row[F];
  uint32_t reg[F];
  __device__ __forceinline__ void load(int64_t kcol, int kvalid) {
#pragma unroll
    for (int f = 0; f < F; ++f) {
      uint32_t s = 0;
      if (row[f]) {
        if (ALIGNED && kvalid == kBK) {
          s = *reinterpret_cast<const uint32_t*>(row[f] + (kcol >> 5));
        } else {
          for (int g = 0; g < 4; ++g)
            if (g * 32 < kvalid) s |= uint32_t(row[f][(kcol >> 5) + g]) << (8 * g);
        }
      }
      reg[f] = s;
    }
  }
};

template <int BM, int BN, bool SALIGN>
struct TileOperandsBf16 {
  static constexpr int FM = BM / 64, FN = BN / 64;
  Stager<BM> a;
  Stager<BN> b;
  RawScales<FM, SALIGN> sa;
  RawScales<FN, SALIGN> sb;
};

template <int BM, int BN, int FA, int FB, bool SALIGN, class KMap>
__device__ __forceinline__ void mx_mainloop_bf16(TileOperandsBf16<BM, BN, SALIGN>& op, int nstages, const KMap& kmap,
                                                 uint8_t* smem, v16f (&acc)[BM / 64][BN / 64]) {
  constexpr int FM = BM / 64, FN = BN / 64;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
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

  uint8_t* buf[2] = {smem, smem + (BM + BN) * kBK};
  {
    int64_t kc;
    int kv;
    kmap(0, kc, kv);
    op.a.load(kc, kv);
    op.b.load(kc, kv);
    op.sa.load(kc, kv);
    op.sb.load(kc, kv);
    op.a.store(buf[0]);
    op.b.store(buf[0] + BM * kBK);
  }
  __syncthreads();
  uint32_t sa_cur[FM], sb_cur[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) sa_cur[i] = op.sa.reg[i];
#pragma unroll
  for (int j = 0; j < FN; ++j) sb_cur[j] = op.sb.reg[j];

  for (int s = 0; s < nstages; ++s) {
    const bool more = s + 1 < nstages;
    if (more) {
      int64_t kc;
      int kv;
      kmap(s + 1, kc, kv);
      op.a.load(kc, kv);
      op.b.load(kc, kv);
      op.sa.load(kc, kv);
      op.sb.load(kc, kv);
    }
    const uint8_t* At = buf[s & 1];
    const uint8_t* Bt = At + BM * kBK;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      // lane holds G0[16h, 16h+16) and G1[16h, 16h+16) of the 64-element step;
      // bf16 step t covers G0[16h, +8), G0[16h+8, +8), G1[16h, +8), G1[16h+8, +8)
      v8bf af[FM][4], bfv[FN][4];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = wrow + i * 32 + r;
        const uint4 lo = *reinterpret_cast<const uint4*>(At + lds_off(row, ks * 4 + h));
        const uint4 hi = *reinterpret_cast<const uint4*>(At + lds_off(row, ks * 4 + 2 + h));
        cvt16<FA>(lo, e8m0_to_f32((sa_cur[i] >> (16 * ks)) & 0xffu), af[i][0], af[i][1]);
        cvt16<FA>(hi, e8m0_to_f32((sa_cur[i] >> (16 * ks + 8)) & 0xffu), af[i][2], af[i][3]);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int row = wcol + j * 32 + r;
        const uint4 lo = *reinterpret_cast<const uint4*>(Bt + lds_off(row, ks * 4 + h));
        const uint4 hi = *reinterpret_cast<const uint4*>(Bt + lds_off(row, ks * 4 + 2 + h));
        cvt16<FB>(lo, e8m0_to_f32((sb_cur[j] >> (16 * ks)) & 0xffu), bfv[j][0], bfv[j][1]);
        cvt16<FB>(hi, e8m0_to_f32((sb_cur[j] >> (16 * ks + 8)) & 0xffu), bfv[j][2], bfv[j][3]);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i][t], bfv[j][t], acc[i][j], 0, 0, 0);
    }
    if (more) {
      op.a.store(buf[(s + 1) & 1]);
      op.b.store(buf[(s + 1) & 1] + BM * kBK);
#pragma unroll
      for (int i = 0; i < FM; ++i) sa_cur[i] = op.sa.reg[i];
#pragma unroll
      for (int j = 0; j < FN; ++j) sb_cur[j] = op.sb.reg[j];
    }
    __syncthreads();
  }
}

// Row / column of accumulator register q of fragment (i, j) for this lane,
// relative to the block tile origin.
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

}  // namespace mx
