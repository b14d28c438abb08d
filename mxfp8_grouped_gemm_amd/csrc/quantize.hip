// quantize.hip -- MXFP8 quantisers for gfx950 (HBM-bound; no MFMA).
//
// Three kernels share the E8M0 rule and the encoders of mx_device.hpp:
//   quant_rows : groups of 32 along the contiguous axis (codes in place).
//   quant_cols : groups of 32 along the strided axis (codes in place).
//   quant_tok  : groups of 32 along the strided axis, written transposed so the
//                quantised axis becomes contiguous (the K-contiguous operand a
//                scaled MFMA reads), with optional row gather by index, optional
//                per-row fp32 scale (bf16(fp32(a * v))), used for the dense
//                backward's dY^T / W^T / X^T and the MoE token-axis operands.
// Group size, scale rule and rounding: P1 ("Blockwise MM Backward MXFP8 Kernel
// API Reference": 32-element MXFP8 quantization groups).
//
// Scale layouts: row-major [rows][K/32] (one byte per group), or -- for
// operands of the ring GEMM loop -- pair-major [K/128][rows][4], where word
// (p, r) holds row r's four groups of K elements [128p, 128p + 128).
#include <type_traits>

#include "gemm_v2.hpp"
#include "kernels.hpp"
#include "mx_device.hpp"

namespace mx {

// ---------------------------------------------------------------------------
// quant_rows: 4 lanes per group, 8 bf16 (16 B) per lane.  A wave covers 16
// groups = 1 KiB of input per load instruction, fully coalesced.
// fp8 codes -> bf16 values times 2^X (exact: at most 4 significant bits).
typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float pow2_f32(int X) {
  return X > -127 ? __uint_as_float(uint32_t(X + 127) << 23) : __uint_as_float(0x00400000u);
}
template <int FMT, bool HI>
__device__ __forceinline__ uint32_t deq_pk(uint32_t codes, float scale) {
  v2bf_t r = FMT == kE4M3 ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, scale, HI)
                          : __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(codes, scale, HI);
  return __builtin_bit_cast(uint32_t, r);
}

// One chunk c (8 values of a row) from its loaded 16 bytes v.  The four lanes of
// a group (c = 4g .. 4g + 3, consecutive lanes) exchange their maxima.
// stage_major (with PAIRS): codes stage-major (stage_major_off, rows rows over
// 32 * gpr columns) instead of row-major; rows * gpr < 2^32.
template <int FMT, bool DEQ, bool PAIRS>
__device__ __forceinline__ void quant_rows_chunk(const uint4 v, int64_t c, uint2* __restrict__ codes,
                                                 uint8_t* __restrict__ scales, uint4* __restrict__ deq,
                                                 int64_t rows, int64_t gpr, int stage_major) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t amax = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    amax = max(amax, abs_bits_bf16(uint16_t(w[k] & 0xffffu)));
    amax = max(amax, abs_bits_bf16(uint16_t(w[k] >> 16)));
  }
  amax = max(amax, uint32_t(__shfl_xor(int(amax), 1, 64)));
  amax = max(amax, uint32_t(__shfl_xor(int(amax), 2, 64)));
  const int X = scale_exp<FMT>(amax);
  const float inv = inv_scale(X);
  uint32_t out[2];
#pragma unroll
  for (int k = 0; k < 2; ++k)
    out[k] = encode4<FMT>(__uint_as_float(w[2 * k] << 16), __uint_as_float(w[2 * k] & 0xffff0000u),
                          __uint_as_float(w[2 * k + 1] << 16), __uint_as_float(w[2 * k + 1] & 0xffff0000u), inv);
  if (PAIRS && stage_major) {   // chunk c = 8 codes of row c / (4 gpr)
    const uint32_t row = uint32_t(c >> 2) / uint32_t(gpr);
    const int64_t col = (c - int64_t(row) * gpr * 4) * 8;
    codes[stage_major_off(row, col, rows, gpr * 32) >> 3] = make_uint2(out[0], out[1]);
  } else {
    codes[c] = make_uint2(out[0], out[1]);
  }
  if ((c & 3) == 0) {
    if (PAIRS) {   // group G = row * gpr + g  ->  word (g / 4, row), byte g % 4
      const int64_t G = c >> 2, row = G / gpr, g = G - row * gpr;
      scales[((g >> 2) * rows + row) * 4 + (g & 3)] = uint8_t(X + 127);
    } else {
      scales[c >> 2] = uint8_t(X + 127);
    }
  }
  if (DEQ) {
    const float sc = pow2_f32(X);
    deq[c] = make_uint4(deq_pk<FMT, false>(out[0], sc), deq_pk<FMT, true>(out[0], sc),
                        deq_pk<FMT, false>(out[1], sc), deq_pk<FMT, true>(out[1], sc));
  }
}

// U chunks per thread and pass, their loads issued together (U = 4 for small
// inputs, where a thread per chunk leaves the kernel mostly workgroup start-up:
// measured on [4096, 4096]).  nchunks is a multiple of 4, so a group's lanes
// are all in range or all out.
template <int FMT, bool DEQ, bool PAIRS, int U>
__global__ void __launch_bounds__(256) quant_rows_kernel(const uint4* __restrict__ x,
                                                          uint2* __restrict__ codes,
                                                          uint8_t* __restrict__ scales,
                                                          int64_t nchunks, uint4* __restrict__ deq,
                                                          int64_t rows, int64_t gpr, int stage_major) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t c0 = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; c0 < nchunks; c0 += U * stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * stride;
      v[u] = c < nchunks ? x[c] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * stride;
      if (c < nchunks) quant_rows_chunk<FMT, DEQ, PAIRS>(v[u], c, codes, scales, deq, rows, gpr, stage_major);
    }
  }
}

// codes [rows][cols] with scales along cols -> bf16; one thread per 16 codes.
template <int FMT>
__global__ void __launch_bounds__(256) dequant_rows_kernel(const uint4* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales, int64_t n16,
                                                            uint4* __restrict__ out) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t c = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; c < n16; c += stride) {
    const uint4 v = codes[c];
    const float sc = pow2_f32(int(scales[c >> 1]) - 127);
    out[2 * c] = make_uint4(deq_pk<FMT, false>(v.x, sc), deq_pk<FMT, true>(v.x, sc), deq_pk<FMT, false>(v.y, sc),
                            deq_pk<FMT, true>(v.y, sc));
    out[2 * c + 1] = make_uint4(deq_pk<FMT, false>(v.z, sc), deq_pk<FMT, true>(v.z, sc),
                                deq_pk<FMT, false>(v.w, sc), deq_pk<FMT, true>(v.w, sc));
  }
}

// ---------------------------------------------------------------------------
// quant_cols: a thread owns 8 adjacent columns and one group of 32 rows.  VEC
// (cols % 8 == 0, so every row segment is 16-byte aligned): one 16-byte load
// per row for the amax, a second (from L2) to encode, 8-byte code and scale
// stores.  Otherwise element by element.
template <int FMT, bool VEC>
__global__ void __launch_bounds__(256) quant_cols_kernel(const uint16_t* __restrict__ x,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales,
                                                          int64_t rows, int64_t cols) {
  const int64_t c0 = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) * 8;
  const int64_t g = blockIdx.y;
  if (c0 >= cols) return;
  if (VEC) {
    const int64_t ld = cols / 8;   // row stride in 16-byte chunks
    const uint4* src = reinterpret_cast<const uint4*>(x + g * 32 * cols + c0);
    uint32_t am[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll 8
    for (int r = 0; r < 32; ++r) {
      const uint4 v = src[r * ld];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        am[2 * k] = max(am[2 * k], (w[k] << 16) & 0x7fffffffu);
        am[2 * k + 1] = max(am[2 * k + 1], w[k] & 0x7fff0000u);
      }
    }
    float inv[8];
    uint32_t sw[2] = {0, 0};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int X = scale_exp<FMT>(am[k]);
      inv[k] = inv_scale(X);
      sw[k >> 2] |= uint32_t(X + 127) << (8 * (k & 3));
    }
    *reinterpret_cast<uint2*>(scales + g * cols + c0) = make_uint2(sw[0], sw[1]);
    uint2* dst = reinterpret_cast<uint2*>(codes + g * 32 * cols + c0);
#pragma unroll 8
    for (int r = 0; r < 32; ++r) {
      const uint4 v = src[r * ld];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      const uint32_t lo = encode4s<FMT>(__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                                        __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u), inv[0],
                                        inv[1], inv[2], inv[3]);
      const uint32_t hi = encode4s<FMT>(__uint_as_float(w[2] << 16), __uint_as_float(w[2] & 0xffff0000u),
                                        __uint_as_float(w[3] << 16), __uint_as_float(w[3] & 0xffff0000u), inv[4],
                                        inv[5], inv[6], inv[7]);
      dst[r * ld] = make_uint2(lo, hi);
    }
    return;
  }
  const int ncol = cols - c0 >= 8 ? 8 : int(cols - c0);
  uint32_t amax[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int r = 0; r < 32; ++r) {
    const uint16_t* row = x + (g * 32 + r) * cols + c0;
    for (int k = 0; k < ncol; ++k) amax[k] = max(amax[k], abs_bits_bf16(row[k]));
  }
  int X[8];
  for (int k = 0; k < ncol; ++k) {
    X[k] = scale_exp<FMT>(amax[k]);
    scales[g * cols + c0 + k] = uint8_t(X[k] + 127);
  }
  for (int r = 0; r < 32; ++r) {
    const uint16_t* row = x + (g * 32 + r) * cols + c0;
    uint8_t* crow = codes + (g * 32 + r) * cols + c0;
    for (int k = 0; k < ncol; ++k) crow[k] = uint8_t(encode<FMT>(uint32_t(row[k]) << 16, X[k]));
  }
}

// The 32 rows row0 .. row0 + 31 of columns colA, colA + 1 (w[r]: bf16 of colA
// in the low half, colA + 1 in the high half) as one scale group each: codes
// to codes_t [cols][rows] (or stage-major, see stage_major_off, with cols rows
// contracted over rows elements), scale bytes to scales_t.
template <int FMT, bool PAIRS>
__device__ __forceinline__ void tok_encode_pair(const uint32_t (&w)[32], int64_t rows, int64_t cols, int64_t colA,
                                                int64_t row0, uint8_t* __restrict__ codes_t,
                                                uint8_t* __restrict__ scales_t, bool stage_major) {
  uint32_t m = 0;   // |bf16| maxima of both columns
#pragma unroll
  for (int r = 0; r < 32; ++r) m = absmax_bf16x2(m, w[r]);
  const int X0 = scale_exp<FMT>(m << 16), X1 = scale_exp<FMT>(m & 0xffff0000u);
  const uint32_t lim = bf16_limit<FMT>(X0) | (bf16_limit<FMT>(X1) << 16);
  const float s0 = cvt_scale(X0), s1 = cvt_scale(X1);
  uint32_t p0[8], p1[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint32_t w0 = clamp_bf16x2(w[4 * q], lim), w1 = clamp_bf16x2(w[4 * q + 1], lim);
    const uint32_t w2 = clamp_bf16x2(w[4 * q + 2], lim), w3 = clamp_bf16x2(w[4 * q + 3], lim);
    p0[q] = encode_bf16x4<FMT>(lo_halves(w0, w1), lo_halves(w2, w3), s0);
    p1[q] = encode_bf16x4<FMT>(hi_halves(w0, w1), hi_halves(w2, w3), s1);
  }
  const int64_t o0 = stage_major ? stage_major_off(colA, row0, cols, rows) : colA * rows + row0;
  const int64_t o1 = stage_major ? stage_major_off(colA + 1, row0, cols, rows) : o0 + rows;
  uint4* dst0 = reinterpret_cast<uint4*>(codes_t + o0);
  uint4* dst1 = reinterpret_cast<uint4*>(codes_t + o1);
  dst0[0] = make_uint4(p0[0], p0[1], p0[2], p0[3]);
  dst0[1] = make_uint4(p0[4], p0[5], p0[6], p0[7]);
  dst1[0] = make_uint4(p1[0], p1[1], p1[2], p1[3]);
  dst1[1] = make_uint4(p1[4], p1[5], p1[6], p1[7]);
  if (PAIRS) {
    const int64_t g = row0 / 32;
    scales_t[((g >> 2) * cols + colA) * 4 + (g & 3)] = uint8_t(X0 + 127);
    scales_t[((g >> 2) * cols + colA + 1) * 4 + (g & 3)] = uint8_t(X1 + 127);
  } else {
    scales_t[colA * (rows / 32) + row0 / 32] = uint8_t(X0 + 127);
    scales_t[(colA + 1) * (rows / 32) + row0 / 32] = uint8_t(X1 + 127);
  }
}

// ---------------------------------------------------------------------------
// quant_tok: a workgroup covers 128 logical rows x 128 columns; wave w takes
// rows 32w .. 32w+31 (one scale group) and lane l the column pair 2l, 2l+1.
// Logical row r reads source row idx[r] (or r without an index; with
// self_rows, row r itself where idx[r] >= 0); a source outside [0, src_rows)
// contributes zeros (a padding slot).  With a row scale,
// the value is bf16(fp32(scale[r] * v)).  Output: codes_t [cols][rows] and
// scales_t [cols][rows/32] (or pair-major [rows/128][cols][4] with PAIRS);
// rows % 32 == 0 (% 128 with PAIRS) and cols % 8 == 0.
// A row and its source index are the same for every lane of a wave, so each
// of the 32 row loads is one 256-byte coalesced read (the index and the row
// scale are scalar loads); the 32 values a lane needs stay in registers and
// no LDS staging or barrier stands between the loads and the stores.
constexpr int kTokRows = 128;
constexpr int kTokCols = 128;

// BIAS (the gathered dY rows of the MoE backward with a down-projection bias;
// ROWSCALE and OFF32 hold, rows % 128 == 0, cols % 128 == 0, and a
// workgroup's 128 rows are slots of one block of bias.B slots): from the raw
// dY values already in registers, also
//   db2[e][h]  += sum over the workgroup's slots of a * dY   (fp32; one atomic
//                 per workgroup and column, the waves' sums added in order)
//   part[c][s]  = sum over the 128 columns of column tile c of dY[s][h] * b2[e][h]
//                 (each slot's share of <dY, b2>; the finalisation adds the
//                 H/128 shares in order, so d(a) stays reproducible)
// P3 (sonic-moe functional/backward.py, db2_and_ds_kernel): db2 and the bias
// term of the affinity gradient.
template <int FMT, bool GATHER, bool ROWSCALE, bool PAIRS, bool OFF32, bool BIAS>
__global__ void __launch_bounds__(256) quant_tok_kernel(const uint16_t* __restrict__ x,
                                                         int64_t src_rows, int64_t cols,
                                                         const int32_t* __restrict__ idx,
                                                         const float* __restrict__ rowscale,
                                                         int64_t rows, uint8_t* __restrict__ codes_t,
                                                         uint8_t* __restrict__ scales_t, int self_rows,
                                                         TokBias bias, int stage_major) {
  const int cp = threadIdx.x & 63;
  const int grp = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row0 = int64_t(blockIdx.y) * kTokRows + grp * 32;
  const int64_t colA = int64_t(blockIdx.x) * kTokCols + 2 * cp;
  if (!BIAS && (row0 >= rows || colA >= cols)) return;   // BIAS: every lane reaches the barrier
  uint32_t w[32];   // bf16 of columns colA (low half) and colA + 1 (high half), rows row0 ..
  float dot[BIAS ? 32 : 1];        // BIAS: this lane's two columns' share of <dY, b2> per row
  float db0 = 0.f, db1 = 0.f;      // BIAS: sums of a * dY over the wave's rows, columns colA, colA + 1
  float b2lo = 0.f, b2hi = 0.f;
#pragma unroll
  for (int r = 0; r < (BIAS ? 32 : 1); ++r) dot[r] = 0.f;
  if (BIAS) {
    const int64_t e = bias.b2e[(int64_t(blockIdx.y) * kTokRows) / bias.B];
    const uint32_t bw = *reinterpret_cast<const uint32_t*>(bias.b2 + e * cols + colA);
    b2lo = __uint_as_float(bw << 16);
    b2hi = __uint_as_float(bw & 0xffff0000u);
  }
  if (src_rows > 0) {
#if defined(__HIP_DEVICE_COMPILE__)
    // OFF32 (source under 2 GiB): buffer loads at 32-bit offsets, a padding row
    // at an offset past the buffer, which reads zeros; the 32 row offsets live
    // in vector registers (as 64-bit scalar addresses they spilled)
    const auto rx = MX_RSRC(v2::make_rsrc(x, OFF32 ? uint32_t(src_rows * cols * 2) : 0u));
    const uint32_t row_bytes = uint32_t(cols * 2), lane_bytes = uint32_t(colA * 2);
#endif
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      uint32_t v = 0u;
#if defined(__HIP_DEVICE_COMPILE__)
      if (OFF32) {   // rows and sources fit in 32 bits: one scalar register per row index
        const int32_t lr = int32_t(row0) + r;
        const int32_t id = GATHER ? idx[lr] : lr;
        const int32_t src = self_rows ? (id >= 0 ? lr : -1) : id;
        const bool ok = src >= 0 && src < src_rows;
        v = __builtin_amdgcn_raw_buffer_load_b32(rx, ok ? uint32_t(src) * row_bytes + lane_bytes : v2::kOOB, 0, 0);
      } else {
        const int64_t id = GATHER ? int64_t(idx[row0 + r]) : row0 + r;
        const int64_t src = self_rows ? (id >= 0 ? row0 + r : -1) : id;
        const bool ok = src >= 0 && src < src_rows;
        // invalid rows read row 0's word and are zeroed: no branch per row
        v = *reinterpret_cast<const uint32_t*>(x + (ok ? src : 0) * cols + colA);
        v = ok ? v : 0u;
      }
#endif
      w[r] = v;
      if (ROWSCALE) {   // bf16(a * x), round to nearest even
        const float a = rowscale[row0 + r];
        const float x0 = __uint_as_float(w[r] << 16), x1 = __uint_as_float(w[r] & 0xffff0000u);
        if (BIAS) {
          dot[BIAS ? r : 0] = x0 * b2lo + x1 * b2hi;
          db0 += a * x0;
          db1 += a * x1;
        }
        w[r] = bf16x2_pack(a * x0, a * x1);
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < 32; ++r) w[r] = 0u;
  }
  if constexpr (BIAS) {
    // <dY, b2> shares: the 32 rows' values summed over the wave's 64 lanes by
    // halving exchanges (stride 32 keeps rows 16..31 in the upper lanes, ...,
    // stride 2 leaves row (lane >> 1) & 31), then lanes l and l ^ 1 add up.
    const int lane = threadIdx.x & 63;
    v2::static_for<5>([&](auto S) {
      constexpr int n = 16 >> int(S);                // values kept after this stage
      constexpr int stride = 32 >> int(S);
      const bool up = (lane & stride) != 0;
      v2::static_for<n>([&](auto I) {
        const float send = up ? dot[I] : dot[I + n];
        const float keep = up ? dot[I + n] : dot[I];
        dot[I] = keep + __shfl_xor(send, stride, 64);
      });
    });
    const float sum = dot[0] + __shfl_xor(dot[0], 1, 64);
    const int64_t ct = int64_t(blockIdx.x);            // column tile of kTokCols columns
    if ((lane & 1) == 0) bias.part[ct * rows + row0 + ((lane >> 1) & 31)] = sum;
    // db2: the four waves' column sums added in wave order, one atomic per column
    __shared__ float colsum[4][kTokCols];
    colsum[grp][2 * cp] = db0;
    colsum[grp][2 * cp + 1] = db1;
    __syncthreads();
    if (threadIdx.x < kTokCols) {
      const float t = ((colsum[0][threadIdx.x] + colsum[1][threadIdx.x]) + colsum[2][threadIdx.x]) +
                      colsum[3][threadIdx.x];
      const int64_t e = bias.b2e[(int64_t(blockIdx.y) * kTokRows) / bias.B];
      atomicAdd(bias.db2_acc + e * cols + int64_t(blockIdx.x) * kTokCols + threadIdx.x, t);
    }
  }
  tok_encode_pair<FMT, PAIRS>(w, rows, cols, colA, row0, codes_t, scales_t, stage_major != 0);
}

// ---------------------------------------------------------------------------
// quant_dual: one matrix [rows][cols] quantised along both axes from one read,
// as quant_rows (groups of 32 along a row: codes [rows][cols], scales
// pair-major [cols/128][rows][4]) and quant_tok without an index (groups of
// 32 along a column: codes_t [cols][rows], scales_t pair-major
// [rows/128][cols][4], or [cols][rows/32] when rows % 128 != 0), bit for bit.
// Wave w of a workgroup takes rows 32w .. 32w+31 of its 128, lane l columns
// 8l .. 8l+7 of its 512: 32 loads of 16 bytes, then the row groups (4 lanes
// each) and the column groups (a lane's 8 columns over the wave's 32 rows)
// from the same registers.  rows % 32 == 0, cols % 512 == 0.
constexpr int kDualCols = 512;

// sm / sm_t: codes / codes_t stage-major (stage_major_off) instead of row-major.
template <int FMT, bool PAIRS_T>
__global__ void __launch_bounds__(256) quant_dual_kernel(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                          uint2* __restrict__ codes, uint8_t* __restrict__ scales,
                                                          uint8_t* __restrict__ codes_t,
                                                          uint8_t* __restrict__ scales_t, int sm, int sm_t) {
  const int lane = threadIdx.x & 63;
  const int64_t row0 = int64_t(blockIdx.y) * 128 + (threadIdx.x >> 6) * 32;
  if (row0 >= rows) return;   // a partial last workgroup of rows (no barrier below)
  const int64_t col0 = int64_t(blockIdx.x) * kDualCols + 8 * lane;
  uint32_t w[32][4];
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    const uint4 v = *reinterpret_cast<const uint4*>(x + (row0 + r) * cols + col0);
    w[r][0] = v.x; w[r][1] = v.y; w[r][2] = v.z; w[r][3] = v.w;
  }
  // groups along the rows: this lane's 8 values and its 3 neighbours' (quant_rows)
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    uint32_t amax = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      amax = max(amax, abs_bits_bf16(uint16_t(w[r][k] & 0xffffu)));
      amax = max(amax, abs_bits_bf16(uint16_t(w[r][k] >> 16)));
    }
    amax = max(amax, uint32_t(__shfl_xor(int(amax), 1, 64)));
    amax = max(amax, uint32_t(__shfl_xor(int(amax), 2, 64)));
    const int X = scale_exp<FMT>(amax);
    const float inv = inv_scale(X);
    uint32_t out[2];
#pragma unroll
    for (int k = 0; k < 2; ++k)
      out[k] = encode4<FMT>(__uint_as_float(w[r][2 * k] << 16), __uint_as_float(w[r][2 * k] & 0xffff0000u),
                            __uint_as_float(w[r][2 * k + 1] << 16), __uint_as_float(w[r][2 * k + 1] & 0xffff0000u),
                            inv);
    const int64_t row = row0 + r;
    codes[(sm ? stage_major_off(row, col0, rows, cols) : row * cols + col0) / 8] = make_uint2(out[0], out[1]);
    if ((lane & 3) == 0) {   // group g of the row -> word (g / 4, row), byte g % 4
      const int64_t g = col0 / 32;
      scales[((g >> 2) * rows + row) * 4 + (g & 3)] = uint8_t(X + 127);
    }
  }
  // groups along the columns: the lane's four column pairs (quant_tok)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t wq[32];
#pragma unroll
    for (int r = 0; r < 32; ++r) wq[r] = w[r][q];
    tok_encode_pair<FMT, PAIRS_T>(wq, rows, cols, col0 + 2 * q, row0, codes_t, scales_t, sm_t != 0);
  }
}

// ---------------------------------------------------------------------------
// Row-major scales of `groups` matrices [rows][k/32] -> pair-major
// [groups][k/128][rows][4]; k % 128 == 0.  A transpose of 4-byte words
// ([rows][kp] -> [kp][rows] per group) through LDS: a workgroup moves 64 rows x
// 32 words, reading 128-byte row runs and writing 256-byte column runs.
__global__ void __launch_bounds__(256) scales_to_pairs_kernel(const uint32_t* __restrict__ in, int64_t rows,
                                                              int64_t kp, uint32_t* __restrict__ out) {
  __shared__ uint32_t tile[32][65];
  const int64_t p0 = int64_t(blockIdx.x) * 32, r0 = int64_t(blockIdx.y) * 64, g = blockIdx.z;
  const uint32_t* src = in + g * rows * kp;
  uint32_t* dst = out + g * rows * kp;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int i = threadIdx.x + 256 * k, r = i >> 5, p = i & 31;
    if (r0 + r < rows && p0 + p < kp) tile[p][r] = src[(r0 + r) * kp + p0 + p];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int i = threadIdx.x + 256 * k, p = i >> 6, r = i & 63;
    if (r0 + r < rows && p0 + p < kp) dst[(p0 + p) * rows + r0 + r] = tile[p][r];
  }
}

// ---------------------------------------------------------------------------
// host launchers
template <int FMT, int U>
static void rows_dispatch(int blocks, hipStream_t st, const uint4* xs, uint2* cs, uint8_t* scales, int64_t nchunks,
                          uint4* ds, int64_t rows, int64_t gpr, bool pairs, int sm) {
  if (ds) quant_rows_kernel<FMT, true, false, U><<<blocks, 256, 0, st>>>(xs, cs, scales, nchunks, ds, rows, gpr, 0);
  else if (pairs)
    quant_rows_kernel<FMT, false, true, U><<<blocks, 256, 0, st>>>(xs, cs, scales, nchunks, ds, rows, gpr, sm);
  else quant_rows_kernel<FMT, false, false, U><<<blocks, 256, 0, st>>>(xs, cs, scales, nchunks, ds, rows, gpr, 0);
}
template <int FMT>
static void rows_dispatch(int64_t nchunks, hipStream_t st, const uint4* xs, uint2* cs, uint8_t* scales, uint4* ds,
                          int64_t rows, int64_t gpr, bool pairs, int sm) {
  const bool small = nchunks <= (int64_t(1) << 22);
  const int64_t want = small ? (nchunks + 1023) / 1024 : (nchunks + 255) / 256;
  const int blocks = int(want < 65536 ? want : 65536);
  if (small) rows_dispatch<FMT, 4>(blocks, st, xs, cs, scales, nchunks, ds, rows, gpr, pairs, sm);
  else rows_dispatch<FMT, 1>(blocks, st, xs, cs, scales, nchunks, ds, rows, gpr, pairs, sm);
}

hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int64_t cols, int fmt, uint8_t* codes,
                             uint8_t* scales, hipStream_t st, uint16_t* deq, bool pairs, bool stage_major) {
  const int64_t nchunks = rows * cols / 8;
  if (nchunks == 0) return hipSuccess;
  if (deq && pairs) return hipErrorInvalidValue;   // no caller needs both
  if (stage_major && (!pairs || rows * (cols / 32) > int64_t(UINT32_MAX))) return hipErrorInvalidValue;
  const uint4* xs = reinterpret_cast<const uint4*>(x);
  uint2* cs = reinterpret_cast<uint2*>(codes);
  uint4* ds = reinterpret_cast<uint4*>(deq);
  const int sm = stage_major ? 1 : 0;
  if (fmt == kE4M3) rows_dispatch<kE4M3>(nchunks, st, xs, cs, scales, ds, rows, cols / 32, pairs, sm);
  else rows_dispatch<kE5M2>(nchunks, st, xs, cs, scales, ds, rows, cols / 32, pairs, sm);
  return hipGetLastError();
}

hipError_t launch_scales_to_pairs(const uint8_t* in, int64_t groups, int64_t rows, int64_t k, uint8_t* out,
                                  hipStream_t st) {
  if (k % 128) return hipErrorInvalidValue;
  const int64_t kp = k / 128;
  if (groups == 0 || rows == 0 || kp == 0) return hipSuccess;
  if (groups > 65535 || (rows + 63) / 64 > 65535 || (kp + 31) / 32 > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid(unsigned((kp + 31) / 32), unsigned((rows + 63) / 64), unsigned(groups));
  scales_to_pairs_kernel<<<grid, 256, 0, st>>>(reinterpret_cast<const uint32_t*>(in), rows, kp,
                                               reinterpret_cast<uint32_t*>(out));
  return hipGetLastError();
}

hipError_t launch_dequant_rows(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols, int fmt,
                               uint16_t* out, hipStream_t st) {
  const int64_t n16 = rows * cols / 16;
  if (n16 == 0) return hipSuccess;
  const int64_t want = (n16 + 255) / 256;
  const int blocks = int(want < 65536 ? want : 65536);
  if (fmt == kE4M3)
    dequant_rows_kernel<kE4M3><<<blocks, 256, 0, st>>>(reinterpret_cast<const uint4*>(codes), scales, n16,
                                                        reinterpret_cast<uint4*>(out));
  else
    dequant_rows_kernel<kE5M2><<<blocks, 256, 0, st>>>(reinterpret_cast<const uint4*>(codes), scales, n16,
                                                        reinterpret_cast<uint4*>(out));
  return hipGetLastError();
}

hipError_t launch_quant_cols(const uint16_t* x, int64_t rows, int64_t cols, int fmt, uint8_t* codes,
                             uint8_t* scales, hipStream_t st) {
  if (rows == 0 || cols == 0) return hipSuccess;
  dim3 grid(unsigned((cols + 8 * 256 - 1) / (8 * 256)), unsigned(rows / 32));
  const bool vec = cols % 8 == 0;
  if (fmt == kE4M3) {
    if (vec) quant_cols_kernel<kE4M3, true><<<grid, 256, 0, st>>>(x, codes, scales, rows, cols);
    else quant_cols_kernel<kE4M3, false><<<grid, 256, 0, st>>>(x, codes, scales, rows, cols);
  } else {
    if (vec) quant_cols_kernel<kE5M2, true><<<grid, 256, 0, st>>>(x, codes, scales, rows, cols);
    else quant_cols_kernel<kE5M2, false><<<grid, 256, 0, st>>>(x, codes, scales, rows, cols);
  }
  return hipGetLastError();
}

template <int FMT, bool PAIRS, bool OFF32>
static void tok_dispatch(dim3 grid, hipStream_t st, const uint16_t* x, int64_t src_rows, int64_t cols,
                         const int32_t* idx, const float* rs, int64_t rows, uint8_t* ct, uint8_t* sct, int self_rows,
                         const TokBias& b, int sm) {
  if (b.part && OFF32 && idx && rs)
    quant_tok_kernel<FMT, true, true, PAIRS, OFF32, true>
        <<<grid, 256, 0, st>>>(x, src_rows, cols, idx, rs, rows, ct, sct, self_rows, b, sm);
  else if (idx && rs)
    quant_tok_kernel<FMT, true, true, PAIRS, OFF32, false>
        <<<grid, 256, 0, st>>>(x, src_rows, cols, idx, rs, rows, ct, sct, self_rows, b, sm);
  else if (idx)
    quant_tok_kernel<FMT, true, false, PAIRS, OFF32, false>
        <<<grid, 256, 0, st>>>(x, src_rows, cols, idx, rs, rows, ct, sct, self_rows, b, sm);
  else if (rs)
    quant_tok_kernel<FMT, false, true, PAIRS, OFF32, false>
        <<<grid, 256, 0, st>>>(x, src_rows, cols, idx, rs, rows, ct, sct, self_rows, b, sm);
  else
    quant_tok_kernel<FMT, false, false, PAIRS, OFF32, false>
        <<<grid, 256, 0, st>>>(x, src_rows, cols, idx, rs, rows, ct, sct, self_rows, b, sm);
}
template <int FMT, bool PAIRS>
static void tok_dispatch(dim3 grid, hipStream_t st, const uint16_t* x, int64_t src_rows, int64_t cols,
                         const int32_t* idx, const float* rs, int64_t rows, uint8_t* ct, uint8_t* sct, int self_rows,
                         const TokBias& b, int sm) {
  const bool off32 = src_rows * cols * 2 < int64_t(v2::kOOB) && rows <= int64_t(INT32_MAX);
  if (off32)
    tok_dispatch<FMT, PAIRS, true>(grid, st, x, src_rows, cols, idx, rs, rows, ct, sct, self_rows, b, sm);
  else
    tok_dispatch<FMT, PAIRS, false>(grid, st, x, src_rows, cols, idx, rs, rows, ct, sct, self_rows, b, sm);
}

hipError_t launch_quant_tok(const uint16_t* x, int64_t src_rows, int64_t cols, const int32_t* idx,
                            const float* rowscale, int64_t rows, int fmt, uint8_t* codes_t,
                            uint8_t* scales_t, hipStream_t st, bool pairs, bool self_rows, const TokBias* bias,
                            bool stage_major) {
  if (rows == 0 || cols == 0) return hipSuccess;
  if ((pairs || stage_major) && rows % 128) return hipErrorInvalidValue;
  if (self_rows && !idx) return hipErrorInvalidValue;
  TokBias b{};
  if (bias) {   // the fused bias reductions need whole tiles, row scales and 32-bit offsets
    if (cols % kTokCols || rows % kTokRows || bias->B % kTokRows || !idx || !rowscale || self_rows ||
        src_rows * cols * 2 >= int64_t(v2::kOOB) || rows > int64_t(INT32_MAX))
      return hipErrorInvalidValue;
    b = *bias;
  }
  const int self = self_rows ? 1 : 0, sm = stage_major ? 1 : 0;
  dim3 grid(unsigned((cols + kTokCols - 1) / kTokCols), unsigned((rows + kTokRows - 1) / kTokRows));
  auto go = [&](auto F, auto PAIRS) {
    tok_dispatch<decltype(F)::value, decltype(PAIRS)::value>(grid, st, x, src_rows, cols, idx, rowscale, rows,
                                                             codes_t, scales_t, self, b, sm);
  };
  using E4 = std::integral_constant<int, kE4M3>;
  using E5 = std::integral_constant<int, kE5M2>;
  if (fmt == kE4M3) {
    if (pairs) go(E4{}, std::true_type{});
    else go(E4{}, std::false_type{});
  } else {
    if (pairs) go(E5{}, std::true_type{});
    else go(E5{}, std::false_type{});
  }
  return hipGetLastError();
}

bool quant_dual_fits(int64_t rows, int64_t cols) {
  return rows > 0 && cols > 0 && rows % 32 == 0 && cols % kDualCols == 0 && (rows + 127) / 128 <= 65535;
}

hipError_t launch_quant_dual(const uint16_t* x, int64_t rows, int64_t cols, int fmt, uint8_t* codes,
                             uint8_t* scales, uint8_t* codes_t, uint8_t* scales_t, hipStream_t st, bool stage_major,
                             bool stage_major_t) {
  if (!quant_dual_fits(rows, cols)) return hipErrorInvalidValue;
  const bool pt = rows % 128 == 0;
  if (stage_major_t && !pt) return hipErrorInvalidValue;
  const dim3 grid(unsigned(cols / kDualCols), unsigned((rows + 127) / 128));
  uint2* cs = reinterpret_cast<uint2*>(codes);
  const int sm = stage_major ? 1 : 0, smt = stage_major_t ? 1 : 0;
  if (fmt == kE4M3) {
    if (pt) quant_dual_kernel<kE4M3, true><<<grid, 256, 0, st>>>(x, rows, cols, cs, scales, codes_t, scales_t, sm, smt);
    else quant_dual_kernel<kE4M3, false><<<grid, 256, 0, st>>>(x, rows, cols, cs, scales, codes_t, scales_t, sm, smt);
  } else {
    if (pt) quant_dual_kernel<kE5M2, true><<<grid, 256, 0, st>>>(x, rows, cols, cs, scales, codes_t, scales_t, sm, smt);
    else quant_dual_kernel<kE5M2, false><<<grid, 256, 0, st>>>(x, rows, cols, cs, scales, codes_t, scales_t, sm, smt);
  }
  return hipGetLastError();
}

}  // namespace mx
