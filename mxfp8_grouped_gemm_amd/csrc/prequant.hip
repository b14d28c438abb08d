// prequant.hip -- layout kernels for operands that arrive already quantised
// ([P2] "Matmul MXFP8 Backward Kernel API Reference", API Reference: the
// pre-computed output_grad / weight / input scales and the pre-swizzled
// inputs).  An operand quantised along its rows' axis (axis 0: codes [R][C],
// E8M0 scales [R/32][C], as mxfp8_quantize writes them) is turned into the
// GEMM's operand layout, which keeps the contraction axis contiguous: codes
// [C][R] and scales [C][R/32] or pair-major [R/128][C][4].  Row-major scales
// of an operand already in that layout become pair-major through
// launch_scales_to_pairs (quantize.hip).  Pure data movement.
#include "kernels.hpp"

namespace mx {

// codes [R][C] -> [C][R] (R % 32 == 0, C % 32 == 0): a workgroup moves a
// 64 x 64 tile through LDS, reading and writing 16-byte runs; runs past the
// matrix are skipped (whole runs: both sizes are multiples of 16).
__global__ void __launch_bounds__(256) transpose_u8_kernel(const uint8_t* __restrict__ in, int64_t R, int64_t C,
                                                           uint8_t* __restrict__ out) {
  __shared__ uint8_t tile[64][64 + 4];
  const int64_t r0 = int64_t(blockIdx.y) * 64, c0 = int64_t(blockIdx.x) * 64;
  const int t = threadIdx.x, row = t >> 2, chunk = t & 3;
  if (r0 + row < R && c0 + 16 * chunk < C) {
    const uint4 v = *reinterpret_cast<const uint4*>(in + (r0 + row) * C + c0 + 16 * chunk);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 16; ++k) tile[row][16 * chunk + k] = uint8_t(w[k >> 2] >> (8 * (k & 3)));
  }
  __syncthreads();
  // output row c0 + row (a column of the input), bytes r0 + 16 * chunk ..
  if (c0 + row < C && r0 + 16 * chunk < R) {
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < 16; ++k) w[k >> 2] |= uint32_t(tile[16 * chunk + k][row]) << (8 * (k & 3));
    *reinterpret_cast<uint4*>(out + (c0 + row) * R + r0 + 16 * chunk) = uint4{w[0], w[1], w[2], w[3]};
  }
}

// scales [R/32][C] (groups along R) -> pair-major [R/128][C][4]: word (p, c)
// holds column c's bytes of groups 4p .. 4p + 3 (R % 128 == 0).
__global__ void __launch_bounds__(256) scales_axis0_to_pairs_kernel(const uint8_t* __restrict__ in, int64_t R,
                                                                    int64_t C, uint32_t* __restrict__ out) {
  const int64_t n = (R / 128) * C;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
    const int64_t p = i / C, c = i - p * C;
    const uint8_t* s = in + 4 * p * C + c;
    out[i] = uint32_t(s[0]) | (uint32_t(s[C]) << 8) | (uint32_t(s[2 * C]) << 16) | (uint32_t(s[3 * C]) << 24);
  }
}

// scales [R/32][C] -> row-major [C][R/32] (a byte transpose; R % 32 == 0).
__global__ void __launch_bounds__(256) scales_axis0_to_rows_kernel(const uint8_t* __restrict__ in, int64_t R,
                                                                   int64_t C, uint8_t* __restrict__ out) {
  const int64_t G = R / 32, n = G * C;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
    const int64_t g = i / C, c = i - g * C;
    out[c * G + g] = in[i];
  }
}

hipError_t launch_transpose_codes(const uint8_t* in, int64_t R, int64_t C, uint8_t* out, hipStream_t st) {
  if (R == 0 || C == 0) return hipSuccess;
  if (R % 32 || C % 32 || (C + 63) / 64 > INT32_MAX || (R + 63) / 64 > 65535) return hipErrorInvalidValue;
  transpose_u8_kernel<<<dim3(unsigned((C + 63) / 64), unsigned((R + 63) / 64)), 256, 0, st>>>(in, R, C, out);
  return hipGetLastError();
}

hipError_t launch_scales_axis0(const uint8_t* in, int64_t R, int64_t C, uint8_t* out, bool pairs, hipStream_t st) {
  if (R == 0 || C == 0) return hipSuccess;
  if (R % 32 || (pairs && R % 128)) return hipErrorInvalidValue;
  const int64_t n = pairs ? (R / 128) * C : (R / 32) * C;
  const int64_t want = (n + 255) / 256;
  const unsigned grid = unsigned(want < 16384 ? want : 16384);
  if (pairs) scales_axis0_to_pairs_kernel<<<grid, 256, 0, st>>>(in, R, C, reinterpret_cast<uint32_t*>(out));
  else scales_axis0_to_rows_kernel<<<grid, 256, 0, st>>>(in, R, C, out);
  return hipGetLastError();
}

}  // namespace mx
