// kernels.hpp -- host-side launchers of the gfx950 kernels (internal to the
// library; the public interface is include/mxfp8_moe.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mx {

// quantize.hip
hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int64_t cols, int fmt, uint8_t* codes,
                             uint8_t* scales, hipStream_t st);
hipError_t launch_quant_cols(const uint16_t* x, int64_t rows, int64_t cols, int fmt, uint8_t* codes,
                             uint8_t* scales, hipStream_t st);
hipError_t launch_quant_tok(const uint16_t* x, int64_t src_rows, int64_t cols, const int32_t* idx,
                            const float* rowscale, int64_t rows, int fmt, uint8_t* codes_t,
                            uint8_t* scales_t, hipStream_t st);

// gemm_dense.hip: C[m][n] = sum_k A[m][k] B[n][k] -> bf16 out[g][m][n].
// A [M][lda] and B [N][ldb] fp8 codes, K-contiguous, scales [rows][ld/32].
// Without blk_list the contraction is [0, K); with it, group g contracts over
// the columns of blocks blk_list[blk_off[g] .. blk_off[g+1]) of blk bytes each.
struct GemmStoreArgs {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  int64_t lda;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  int64_t ldb;
  int64_t M, N, K;
  uint16_t* out;
  int64_t ldo;
  int64_t out_gstride;
  const int32_t* blk_off;
  const int32_t* blk_list;
  int blk;
  int tiles_m, tiles_n;
};
hipError_t launch_gemm_store(GemmStoreArgs p, int groups, int fa, int fb, hipStream_t st);

}  // namespace mx
