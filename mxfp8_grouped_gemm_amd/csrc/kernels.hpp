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

}  // namespace mx
