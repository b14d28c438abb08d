// api.cpp -- the C ABI (include/mxfp8_moe.h): argument validation, workspace
// carving and the launch sequence on the caller's stream.  No device memory is
// allocated here and nothing is synchronised.
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/mxfp8_moe.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return MXFP8_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MXFP8_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool valid_fmt(int f) { return f == MXFP8_E4M3 || f == MXFP8_E5M2; }

}  // namespace

extern "C" {

const char* mxfp8_last_error(void) { return g_last_error.c_str(); }

const char* mxfp8_version(void) { return "mxfp8_moe 0.1.0 (gfx950)"; }

int mxfp8_quantize(const uint16_t* x, int64_t rows, int64_t cols, int axis, int fmt, uint8_t* codes,
                   uint8_t* scales, void* stream) {
  if (rows < 0 || cols < 0) return fail(MXFP8_ERR_INVALID_ARG, "mxfp8_quantize: negative shape");
  if (!valid_fmt(fmt)) return fail(MXFP8_ERR_INVALID_ARG, "mxfp8_quantize: fmt %d is not E4M3/E5M2", fmt);
  if (axis != 0 && axis != 1) return fail(MXFP8_ERR_INVALID_ARG, "mxfp8_quantize: axis must be 0 or 1");
  if (axis == 1 && cols % 32) return fail(MXFP8_ERR_INVALID_ARG, "mxfp8_quantize: cols %% 32 != 0");
  if (axis == 0 && rows % 32) return fail(MXFP8_ERR_INVALID_ARG, "mxfp8_quantize: rows %% 32 != 0");
  if (rows == 0 || cols == 0) return ok();
  if (!x || !codes || !scales) return fail(MXFP8_ERR_INVALID_ARG, "mxfp8_quantize: null pointer");
  if (!aligned16(x) || !aligned16(codes))
    return fail(MXFP8_ERR_INVALID_ARG, "mxfp8_quantize: x and codes must be 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (axis == 1) return hip_status(mx::launch_quant_rows(x, rows, cols, fmt, codes, scales, st), "quant_rows");
  return hip_status(mx::launch_quant_cols(x, rows, cols, fmt, codes, scales, st), "quant_cols");
}

int64_t moe_num_blocks(int64_t T, int64_t K, int64_t E, int64_t B) {
  if (T <= 0 || K <= 0 || E <= 0 || B <= 0 || T * K < E) return -1;
  // P1 "Dimensions": N = (T*TopK - (E-1))/B + E - 1, the division rounded up.
  return (T * K - (E - 1) + B - 1) / B + E - 1;
}

}  // extern "C"
