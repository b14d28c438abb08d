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

static size_t up256(size_t v) { return (v + 255) & ~size_t(255); }

/* Dense workspace: four quantised operands, codes then scales, 256-aligned. */
static void dense_regions(int64_t M, int64_t N, int64_t K, size_t off[8], size_t* total) {
  const int64_t codes[4] = {M * N, K * N, N * M, K * M};
  size_t o = 0;
  for (int i = 0; i < 4; ++i) {
    off[2 * i] = o;
    o = up256(o + size_t(codes[i]));
    off[2 * i + 1] = o;
    o = up256(o + size_t(codes[i] / 32));
  }
  *total = o;
}

size_t matmul_mxfp8_bwd_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  size_t off[8], total;
  dense_regions(M, N, K, off, &total);
  return total;
}

int matmul_mxfp8_bwd(const uint16_t* dy, const uint16_t* w, const uint16_t* x, int64_t M, int64_t N,
                     int64_t K, int fmt_dy, int fmt_w, int fmt_x, uint16_t* dx, uint16_t* dw, void* ws,
                     size_t ws_bytes, void* stream) {
  if (M <= 0 || N <= 0 || K <= 0) return fail(MXFP8_ERR_INVALID_ARG, "matmul_mxfp8_bwd: non-positive shape");
  if (M % 32 || N % 32 || K % 32)
    return fail(MXFP8_ERR_INVALID_ARG, "matmul_mxfp8_bwd: M, N, K must be multiples of 32 (got %lld %lld %lld)",
                (long long)M, (long long)N, (long long)K);
  if (!valid_fmt(fmt_dy) || !valid_fmt(fmt_w) || !valid_fmt(fmt_x))
    return fail(MXFP8_ERR_INVALID_ARG, "matmul_mxfp8_bwd: formats must be E4M3 (0) or E5M2 (1)");
  if (!dy || !w || !x || !dx || !dw || !ws) return fail(MXFP8_ERR_INVALID_ARG, "matmul_mxfp8_bwd: null pointer");
  if (!aligned16(dy) || !aligned16(w) || !aligned16(x) || !aligned16(dx) || !aligned16(dw))
    return fail(MXFP8_ERR_INVALID_ARG, "matmul_mxfp8_bwd: tensors must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(ws) & 255u)
    return fail(MXFP8_ERR_INVALID_ARG, "matmul_mxfp8_bwd: workspace must be 256-byte aligned");
  size_t off[8], total;
  dense_regions(M, N, K, off, &total);
  if (ws_bytes < total)
    return fail(MXFP8_ERR_WORKSPACE, "matmul_mxfp8_bwd: workspace %zu < %zu bytes", ws_bytes, total);
  uint8_t* base = static_cast<uint8_t*>(ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  // dX = dY W: dY along N [M,N]; W along N, transposed to [K,N]
  if ((e = mx::launch_quant_rows(dy, M, N, fmt_dy, base + off[0], base + off[1], st)) != hipSuccess)
    return hip_status(e, "quantize dY along N");
  if ((e = mx::launch_quant_tok(w, N, K, nullptr, nullptr, N, fmt_w, base + off[2], base + off[3], st)) !=
      hipSuccess)
    return hip_status(e, "quantize W along N");
  // dW = dY^T X: dY along M, transposed to [N,M]; X along M, transposed to [K,M]
  if ((e = mx::launch_quant_tok(dy, M, N, nullptr, nullptr, M, fmt_dy, base + off[4], base + off[5], st)) !=
      hipSuccess)
    return hip_status(e, "quantize dY along M");
  if ((e = mx::launch_quant_tok(x, M, K, nullptr, nullptr, M, fmt_x, base + off[6], base + off[7], st)) !=
      hipSuccess)
    return hip_status(e, "quantize X along M");
  mx::GemmStoreArgs g{};
  g.a_codes = base + off[0]; g.a_scales = base + off[1]; g.lda = N;
  g.b_codes = base + off[2]; g.b_scales = base + off[3]; g.ldb = N;
  g.M = M; g.N = K; g.K = N; g.out = dx; g.ldo = K;
  if ((e = mx::launch_gemm_store(g, 1, fmt_dy, fmt_w, st)) != hipSuccess) return hip_status(e, "dX GEMM");
  g.a_codes = base + off[4]; g.a_scales = base + off[5]; g.lda = M;
  g.b_codes = base + off[6]; g.b_scales = base + off[7]; g.ldb = M;
  g.M = N; g.N = K; g.K = M; g.out = dw; g.ldo = K;
  if ((e = mx::launch_gemm_store(g, 1, fmt_dy, fmt_x, st)) != hipSuccess) return hip_status(e, "dW GEMM");
  return ok();
}

int64_t moe_num_blocks(int64_t T, int64_t K, int64_t E, int64_t B) {
  if (T <= 0 || K <= 0 || E <= 0 || B <= 0 || T * K < E) return -1;
  // P1 "Dimensions": N = (T*TopK - (E-1))/B + E - 1, the division rounded up.
  return (T * K - (E - 1) + B - 1) / B + E - 1;
}

}  // extern "C"
