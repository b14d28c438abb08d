// api.cpp -- the C ABI (include/mxfp8_moe.h): argument validation, workspace
// carving and the launch sequence on the caller's stream.  No device memory is
// allocated here and nothing is synchronised.
#include <climits>
#include <atomic>
#include <mutex>
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

// The four GEMM operand streams of the dense backward: rows, contraction, and
// the workspace regions (codes, scales) they are built in when the caller does
// not supply them in the GEMM's layout.
struct DenseOperand {
  const uint8_t* codes;    // what the GEMM reads
  const uint8_t* scales;
};

static int dense_check(const matmul_mxfp8_bwd_args* a) {
  if (!a) return fail(MXFP8_ERR_INVALID_ARG, "matmul_mxfp8_bwd: null args");
  const int64_t M = a->M, N = a->N, K = a->K;
  if (M <= 0 || N <= 0 || K <= 0) return fail(MXFP8_ERR_INVALID_ARG, "matmul_mxfp8_bwd: non-positive shape");
  if (M % 32 || N % 32 || K % 32)
    return fail(MXFP8_ERR_INVALID_ARG, "matmul_mxfp8_bwd: M, N, K must be multiples of 32 (got %lld %lld %lld)",
                (long long)M, (long long)N, (long long)K);
  if (!valid_fmt(a->fmt_output_grad) || !valid_fmt(a->fmt_weights) || !valid_fmt(a->fmt_input))
    return fail(MXFP8_ERR_INVALID_ARG, "matmul_mxfp8_bwd: formats must be E4M3 (0) or E5M2 (1)");
  const int flags[4] = {a->output_grad_is_swizzled, a->weights_is_swizzled, a->input_is_swizzled,
                        a->use_scale_packing};
  for (int f : flags)
    if (f != 0 && f != 1) return fail(MXFP8_ERR_INVALID_ARG, "matmul_mxfp8_bwd: flags must be 0 or 1");
  struct Pre { const uint8_t* c; const uint8_t* s; int swz; int64_t kdim; const char* name; };
  const Pre pre[4] = {{a->output_grad_codes_n, a->output_grad_scales_n, a->output_grad_is_swizzled, N, "output_grad (along N)"},
                      {a->weight_codes, a->weight_scales, a->weights_is_swizzled, N, "weights"},
                      {a->output_grad_codes_m, a->output_grad_scales_m, a->output_grad_is_swizzled, M, "output_grad (along M)"},
                      {a->input_codes, a->input_scales, a->input_is_swizzled, M, "input_activation"}};
  for (const Pre& q : pre) {
    if ((q.c == nullptr) != (q.s == nullptr))
      return fail(MXFP8_ERR_INVALID_ARG, "matmul_mxfp8_bwd: %s: pre-quantised codes and scales go together", q.name);
    if (q.c && (!aligned16(q.c) || !aligned16(q.s)))
      return fail(MXFP8_ERR_INVALID_ARG, "matmul_mxfp8_bwd: %s: codes and scales must be 16-byte aligned", q.name);
    if (q.c && a->use_scale_packing && !q.swz)
      return fail(MXFP8_ERR_INVALID_ARG, "matmul_mxfp8_bwd: %s: packed scales come with the swizzled layout", q.name);
    if (q.c && q.swz && a->use_scale_packing && q.kdim % 128)
      return fail(MXFP8_ERR_INVALID_ARG, "matmul_mxfp8_bwd: %s: packed scales need a contraction that is a "
                  "multiple of 128", q.name);
  }
  if (a->output_grad_is_swizzled && !a->output_grad_codes_n && !a->output_grad_codes_m)
    return fail(MXFP8_ERR_INVALID_ARG, "matmul_mxfp8_bwd: output_grad_is_swizzled without pre-quantised output_grad");
  if (a->weights_is_swizzled && !a->weight_codes)
    return fail(MXFP8_ERR_INVALID_ARG, "matmul_mxfp8_bwd: weights_is_swizzled without pre-quantised weights");
  if (a->input_is_swizzled && !a->input_codes)
    return fail(MXFP8_ERR_INVALID_ARG, "matmul_mxfp8_bwd: input_is_swizzled without pre-quantised input_activation");
  if (a->use_scale_packing && !a->output_grad_codes_n && !a->output_grad_codes_m && !a->weight_codes && !a->input_codes)
    return fail(MXFP8_ERR_INVALID_ARG, "matmul_mxfp8_bwd: use_scale_packing without a pre-quantised input");
  const bool need_dy = !a->output_grad_codes_n || !a->output_grad_codes_m;
  if ((need_dy && !a->output_grad) || (!a->weight_codes && !a->weights) || (!a->input_codes && !a->input_activation) ||
      !a->input_grad || !a->weight_grad)
    return fail(MXFP8_ERR_INVALID_ARG, "matmul_mxfp8_bwd: null pointer (a bf16 input that is not given pre-quantised, "
                "or an output)");
  const void* al[5] = {need_dy ? a->output_grad : nullptr, a->weight_codes ? nullptr : a->weights,
                       a->input_codes ? nullptr : a->input_activation, a->input_grad, a->weight_grad};
  for (const void* q : al)
    if (q && !aligned16(q)) return fail(MXFP8_ERR_INVALID_ARG, "matmul_mxfp8_bwd: tensors must be 16-byte aligned");
  return MXFP8_OK;
}

static int dense_run(const matmul_mxfp8_bwd_args* a, void* ws, size_t ws_bytes, void* stream, int lo, int hi) {
  int rc = dense_check(a);
  if (rc) return rc;
  const int64_t M = a->M, N = a->N, K = a->K;
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255u))
    return fail(MXFP8_ERR_INVALID_ARG, "matmul_mxfp8_bwd: workspace must be non-null and 256-byte aligned");
  size_t off[8], total;
  dense_regions(M, N, K, off, &total);
  if (ws_bytes < total)
    return fail(MXFP8_ERR_WORKSPACE, "matmul_mxfp8_bwd: workspace %zu < %zu bytes", ws_bytes, total);
  uint8_t* base = static_cast<uint8_t*>(ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  // Operands of a GEMM whose contraction is a multiple of 128 feed the ring
  // loop and get pair-major scales.  Stream i of the GEMMs (rows x contraction): 0 dY along N (M x N), 1 W^T
  // (K x N), 2 dY^T (N x M), 3 X^T (K x M).  Each is quantised from bf16 into
  // workspace region i, or built there from a pre-quantised operand, or read
  // in place when the caller's operand already has the GEMM's layout.
  DenseOperand op[4];
  for (int i = 0; i < 4; ++i) op[i] = {base + off[2 * i], base + off[2 * i + 1]};
  const int64_t rows[4] = {M, K, N, K}, kdim[4] = {N, N, M, M};
  const uint8_t* pc[4] = {a->output_grad_codes_n, a->weight_codes, a->output_grad_codes_m, a->input_codes};
  const uint8_t* ps[4] = {a->output_grad_scales_n, a->weight_scales, a->output_grad_scales_m, a->input_scales};
  const int swz[4] = {a->output_grad_is_swizzled, a->weights_is_swizzled, a->output_grad_is_swizzled,
                      a->input_is_swizzled};
  // natural (unswizzled) source of streams 1-3: codes [kdim][rows], scales [kdim/32][rows]
  for (int i = 0; i < 4; ++i) {
    if (!pc[i]) continue;
    const bool pairs = kdim[i] % 128 == 0;
    if (i == 0 || swz[i]) {   // codes already [rows][kdim]
      op[i].codes = pc[i];
      if (!pairs || a->use_scale_packing) op[i].scales = ps[i];   // the GEMM's scale layout as given
    }
  }
  const uint16_t* dy = a->output_grad;
  const int fdy = a->fmt_output_grad, fw = a->fmt_weights, fx = a->fmt_input;
  // A GEMM whose two operands are both quantised here from bf16, on the ring
  // loop (contraction a multiple of 128), gets them stage-major and runs the
  // four-slot ring: whole cache lines per DMA instruction (mx_device.hpp,
  // stage_major_off).  Operands the caller hands in keep their row-major layout.
  const bool sm_dx = !pc[0] && !pc[1] && N % 128 == 0 && N < (int64_t(1) << 24) &&
                     M * (N / 32) <= int64_t(UINT32_MAX);
  const bool sm_dw = !pc[2] && !pc[3] && M % 128 == 0 && M < (int64_t(1) << 24);
  const bool sm[4] = {sm_dx, sm_dx, sm_dw, sm_dw};
  // dY along both axes from one read where the shapes allow (stage 0 then makes stream 2 too)
  const bool dual = !pc[0] && !pc[2] && mx::quant_dual_fits(M, N);
  auto prep = [&](int i) -> hipError_t {
    const bool pairs = kdim[i] % 128 == 0;
    uint8_t* wc = base + off[2 * i];
    uint8_t* wsc = base + off[2 * i + 1];
    if (dual && i == 0)
      return mx::launch_quant_dual(dy, M, N, fdy, wc, wsc, base + off[4], base + off[5], st, sm[0], sm[2]);
    if (dual && i == 2) return hipSuccess;
    if (!pc[i]) {   // quantise from bf16 along the contraction
      switch (i) {
        case 0: return mx::launch_quant_rows(dy, M, N, fdy, wc, wsc, st, nullptr, pairs, sm[0]);
        case 1:
          return mx::launch_quant_tok(a->weights, N, K, nullptr, nullptr, N, fw, wc, wsc, st, pairs, false, nullptr,
                                      sm[1]);
        case 2:
          return mx::launch_quant_tok(dy, M, N, nullptr, nullptr, M, fdy, wc, wsc, st, pairs, false, nullptr, sm[2]);
        default:
          return mx::launch_quant_tok(a->input_activation, M, K, nullptr, nullptr, M, fx, wc, wsc, st, pairs, false,
                                      nullptr, sm[3]);
      }
    }
    if (i == 0 || swz[i]) {   // GEMM layout: at most the row-major scales become pair-major
      if (pairs && !a->use_scale_packing) return mx::launch_scales_to_pairs(ps[i], 1, rows[i], kdim[i], wsc, st);
      return hipSuccess;
    }
    hipError_t r = mx::launch_transpose_codes(pc[i], kdim[i], rows[i], wc, st);
    if (r != hipSuccess) return r;
    return mx::launch_scales_axis0(ps[i], kdim[i], rows[i], wsc, pairs, st);
  };
  // stage 0 -- the dX operands (dY along N; W along N); stage 1 -- the dW operands
  for (int i = 0; i < 4; ++i) {
    const int stage = i < 2 ? 0 : 1;
    if (lo <= stage && stage <= hi && (e = prep(i)) != hipSuccess) return hip_status(e, "operand preparation");
  }
  mx::GemmStoreArgs g{};
  g.a_codes = op[0].codes; g.a_scales = op[0].scales; g.lda = N;
  g.b_codes = op[1].codes; g.b_scales = op[1].scales; g.ldb = N;
  g.M = M; g.N = K; g.K = N; g.out = a->input_grad; g.ldo = K;
  // row-major operands: the pair-slot ring, measured 6% faster than the
  // four-slot ring on 8192^3, 5% on 4096^3
  g.stage_major = sm_dx;
  g.pair = sm_dx ? 0 : 1;
  // stage 2 -- dX GEMM
  if (lo <= 2 && 2 <= hi && (e = mx::launch_gemm_store(g, 1, fdy, fw, st)) != hipSuccess)
    return hip_status(e, "dX GEMM");
  g.a_codes = op[2].codes; g.a_scales = op[2].scales; g.lda = M;
  g.b_codes = op[3].codes; g.b_scales = op[3].scales; g.ldb = M;
  g.M = N; g.N = K; g.K = M; g.out = a->weight_grad; g.ldo = K;
  g.stage_major = sm_dw;
  g.pair = sm_dw ? 0 : 1;
  // stage 3 -- dW GEMM
  if (lo <= 3 && 3 <= hi && (e = mx::launch_gemm_store(g, 1, fdy, fx, st)) != hipSuccess)
    return hip_status(e, "dW GEMM");
  return ok();
}

static matmul_mxfp8_bwd_args dense_plain_args(const uint16_t* dy, const uint16_t* w, const uint16_t* x, int64_t M,
                                              int64_t N, int64_t K, int fmt_dy, int fmt_w, int fmt_x, uint16_t* dx,
                                              uint16_t* dw) {
  matmul_mxfp8_bwd_args a{};
  a.M = M; a.N = N; a.K = K;
  a.output_grad = dy; a.weights = w; a.input_activation = x;
  a.fmt_output_grad = fmt_dy; a.fmt_weights = fmt_w; a.fmt_input = fmt_x;
  a.input_grad = dx; a.weight_grad = dw;
  return a;
}

int matmul_mxfp8_bwd(const uint16_t* dy, const uint16_t* w, const uint16_t* x, int64_t M, int64_t N, int64_t K,
                     int fmt_dy, int fmt_w, int fmt_x, uint16_t* dx, uint16_t* dw, void* ws, size_t ws_bytes,
                     void* stream) {
  const matmul_mxfp8_bwd_args a = dense_plain_args(dy, w, x, M, N, K, fmt_dy, fmt_w, fmt_x, dx, dw);
  return dense_run(&a, ws, ws_bytes, stream, 0, 3);
}

int matmul_mxfp8_bwd_ex(const matmul_mxfp8_bwd_args* a, void* ws, size_t ws_bytes, void* stream) {
  return dense_run(a, ws, ws_bytes, stream, 0, 3);
}

int matmul_mxfp8_bwd_stage(const uint16_t* dy, const uint16_t* w, const uint16_t* x, int64_t M, int64_t N,
                           int64_t K, int fmt_dy, int fmt_w, int fmt_x, uint16_t* dx, uint16_t* dw, void* ws,
                           size_t ws_bytes, int stage, void* stream) {
  if (stage < 0 || stage > 3) return fail(MXFP8_ERR_INVALID_ARG, "matmul_mxfp8_bwd_stage: stage %d outside [0,4)", stage);
  const matmul_mxfp8_bwd_args a = dense_plain_args(dy, w, x, M, N, K, fmt_dy, fmt_w, fmt_x, dx, dw);
  return dense_run(&a, ws, ws_bytes, stream, stage, stage);
}

int64_t moe_num_blocks(int64_t T, int64_t K, int64_t E, int64_t B) {
  if (T <= 0 || K <= 0 || E <= 0 || B <= 0 || T * K < E) return -1;
  // P1 "Dimensions": N = (T*TopK - (E-1))/B + E - 1, the division rounded up.
  return (T * K - (E - 1) + B - 1) / B + E - 1;
}

size_t moe_build_blocks_workspace_size(int64_t E) {
  return E > 0 ? up256(size_t(mx::build_blocks_workspace_bytes(E))) : 0;
}

int moe_build_blocks(const int32_t* topk, int64_t T, int64_t K, int64_t E, int64_t B, int64_t N, int32_t* tpid,
                     int32_t* b2e, void* ws, size_t ws_bytes, void* stream) {
  if (T <= 0 || K <= 0 || E <= 0 || B <= 0 || N <= 0)
    return fail(MXFP8_ERR_INVALID_ARG, "moe_build_blocks: sizes must be positive");
  const int64_t need = moe_num_blocks(T, K, E, B);
  if (need < 0) return fail(MXFP8_ERR_INVALID_ARG, "moe_build_blocks: T*K (%lld) < E (%lld)", (long long)(T * K), (long long)E);
  if (N < need)
    return fail(MXFP8_ERR_INVALID_ARG, "moe_build_blocks: N = %lld is below the worst case %lld", (long long)N,
                (long long)need);
  if (!topk || !tpid || !b2e || !ws) return fail(MXFP8_ERR_INVALID_ARG, "moe_build_blocks: null pointer");
  if (ws_bytes < moe_build_blocks_workspace_size(E))
    return fail(MXFP8_ERR_WORKSPACE, "moe_build_blocks: workspace too small");
  if (T * K > INT32_MAX || N * B > INT32_MAX)
    return fail(MXFP8_ERR_UNSUPPORTED, "moe_build_blocks: sizes beyond int32 indexing");
  return hip_status(mx::launch_build_blocks(topk, T, K, E, B, N, tpid, b2e, static_cast<int32_t*>(ws),
                                            static_cast<hipStream_t>(stream)),
                    "moe_build_blocks");
}

int moe_build_blocks_noalloc(const int32_t* topk, int64_t T, int64_t K, int64_t E, int64_t B, int64_t N,
                             int32_t* tpid, int32_t* b2e, void* stream) {
  if (T <= 0 || K <= 0 || E <= 0 || B <= 0 || N <= 0)
    return fail(MXFP8_ERR_INVALID_ARG, "moe_build_blocks_noalloc: sizes must be positive");
  if (E > MOE_BUILD_BLOCKS_NOALLOC_MAX_EXPERTS || E > mx::build_blocks_noalloc_max_experts())
    return fail(MXFP8_ERR_UNSUPPORTED,
                "moe_build_blocks_noalloc: E = %lld is above the %d experts its scratch holds "
                "(use moe_build_blocks with a workspace)",
                (long long)E, MOE_BUILD_BLOCKS_NOALLOC_MAX_EXPERTS);
  const int64_t need = moe_num_blocks(T, K, E, B);
  if (need < 0)
    return fail(MXFP8_ERR_INVALID_ARG, "moe_build_blocks_noalloc: T*K (%lld) < E (%lld)", (long long)(T * K),
                (long long)E);
  if (N < need)
    return fail(MXFP8_ERR_INVALID_ARG, "moe_build_blocks_noalloc: N = %lld is below the worst case %lld",
                (long long)N, (long long)need);
  if (!topk || !tpid || !b2e) return fail(MXFP8_ERR_INVALID_ARG, "moe_build_blocks_noalloc: null pointer");
  if (T * K > INT32_MAX || N * B > INT32_MAX)
    return fail(MXFP8_ERR_UNSUPPORTED, "moe_build_blocks_noalloc: sizes beyond int32 indexing");
  hipStream_t st = static_cast<hipStream_t>(stream);
  int device = -1;
  hipError_t e = st ? hipStreamGetDevice(st, &device) : hipGetDevice(&device);
  if (e != hipSuccess) return hip_status(e, "moe_build_blocks_noalloc: device of the stream");
  int32_t* scratch = nullptr;
  if ((e = mx::build_blocks_scratch(device, &scratch)) != hipSuccess)
    return hip_status(e, "moe_build_blocks_noalloc: address of the scratch array");
  return hip_status(mx::launch_build_blocks(topk, T, K, E, B, N, tpid, b2e, scratch, st), "moe_build_blocks_noalloc");
}

/* ---- MoE backward -------------------------------------------------------- */

// A whole backward with few rounds of Phase-3 tiles runs the steps that do
// not depend on each other on two streams: the caller's carries routing
// set-up, dY along H, Phase 1 with its epilogue, Phase 3 and the
// finalisation; a second stream of the library's carries the token-axis
// gathers (with the bias reductions) and then Phases 2 and 4, which fill the
// CUs that the last, partial round of Phase 3's tiles leaves idle.  Measured:
// 3.5% faster on the medium workload (Phase 3 in 4.6 rounds of tiles over the
// CUs), 0.3% and 1% slower with 9.8 and 51 rounds (large, fine), where the
// two streams' GEMMs share the L2s for little idle time; hence the rule of
// fewer than 8 rounds (kOverlapRounds).  Below one round the work is too
// short for the events to pay (the tiny workload's step went 0.096 -> 0.150
// ms), so from one round on.  The second stream (default
// priority, non-blocking) and its four events are made per device on first
// use and kept until the process ends; whole backwards on one device take its
// mutex while they enqueue, and the caller's stream waits for the second one
// before the call returns, so stream order is as if one stream did it all.
constexpr int64_t kOverlapRounds = 8;
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t ev[4] = {};   // after dY along H; after the epilogue; after the gathers; at the end
  std::mutex mu;
  bool made = false, ok = false;
};
static SideStream* side_stream(int device) {
  constexpr int kMaxDevices = 64;
  static SideStream per[kMaxDevices];
  static std::mutex init_mu;
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(init_mu);
  SideStream& x = per[device];
  if (!x.made) {
    x.made = true;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != device && hipSetDevice(device) != hipSuccess) return nullptr;
    bool good = hipStreamCreateWithFlags(&x.s, hipStreamNonBlocking) == hipSuccess;
    for (int i = 0; i < 4 && good; ++i) good = hipEventCreateWithFlags(&x.ev[i], hipEventDisableTiming) == hipSuccess;
    if (cur != device) good = hipSetDevice(cur) == hipSuccess && good;
    x.ok = good;
  }
  return x.ok ? &x : nullptr;
}
// CUs of the device that `st` runs on (0 if unknown), looked up once per device.
static int device_cus(hipStream_t st) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int device = -1;
  if ((st ? hipStreamGetDevice(st, &device) : hipGetDevice(&device)) != hipSuccess || device < 0 ||
      device >= kMaxDevices)
    return 0;
  int c = cache[device].load(std::memory_order_relaxed);
  if (c <= 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || c <= 0) return 0;
    cache[device].store(c, std::memory_order_relaxed);
  }
  return c;
}
// An expert weight operand at least this large (8x one XCD's 4 MB L2) is shared
// by all XCDs through the infinity cache: its GEMM hands tiles out round robin
// (moe_tiles.hpp).
constexpr int64_t kRoundRobinWeightBytes = int64_t(32) << 20;

// The bias reductions ride on the gather of dY rows (one read of each row)
// when H is a multiple of 128 and those rows are gathered, i.e. no a*dY
// checkpoint replaces them, and dY is under 2 GiB (that gather then reads it
// at 32-bit offsets); otherwise they run as kernels of their own.
static bool moe_fuse_bias(const moe_bwd_mxfp8_args* a) {
  return a->has_bias && a->H % 128 == 0 && !a->down_proj_act_checkpoint && a->T * a->H * 2 <= INT32_MAX;
}

// Phase 1 with its epilogue in one kernel (the conditions of mx::phase1_fusable,
// which its launcher checks again): no dS in HBM, and no tile ranges.
static bool moe_phase1_fused(const moe_bwd_mxfp8_args* a) {
  return a->H % 128 == 0 && a->H <= 2048 && a->I <= 512 && !a->gate_act_checkpoint_T &&
         !a->intermediate_checkpoint_T && !a->scaled_intermediate_checkpoint_T;
}

static int moe_layout(const moe_bwd_mxfp8_args* a, moe_bwd_mxfp8_workspace_layout* L) {
  const int64_t T = a->T, H = a->H, I = a->I, E = a->E, N = a->N, B = a->block_size, P = N * B;
  size_t o = 0;
  auto put = [&](size_t& field, int64_t bytes) {
    field = o;
    o = up256(o + size_t(bytes));
  };
  const bool h_pairs = H % 128 == 0;   // Phase 1 reads the codes (else their bf16 values)
  put(L->dy_codes, T * H);
  put(L->dy_scales, T * H / 32);
  put(L->dy_deq, h_pairs ? 0 : T * H * 2);
  put(L->wd_deq, h_pairs ? 0 : E * I * H * 2);
  put(L->x_tok_codes, H * P);
  put(L->x_tok_scales, H * P / 32);
  put(L->gy_tok_codes, H * P);
  put(L->gy_tok_scales, H * P / 32);
  put(L->inter_tok_codes, I * P);
  put(L->inter_tok_scales, I * P / 32);
  put(L->dgu_row_codes, P * 2 * I);
  put(L->dgu_row_scales, P * 2 * I / 32);
  put(L->dgu_tok_codes, 2 * I * P);
  put(L->dgu_tok_scales, 2 * I * P / 32);
  put(L->wgu_scales_pairs, E * H * 2 * I / 32);
  put(L->wd_scales_pairs, h_pairs ? E * I * H / 32 : 0);
  const bool fused = moe_phase1_fused(a);
  put(L->phase1_ds, fused ? 0 : N * I * B * 4);
  // tile starts [N+1], then the tile -> block map over every tile a block can
  // have at the smallest tile (128 x 128)
  put(L->phase1_tiles, fused ? 0 : (N + 1 + N * ((I + 127) / 128) * ((B + 127) / 128)) * 4);
  put(L->phase3_tiles, (N + 1 + N * ((B + 127) / 128) * ((H + 127) / 128)) * 4);
  put(L->dx_slot, N * B * H * 4);
  {
    mx::Phase3Args q{};
    q.H = H; q.I = I; q.N = N; q.B = B;
    put(L->phase3_parts, mx::phase3_parts_bytes(q));
  }
  put(L->slot_of, T * E * 4);
  put(L->daff_slot, P * 4);
  put(L->daff_part, (I / 32 + (moe_fuse_bias(a) ? H / 128 : 0)) * P * 4);
  put(L->db1_acc, E * 2 * I * 4);
  put(L->db2_acc, E * H * 4);
  put(L->expert_block_offsets, (E + 1) * 4);
  put(L->expert_block_list, N * 4);
  put(L->slot_token, P * 4);
  put(L->slot_affinity, P * 4);
  put(L->block_flag, N * 4);
  L->total = o;
  return MXFP8_OK;
}

static int moe_check_shapes(const moe_bwd_mxfp8_args* a) {
  if (!a) return fail(MXFP8_ERR_INVALID_ARG, "moe_bwd_mxfp8: null args");
  if (a->T <= 0 || a->H <= 0 || a->I <= 0 || a->E <= 0 || a->N <= 0 || a->block_size <= 0)
    return fail(MXFP8_ERR_INVALID_ARG, "moe_bwd_mxfp8: sizes must be positive");
  if (a->H % 32 || a->I % 32)
    return fail(MXFP8_ERR_INVALID_ARG, "moe_bwd_mxfp8: H and I must be multiples of 32 (got %lld, %lld)",
                (long long)a->H, (long long)a->I);
  const int64_t B = a->block_size;
  if (B != 128 && B != 256 && B != 512 && B != 1024)
    return fail(MXFP8_ERR_UNSUPPORTED, "moe_bwd_mxfp8: block_size %lld not in {128,256,512,1024}", (long long)B);
  if (a->N * B > INT32_MAX || a->T * a->E > INT32_MAX || a->T * a->H > INT32_MAX)
    return fail(MXFP8_ERR_UNSUPPORTED, "moe_bwd_mxfp8: sizes beyond 32-bit indexing");
  // Phase 1 gathers dY's code rows ([T, H] bytes) through one buffer at 32-bit
  // offsets: T * H < 2^31.  Where H is not a multiple of 128 it gathers dY's
  // bf16 values (twice the bytes) that way instead.
  if (a->T * a->H * 2 > INT32_MAX && a->H % 128)
    return fail(MXFP8_ERR_UNSUPPORTED,
                "moe_bwd_mxfp8: a [T,H] bf16 tensor of 2 GiB or more needs H %% 128 == 0 (32-bit indexing)");
  // the stage-major operands' panels (256 rows over P slots or 2I) are read through one buffer
  if (a->N * B * 256 > int64_t(UINT32_MAX) || 2 * a->I * 256 > int64_t(UINT32_MAX))
    return fail(MXFP8_ERR_UNSUPPORTED, "moe_bwd_mxfp8: N * block_size = %lld slots beyond 2^24 or I = %lld beyond 2^23",
                (long long)(a->N * B), (long long)a->I);
  if (a->I * B * 4 > INT32_MAX)   // a block's checkpoint / product is read through one buffer
    return fail(MXFP8_ERR_UNSUPPORTED, "moe_bwd_mxfp8: I * block_size * 4 = %lld bytes beyond 2 GiB",
                (long long)(a->I * B * 4));
  return MXFP8_OK;
}

int moe_bwd_mxfp8_workspace_query(const moe_bwd_mxfp8_args* a, moe_bwd_mxfp8_workspace_layout* L) {
  int rc = moe_check_shapes(a);
  if (rc) return rc;
  if (!L) return fail(MXFP8_ERR_INVALID_ARG, "moe_bwd_mxfp8_workspace_query: null layout");
  moe_layout(a, L);
  return ok();
}

size_t moe_bwd_mxfp8_workspace_size(const moe_bwd_mxfp8_args* a) {
  moe_bwd_mxfp8_workspace_layout L;
  if (moe_bwd_mxfp8_workspace_query(a, &L)) return 0;
  return L.total;
}

static int moe_run(const moe_bwd_mxfp8_args* a, void* ws, size_t ws_bytes, void* stream, int lo, int hi) {
  int rc = moe_check_shapes(a);
  if (rc) return rc;
  if (!valid_fmt(a->fmt_weight) || !valid_fmt(a->fmt_act) || !valid_fmt(a->fmt_grad))
    return fail(MXFP8_ERR_INVALID_ARG, "moe_bwd_mxfp8: formats must be E4M3 (0) or E5M2 (1)");
  if (a->affinity_on != 0 && a->affinity_on != 1)
    return fail(MXFP8_ERR_INVALID_ARG, "moe_bwd_mxfp8: affinity_on must be 0 (H) or 1 (I)");
  if (a->has_bias != 0 && a->has_bias != 1) return fail(MXFP8_ERR_INVALID_ARG, "moe_bwd_mxfp8: has_bias must be 0/1");
  if (a->accumulate != 0 && a->accumulate != 1)
    return fail(MXFP8_ERR_INVALID_ARG, "moe_bwd_mxfp8: accumulate must be 0/1");
  if (a->activation != MXFP8_ACT_SWIGLU && a->activation != MXFP8_ACT_GEGLU)
    return fail(MXFP8_ERR_INVALID_ARG, "moe_bwd_mxfp8: activation must be 0 (SwiGLU) or 1 (GeGLU)");
  if (a->affinity_on == 1 && a->has_bias)
    return fail(MXFP8_ERR_UNSUPPORTED, "moe_bwd_mxfp8: a bias with the affinity on I is not supported");
  const void* req[] = {a->hidden_states, a->expert_affinities_masked, a->gate_up_codes, a->gate_up_scales,
                       a->down_codes, a->down_scales, a->token_position_to_id, a->block_to_expert,
                       a->output_hidden_states_grad, a->gate_up_proj_act_checkpoint_T, a->hidden_states_grad,
                       a->expert_affinities_masked_grad, a->gate_up_proj_weight_grad, a->down_proj_weight_grad};
  for (const void* q : req)
    if (!q) return fail(MXFP8_ERR_INVALID_ARG, "moe_bwd_mxfp8: a required pointer is null");
  for (const void* q : req)
    if (!aligned16(q)) return fail(MXFP8_ERR_INVALID_ARG, "moe_bwd_mxfp8: tensors must be 16-byte aligned");
  if (a->has_bias) {
    if (!a->down_proj_bias || !a->gate_and_up_proj_bias_grad || !a->down_proj_bias_grad)
      return fail(MXFP8_ERR_INVALID_ARG, "moe_bwd_mxfp8: has_bias needs down_proj_bias and both bias grads");
    if (!aligned16(a->down_proj_bias) || !aligned16(a->gate_and_up_proj_bias_grad) ||
        !aligned16(a->down_proj_bias_grad))
      return fail(MXFP8_ERR_INVALID_ARG, "moe_bwd_mxfp8: bias tensors must be 16-byte aligned");
  }
  if (a->scaled_intermediate_checkpoint_T && a->affinity_on != 1)
    return fail(MXFP8_ERR_INVALID_ARG, "moe_bwd_mxfp8: scaled_intermediate_checkpoint_T needs the affinity on I");
  if (a->down_proj_act_checkpoint && a->affinity_on != 0)
    return fail(MXFP8_ERR_INVALID_ARG, "moe_bwd_mxfp8: down_proj_act_checkpoint needs the affinity on H");
  const void* opt[] = {a->gate_act_checkpoint_T, a->intermediate_checkpoint_T, a->scaled_intermediate_checkpoint_T,
                       a->down_proj_act_checkpoint};
  for (const void* q : opt)
    if (q && !aligned16(q)) return fail(MXFP8_ERR_INVALID_ARG, "moe_bwd_mxfp8: checkpoints must be 16-byte aligned");
  if (a->num_valid_tokens && (reinterpret_cast<uintptr_t>(a->num_valid_tokens) & 3u))
    return fail(MXFP8_ERR_INVALID_ARG, "moe_bwd_mxfp8: num_valid_tokens must be 4-byte aligned");
  if (a->down_proj_act_checkpoint && a->N * a->block_size * a->H * 2 >= int64_t(0x80000000u))
    return fail(MXFP8_ERR_INVALID_ARG, "moe_bwd_mxfp8: down_proj_act_checkpoint must be under 2 GiB");
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255u))
    return fail(MXFP8_ERR_INVALID_ARG, "moe_bwd_mxfp8: workspace must be non-null and 256-byte aligned");
  moe_bwd_mxfp8_workspace_layout L;
  moe_layout(a, &L);
  if (ws_bytes < L.total) return fail(MXFP8_ERR_WORKSPACE, "moe_bwd_mxfp8: workspace %zu < %zu bytes", ws_bytes, L.total);

  const int64_t T = a->T, H = a->H, I = a->I, E = a->E, N = a->N, B = a->block_size, P = N * B;
  uint8_t* w = static_cast<uint8_t*>(ws);
  auto at = [&](size_t off) { return w + off; };
  int32_t* slot_tok = reinterpret_cast<int32_t*>(at(L.slot_token));
  float* slot_aff = reinterpret_cast<float*>(at(L.slot_affinity));
  int32_t* flag = reinterpret_cast<int32_t*>(at(L.block_flag));
  int32_t* boff = reinterpret_cast<int32_t*>(at(L.expert_block_offsets));
  int32_t* blist = reinterpret_cast<int32_t*>(at(L.expert_block_list));
  float* dx_slot = reinterpret_cast<float*>(at(L.dx_slot));
  int32_t* slot_of = reinterpret_cast<int32_t*>(at(L.slot_of));
  float* daff_slot = reinterpret_cast<float*>(at(L.daff_slot));
  float* db1_acc = reinterpret_cast<float*>(at(L.db1_acc));
  float* db2_acc = reinterpret_cast<float*>(at(L.db2_acc));
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  // the second stream, for a whole backward (stages in order keep to the caller's)
  SideStream* side = nullptr;
  std::unique_lock<std::mutex> side_lock;
  if (lo == 0 && hi == MOE_BWD_NUM_STAGES - 1) {
    int device = -1, cus = 0;
    if ((st ? hipStreamGetDevice(st, &device) : hipGetDevice(&device)) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) == hipSuccess && cus > 0) {
      mx::Phase3Args q{};
      q.H = H; q.I = I; q.N = N; q.B = B;
      const int64_t tiles = mx::phase3_max_tiles(q);
      if (tiles >= int64_t(cus) && tiles < kOverlapRounds * int64_t(cus)) side = side_stream(device);
    }
    if (side) side_lock = std::unique_lock<std::mutex>(side->mu);
  }
  hipStream_t s2 = side ? side->s : st;
  // the stream `to` waits for what `from` has enqueued so far (nothing without a second stream)
  auto order = [&](hipEvent_t* ev, hipStream_t from, hipStream_t to) -> hipError_t {
    if (!side) return hipSuccess;
    hipError_t r = hipEventRecord(*ev, from);
    return r != hipSuccess ? r : hipStreamWaitEvent(to, *ev, 0);
  };
  int stage = -1;
#define STEP(call, what) \
  if (stage >= lo && stage <= hi && (e = (call)) != hipSuccess) return hip_status(e, what);

  stage = 0;
  STEP(mx::launch_fill_u32(daff_slot, P, 0u, st), "zero the d(affinity) bias term");
  if (a->has_bias) {
    STEP(mx::launch_fill_u32(db1_acc, E * 2 * I, 0u, st), "zero db1 accumulator");
    STEP(mx::launch_fill_u32(db2_acc, E * H, 0u, st), "zero db2 accumulator");
  }
  STEP(mx::launch_slot_setup(a->token_position_to_id, a->block_to_expert, a->expert_affinities_masked, T, E, N, B,
                             a->num_valid_tokens, slot_tok, slot_aff, slot_of, flag, boff, blist, st),
       "slot setup");
  stage = 1;
  // S1: dY quantised along H per token row (Phase-1 operand, gathered by token later).
  // H % 128 == 0: Phase 1 streams the codes with pair-major scales (dY's written so,
  // W_down's re-laid); otherwise it reads their exact bf16 values.
  const bool h_pairs = H % 128 == 0;
  STEP(mx::launch_quant_rows(a->output_hidden_states_grad, T, H, a->fmt_grad, at(L.dy_codes), at(L.dy_scales), st,
                             h_pairs ? nullptr : reinterpret_cast<uint16_t*>(at(L.dy_deq)), h_pairs),
       "quantize dY");
  if (h_pairs) {
    STEP(mx::launch_scales_to_pairs(a->down_scales, E, I, H, at(L.wd_scales_pairs), st), "W_down scales to pairs");
  } else {
    STEP(mx::launch_dequant_rows(a->down_codes, a->down_scales, E * I, H, a->fmt_weight,
                                 reinterpret_cast<uint16_t*>(at(L.wd_deq)), st),
         "dequantize W_down");
  }
  // Phase 3 on the ring loop reads W_gate_up's scales pair-major
  const bool gu_pairs = (2 * I) % 128 == 0;
  if (gu_pairs)
    STEP(mx::launch_scales_to_pairs(a->gate_up_scales, E, H, 2 * I, at(L.wgu_scales_pairs), st),
         "W_gate_up scales to pairs");
  stage = 2;
  STEP(order(side ? &side->ev[0] : nullptr, st, s2), "second stream after the set-up");
  // token-axis operands of Phases 2 and 4: X, a*dY (on H) or dY (on I); the intermediate
  // operand comes out of the Phase-1 epilogue
  STEP(mx::launch_quant_tok(a->hidden_states, T, H, slot_tok, nullptr, P, a->fmt_act, at(L.x_tok_codes),
                            at(L.x_tok_scales), s2, true, false, nullptr, true),
       "gather-quantize X");
  if (a->down_proj_act_checkpoint) {   // a*dY supplied per slot: each routed slot reads its own row
    STEP(mx::launch_quant_tok(a->down_proj_act_checkpoint, P, H, slot_tok, nullptr, P, a->fmt_grad,
                              at(L.gy_tok_codes), at(L.gy_tok_scales), s2, true, true, nullptr, true),
         "quantize the a*dY checkpoint");
  } else {
    // with a bias: db2 and the <dY, b2> shares of d(a) from the same row reads
    // (rows I/32 .. I/32 + H/128 of daff_part)
    const mx::TokBias tb{a->down_proj_bias, a->block_to_expert, B, db2_acc,
                         reinterpret_cast<float*>(at(L.daff_part)) + (I / 32) * P};
    STEP(mx::launch_quant_tok(a->output_hidden_states_grad, T, H, slot_tok, a->affinity_on == 0 ? slot_aff : nullptr,
                              P, a->fmt_grad, at(L.gy_tok_codes), at(L.gy_tok_scales), s2, true, false,
                              moe_fuse_bias(a) ? &tb : nullptr, true),
         "gather-quantize dY");
  }
  stage = 3;
  if (a->has_bias && !moe_fuse_bias(a))
    STEP(mx::launch_bias(a->output_hidden_states_grad, a->down_proj_bias, slot_tok, slot_aff, a->block_to_expert,
                         flag, H, B, N, daff_slot, db2_acc, s2),
         "bias reductions");
  // the finalisation reads the bias terms: it waits for this point of the second stream
  if (side && stage >= lo && stage <= hi && (e = hipEventRecord(side->ev[2], s2)) != hipSuccess)
    return hip_status(e, "second stream after the gathers");
  stage = 4;
  // Phase 1: the product dS, fp32
  mx::Phase1Args p1{};
  if (h_pairs) {
    p1.wd_codes = a->down_codes; p1.wd_scales = at(L.wd_scales_pairs);
    p1.dy_codes = at(L.dy_codes); p1.dy_scales = at(L.dy_scales);
  } else {
    p1.wd_deq = reinterpret_cast<const uint16_t*>(at(L.wd_deq));
    p1.dy_deq = reinterpret_cast<const uint16_t*>(at(L.dy_deq));
  }
  p1.ds = reinterpret_cast<float*>(at(L.phase1_ds));
  p1.tile_start = reinterpret_cast<int32_t*>(at(L.phase1_tiles));
  p1.slot_tok = slot_tok; p1.slot_aff = slot_aff; p1.b2e = a->block_to_expert; p1.flag = flag;
  p1.ckpt = a->gate_up_proj_act_checkpoint_T;
  p1.ga_ckpt = a->gate_act_checkpoint_T;
  p1.in_ckpt = a->intermediate_checkpoint_T;
  p1.sc_ckpt = a->scaled_intermediate_checkpoint_T;
  p1.T = T; p1.H = H; p1.I = I; p1.E = E; p1.N = N; p1.B = B;
  p1.dgu_row_codes = at(L.dgu_row_codes); p1.dgu_row_scales = at(L.dgu_row_scales);
  p1.dgu_tok_codes = at(L.dgu_tok_codes); p1.dgu_tok_scales = at(L.dgu_tok_scales);
  p1.inter_tok_codes = at(L.inter_tok_codes); p1.inter_tok_scales = at(L.inter_tok_scales);
  p1.daff_part = reinterpret_cast<float*>(at(L.daff_part)); p1.db1_acc = db1_acc;
  p1.affinity_on_i = a->affinity_on; p1.has_bias = a->has_bias; p1.fmt_act = a->fmt_act;
  p1.geglu = a->activation == MXFP8_ACT_GEGLU;
  p1.dgu_row_pairs = gu_pairs;
  // Tile order over the XCDs (measured: round robin 2.6% faster on Phase 1 with
  // 58 MB W_down experts; the contiguous ranges 6% faster with 0.4-3 MB ones)
  p1.rr_tiles = I * H >= kRoundRobinWeightBytes;
  // With the epilogue fused stage 4 does both and stage 5 nothing.
  const bool fused = moe_phase1_fused(a);
  if (fused) {
    STEP(mx::launch_phase1_fused(p1, a->fmt_grad, a->fmt_weight, st), "phase 1 (with its epilogue)");
  } else {
    STEP(mx::launch_phase1(p1, a->fmt_grad, a->fmt_weight, st), "phase 1");
  }
  stage = 5;
  // the SwiGLU backward on dS: dGU along both axes, the intermediate operand, d(a), db1
  if (!fused) STEP(mx::launch_phase1_epi(p1, a->fmt_grad, st), "phase 1 epilogue");
  stage = 6;
  STEP(order(side ? &side->ev[1] : nullptr, st, s2), "second stream after the epilogue");
  // Phase 3: dX scatter-add
  mx::Phase3Args p3{};
  p3.dgu_row_codes = at(L.dgu_row_codes); p3.dgu_row_scales = at(L.dgu_row_scales);
  p3.wgu_codes = a->gate_up_codes; p3.wgu_scales = gu_pairs ? at(L.wgu_scales_pairs) : a->gate_up_scales;
  p3.slot_tok = slot_tok; p3.b2e = a->block_to_expert; p3.flag = flag;
  p3.tile_start = reinterpret_cast<int32_t*>(at(L.phase3_tiles));
  p3.H = H; p3.I = I; p3.N = N; p3.B = B; p3.dx_slot = dx_slot;
  // the last round of tiles cut along K over the device's CUs
  p3.conc = device_cus(st);
  p3.parts = mx::phase3_parts_bytes(p3) > 0 ? at(L.phase3_parts) : nullptr;
  // measured: round robin 4.8% faster with 117 MB W_gate_up experts, the
  // contiguous ranges 6-14% faster with 0.8-6 MB ones
  p3.rr_tiles = H * 2 * I >= kRoundRobinWeightBytes;
  STEP(mx::launch_phase3(p3, a->fmt_grad, a->fmt_weight, st), "phase 3");
  stage = 7;
  // Phase 2: dW_gate_up[e] = X_tok . dGU_tok^T over the expert's blocks
  mx::GemmStoreArgs g{};
  g.a_codes = at(L.x_tok_codes); g.a_scales = at(L.x_tok_scales); g.lda = P;
  g.b_codes = at(L.dgu_tok_codes); g.b_scales = at(L.dgu_tok_scales); g.ldb = P;
  g.M = H; g.N = 2 * I; g.K = 0; g.out = a->gate_up_proj_weight_grad; g.ldo = 2 * I; g.out_gstride = H * 2 * I;
  g.blk_off = boff; g.blk_list = blist; g.blk = int(B);
  g.blk_ext = flag;   // the expert's last block ends at its last routed slot (rounded up to 128)
  // the token-axis operands are stage-major (whole cache lines per DMA
  // instruction), which only the four-slot ring reads; measured on the large
  // workload against row-major operands, Phase 2 on the pair-slot ring and
  // Phase 4 on the four-slot ring: 9% and 10% faster
  g.pair = 0;
  g.stage_major = 1;
  g.accumulate = a->accumulate;
  STEP(mx::launch_gemm_store(g, int(E), a->fmt_act, a->fmt_grad, s2), "phase 2");
  stage = 8;
  // Phase 4: dW_down[e] = inter_tok . gy_tok^T
  g.a_codes = at(L.inter_tok_codes); g.a_scales = at(L.inter_tok_scales); g.lda = P;
  g.b_codes = at(L.gy_tok_codes); g.b_scales = at(L.gy_tok_scales); g.ldb = P;
  g.M = I; g.N = H; g.out = a->down_proj_weight_grad; g.ldo = H; g.out_gstride = I * H;
  STEP(mx::launch_gemm_store(g, int(E), a->fmt_act, a->fmt_grad, s2), "phase 4");
  stage = 9;
  // finalisation (after the second stream's gathers and bias terms)
  if (side && stage >= lo && stage <= hi && (e = hipStreamWaitEvent(st, side->ev[2], 0)) != hipSuccess)
    return hip_status(e, "caller's stream after the gathers");
  const bool acc = a->accumulate != 0;
  STEP(mx::launch_dx_reduce(dx_slot, slot_of, T, E, H, a->hidden_states_grad, st, acc), "dX per-token sums");
  STEP(mx::launch_daff_scatter(daff_slot, reinterpret_cast<const float*>(at(L.daff_part)),
                               I / 32 + (moe_fuse_bias(a) ? H / 128 : 0), slot_tok,
                               a->block_to_expert, T, E, B, N, a->expert_affinities_masked_grad,
                               st, acc),
       "d(affinity) scatter");
  if (a->has_bias) {
    STEP(mx::launch_f32_to_bf16(db1_acc, a->gate_and_up_proj_bias_grad, E * 2 * I, st, acc), "db1 to bf16");
    STEP(mx::launch_f32_to_bf16(db2_acc, a->down_proj_bias_grad, E * H, st, acc), "db2 to bf16");
  }
  // the caller's stream waits for Phases 2 and 4
  STEP(order(side ? &side->ev[3] : nullptr, s2, st), "join of the second stream");
#undef STEP
  return ok();
}

int moe_bwd_mxfp8(const moe_bwd_mxfp8_args* a, void* ws, size_t ws_bytes, void* stream) {
  return moe_run(a, ws, ws_bytes, stream, 0, MOE_BWD_NUM_STAGES - 1);
}

int moe_bwd_mxfp8_stage(const moe_bwd_mxfp8_args* a, void* ws, size_t ws_bytes, int stage, void* stream) {
  if (stage < 0 || stage >= MOE_BWD_NUM_STAGES)
    return fail(MXFP8_ERR_INVALID_ARG, "moe_bwd_mxfp8_stage: stage %d outside [0,%d)", stage, MOE_BWD_NUM_STAGES);
  return moe_run(a, ws, ws_bytes, stream, stage, stage);
}

int moe_router_bwd(int mode, int64_t T, int64_t E, int64_t K, const int32_t* topk_idx, const float* topk_scores,
                   const float* logits, const float* dscores, const uint16_t* daff, int renorm, float* dlogits,
                   void* stream) {
  if (mode != MXFP8_ROUTER_SOFTMAX_OVER_TOPK && mode != MXFP8_ROUTER_TOPK_OVER_SOFTMAX && mode != MXFP8_ROUTER_TOPK)
    return fail(MXFP8_ERR_INVALID_ARG, "moe_router_bwd: unknown mode %d", mode);
  if (T < 0 || E < 1 || K < 1 || K > E || K > MXFP8_ROUTER_MAX_K)
    return fail(MXFP8_ERR_INVALID_ARG, "moe_router_bwd: need T >= 0 and 1 <= K <= min(E, %d) (T %lld, E %lld, K %lld)",
                MXFP8_ROUTER_MAX_K, (long long)T, (long long)E, (long long)K);
  if (E > INT32_MAX / 2) return fail(MXFP8_ERR_INVALID_ARG, "moe_router_bwd: E %lld too large", (long long)E);
  if (renorm && mode != MXFP8_ROUTER_TOPK_OVER_SOFTMAX)
    return fail(MXFP8_ERR_INVALID_ARG, "moe_router_bwd: renorm applies to the top-k-over-softmax mode only");
  if ((dscores == nullptr) == (daff == nullptr))
    return fail(MXFP8_ERR_INVALID_ARG, "moe_router_bwd: pass exactly one of dscores and daff");
  if (T == 0) return ok();
  const bool need_scores = mode == MXFP8_ROUTER_SOFTMAX_OVER_TOPK || (mode == MXFP8_ROUTER_TOPK_OVER_SOFTMAX && renorm);
  const bool need_logits = mode == MXFP8_ROUTER_TOPK_OVER_SOFTMAX;
  if (!topk_idx || !dlogits || (need_scores && !topk_scores) || (need_logits && !logits))
    return fail(MXFP8_ERR_INVALID_ARG, "moe_router_bwd: null pointer for a tensor this mode reads or writes");
  const void* ptrs[6] = {topk_idx, topk_scores, logits, dscores, daff, dlogits};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return fail(MXFP8_ERR_INVALID_ARG, "moe_router_bwd: tensors must be 16-byte aligned");
  mx::RouterArgs r{};
  r.mode = mode; r.renorm = renorm ? 1 : 0; r.T = T; r.E = E; r.K = K;
  r.idx = topk_idx; r.scores = topk_scores; r.logits = logits; r.dscores = dscores; r.daff = daff;
  r.dlogits = dlogits;
  return hip_status(mx::launch_router_bwd(r, static_cast<hipStream_t>(stream)), "router backward");
}

}  // extern "C"
