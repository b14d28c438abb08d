// kernels.hpp -- host-side launchers of the gfx950 kernels (internal to the
// library; the public interface is include/mxfp8_moe.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mx {

// quantize.hip
// Scale layouts: row-major [rows][K/32], or pair-major [K/128][rows][4] (pairs
// = true) for operands of the ring GEMM loop; see gemm_v3.hpp.
// stage_major (with pairs): codes stage-major (mx_device.hpp, stage_major_off), rows rows over cols
hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int64_t cols, int fmt, uint8_t* codes,
                             uint8_t* scales, hipStream_t st, uint16_t* deq = nullptr, bool pairs = false,
                             bool stage_major = false);
// codes [rows][cols] + scales [rows][cols/32] (groups along cols) -> exact bf16 values
hipError_t launch_dequant_rows(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols, int fmt,
                               uint16_t* out, hipStream_t st);
hipError_t launch_quant_cols(const uint16_t* x, int64_t rows, int64_t cols, int fmt, uint8_t* codes,
                             uint8_t* scales, hipStream_t st);
// The bias reductions fused into the gather of dY rows (see quant_tok_kernel):
// db2_acc [E][cols] += a * dY sums; part [cols/128][rows] = <dY, b2> shares.
struct TokBias {
  const uint16_t* b2;      // [E][cols] bf16
  const int32_t* b2e;      // [rows / B]
  int64_t B;               // slots per block (a multiple of 128)
  float* db2_acc;
  float* part;             // null: no bias work
};
// x [rows][cols] along both axes in one pass, the same bytes as launch_quant_rows
// (pairs) and launch_quant_tok (no index) each give: rows % 32 == 0, cols % 512 == 0
bool quant_dual_fits(int64_t rows, int64_t cols);
// stage_major / stage_major_t: codes / codes_t stage-major (codes_t needs rows % 128 == 0)
hipError_t launch_quant_dual(const uint16_t* x, int64_t rows, int64_t cols, int fmt, uint8_t* codes,
                             uint8_t* scales, uint8_t* codes_t, uint8_t* scales_t, hipStream_t st,
                             bool stage_major = false, bool stage_major_t = false);
// stage_major: codes_t stage-major, cols rows over rows elements (rows % 128 == 0)
hipError_t launch_quant_tok(const uint16_t* x, int64_t src_rows, int64_t cols, const int32_t* idx,
                            const float* rowscale, int64_t rows, int fmt, uint8_t* codes_t,
                            uint8_t* scales_t, hipStream_t st, bool pairs = false, bool self_rows = false,
                            const TokBias* bias = nullptr, bool stage_major = false);
// prequant.hip: an operand quantised along its rows (codes [R][C], scales
// [R/32][C]) into the GEMM layout: codes [C][R]; scales pair-major
// [R/128][C][4] (pairs) or row-major [C][R/32]
hipError_t launch_transpose_codes(const uint8_t* in, int64_t R, int64_t C, uint8_t* out, hipStream_t st);
hipError_t launch_scales_axis0(const uint8_t* in, int64_t R, int64_t C, uint8_t* out, bool pairs, hipStream_t st);
// gate/up weight scales [E][H][2I/32] -> pair-major per expert [E][2I/128][H][4]
hipError_t launch_scales_to_pairs(const uint8_t* in, int64_t groups, int64_t rows, int64_t k, uint8_t* out,
                                  hipStream_t st);

// gemm_dense.hip: C[m][n] = sum_k A[m][k] B[n][k] -> bf16 out[g][m][n].
// A [M][lda] and B [N][ldb] fp8 codes, K-contiguous.  Scales pair-major
// ([ld/128][rows][4]) when lda, ldb and K (or blk) are multiples of 128 (the
// ring loop), else row-major [rows][ld/32].
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
  const int32_t* blk_ext;   // optional: per block, one past its last routed column; a group's
                            // last block then contributes only that many columns, rounded up to 128
  int blk;
  int accumulate;                 // 1: out = bf16(out + C) instead of bf16(C)
  int pair;                       // 1: 256 x 256 tiles run the pair-slot ring (128-byte rows), 0: the
                                  // four-slot ring (deeper look-ahead, for operands streamed from HBM)
  int stage_major;                // 1: both operands' codes are stage-major (stage_major_off; lda and
                                  // ldb are then their K); needs the four-slot ring: pair == 0, every
                                  // ld a multiple of 128 and, with a block list, blk too
  int tiles_m, tiles_n;
  int total;                      // tiles over all groups
  int groups;                     // set by the launcher
};
hipError_t launch_gemm_store(GemmStoreArgs p, int groups, int fa, int fb, hipStream_t st);

// router.hip -- the router backward (modes as mxfp8_router_mode in the public header)
constexpr int kRouterSoftmaxOverTopk = 0;
constexpr int kRouterTopkOverSoftmax = 1;
constexpr int kRouterTopk = 2;
struct RouterArgs {
  int mode;
  int renorm;                 // top-k over softmax: the selected probabilities were renormalised
  int64_t T, E, K;
  const int32_t* idx;         // [T,K] selected experts
  const float* scores;        // [T,K] forward scores (softmax over top-k; renormalised top-k over softmax)
  const float* logits;        // [T,E] router logits (top-k over softmax)
  const float* dscores;       // [T,K] upstream score gradients, or null when
  const uint16_t* daff;       // [T,E] bf16 affinity gradient is read at idx instead
  float* dlogits;             // [T,E] output
};
hipError_t launch_router_bwd(const RouterArgs& p, hipStream_t st);

// moe_aux.hip
hipError_t launch_fill_u32(void* p, int64_t n, uint32_t v, hipStream_t st);
hipError_t launch_fill_u16(void* p, int64_t n, uint16_t v, hipStream_t st);
// ws: build_blocks_workspace_bytes(E) bytes (per expert and token chunk: counts, first slots)
int64_t build_blocks_workspace_bytes(int64_t E);
hipError_t launch_build_blocks(const int32_t* topk, int64_t T, int64_t K, int64_t E, int64_t B, int64_t N,
                               int32_t* tpid, int32_t* b2e, int32_t* ws, hipStream_t st);
// the allocation-free variant: the most experts its file-scope scratch holds,
// and that scratch's device address on `device` (looked up once per device)
int64_t build_blocks_noalloc_max_experts();
hipError_t build_blocks_scratch(int device, int32_t** out);
struct TailCut;
// rr: the tiles handed out round robin over the XCDs (the blocks whose slot
// tiles are all live first, blk = the block size); cut: Phase 3's tail cut
hipError_t launch_tile_ranges(const int32_t* ext, int64_t N, int W, int other, int32_t* start, hipStream_t st,
                              TailCut* cut, int conc, int npairs, int rr, int blk);
hipError_t launch_slot_setup(const int32_t* tpid, const int32_t* b2e, const float* aff, int64_t T, int64_t E,
                             int64_t N, int64_t B, const int32_t* nvalid, int32_t* slot_tok, float* slot_aff,
                             int32_t* slot_of, int32_t* flag, int32_t* off, int32_t* list, hipStream_t st);
// accumulate: each bf16 output becomes bf16(old + value) (else bf16(value))
hipError_t launch_dx_reduce(const float* dx_slot, const int32_t* slot_of, int64_t T, int64_t E, int64_t H,
                            uint16_t* dx, hipStream_t st, bool accumulate = false);
hipError_t launch_bias(const uint16_t* dy, const uint16_t* b2, const int32_t* slot_tok, const float* slot_aff,
                       const int32_t* b2e, const int32_t* flag, int64_t H, int64_t B, int64_t N, float* daff_slot,
                       float* db2_acc, hipStream_t st);
hipError_t launch_f32_to_bf16(const float* src, uint16_t* dst, int64_t n, hipStream_t st, bool accumulate = false);
hipError_t launch_daff_scatter(const float* daff_slot, const float* daff_part, int64_t nparts,
                               const int32_t* slot_tok, const int32_t* b2e, int64_t T, int64_t E, int64_t B,
                               int64_t N, uint16_t* daff, hipStream_t st, bool accumulate = false);

// moe_phase1_*.hip (product, epilogue), moe_phase3.hip
struct Phase1Args {
  // H % 128 == 0: the MX operands themselves, scales pair-major
  const uint8_t* wd_codes;      // [E][I][H]
  const uint8_t* wd_scales;     // [E][H/128][I][4]
  const uint8_t* dy_codes;      // [T][H]: Q_H(dY)
  const uint8_t* dy_scales;     // [H/128][T][4]
  // otherwise their exact bf16 values
  const uint16_t* wd_deq;       // [E][I][H] bf16: dequantised W_down
  const uint16_t* dy_deq;       // [T][H] bf16: dequantised Q_H(dY)
  float* ds;                    // [N][I][B] fp32: the product, written by Phase 1, read by its epilogue
  const int32_t* slot_tok;      // [P]
  const float* slot_aff;        // [P]
  const int32_t* b2e;           // [N]
  const int32_t* flag;          // [N]: the block's extent (one past its last routed slot)
  int32_t* tile_start;          // [N+1]: tile ranges over the blocks' live slot tiles (moe_tiles.hpp)
  const uint16_t* ckpt;         // [N][2][I][B]
  // optional checkpoints supplied by the caller ([N][I][B] bf16 each), read in
  // place of recomputing the value: silu(gate), the intermediate, and the
  // intermediate times the affinity (affinity on I)
  const uint16_t* ga_ckpt;
  const uint16_t* in_ckpt;
  const uint16_t* sc_ckpt;
  int64_t T, H, I, E, N, B;
  // stage-major codes: the four-slot ring's layout (mx_device.hpp, stage_major_off)
  uint8_t* dgu_row_codes;       // stage-major, P rows over 2I (dgu_row_pairs), or row-major [P][2I]
  uint8_t* dgu_row_scales;      // pair-major [2I/128][P][4] (dgu_row_pairs) or row-major [P][2I/32]
  uint8_t* dgu_tok_codes;       // stage-major, 2I rows over P
  uint8_t* dgu_tok_scales;      // pair-major [P/128][2I][4]
  uint8_t* inter_tok_codes;     // stage-major, I rows over P: the intermediate (times a with the
                                // affinity on I), slot groups
  uint8_t* inter_tok_scales;    // pair-major [P/128][I][4]
  float* daff_part;             // [I/32][P]: d(a) partial sums per 32 rows i
  float* db1_acc;               // [E][2][I]
  int affinity_on_i;            // 1: the intermediate operand carries the affinity
  int has_bias;                 // 1: accumulate db1
  int fmt_act;                  // format of the intermediate operand (activation format)
  int geglu;                    // gated activation: 0 SwiGLU (silu), 1 GeGLU (gelu, erf form)
  int dgu_row_pairs;            // 1: dGU along I feeds the ring loop (2I % 128 == 0): stage-major
                                // codes, pair-major scales
  int rr_tiles;                 // tile order over the XCDs (moe_tiles.hpp)
  int tiles_m, tiles_n;
};
hipError_t launch_phase1(const Phase1Args& p, int fmt_grad, int fmt_weight, hipStream_t st);
hipError_t launch_phase1_epi(const Phase1Args& p, int fmt_grad, hipStream_t st);
// Phase 1 and its epilogue in one kernel, where phase1_fusable: the same outputs
// as launch_phase1 followed by launch_phase1_epi, without dS in HBM
bool phase1_fusable(const Phase1Args& p);
hipError_t launch_phase1_fused(const Phase1Args& p, int fmt_grad, int fmt_weight, hipStream_t st);

struct Phase3Args {
  const uint8_t* dgu_row_codes;   // 2I % 128 == 0: stage-major, P rows over 2I; else row-major [P][2I]
  const uint8_t* dgu_row_scales;  // 2I % 128 == 0: pair-major [2I/128][P][4]; else row-major [P][2I/32]
  const uint8_t* wgu_codes;       // [E][H][2I]
  const uint8_t* wgu_scales;      // 2I % 128 == 0: pair-major [E][2I/128][H][4]; else row-major [E][H][2I/32]
  const int32_t* slot_tok;
  const int32_t* b2e;
  const int32_t* flag;            // [N]: the block's extent (one past its last routed slot)
  int32_t* tile_start;            // [N+1]: tile ranges over the blocks' live slot tiles (moe_tiles.hpp)
  int64_t H, I, N, B;
  float* dx_slot;                 // [P][H] fp32: each routed slot's row of dX
  int rr_tiles;                   // tile order over the XCDs (moe_tiles.hpp)
  // The last round of tiles cut along K (moe_tiles.hpp, TailCut): conc =
  // workgroups resident at once (0: no cut); parts = phase3_parts_bytes(...)
  // bytes: the cut of each XCD (8 TailCut, 256 bytes), then the later parts'
  // fp32 tiles
  int conc;
  uint8_t* parts;
  int tiles_m, tiles_n, grid_main, npairs;   // set by the launcher
};
hipError_t launch_phase3(const Phase3Args& p, int fg, int fw, hipStream_t st);
// Phase 3 tiles when every slot tile of every block is live (an upper bound)
int64_t phase3_max_tiles(const Phase3Args& p);
// bytes of the parts buffer (H, I, N, B set)
int64_t phase3_parts_bytes(const Phase3Args& p);

}  // namespace mx
