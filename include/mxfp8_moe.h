/*
 * mxfp8_moe.h -- C ABI of the MI355X (gfx950) MXFP8 MoE-backward library
 * (libmxfp8_moe.so).
 *
 * What it computes is defined by three pages:
 *   [P1] AWS Neuron NKI library, "Blockwise MM Backward MXFP8 Kernel API
 *        Reference": gradients of a blockwise Mixture-of-Experts SwiGLU layer
 *        from BF16 activations, MXFP8 weights and block routing indices.
 *   [P2] AWS Neuron NKI library, "Matmul MXFP8 Backward Kernel API
 *        Reference": dX and dW of a linear layer Y = X W^T with MXFP8
 *        quantised operands.
 *   [P3] sonic-moe, functional/backward.py: the fused gated-activation
 *        backward epilogue and the bias / affinity reductions.
 *
 * Conventions for every entry point
 *  - Pointers named in a signature are DEVICE pointers unless marked "host".
 *    bf16 tensors are passed as uint16_t bit patterns; all tensors are dense,
 *    row-major and must be 16-byte aligned.
 *  - The caller owns every buffer, including the workspace.  The library never
 *    allocates or frees device memory and keeps no state between calls, except
 *    the allocation-free routing entry point's file-scope device scratch (one
 *    1 MiB copy per GPU, part of the loaded library) and its address per device.
 *  - Calls are asynchronous: work is enqueued on `stream` (a hipStream_t, NULL
 *    for the default stream) and the call returns without synchronising.  A
 *    device fault surfaces at the caller's next synchronisation.
 *  - Arguments are validated before anything is enqueued.  On a validation
 *    failure the call returns a non-zero mxfp8_status, records a message that
 *    mxfp8_last_error() returns on the calling thread, and leaves every output
 *    untouched.  No C++ exception crosses this interface.
 *  - Outputs are fully overwritten, except where moe_bwd_mxfp8's `accumulate`
 *    flag asks for the gradients to be added into them.
 *
 * MXFP8 (P1: "32-element quantization group"): a group of 32 consecutive
 * elements along the quantised axis shares one E8M0 scale byte S (value
 * 2^(S-127)); each element is an 8-bit OCP E4M3 or E5M2 code.  The scale is
 * X = floor(log2(amax)) - emax (emax 8 for E4M3, 15 for E5M2), clamped to
 * [-127,127], with X = -127 for an all-zero group; codes round v*2^-X to
 * nearest-even and saturate at the format maximum.  Inputs are expected to be
 * finite: the codes and scales of a group holding a NaN or an infinity are
 * unspecified (no error is raised and other groups are unaffected).
 */
#ifndef MXFP8_MOE_H
#define MXFP8_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MXFP8_E4M3 = 0, MXFP8_E5M2 = 1 } mxfp8_fmt;

typedef enum {
  MXFP8_OK = 0,
  MXFP8_ERR_INVALID_ARG = 1, /* bad shape, null pointer, misalignment, bad enum   */
  MXFP8_ERR_UNSUPPORTED = 2, /* a valid combination this library does not run    */
  MXFP8_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the size query */
  MXFP8_ERR_HIP = 4          /* the HIP runtime refused a launch                 */
} mxfp8_status;

/* Host.  Message of the last failing call on this thread ("" if none). */
const char* mxfp8_last_error(void);

/* Host.  Library version string. */
const char* mxfp8_version(void);

/* ---------------------------------------------------------------------------
 * mxfp8_quantize -- P1's 32-element MXFP8 group quantisation of a BF16 tensor.
 *   x      [rows, cols] bf16.
 *   axis 1: groups of 32 along cols;  scales [rows, cols/32]  (cols % 32 == 0).
 *   axis 0: groups of 32 along rows;  scales [rows/32, cols]  (rows % 32 == 0).
 *   fmt    MXFP8_E4M3 or MXFP8_E5M2.
 *   codes  [rows, cols] u8, in x's layout;  scales: E8M0 bytes as above.
 * Errors: INVALID_ARG for a negative size, a bad axis or fmt, a size along the
 * quantised axis that is not a multiple of 32, a null pointer, or x / codes
 * not 16-byte aligned; HIP if the launch fails.  rows * cols == 0 is not an
 * error: nothing is enqueued and the pointers are not read (they may be NULL).
 * ------------------------------------------------------------------------- */
int mxfp8_quantize(const uint16_t* x, int64_t rows, int64_t cols, int axis, int fmt,
                   uint8_t* codes, uint8_t* scales, void* stream);

/* ---------------------------------------------------------------------------
 * matmul_mxfp8_bwd -- P2: the backward of Y = X W^T with X [M,K], W [N,K]:
 *   input_grad  dX = dY W    [M,K]  (contraction over N)
 *   weight_grad dW = dY^T X  [N,K]  (contraction over M)
 * Each operand is quantised in groups of 32 along the contraction axis of the
 * product it feeds (dY twice: along N for dX, along M for dW), products are
 * accumulated in fp32 and the outputs are bf16 (P2: output_dtype bf16).
 *   output_grad [M,N], weights [N,K], input_activation [M,K]: bf16.
 *   fmt_*: element format per operand (P2's default float8_e5m2; the common
 *          training choice is E5M2 for dY, E4M3 for W and X).
 *   M % 32 == 0, N % 32 == 0, K % 32 == 0.
 *   workspace: >= matmul_mxfp8_bwd_workspace_size(M,N,K) bytes of device
 *   memory, 256-byte aligned; it holds the quantised operands (P2:
 *   "spill quantized blocks to HBM for reuse"):
 *     [0]  dY codes along N  [M,N]  + scales [M,N/32]
 *     [1]  W^T codes along N [K,N]  + scales [K,N/32]
 *     [2]  dY^T codes along M [N,M] + scales [N,M/32]
 *     [3]  X^T codes along M [K,M]  + scales [K,M/32]
 *   Scales of [0],[1] are pair-major ([N/128][rows][4]: word (p, r) = row r's
 *   bytes for elements [128p, 128p+128)) when N % 128 == 0, and those of
 *   [2],[3] ([M/128][rows][4]) when M % 128 == 0.  The codes of a product's
 *   two operands are stage-major (S64, as defined with
 *   moe_bwd_mxfp8_workspace_layout: 256-row panels, each [C/64][rows][64],
 *   C the contraction) when both are quantised here from bf16 and C is a
 *   multiple of 128 below 2^24 (N for [0],[1], M for [2],[3]); otherwise
 *   row-major as shown.  The region sizes are the same either way, each
 *   region starting on a 256-byte boundary, in this order, codes first.
 * ------------------------------------------------------------------------- */
size_t matmul_mxfp8_bwd_workspace_size(int64_t M, int64_t N, int64_t K);

/* matmul_mxfp8_bwd_ex -- the same backward with [P2]'s optional pre-quantised
 * operands ("API Reference": output_grad_scales, weight_scales, input_scales,
 * use_scale_packing and the *_is_swizzled flags).  Reading: a pre-quantised
 * operand is given as its codes and E8M0 scales, grouped along the
 * contraction axis of the product it feeds.  dY feeds two products that
 * contract different axes, so it takes one set per axis (along N for dX,
 * along M for dW); either or both may be given, and the bf16 output_grad is
 * needed only for a set that is not.  An operand given pre-quantised needs no
 * bf16 tensor (its pointer may be NULL).  The codes' format is the operand's
 * fmt_*.  Layouts, for an operand with contraction length C:
 *   not swizzled (what mxfp8_quantize writes):
 *     output_grad along N  codes [M,N], scales [M, N/32]   (axis 1)
 *     output_grad along M  codes [M,N], scales [M/32, N]   (axis 0)
 *     weights (along N)    codes [N,K], scales [N/32, K]   (axis 0)
 *     input (along M)      codes [M,K], scales [M/32, K]   (axis 0)
 *   swizzled (*_is_swizzled = 1; the GEMM's operand layout, contraction
 *   contiguous, as workspace regions [0]-[3] of matmul_mxfp8_bwd hold it
 *   when they are not stage-major):
 *     output_grad along N  codes [M,N], scales [M, N/32]
 *     output_grad along M  codes [N,M], scales [N, M/32]
 *     weights              codes [K,N], scales [K, N/32]
 *     input                codes [K,M], scales [K, M/32]
 *   use_scale_packing = 1 (swizzled operands only, C % 128 == 0): the scales
 *     of every pre-quantised operand are packed as [C/128][rows][4], word
 *     (p, r) holding row r's E8M0 bytes for elements [128p, 128p + 128).
 * A swizzled operand (with packed scales, or with C % 128 != 0) is read in
 * place; any other is rearranged into its workspace region first.
 * Workspace: matmul_mxfp8_bwd_workspace_size(M, N, K) bytes, as above.
 * Errors: those of matmul_mxfp8_bwd, and INVALID_ARG for codes without scales
 * (or the reverse), a flag outside {0,1}, a *_is_swizzled flag or
 * use_scale_packing without a pre-quantised operand it applies to, packed
 * scales on an unswizzled operand or with C % 128 != 0, or a missing bf16
 * tensor that some product still needs.                                     */
typedef struct {
  int64_t M, N, K;
  const uint16_t* output_grad;         /* [M,N] bf16 (NULL if both dY sets are given) */
  const uint16_t* weights;             /* [N,K] bf16 (NULL if weight_codes is given)  */
  const uint16_t* input_activation;    /* [M,K] bf16 (NULL if input_codes is given)   */
  int fmt_output_grad, fmt_weights, fmt_input;
  const uint8_t* output_grad_codes_n;  /* dY quantised along N (feeds dX), or NULL    */
  const uint8_t* output_grad_scales_n;
  const uint8_t* output_grad_codes_m;  /* dY quantised along M (feeds dW), or NULL    */
  const uint8_t* output_grad_scales_m;
  const uint8_t* weight_codes;         /* W quantised along N, or NULL               */
  const uint8_t* weight_scales;
  const uint8_t* input_codes;          /* X quantised along M, or NULL               */
  const uint8_t* input_scales;
  int output_grad_is_swizzled, weights_is_swizzled, input_is_swizzled;
  int use_scale_packing;
  uint16_t* input_grad;                /* [M,K] bf16 */
  uint16_t* weight_grad;               /* [N,K] bf16 */
} matmul_mxfp8_bwd_args;
int matmul_mxfp8_bwd_ex(const matmul_mxfp8_bwd_args* args, void* workspace, size_t workspace_bytes,
                        void* stream);
/* Profiling aid: one stage of matmul_mxfp8_bwd on a workspace a full call has
 * filled: 0 quantise dY along N and W along N (and dY along M as well when
 * one pass does both: M % 32 == 0, N % 512 == 0), 1 quantise X (and dY, if
 * stage 0 did not) along M, 2 the dX GEMM, 3 the dW GEMM.  INVALID_ARG for
 * another stage. */
int matmul_mxfp8_bwd_stage(const uint16_t* output_grad, const uint16_t* weights,
                           const uint16_t* input_activation, int64_t M, int64_t N, int64_t K,
                           int fmt_output_grad, int fmt_weights, int fmt_input,
                           uint16_t* input_grad, uint16_t* weight_grad,
                           void* workspace, size_t workspace_bytes, int stage, void* stream);
int matmul_mxfp8_bwd(const uint16_t* output_grad, const uint16_t* weights,
                     const uint16_t* input_activation, int64_t M, int64_t N, int64_t K,
                     int fmt_output_grad, int fmt_weights, int fmt_input,
                     uint16_t* input_grad, uint16_t* weight_grad,
                     void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Routing blocks (P1 parameters token_position_to_id [N*B], block_to_expert
 * [N,1] and the "Dimensions" paragraph).  P1 leaves their construction to
 * the caller; this helper builds them from top-k expert ids:
 *   expert e owns ceil(n_e/B) consecutive blocks, experts in ascending id,
 *   tokens in ascending id within an expert; empty slots hold -1; blocks past
 *   the last used one hold -1 everywhere and map to expert E-1.
 * moe_num_blocks (host) returns P1's N = (T*TopK - (E-1))/B + E - 1 with the
 * division rounded up -- the worst case over all routings -- or -1 when
 * T*K < E or a size is not positive.
 *   topk_ids [T,K] int32, distinct per row, each in [0,E).  A negative id is
 *   a dropped selection ([P3]'s varlen-K routing: a token may activate fewer
 *   than K experts, down to none); ids of E or more are ignored as well.  A
 *   token with no expert gets a zero dX row and zero d(a) from the backward.
 *   N >= moe_num_blocks(T,K,E,B) (checked).
 *   workspace >= moe_build_blocks_workspace_size(E) bytes.
 * ------------------------------------------------------------------------- */
int64_t moe_num_blocks(int64_t T, int64_t K, int64_t E, int64_t block_size);
size_t moe_build_blocks_workspace_size(int64_t E);
int moe_build_blocks(const int32_t* topk_ids, int64_t T, int64_t K, int64_t E,
                     int64_t block_size, int64_t N, int32_t* token_position_to_id,
                     int32_t* block_to_expert, void* workspace, size_t workspace_bytes,
                     void* stream);

/* moe_build_blocks_noalloc -- for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): moe_build_blocks without a workspace argument.  Its scratch
 * (the counts and first slots per expert and token chunk) is a file-scope
 * device array of 1 MiB inside the library, one copy per GPU, held until the
 * process ends; its address is looked up once per device on the first call
 * there.  Nothing is allocated and nothing is cleared: every scratch word the
 * call reads it has written first.  Arguments, outputs and errors as for
 * moe_build_blocks, except: E above MOE_BUILD_BLOCKS_NOALLOC_MAX_EXPERTS is
 * UNSUPPORTED (use moe_build_blocks), and HIP if the scratch's address cannot
 * be found.  The kernels run on `stream`'s device (the current device for
 * NULL).  Every call on one GPU shares its scratch: calls that can overlap on
 * one GPU (concurrent streams, several host threads) race and must be
 * serialised by the caller; calls in order on one stream are safe. */
#define MOE_BUILD_BLOCKS_NOALLOC_MAX_EXPERTS 4096
int moe_build_blocks_noalloc(const int32_t* topk_ids, int64_t T, int64_t K, int64_t E,
                             int64_t block_size, int64_t N, int32_t* token_position_to_id,
                             int32_t* block_to_expert, void* stream);

/* ---------------------------------------------------------------------------
 * moe_bwd_mxfp8 -- P1's blockwise_mm_bwd_mxfp8: all gradients of a blockwise
 * MoE SwiGLU (or GeGLU, see `activation`) layer.  Forward, per routed (token t,
 * expert e) with affinity a:
 *   g = x_t Wgu[e][:,0,:] (+b1),  u = x_t Wgu[e][:,1,:] (+b1),  inter = silu(g)*u
 *   affinity on H (0): y_t += a * (inter Wd[e] + b2[e])
 *   affinity on I (1): y_t += (a * inter) Wd[e]            (no bias)
 * Backward (P1 phases; P3's epilogue):
 *   Phase 1  dS = dY_t Wd[e]^T (quantised along H), then the SwiGLU-backward
 *            epilogue on the fp32 product (a kernel of its own, or inside
 *            Phase 1's kernel where that measured faster, see phase1_ds):
 *            d(a) = sum_i dS*inter + <dY_t, b2[e]>,  dInter = a*dS,
 *            dGate = dInter*up*silu'(g),  dUp = dInter*silu(g)
 *   Phase 3  dX_t += [dGate,dUp] Wgu[e]^T    (quantised along I)
 *   Phase 2  dWgu[e] = sum over the expert's slots of x^T [dGate,dUp]
 *   Phase 4  dWd[e]  = sum of inter^T (a*dY)   (on H)  or  (a*inter)^T dY (on I)
 *   bias     db1[e] = sum [dGate,dUp],  db2[e] = sum a*dY
 * Phases 2 and 4 quantise along the token axis in groups of 32 consecutive
 * slots of one block.  Rounding points: gate_act, inter, a*inter, a*dY, dGate
 * and dUp are bf16 (the precision of the checkpoints P1 accepts); dS, dInter,
 * d(a) and every accumulator are fp32; outputs are bf16.
 * ------------------------------------------------------------------------- */
typedef struct {
  int64_t T, H, I, E, N, block_size;   /* I is P1's I_TP; block_size in {128,256,512,1024};
                                          H % 32 == 0, I % 32 == 0, N >= moe_num_blocks  */
  const uint16_t* hidden_states;                  /* [T,H] bf16                          */
  const float*    expert_affinities_masked;       /* [T*E] fp32, index t*E+e             */
  const uint8_t*  gate_up_codes;                  /* [E,H,2,I] codes, fmt_weight         */
  const uint8_t*  gate_up_scales;                 /* [E,H,2,I/32]: groups along I        */
  const uint8_t*  down_codes;                     /* [E,I,H] codes, fmt_weight           */
  const uint8_t*  down_scales;                    /* [E,I,H/32]: groups along H          */
  const int32_t*  token_position_to_id;           /* [N*B]; outside [0,T) = padding slot */
  const int32_t*  block_to_expert;                /* [N], each in [0,E)                  */
  const uint16_t* output_hidden_states_grad;      /* [T,H] bf16                          */
  const uint16_t* gate_up_proj_act_checkpoint_T;  /* [N,2,I,B] bf16, required:
                                                     [b,0,i,p] = gate_pre, [b,1,i,p] = up;
                                                     padding slots' values are ignored  */
  const uint16_t* down_proj_bias;                 /* [E,H] bf16, required iff has_bias   */
  int affinity_on;      /* 0 = affinity on H (output), 1 = on I (intermediate)          */
  int has_bias;         /* 1: add <dY,b2> to d(a) and write both bias gradients         */
  int fmt_weight;       /* element format of the pre-quantised weights (E4M3)           */
  int fmt_act;          /* activations X, inter, a*inter in Phases 2/4 (E4M3)          */
  int fmt_grad;         /* dY, a*dY, dGate/dUp (E5M2)                                   */
  uint16_t* hidden_states_grad;                   /* [T,H] bf16; unrouted tokens -> 0   */
  uint16_t* expert_affinities_masked_grad;        /* [T*E] bf16; unrouted pairs -> 0    */
  uint16_t* gate_up_proj_weight_grad;             /* [E,H,2,I] bf16; empty experts -> 0 */
  uint16_t* down_proj_weight_grad;                /* [E,I,H] bf16                        */
  uint16_t* gate_and_up_proj_bias_grad;           /* [E,2,I] bf16 (has_bias)             */
  uint16_t* down_proj_bias_grad;                  /* [E,H] bf16 (has_bias)               */
  /* Optional checkpoints ([P1] "Parameters": gate_act_checkpoint_T,
   * intermediate_checkpoint_T, scaled_intermediate_checkpoint_T,
   * down_proj_act_checkpoint).  NULL: the value is recomputed from the
   * gate/up checkpoint, dY and the affinities.  Supplied: it is read instead;
   * it must hold the value the recomputation rounds to (padding slots are
   * ignored), and the gradients are then the same.  All bf16.               */
  const uint16_t* gate_act_checkpoint_T;          /* [N,I,B] bf16(silu(gate_pre))        */
  const uint16_t* intermediate_checkpoint_T;      /* [N,I,B] bf16(gate_act * up)         */
  const uint16_t* scaled_intermediate_checkpoint_T; /* [N,I,B] bf16(a * intermediate);
                                                     affinity on I only                 */
  const uint16_t* down_proj_act_checkpoint;       /* [N,B,H] bf16(a * dY[token]) per slot;
                                                     affinity on H only (the Phase-4
                                                     operand)                           */
  /* [P1] num_valid_tokens: [1] int32 in device memory, optional (NULL: T).
   * Only the leading rows hold real tokens; a count above T means T, below 0
   * means 0.  Slots of tokens at or past the count are padding, so those
   * tokens' dX rows and d(a) entries are written as 0.  Read on the device by
   * the first stage, so the count may be produced by earlier work on the
   * stream.  With E = 1 and token_position_to_id = 0, 1, 2, ... (P1's
   * single_expert_dense) it is P1's dynamic block loop.                     */
  const int32_t* num_valid_tokens;
  /* [P1] accumulation flag (its meaning is not spelled out there; reading:
   * accumulate into the gradients instead of initialising them).  0: every
   * output above is overwritten.  1: each output element becomes
   * bf16(old + g), the value the caller's buffer holds plus the fp32 gradient,
   * rounded once; entries the overwrite mode writes as 0 (unrouted tokens and
   * pairs, empty experts) keep their old value.  For gradient accumulation
   * over micro-batches.                                                      */
  int accumulate;
  /* Gated activation of the gate projection ([P3] _down_projection_backward_act
   * accepts "swiglu" and "geglu"): MXFP8_ACT_SWIGLU (0, act = silu) or
   * MXFP8_ACT_GEGLU (1, act = gelu in its erf form, g * Phi(g) with Phi the
   * standard normal CDF; the pages do not say which GELU, and this is its
   * definition).  inter = act(gate_pre) * up, dGate = dInter * up * act'(g),
   * dUp = dInter * act(g); gate_act_checkpoint_T then holds bf16(act(g)).   */
  int activation;
} moe_bwd_mxfp8_args;
typedef enum { MXFP8_ACT_SWIGLU = 0, MXFP8_ACT_GEGLU = 1 } mxfp8_activation;

/* Byte offsets of the workspace regions (each 256-byte aligned).  The quantised
 * operands can be read back from them after a call:
 *   dy_codes/dy_scales        [T,H] / P4[H,T]         dY along H (Phase 1); scales
 *                                                     [T,H/32] when H % 128 != 0
 *   dy_deq                    [T,H] bf16              exact values of those codes
 *                                                     (H % 128 != 0; else empty)
 *   wd_deq                    [E,I,H] bf16            exact values of the W_down codes
 *                                                     (H % 128 != 0; else empty)
 *   x_tok_codes/scales        S64[P,H] / P4[P,H]      X along slots (Phase 2), P = N*B
 *   gy_tok_codes/scales       S64[P,H] / P4[P,H]      a*dY (on H) or dY (on I), Phase 4
 *   inter_tok_codes/scales    S64[P,I] / P4[P,I]      inter (on H) or a*inter (on I)
 *   dgu_row_codes/scales      S64[2I,P] / P4[2I,P]    [dGate|dUp] along I (Phase 3);
 *                                                     [P,2I] / [P,2I/32] when 2I % 128 != 0
 *   dgu_tok_codes/scales      S64[P,2I] / P4[P,2I]    [dGate;dUp] along slots (Phase 2)
 *   wgu_scales_pairs          P4 of gate_up_scales per expert, [E][2I/128][H][4]
 *                                                     (written when 2I % 128 == 0)
 *   wd_scales_pairs           P4 of down_scales per expert, [E][H/128][I][4]
 *                                                     (H % 128 == 0; else empty)
 *   phase1_ds                 [N,I,B] fp32            Phase 1's product dS per block
 *                                                     (slots past a block's extent unwritten;
 *                                                     empty, like phase1_tiles, where Phase 1
 *                                                     runs with its epilogue in one kernel:
 *                                                     H % 128 == 0, H <= 2048, I <= 512 and
 *                                                     no caller checkpoints)
 *   phase1_tiles/phase3_tiles [N+1 + tiles] int32     first tile of each block over its
 *                                                     live slot tiles (with round-robin tile
 *                                                     order the blocks whose slot tiles are
 *                                                     all live first), and the total; then
 *                                                     each tile's block
 *   dx_slot [P,H] fp32 (each routed slot's dX row, summed per token at the end),
 *   phase3_parts: Phase 3's last, partly filled round of tiles cut along K: each
 *   XCD's cut (256 bytes), then fp32 tiles (up to 256 of 256 x 256 or 128 x 256)
 *   holding the later K parts of the cut tiles, which are added into dx_slot
 *   before the stage ends (empty when 2I % 128 != 0 or 2I < 4096),
 *   slot_of [T,E] int32 (the slot of pair (t, e), -1 = none),
 *   daff_slot [P] fp32 (the <dY, b2> term when it is computed on its own, else 0),
 *   daff_part [I/32 (+ H/128), P] fp32 (d(a) partials per 32 rows i; with a bias,
 *   H % 128 == 0 and no down_proj_act_checkpoint, then the <dY, b2> shares per
 *   128 columns h), db1_acc [E,2,I] fp32, db2_acc [E,H] fp32,
 *   expert_block_offsets [E+1] int32 and expert_block_list [N] int32: the blocks of
 *   expert e holding at least one routed slot are list[off[e] .. off[e+1]), ascending;
 *   slot_token [P] int32 (-1 = padding), slot_affinity [P] fp32, block_flag [N] int32
 *   (one past the block's last routed slot; 0 = no routed slot).
 * P4[K,R] is the pair-major scale layout of an operand with R rows contracted
 * over K elements: [K/128][R][4] bytes, word (p, r) holding row r's E8M0 bytes
 * for elements [128p, 128p+128) (so one stage pair's words for consecutive rows
 * are contiguous).  S64[K,R] is the stage-major code layout of such an
 * operand: the rows in panels of 256 (the last one holds R % 256 when that is
 * not 0), panel rows r0 .. r0+n-1 at bytes [r0*K, (r0+n)*K) as [K/64][n][64], so
 * that code (r, k) sits at r0*K + ((k/64)*n + r - r0)*64 + k%64 (64 elements of
 * every row of a panel in one contiguous run: whole cache lines per load).
 * Pad slots hold code 0.  Otherwise, rows of a region are contiguous. */
typedef struct {
  size_t dy_codes, dy_scales, dy_deq, wd_deq, x_tok_codes, x_tok_scales, gy_tok_codes, gy_tok_scales,
      inter_tok_codes, inter_tok_scales, dgu_row_codes, dgu_row_scales, dgu_tok_codes,
      dgu_tok_scales, wgu_scales_pairs, wd_scales_pairs, phase1_ds, phase1_tiles, phase3_tiles, dx_slot,
      phase3_parts, slot_of, daff_slot, daff_part, db1_acc, db2_acc, expert_block_offsets,
      expert_block_list, slot_token, slot_affinity, block_flag, total;
} moe_bwd_mxfp8_workspace_layout;

/* Host.  Fills *layout for the shapes in *args (pointers are not read).
 * Returns MXFP8_OK or INVALID_ARG. */
int moe_bwd_mxfp8_workspace_query(const moe_bwd_mxfp8_args* args,
                                  moe_bwd_mxfp8_workspace_layout* layout);
/* Host.  Workspace size in bytes (0 on invalid shapes). */
size_t moe_bwd_mxfp8_workspace_size(const moe_bwd_mxfp8_args* args);

/* Enqueues the whole backward on `stream`.  When Phase 3 has between one and
 * eight rounds of tiles over the device's CUs, part of the work (the
 * token-axis gathers and Phases 2 and 4) runs on a second stream that the
 * library creates once per device (default priority) and keeps; `stream`
 * waits for it before the call returns, so work enqueued on `stream` later is
 * ordered after the whole backward, as with one stream.  Host threads that
 * call this on one device at the same time are serialised while they enqueue.
 * Errors: INVALID_ARG (shapes, null required
 * pointers, alignment, formats, accumulate or activation outside {0,1}), UNSUPPORTED
 * (block_size outside the set, affinity on I together with a bias, or sizes
 * beyond 32-bit indexing: N * block_size, T * E or T * H above 2^31 - 1 (dY's
 * [T,H] codes are gathered through one buffer descriptor), a [T,H] bf16 tensor
 * of 2 GiB or more (T * H * 2 > 2^31 - 1) when H is not a multiple of 128
 * (Phase 1 then gathers dY's bf16 values that way), I * block_size * 4 beyond 2 GiB, or a
 * 256-row panel of a stage-major operand, 256 * N * block_size or 256 * 2I
 * bytes, beyond 2^32 - 1), WORKSPACE (too small).  Device-side
 * preconditions (not checked): block_to_expert entries in [0,E) (blocks with
 * other values are skipped); each (t,e) pair appears in at most one slot. */
int moe_bwd_mxfp8(const moe_bwd_mxfp8_args* args, void* workspace, size_t workspace_bytes,
                  void* stream);

/* Profiling aid: enqueue only one stage of moe_bwd_mxfp8, on a workspace that a
 * full call with the same arguments has already filled (stages read what the
 * earlier ones wrote there).  Running stages in order 0..MOE_BWD_NUM_STAGES-1
 * is exactly one full call.  Stages:
 *   0 setup (zero accumulators, slot routing info, per-expert block lists)
 *   1 quantise dY along H (and lay out W_down's scales for Phase 1)
 *   2 gather-quantise X and a*dY (or dY) along slots (and, with a bias, db2
 *     and the <dY, b2> shares of d(a) from the same dY rows)
 *   3 bias reductions (has_bias only; nothing when stage 2 does them: H a
 *     multiple of 128 and no down_proj_act_checkpoint)
 *   4 Phase 1 (the product dS)
 *   5 Phase 1 epilogue (SwiGLU backward; dGU along I and along slots, the
 *     intermediate along slots, d(affinity) and db1 partial sums); where the
 *     layout has no phase1_ds (see there) stage 4 does this too and stage 5
 *     nothing
 *   6 Phase 3 (dX rows per slot)  7 Phase 2 (dW_gate_up)       8 Phase 4 (dW_down)
 *   9 finalise (dX summed per token in expert order, the rest to bf16)
 * Errors as for moe_bwd_mxfp8, plus INVALID_ARG for a stage outside the range. */
#define MOE_BWD_NUM_STAGES 10
int moe_bwd_mxfp8_stage(const moe_bwd_mxfp8_args* args, void* workspace, size_t workspace_bytes,
                        int stage, void* stream);

/* ---------------------------------------------------------------------------
 * moe_router_bwd -- the router backward that consumes the affinity gradient
 * ([P3] sonic-moe functional/backward.py: the softmax-over-top-k, top-k-over-
 * softmax and top-k scatter backward kernels).  Per token t, with selected
 * experts idx[t][0..K) (distinct, in [0,E); an entry outside that range is
 * skipped) and upstream score gradients g[t][k], it writes the gradient of the
 * router logits d[t][0..E):
 *   MXFP8_ROUTER_SOFTMAX_OVER_TOPK  scores y = softmax over the K selected
 *       logits (topk_scores = y, required):
 *       d[idx_k] = y_k (g_k - sum_m g_m y_m), 0 elsewhere.
 *   MXFP8_ROUTER_TOPK_OVER_SOFTMAX  p = softmax over all E logits (logits,
 *       required), scores p[idx_k], or with renorm != 0 s_k = p[idx_k] / S,
 *       S = sum_k p[idx_k] (topk_scores = s, required with renorm):
 *       dp_k = g_k, or (g_k - sum_m g_m s_m) / S with renorm;
 *       d[e] = p_e (dp(e) - sum_k dp_k p[idx_k]) for every e, where dp(e) is
 *       dp_k at e = idx_k and 0 elsewhere.
 *   MXFP8_ROUTER_TOPK  scores = the selected logits: d[idx_k] = g_k, 0 elsewhere.
 * Arguments:
 *   T, E, K      tokens, experts, selections per token; 1 <= K <= min(E, 32).
 *   topk_idx     [T,K] int32.
 *   topk_scores  [T,K] fp32 forward scores (see the modes), else may be NULL.
 *   logits       [T,E] fp32 router logits (top-k over softmax), else may be NULL.
 *   dscores      [T,K] fp32 upstream score gradients, or NULL and
 *   daff         [T,E] bf16 affinity gradient in the masked layout (index
 *                t*E + e, as moe_bwd_mxfp8 writes expert_affinities_masked_grad),
 *                read at the selected experts: exactly one of the two.
 *   renorm       0 or 1; non-zero only with MXFP8_ROUTER_TOPK_OVER_SOFTMAX.
 *   dlogits      [T,E] fp32 output, every entry written.
 * Arithmetic is fp32 (exp through the device math library).
 * Errors: INVALID_ARG for an unknown mode, a shape outside the bounds above,
 * renorm with another mode, both or neither of dscores/daff, a NULL pointer
 * for a tensor the mode reads or writes, or a tensor not 16-byte aligned;
 * HIP if the launch fails. */
typedef enum {
  MXFP8_ROUTER_SOFTMAX_OVER_TOPK = 0,
  MXFP8_ROUTER_TOPK_OVER_SOFTMAX = 1,
  MXFP8_ROUTER_TOPK = 2
} mxfp8_router_mode;
#define MXFP8_ROUTER_MAX_K 32
int moe_router_bwd(int mode, int64_t T, int64_t E, int64_t K, const int32_t* topk_idx, const float* topk_scores,
                   const float* logits, const float* dscores, const uint16_t* daff, int renorm, float* dlogits,
                   void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MXFP8_MOE_H */
