/*
 * mxfp8_oracle.h -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow CPU implementation of what the MXFP8 MoE backward computes.
 * It is the reference that the HIP library is checked against and is never
 * part of the product path: only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load it.  It shares no code, header,
 * table or constant with the GPU library.
 *
 * Sources (page titles; sections named, no line numbers):
 *   [P1] AWS Neuron NKI library, "Blockwise MM Backward MXFP8 Kernel API
 *        Reference" (nkilib.experimental.moe_mxfp8.bwd): the parameter list,
 *        the return tuple and the "Dimensions" paragraph.
 *   [P2] AWS Neuron NKI library, "Matmul MXFP8 Backward Kernel API
 *        Reference" (nkilib.experimental.matmul_mxfp8): the forward/backward
 *        convention paragraph and the parameter list.
 *   [P3] sonic-moe, functional/backward.py: _down_projection_backward_act,
 *        _up_projection_backward_act/_weight, _down_projection_backward_weight,
 *        db1_kernel and db2_and_ds_kernel.
 *
 * Every value crossing this interface is a host pointer.  bf16 tensors are
 * passed as their uint16_t bit patterns.  Nothing here allocates memory the
 * caller must free.
 *
 * Format codes: 0 = OCP E4M3 (E4M3FN), 1 = OCP E5M2, -1 = "no quantisation"
 * (test hook: dequantised value == input value; used to pin the algebra of
 * the quantised path against the exact path).
 */
#ifndef MXFP8_ORACLE_H
#define MXFP8_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- element codec (MX element formats; P1 names "MXFP8", P2 "float8_e5m2") ---- */
double  orc_fp8_decode(int code, int fmt);           /* value of one 8-bit code          */
int     orc_fp8_encode(double y, int fmt);           /* RNE, saturating, sign kept       */
int     orc_fp8_encode_array(const double* y, int64_t n, int fmt, uint8_t* out);
int     orc_fp8_emax(int fmt);                       /* exponent of the largest binade   */
double  orc_bf16_to_double(uint16_t b);
uint16_t orc_double_to_bf16(double x);               /* one RNE rounding from fp64       */

/* ---- one 32-element group: E8M0 scale byte + codes; deq gets decode(code)*2^X ---- */
int orc_quantize_group(const double* v, int n, int fmt, uint8_t* codes, double* deq);

/* ---- whole-tensor quantiser (P1: "32-element quantization group")
 * x [R][C] bf16.  axis 1: groups of 32 along C, scales [R][C/32].
 *                 axis 0: groups of 32 along R, scales [R/32][C].
 * codes [R][C] always in x's layout.  Returns 0, or -1 on bad sizes. */
int orc_quantize(const uint16_t* x, int64_t R, int64_t C, int axis, int fmt,
                 uint8_t* codes, uint8_t* scales);

/* ---- MX GEMM emulation: C[m][n] = fp32( sum_k deqA[m][k] * deqB[n][k] ),
 * exact products summed in fp64.  A [M][K] codes + scales [M][K/32],
 * B [N][K] codes + scales [N][K/32]. */
int orc_mx_gemm_nt(const uint8_t* a_codes, const uint8_t* a_scales, int fmt_a,
                   const uint8_t* b_codes, const uint8_t* b_scales, int fmt_b,
                   int64_t M, int64_t N, int64_t K, float* C, int nthreads);

/* ---- dense backward (P2): forward Y = X W^T with X [M][K], W [N][K].
 * dX = dY W   [M][K]  (contraction over N: dY and W quantised along N)
 * dW = dY^T X [N][K]  (contraction over M: dY and X quantised along M)
 * dx_rows / dw_rows select output rows (NULL = all rows, n ignored); the
 * outputs are then [n_dx_rows][K] and [n_dw_rows][K] (either may be NULL). */
int orc_dense_bwd(const uint16_t* dY, const uint16_t* W, const uint16_t* X,
                  int64_t M, int64_t N, int64_t K, int fmt_dy, int fmt_w, int fmt_x,
                  const int64_t* dx_rows, int64_t n_dx_rows, uint16_t* dX,
                  const int64_t* dw_rows, int64_t n_dw_rows, uint16_t* dW, int nthreads);

/* ---- routing blocks (P1 "Dimensions": N = (T*TopK - (E-1))/B + E - 1) ---- */
int64_t orc_num_blocks(int64_t T, int64_t K, int64_t E, int64_t B);
/* topk [T][K] expert ids (distinct per row, in [0,E); a negative id is a
 * dropped selection -- page 3's varlen-K routing, where a token activates
 * fewer than K experts -- and is skipped).  Writes token_position_to_id
 * [N*B] (-1 = padding) and block_to_expert [N].
 * Returns 0, or -1 if N is too small / an id is E or larger. */
int orc_build_blocks(const int32_t* topk, int64_t T, int64_t K, int64_t E, int64_t B,
                     int64_t N, int32_t* tpid, int32_t* b2e);

/* ---- MoE backward, MXFP8 mode (P1's kernel; P3's epilogue math) ---- */
typedef struct {
  int64_t T, H, I, E, N, B;
  const uint16_t* hidden;                          /* [T][H] bf16                       */
  const float*    aff;                             /* [T*E] fp32, index t*E+e           */
  const uint8_t*  wgu_codes; const uint8_t* wgu_scales;  /* [E][H][2][I], [E][H][2][I/32] */
  const uint8_t*  wd_codes;  const uint8_t* wd_scales;   /* [E][I][H],    [E][I][H/32]    */
  const int32_t*  tpid;                            /* [N*B], outside [0,T) = padding    */
  const int32_t*  b2e;                             /* [N]                               */
  const uint16_t* dy;                              /* [T][H] bf16                       */
  const uint16_t* ckpt;                            /* [N][2][I][B] bf16 (gate_pre, up)  */
  const uint16_t* b2;                              /* [E][H] bf16 or NULL               */
  int affinity_on;                                 /* 0 = on H (output), 1 = on I       */
  int has_bias;                                    /* adds <dY, b2[e]> to d(affinity)   */
  int fmt_w, fmt_act, fmt_grad;
  int nthreads;                                    /* 0 = all host cores                */
  int accumulate;      /* P1's accumulation flag (reading: add into the gradients):
                          1 = every output element o becomes bf16(fp32(o + g)), the
                          buffer's value plus the exact gradient, rounded as an fp32
                          sum would be; 0 = bf16(fp32(g))                        */
  int activation;      /* gated activation of the gate projection: 0 = SwiGLU
                          (silu), 1 = GeGLU (gelu, the erf form g * Phi(g))       */
} orc_moe_problem;

/* All outputs bf16.  Full problem: dx [T][H], daff [T*E], dwgu [E][H][2][I],
 * dwd [E][I][H], db1 [E][2][I], db2 [E][H] (any may be NULL).  With accumulate
 * the output buffers hold the values to add to on entry. */
int orc_moe_bwd(const orc_moe_problem* p, uint16_t* dx, uint16_t* daff, uint16_t* dwgu,
                uint16_t* dwd, uint16_t* db1, uint16_t* db2);

/* Selected tokens: dx_rows [ntok][H], daff_rows [ntok][E]. */
int orc_moe_token_rows(const orc_moe_problem* p, const int32_t* tokens, int64_t ntok,
                       uint16_t* dx_rows, uint16_t* daff_rows);

/* One expert, selected intermediate columns i: dwgu_cols [H][2][nicol],
 * dwd_rows [nicol][H], db1_cols [2][nicol], db2_row [H] (any may be NULL). */
int orc_moe_expert_cols(const orc_moe_problem* p, int64_t e, const int32_t* icols, int64_t nicol,
                        uint16_t* dwgu_cols, uint16_t* dwd_rows, uint16_t* db1_cols,
                        uint16_t* db2_row);

/* Per-block intermediates of the epilogue (for diagnostics and identities):
 * dS [B][I] fp32, ga/inter/dG/dU [B][I] bf16, daff_slot [B] fp32 (any NULL). */
int orc_moe_block_detail(const orc_moe_problem* p, int64_t b, float* dS, uint16_t* ga,
                         uint16_t* inter, uint16_t* dG, uint16_t* dU, float* daff_slot);

/* Token-axis quantised operands of the weight-gradient GEMMs, [rows][N*B] codes
 * and [rows][N*B/32] scales:  which = 0: X (rows H, fmt_act);
 * 1: a*dY under affinity-on-H, dY under affinity-on-I (rows H, fmt_grad);
 * 2: inter under on-H, a*inter under on-I (rows I, fmt_act);
 * 3: [dG;dU] (rows 2I, fmt_grad). */
int orc_moe_token_operand(const orc_moe_problem* p, int which, uint8_t* codes, uint8_t* scales);

/* ---- MoE exact mode: the plain definition of the layer and its gradients in
 * fp64, with no quantisation and no bf16 rounding (used for finite
 * differences) ---- */
typedef struct {
  int64_t T, H, I, E, N, B;
  const double* x;    /* [T][H]        */
  const double* aff;  /* [T*E]         */
  const double* wgu;  /* [E][H][2][I]  */
  const double* b1;   /* [E][2][I] or NULL */
  const double* wd;   /* [E][I][H]     */
  const double* b2;   /* [E][H] or NULL (must be NULL when affinity_on == 1) */
  const int32_t* tpid;
  const int32_t* b2e;
  int affinity_on;
  int activation;     /* 0 = SwiGLU, 1 = GeGLU */
} orc_moe_exact_problem;

/* y [T][H]; gu_ckpt [N][2][I][B] pre-activations (NULL to skip). */
int orc_moe_fwd_exact(const orc_moe_exact_problem* p, double* y, double* gu_ckpt);
/* Gradients of L = <dy, y>.  Outputs are fully overwritten. */
int orc_moe_bwd_exact(const orc_moe_exact_problem* p, const double* dy, double* dx,
                      double* daff, double* dwgu, double* dwd, double* db1, double* db2);

#ifdef __cplusplus
}
#endif
#endif
