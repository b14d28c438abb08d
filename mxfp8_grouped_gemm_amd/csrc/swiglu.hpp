// swiglu.hpp -- SwiGLU recompute and backward factors for the Phase-1 epilogue.
//
// P1 ("Blockwise MM Backward MXFP8 Kernel API Reference", the checkpoint
// parameters): gate_act = SiLU(gate_pre) and intermediate = gate_act * up are
// recomputed per block from gate_up_proj_act_checkpoint_T; both are tensors
// the caller may also supply, so both are rounded to bf16.
// P3 (sonic-moe functional/backward.py, _down_projection_backward_act): the
// gated-activation backward dGate = dInter * up * silu'(gate_pre) and
// dUp = dInter * silu(gate_pre), with silu'(g) = s * (1 + g * (1 - s)),
// s = sigmoid(g).
#pragma once
#include "mx_device.hpp"

namespace mx {

// sigmoid(g) = 1 / (1 + 2^(-g log2 e)) through v_exp_f32 and v_rcp_f32 (each
// about 1 ulp): a few ulp of fp32, far below the bf16 rounding that follows.
// Large |g| saturates correctly (2^+big = inf -> 0, 2^-big = 0 -> 1).
__device__ __forceinline__ float sigmoid_fast(float g) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f));
}

// silu'(g) from s = sigmoid(g)
__device__ __forceinline__ float dsilu_from(float g, float s) { return s * (1.f + g * (1.f - s)); }

__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) { return bf16x2_pack(a, b); }
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

}  // namespace mx
