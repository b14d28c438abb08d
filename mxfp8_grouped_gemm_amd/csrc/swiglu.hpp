// swiglu.hpp -- gated-activation (SwiGLU, GeGLU) recompute and backward
// factors for the Phase-1 epilogue.
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

// GeGLU's gate activation (P3 accepts "geglu" beside "swiglu"; the GELU taken
// is its definition g * Phi(g), Phi the standard normal CDF):
// Phi(g) = erfc(-g / sqrt 2) / 2 with the device library's erfcf (a few ulp,
// relative, also for negative g, where 1 + erf would cancel), and
// gelu'(g) = Phi(g) + g * exp(-g^2 / 2) / sqrt(2 pi) with v_exp_f32.
__device__ __forceinline__ float normal_cdf(float g) { return 0.5f * erfcf(g * -0.70710678118654752f); }
__device__ __forceinline__ float dgelu_from(float g, float cdf) {
  return cdf + g * (0.39894228040143268f * __builtin_amdgcn_exp2f(g * g * -0.72134752044448170f));
}

__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) { return bf16x2_pack(a, b); }
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

}  // namespace mx
