// swiglu.hpp -- SwiGLU recompute and backward factors, shared by every kernel
// that needs them so that all of them round identically.
//
// P1 ("Blockwise MM Backward MXFP8 Kernel API Reference", the checkpoint
// parameters): gate_act = SiLU(gate_pre) and intermediate = gate_act * up are
// recomputed per block from gate_up_proj_act_checkpoint_T; both are tensors
// the caller may also supply, so both are rounded to bf16 here.
// P3 (sonic-moe functional/backward.py, _down_projection_backward_act): the
// gated-activation backward dGate = dInter * up * silu'(gate_pre) and
// dUp = dInter * silu(gate_pre).
#pragma once
#include "mx_device.hpp"

namespace mx {

__device__ __forceinline__ float sigmoid_f32(float g) { return 1.f / (1.f + expf(-g)); }

// bf16(silu(g))
__device__ __forceinline__ float swiglu_gate_act(float g) { return bf16_to_f32(f32_to_bf16(g * sigmoid_f32(g))); }

// bf16(bf16(silu(g)) * u): the product of two bf16 values is exact in fp32.
__device__ __forceinline__ float swiglu_inter(float g, float u) {
  return bf16_to_f32(f32_to_bf16(swiglu_gate_act(g) * u));
}

// silu'(g) = s * (1 + g * (1 - s)), s = sigmoid(g)
__device__ __forceinline__ float dsilu_f32(float g) {
  const float s = sigmoid_f32(g);
  return s * (1.f + g * (1.f - s));
}

}  // namespace mx
