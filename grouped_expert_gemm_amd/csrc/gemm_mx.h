// MXFP8 grouped MLP forward (MX-scaled fp8 MFMA).
#pragma once

#include "common.h"

namespace moe {
namespace mx {

moe_status forward(const moe_mlp_desc& d, int64_t R, const void* x_perm, const uint8_t* x_perm_scale,
                   const void* const* w_gate_up, const void* const* w_down, const uint8_t* const* w_gate_up_scale,
                   const uint8_t* const* w_down_scale, const int32_t* offsets, const float* prob_perm,
                   void* y_perm, uint8_t* workspace, hipStream_t s, void* z_save = nullptr,
                   void* h_save = nullptr);

// MXFP8 gate_up + ScaledSwiGLU on pre-quantised operands; h written as MXFP8, and
// optionally z [R, 2I] and h [R, I] in bf16 for the backward. step_major: every scale
// array (x's, the weights', h's) in the step-major layout of launch_mxfp8_quantize_step_major
// (the wide-step kernel), else in the public row-major layout.
moe_status gate_up(int E, int64_t R, int H, int I, const uint8_t* x, const uint8_t* x_scale, const void* const* w,
                   const uint8_t* const* w_scale, const int32_t* offsets, const float* prob, uint8_t* h,
                   uint8_t* h_scale, hipStream_t s, void* z_save = nullptr, void* h_save = nullptr,
                   bool step_major = false);

// per-tensor FP8 forward (E4M3 with one float32 scale per tensor: x_perm, each expert's
// W1 and W2, and h, which is stored in bf16 before its scale is known: into h_save when
// given, and z = [G, U] into z_save when given)
size_t fp8_tensor_workspace_bytes(const moe_mlp_desc& d, int64_t R);
moe_status forward_fp8_tensor(const moe_mlp_desc& d, int64_t R, const void* x_perm, const float* x_scale,
                              const void* const* w_gate_up, const void* const* w_down, const float* const* w_gate_up_scale,
                              const float* const* w_down_scale, const int32_t* offsets, const float* prob_perm,
                              void* y_perm, uint8_t* ws, hipStream_t s, void* z_save = nullptr,
                              void* h_save = nullptr);

// MXFP8 backward (bf16 inputs and outputs, every GEMM operand quantised along its K axis)
size_t bwd_workspace_bytes(const moe_mlp_desc& d, int64_t R);
moe_status backward(const moe_mlp_desc& d, int64_t R, const bf16_t* dy, const bf16_t* x, const bf16_t* z,
                    const bf16_t* h, const float* prob, const void* const* w_gate_up, const void* const* w_down,
                    const int32_t* offsets, bf16_t* dx, void* const* dw_gate_up, void* const* dw_down, float* dprob,
                    uint8_t* ws, hipStream_t s);

// per-tensor FP8 backward (bf16 inputs and outputs, one factor per tensor: dY, dZ, h,
// x over all rows, each expert's W1 and W2)
size_t fp8_bwd_workspace_bytes(const moe_mlp_desc& d, int64_t R);
moe_status backward_fp8_tensor(const moe_mlp_desc& d, int64_t R, const bf16_t* dy, const bf16_t* x, const bf16_t* z,
                               const bf16_t* h, const float* prob, const void* const* w_gate_up,
                               const void* const* w_down, const int32_t* offsets, bf16_t* dx, void* const* dw_gate_up,
                               void* const* dw_down, float* dprob, uint8_t* ws, hipStream_t s);

}  // namespace mx
}  // namespace moe
