// Internal declarations shared between the library's translation units.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "moe.h"

namespace moe {

size_t align_up(size_t x, size_t a);

size_t permute_workspace_bytes(int64_t T, int E, int k);

moe_status validate_desc(const moe_mlp_desc& d, bool backward);
size_t mlp_fwd_workspace_bytes(const moe_mlp_desc& d, int64_t R);
size_t mlp_bwd_workspace_bytes(const moe_mlp_desc& d, int64_t R);
size_t grouped_gemm_workspace_bytes();  // split-K tail area of one grouped GEMM call
size_t router_bwd_workspace_bytes(int64_t T, int H, int E);  // dW token-chunk partials

// mxfp8 quantisation launcher used by the forward (weights and activations)
moe_status launch_mxfp8_quantize(const void* in_bf16, int64_t rows, int64_t cols, uint8_t* e4m3,
                                 uint8_t* e8m0, void* stream);
// the same codes, scales written step-major: the 4 scale bytes of 128 values of row r
// form one 32-bit word; the words of K step k of all rows are contiguous (word k * rows
// + r). cols % 128 == 0. This is the scale layout the wide-step MXFP8 GEMM reads.
moe_status launch_mxfp8_quantize_step_major(const void* in_bf16, int64_t rows, int64_t cols, uint8_t* e4m3,
                                            uint8_t* e8m0, void* stream);
// public-layout scales [rows][cols / 32] of n tensors of one shape -> step-major (4-byte
// aligned pointers, n <= MOE_MAX_EXPERTS, cols % 128 == 0)
moe_status launch_mx_scales_step_major(const uint8_t* const* src, uint8_t* const* dst, int n, int64_t rows,
                                       int64_t cols, void* stream);

// column-wise (token-axis) MXFP8 of x [R, C] per expert (rule of mxfp8_quantize_colwise);
// offsets NULL: one expert of R rows; kofs NULL: the padded offsets are not written.
// The caller guarantees C % 64 == 0, pad % 32 == 0, kcap % 32 == 0, kcap >= the padded
// row total, 16-byte aligned x and codes.
// step_major: scales in the step-major layout of launch_mxfp8_quantize_step_major over
// the transposed [C, kcap] output (word (k / 128) * C + c; kcap % 128 == 0).
// rcodes (optional): also the row-wise codes [R, C] of x (those of mxfp8_quantize) from
// the same loads, with the scales in rscales: [R][C / 32] for rstep == 0, else
// step-major over rstep rows (launch_mxfp8_quantize_step_major's layout; C % 128 == 0);
// rcodes 8-byte aligned.
moe_status launch_mxfp8_colwise(const void* x_bf16, int64_t R, int C, int E, const int32_t* offsets, int pad,
                                int64_t kcap, uint8_t* codes, uint8_t* scales, int32_t* kofs, hipStream_t s,
                                bool step_major = false, uint8_t* rcodes = nullptr, uint8_t* rscales = nullptr,
                                int64_t rstep = 0);
// the same for n tensors of one shape (host arrays of device pointers), as few launches
// as possible; kofs, when not NULL, is written once (it depends only on offsets)
moe_status launch_mxfp8_colwise_multi(int n, const void* const* x_bf16, int64_t R, int C, int E,
                                      const int32_t* offsets, int pad, int64_t kcap, uint8_t* const* codes,
                                      uint8_t* const* scales, int32_t* kofs, hipStream_t s, bool step_major,
                                      uint8_t* const* rcodes = nullptr, uint8_t* const* rscales = nullptr,
                                      int64_t rstep = 0);

// per-tensor FP8 (one float32 scale per tensor). A tensor's word holds the float bits
// of its amax between fp8t_amax and fp8t_finalize (cleared first by fp8t_zero), and
// its scale amax / 448 (1 for amax = 0) after fp8t_finalize. n: elements per tensor,
// a multiple of 8; inputs bf16 16-byte aligned, codes 8-byte aligned.
moe_status fp8t_zero(float* words, int n, hipStream_t s);
moe_status fp8t_amax(const void* const* in, int ntensors, int64_t n, float* words, hipStream_t s);
moe_status fp8t_quantize(const void* const* in, uint8_t* const* out, int ntensors, int64_t n, const float* words,
                         hipStream_t s);
moe_status fp8t_finalize(float* words, int n, hipStream_t s);
// Transposed per-tensor FP8 codes of x [R, C] (bf16, rows grouped into E experts by
// offsets; offsets NULL: one expert of R rows): out [C, kcap], expert e's rows at
// columns kofs[e] .. (padded to a multiple of pad, zeros in the padding), with the
// factor of words[t] (amax bits, between fp8t_amax and fp8t_finalize) for tensor t of
// in/out. kofs (E + 1 padded offsets) is written when not NULL. C % 64 == 0, pad and
// kcap multiples of 32, kcap >= R + E * (pad - 1) (without offsets: R rounded up to a
// multiple of pad), at most 64 tensors. rows_out (optional): per tensor, also the
// row-major codes [R, C] (those of fp8t_quantize), from the same loads.
moe_status fp8t_transpose(const void* const* in, uint8_t* const* out, int ntensors, int64_t R, int C, int E,
                          const int32_t* offsets, int pad, int64_t kcap, const float* words, int32_t* kofs,
                          hipStream_t s, uint8_t* const* rows_out = nullptr);

}  // namespace moe
