// MXFP8 block quantisation of bf16 rows: one E8M0 scale per 32 consecutive values,
// E4M3 elements. Source: "Efficient MoE Training for Biological Foundation Models",
// Challenge 2 (block of 32 consecutive values per scaling factor, 8-bit values) and
// Challenge 3 (bf16 weights and activations quantised before the low-precision GEMM).
//
// HBM-bound: 2 bytes in, 1 + 1/32 bytes out per element. Four lanes own one block
// (16 bytes of bf16 each, so a wavefront reads 1 KiB contiguous); the block maximum is
// reduced with two xor-shuffles; each lane writes its 8 codes as one 8-byte store.
#include "common.h"
#include "internal.h"

namespace moe {

__global__ __launch_bounds__(256) void mxfp8_quantize_kernel(const uint4* __restrict__ in, int64_t nblocks,
                                                             uint2* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
  const int64_t lane_global = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  // the loop trip count is uniform across a wavefront (stride and the start differ by
  // lane only inside one multiple of 64), so every lane reaches the shuffles
  const int64_t total = nblocks * 4;
  const int64_t total_padded = (total + 63) / 64 * 64;
  for (int64_t q = lane_global; q < total_padded; q += stride) {
    const bool live = q < total;
    uint4 v = live ? in[q] : make_uint4(0, 0, 0, 0);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
      f[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    const int s = mx_scale_exponent(amax);
    uint32_t c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = e4m3_encode(ldexpf(f[i], -s));
    if (live) {
      codes[q] = make_uint2(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                            c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24));
      if ((q & 3) == 0) scales[q >> 2] = (uint8_t)(s + 127);
    }
  }
}

moe_status launch_mxfp8_quantize(const void* in_bf16, int64_t rows, int64_t cols, uint8_t* e4m3,
                                 uint8_t* e8m0, void* stream) {
  const int64_t nblocks = rows * (cols / 32);
  if (nblocks == 0) return MOE_OK;
  const int threads = 256;
  int64_t want = (nblocks * 4 + threads - 1) / threads;
  const int64_t cap = (int64_t)num_cus() * 16;
  const unsigned grid = (unsigned)(want < cap ? want : cap);
  hipLaunchKernelGGL(mxfp8_quantize_kernel, dim3(grid), dim3(threads), 0, as_stream(stream),
                     (const uint4*)in_bf16, nblocks, (uint2*)e4m3, e8m0);
  return check_launch("mxfp8_quantize");
}

}  // namespace moe

using namespace moe;

extern "C" moe_status mxfp8_quantize(const void* in_bf16, int64_t rows, int64_t cols, uint8_t* e4m3,
                                     uint8_t* e8m0, void* stream) {
  if (rows < 0 || cols < 0) return fail(MOE_ERR_INVALID_ARG, "mxfp8_quantize: negative size");
  if (cols % 32 != 0) return fail(MOE_ERR_INVALID_ARG, "mxfp8_quantize: cols % 32 != 0");
  if (rows == 0 || cols == 0) return MOE_OK;
  if (!in_bf16 || !e4m3 || !e8m0) return fail(MOE_ERR_INVALID_ARG, "mxfp8_quantize: NULL pointer");
  if (!aligned(in_bf16, 16) || !aligned(e4m3, 8))
    return fail(MOE_ERR_INVALID_ARG, "mxfp8_quantize: input must be 16-byte and codes 8-byte aligned");
  return launch_mxfp8_quantize(in_bf16, rows, cols, e4m3, e8m0, stream);
}
