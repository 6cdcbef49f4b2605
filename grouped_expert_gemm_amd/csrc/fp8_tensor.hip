// Per-tensor FP8 quantisation (E4M3 codes, one float32 scale per tensor).
//
// Source: "Efficient MoE Training for Biological Foundation Models", Challenge 2, which
// sets FP8 with one scaling factor for a whole tensor against MXFP8's factor per 32
// values. The pages give no scale rule; the one implemented is current scaling:
// s = amax / 448 in float32 (amax = max |x| over the tensor; s = 1 when amax = 0), and
// each element's code is the E4M3 code (round to nearest, ties to even, saturating)
// of the float32 quotient x / s.
//
// The whole-tensor maximum forces two passes over the input (HBM-bound: 2 + 2 + 1
// bytes per element). Several tensors of one size go through one launch (a pointer
// table, blockIdx.y = tensor). A tensor's 32-bit word holds the float bits of its amax
// while the quantise pass runs (integer atomic max over non-negative float bits keeps
// the order of the values) and is turned into the scale afterwards.
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kTab = 64;  // tensors per launch

struct Fp8Tab {
  const uint4* in[kTab];   // bf16, 8 values per uint4
  uint2* out[kTab];        // E4M3 codes, 8 per uint2
};

__global__ __launch_bounds__(256) void fp8t_zero_kernel(uint32_t* words, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) words[i] = 0u;
}

// max |x| over each tensor: integer max of the bf16 magnitude bits, one atomic per block
__global__ __launch_bounds__(256) void fp8t_amax_kernel(const Fp8Tab tab, int64_t n8, uint32_t* words) {
  const uint4* in = tab.in[blockIdx.y];
  uint32_t m = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    const uint4 v = in[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m = max(m, w[j] & 0x7FFFu);
      m = max(m, (w[j] >> 16) & 0x7FFFu);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  __shared__ uint32_t red[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    if (m) atomicMax(words + blockIdx.y, m << 16);   // float bits of the bf16 magnitude
  }
}

__device__ __forceinline__ float scale_of_amax(uint32_t bits) {
  const float amax = __uint_as_float(bits);
  return amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
}

// The quotient x / s rounded to nearest, with r = 1/s rounded to nearest computed once:
// q1 = x r is within one ulp of x / s, the residual x - q1 s is exact as an fma, and
// q1 + residual * r (one fma) is the correctly rounded quotient (Markstein's theorem;
// it needs s and r in the normal range, checked per tensor). Quotients below the
// float32 normal range, where the theorem does not hold, are far below E4M3's smallest
// step and get code 0 either way.
template <bool kRecip>
__device__ __forceinline__ float quotient(float x, float s, float r) {
  if constexpr (!kRecip) return __fdiv_rn(x, s);
  const float q1 = x * r;
  const float e = __builtin_fmaf(-q1, s, x);
  return __builtin_fmaf(e, r, q1);
}

template <bool kRecip>
__device__ __forceinline__ void quantize_range(const uint4* in, uint2* out, int64_t n8, float s, float r) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    const uint4 v = in[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t c[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[2 * j] = e4m3_encode(quotient<kRecip>(bf16_to_f32(w[j] & 0xFFFFu), s, r));
      c[2 * j + 1] = e4m3_encode(quotient<kRecip>(bf16_to_f32(w[j] >> 16), s, r));
    }
    out[i] = make_uint2(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                        c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24));
  }
}

__global__ __launch_bounds__(256) void fp8t_quantize_kernel(const Fp8Tab tab, int64_t n8, const uint32_t* words) {
  const float s = scale_of_amax(words[blockIdx.y]);
  const float r = __fdiv_rn(1.f, s);
  const float kMinNormal = 1.17549435e-38f, kMaxNormal = 3.40282347e+38f;
  if (s >= kMinNormal && r >= kMinNormal && r <= kMaxNormal)
    quantize_range<true>(tab.in[blockIdx.y], tab.out[blockIdx.y], n8, s, r);
  else
    quantize_range<false>(tab.in[blockIdx.y], tab.out[blockIdx.y], n8, s, r);
}

__global__ __launch_bounds__(256) void fp8t_finalize_kernel(uint32_t* words, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) words[i] = __float_as_uint(scale_of_amax(words[i]));
}

unsigned grid_x(int64_t n8, int ntensors) {
  int64_t want = (n8 + 255) / 256;
  int64_t cap = (int64_t)num_cus() * 8 / ntensors;
  if (cap < 4) cap = 4;
  if (want > cap) want = cap;
  return (unsigned)(want < 1 ? 1 : want);
}

}  // namespace

moe_status fp8t_zero(float* words, int n, hipStream_t s) {
  if (n <= 0) return MOE_OK;
  hipLaunchKernelGGL(fp8t_zero_kernel, dim3((n + 255) / 256), dim3(256), 0, s, (uint32_t*)words, n);
  return check_launch("per-tensor FP8: clear amax");
}

moe_status fp8t_finalize(float* words, int n, hipStream_t s) {
  if (n <= 0) return MOE_OK;
  hipLaunchKernelGGL(fp8t_finalize_kernel, dim3((n + 255) / 256), dim3(256), 0, s, (uint32_t*)words, n);
  return check_launch("per-tensor FP8: scales");
}

moe_status fp8t_amax(const void* const* in, int ntensors, int64_t n, float* words, hipStream_t s) {
  const int64_t n8 = n / 8;
  if (n8 == 0 || ntensors == 0) return MOE_OK;
  for (int t0 = 0; t0 < ntensors; t0 += kTab) {
    const int cnt = ntensors - t0 < kTab ? ntensors - t0 : kTab;
    Fp8Tab tab = {};
    for (int t = 0; t < cnt; ++t) tab.in[t] = (const uint4*)in[t0 + t];
    hipLaunchKernelGGL(fp8t_amax_kernel, dim3(grid_x(n8, cnt), cnt), dim3(256), 0, s, tab, n8,
                       (uint32_t*)words + t0);
    moe_status st = check_launch("per-tensor FP8: amax");
    if (st != MOE_OK) return st;
  }
  return MOE_OK;
}

moe_status fp8t_quantize(const void* const* in, uint8_t* const* out, int ntensors, int64_t n, const float* words,
                         hipStream_t s) {
  const int64_t n8 = n / 8;
  if (n8 == 0 || ntensors == 0) return MOE_OK;
  for (int t0 = 0; t0 < ntensors; t0 += kTab) {
    const int cnt = ntensors - t0 < kTab ? ntensors - t0 : kTab;
    Fp8Tab tab = {};
    for (int t = 0; t < cnt; ++t) {
      tab.in[t] = (const uint4*)in[t0 + t];
      tab.out[t] = (uint2*)out[t0 + t];
    }
    hipLaunchKernelGGL(fp8t_quantize_kernel, dim3(grid_x(n8, cnt), cnt), dim3(256), 0, s, tab, n8,
                       (const uint32_t*)words + t0);
    moe_status st = check_launch("per-tensor FP8: quantise");
    if (st != MOE_OK) return st;
  }
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" moe_status fp8_tensor_quantize(const void* in_bf16, int64_t n, uint8_t* e4m3, float* scale,
                                          void* stream) {
  if (n < 0) return fail(MOE_ERR_INVALID_ARG, "fp8_tensor_quantize: negative size");
  if (n % 8 != 0) return fail(MOE_ERR_INVALID_ARG, "fp8_tensor_quantize: n % 8 != 0");
  if (!scale) return fail(MOE_ERR_INVALID_ARG, "fp8_tensor_quantize: NULL scale");
  if (!aligned(scale, 4)) return fail(MOE_ERR_INVALID_ARG, "fp8_tensor_quantize: scale not 4-byte aligned");
  if (n > 0 && (!in_bf16 || !e4m3)) return fail(MOE_ERR_INVALID_ARG, "fp8_tensor_quantize: NULL pointer");
  if (n > 0 && (!aligned(in_bf16, 16) || !aligned(e4m3, 8)))
    return fail(MOE_ERR_INVALID_ARG, "fp8_tensor_quantize: input must be 16-byte and codes 8-byte aligned");
  const hipStream_t s = as_stream(stream);
  moe_status st;
  if ((st = fp8t_zero(scale, 1, s)) != MOE_OK) return st;
  const void* in_tab[1] = {in_bf16};
  uint8_t* out_tab[1] = {e4m3};
  if ((st = fp8t_amax(in_tab, 1, n, scale, s)) != MOE_OK) return st;
  if ((st = fp8t_quantize(in_tab, out_tab, 1, n, scale, s)) != MOE_OK) return st;
  return fp8t_finalize(scale, 1, s);
}
