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
// step and get code 0 either way. The residual step alone would turn x = -0 into +0
// (q1 = -0, residual +0, and +0 + -0 rounds to +0); the quotient has x's sign (s > 0),
// so x's sign is put back, which keeps the sign of zero as the division does.
template <bool kRecip>
__device__ __forceinline__ float quotient(float x, float s, float r) {
  if constexpr (!kRecip) return __fdiv_rn(x, s);
  const float q1 = x * r;
  const float e = __builtin_fmaf(-q1, s, x);
  return __builtin_copysignf(__builtin_fmaf(e, r, q1), x);
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

// Transposed codes of x [R, C] (bf16, rows grouped by expert): out [C, kcap], expert
// e's rows at columns [kofs[e], kofs[e] + m_e) of every output row, zero-padded to a
// multiple of pad (the weight-gradient GEMMs' token-axis operand). One factor per
// tensor means the codes are those of the row-major quantiser, only transposed. A
// workgroup takes 128 rows x 64 columns of one expert's padded range through LDS
// (16-byte loads, rows past the expert read as zeros; the next item's rows are loaded
// while the current one is encoded); lane (q, c) encodes rows 32q .. 32q + 31 of column
// c and stores them as two 16-byte stores. The codes come from gfx950's E4M3 conversion
// (round to nearest even) of the correctly rounded quotient, as in the row-major
// quantiser's software encoder for every quotient below 464: the largest is
// amax / s = 448 (1 + at most a few ulps). Tensor blockIdx.y of the table; words: the
// tensors' amax bits (before fp8t_finalize).
struct Fp8TTab {
  const uint16_t* in[kTab];
  uint8_t* out[kTab];
  uint8_t* rows[kTab];  // NULL, or the row-major codes [R, C] of the same tensor, written too
};

template <bool kRecip>
__device__ __forceinline__ uint32_t encode4(const float* t, float s, float r) {
  return e4m3_pack4(quotient<kRecip>(t[0], s, r), quotient<kRecip>(t[65], s, r), quotient<kRecip>(t[130], s, r),
                    quotient<kRecip>(t[195], s, r));
}

__global__ __launch_bounds__(256) void fp8t_transpose_kernel(const Fp8TTab tab, int64_t R, int C, int E,
                                                             const int32_t* __restrict__ offsets, int pad,
                                                             int64_t kcap, const uint32_t* __restrict__ words,
                                                             int32_t* __restrict__ kofs_out) {
  __shared__ int32_t s_off[MOE_MAX_EXPERTS + 1];
  __shared__ int32_t s_kofs[MOE_MAX_EXPERTS + 1];
  __shared__ int32_t s_item[MOE_MAX_EXPERTS + 1];
  __shared__ float tile[128][65];
  const int tid = threadIdx.x;
  const int ncb = C / 64;
  const uint16_t* __restrict__ x = tab.in[blockIdx.y];
  uint8_t* __restrict__ codes = tab.out[blockIdx.y];
  uint8_t* __restrict__ row_codes = tab.rows[blockIdx.y];
  const float s = scale_of_amax(words[blockIdx.y]);
  const float rcp = __fdiv_rn(1.f, s);
  const bool fast = s >= 1.17549435e-38f && rcp >= 1.17549435e-38f && rcp <= 3.40282347e+38f;
  if (tid == 0) {  // offsets made nondecreasing inside [0, R] (none: one expert of R rows); padded offsets
    int prev = 0, kacc = 0, iacc = 0;
    for (int e = 0; e <= E; ++e) {
      int v = e == 0 ? 0 : (offsets ? offsets[e] : (int)R);
      v = v < prev ? prev : v;
      v = v > (int)R ? (int)R : v;
      if (e > 0) {
        const int m = v - prev;
        const int kp = (m + pad - 1) / pad * pad;
        s_kofs[e - 1] = kacc;
        s_item[e - 1] = iacc;
        kacc += kp;
        iacc += ((kp / 32 + 3) / 4) * ncb;
      }
      s_off[e] = v;
      prev = v;
    }
    s_kofs[E] = kacc;
    s_item[E] = iacc;
  }
  __syncthreads();
  if (blockIdx.x == 0 && blockIdx.y == 0 && kofs_out)
    for (int e = tid; e <= E; e += 256) kofs_out[e] = s_kofs[e];
  const int total = s_item[E];
  const int r = tid >> 3, c8 = (tid & 7) * 8;  // load: rows r + 32i, columns c8 .. c8 + 7
  const int cc = tid & 63, q = tid >> 6;        // encode: rows 32q .. 32q + 31 of column cc
  // item -> expert, 128-row group j, 64-column block cb
  auto locate = [&](int item, int& e, int& j, int& cb) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_item[mid] <= item) lo = mid; else hi = mid - 1;
    }
    e = lo;
    const int local = item - s_item[e];
    j = local / ncb;
    cb = local - j * ncb;
  };
  uint4 v[4];  // an item's rows (rows past the expert as zeros)
  auto fetch = [&](int item) {
    int e, j, cb;
    locate(item, e, j, cb);
    const int64_t row0 = (int64_t)s_off[e] + 128 * j;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = row0 + r + 32 * i;
      v[i] = make_uint4(0, 0, 0, 0);
      if (row < s_off[e + 1]) v[i] = *reinterpret_cast<const uint4*>(x + row * C + cb * 64 + c8);
    }
  };
  if ((int)blockIdx.x < total) fetch(blockIdx.x);
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    int e, j, cb;
    locate(item, e, j, cb);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
      float f[8];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        f[2 * h] = bf16_to_f32(w[h] & 0xFFFFu);
        f[2 * h + 1] = bf16_to_f32(w[h] >> 16);
        tile[r + 32 * i][c8 + 2 * h] = f[2 * h];
        tile[r + 32 * i][c8 + 2 * h + 1] = f[2 * h + 1];
      }
      const int64_t row = (int64_t)s_off[e] + 128 * j + r + 32 * i;
      if (row_codes && row < s_off[e + 1]) {  // the same codes, row-major: 8 bytes of the row
        uint32_t c0, c1;
        if (fast) {
          c0 = e4m3_pack4(quotient<true>(f[0], s, rcp), quotient<true>(f[1], s, rcp), quotient<true>(f[2], s, rcp),
                          quotient<true>(f[3], s, rcp));
          c1 = e4m3_pack4(quotient<true>(f[4], s, rcp), quotient<true>(f[5], s, rcp), quotient<true>(f[6], s, rcp),
                          quotient<true>(f[7], s, rcp));
        } else {
          c0 = e4m3_pack4(quotient<false>(f[0], s, rcp), quotient<false>(f[1], s, rcp),
                          quotient<false>(f[2], s, rcp), quotient<false>(f[3], s, rcp));
          c1 = e4m3_pack4(quotient<false>(f[4], s, rcp), quotient<false>(f[5], s, rcp),
                          quotient<false>(f[6], s, rcp), quotient<false>(f[7], s, rcp));
        }
        *reinterpret_cast<uint2*>(row_codes + row * C + cb * 64 + c8) = make_uint2(c0, c1);
      }
    }
    __syncthreads();
    if (item + (int)gridDim.x < total) fetch(item + gridDim.x);
    const int nblk = (s_kofs[e + 1] - s_kofs[e]) / 32;        // 32-row groups in the expert's padded range
    if (q < nblk - 4 * j) {
      uint32_t wd[8];
#pragma unroll
      for (int g = 0; g < 8; ++g)
        wd[g] = fast ? encode4<true>(&tile[32 * q + 4 * g][cc], s, rcp) : encode4<false>(&tile[32 * q + 4 * g][cc], s, rcp);
      const int64_t col = (int64_t)cb * 64 + cc;
      const int64_t k = (int64_t)s_kofs[e] + 128 * j + 32 * q;
      uint4* dst = reinterpret_cast<uint4*>(codes + col * kcap + k);
      dst[0] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
      dst[1] = make_uint4(wd[4], wd[5], wd[6], wd[7]);
    }
    __syncthreads();  // the tile is reused by the next item
  }
}

// copies of the finished scales into per-tensor destinations (the weight packs' factors)
struct Fp8Dst {
  float* p[kTab];
};
__global__ __launch_bounds__(64) void fp8t_scatter_kernel(const float* __restrict__ words, const Fp8Dst dst, int n) {
  const int i = threadIdx.x;
  if (i < n) *dst.p[i] = words[i];
}

unsigned grid_x(int64_t n8, int ntensors) {
  int64_t want = (n8 + 255) / 256;
  int64_t cap = (int64_t)num_cus() * 8 / ntensors;
  if (cap < 4) cap = 4;
  if (want > cap) want = cap;
  return (unsigned)(want < 1 ? 1 : want);
}

}  // namespace

moe_status fp8t_transpose(const void* const* in, uint8_t* const* out, int ntensors, int64_t R, int C, int E,
                          const int32_t* offsets, int pad, int64_t kcap, const float* words, int32_t* kofs,
                          hipStream_t s, uint8_t* const* rows_out) {
  if (ntensors <= 0 || C == 0) return MOE_OK;
  // room for every expert's rows padded to a multiple of pad (one expert: R rounded up)
  const int64_t room = offsets ? R + (int64_t)E * (pad - 1) : (R + pad - 1) / pad * pad;
  if (C % 64 != 0 || pad <= 0 || pad % 32 != 0 || kcap % 32 != 0 || kcap < room || E < 1 || E > MOE_MAX_EXPERTS ||
      (!offsets && E != 1) || ntensors > kTab || R > 0x7FFFFFFF)
    return fail(MOE_ERR_UNSUPPORTED, "per-tensor FP8 transpose: unsupported shape");
  Fp8TTab tab = {};
  for (int t = 0; t < ntensors; ++t) {
    tab.in[t] = (const uint16_t*)in[t];
    tab.out[t] = out[t];
    tab.rows[t] = rows_out ? rows_out[t] : nullptr;
  }
  const int64_t items = (kcap / 32 + 3 * E) / 4 * (C / 64) + E * (C / 64);
  int64_t grid = (int64_t)num_cus() * 16 / ntensors;
  if (grid < 4) grid = 4;
  if (items < grid) grid = items;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(fp8t_transpose_kernel, dim3((unsigned)grid, ntensors), dim3(256), 0, s, tab, R, C, E, offsets,
                     pad, kcap, (const uint32_t*)words, kofs);
  return check_launch("per-tensor FP8: transposed codes");
}

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

extern "C" moe_status fp8_tensor_quantize_colwise(const void* x_bf16, int64_t R, int64_t C, int E,
                                                  const int32_t* offsets, int pad, int64_t kcap, uint8_t* e4m3_t,
                                                  float* scale, int32_t* kofs, void* stream) {
  if (R < 0 || C < 0) return fail(MOE_ERR_INVALID_ARG, "fp8_tensor_quantize_colwise: negative size");
  if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_ERR_INVALID_ARG, "fp8_tensor_quantize_colwise: E out of [1, 256]");
  if (pad <= 0 || pad % 32 != 0)
    return fail(MOE_ERR_INVALID_ARG, "fp8_tensor_quantize_colwise: pad must be a positive multiple of 32");
  if (C % 64 != 0) return fail(MOE_ERR_UNSUPPORTED, "fp8_tensor_quantize_colwise: C % 64 != 0");
  if (kcap % 32 != 0 || kcap < R + (int64_t)E * (pad - 1))
    return fail(MOE_ERR_INVALID_ARG,
                "fp8_tensor_quantize_colwise: kcap must be a multiple of 32 and >= R + E * (pad - 1)");
  if (R > 0x7FFFFFFF || kcap > 0x7FFFFFFF) return fail(MOE_ERR_UNSUPPORTED, "fp8_tensor_quantize_colwise: R or kcap >= 2^31");
  if (!offsets || !kofs || !scale || (C > 0 && !e4m3_t) || (R > 0 && C > 0 && !x_bf16))
    return fail(MOE_ERR_INVALID_ARG, "fp8_tensor_quantize_colwise: NULL pointer");
  if (!aligned(offsets, 4) || !aligned(kofs, 4) || !aligned(scale, 4) || (x_bf16 && !aligned(x_bf16, 16)) ||
      (e4m3_t && !aligned(e4m3_t, 16)))
    return fail(MOE_ERR_INVALID_ARG,
                "fp8_tensor_quantize_colwise: x and codes must be 16-byte, offsets, kofs and scale 4-byte aligned");
  const hipStream_t s = as_stream(stream);
  moe_status st;
  if ((st = fp8t_zero(scale, 1, s)) != MOE_OK) return st;
  const void* in[1] = {x_bf16};
  uint8_t* out[1] = {e4m3_t};
  if ((st = fp8t_amax(in, 1, R * C, scale, s)) != MOE_OK) return st;
  if (C > 0 && (st = fp8t_transpose(in, out, 1, R, (int)C, E, offsets, pad, kcap, scale, kofs, s)) != MOE_OK)
    return st;
  return fp8t_finalize(scale, 1, s);
}

extern "C" moe_status fp8_tensor_pack_weight_bwd(const void* w_bf16, int64_t rows, int64_t cols, void* packed,
                                                 void* stream) {
  if (rows < 0 || cols < 0) return fail(MOE_ERR_INVALID_ARG, "fp8_tensor_pack_weight_bwd: negative size");
  if (rows % 32 != 0 || cols % 64 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "fp8_tensor_pack_weight_bwd: needs rows % 32 == 0 and cols % 64 == 0");
  if (rows > 0x7FFFFFFF || rows * cols > 0x7FFFFFFFLL)
    return fail(MOE_ERR_UNSUPPORTED, "fp8_tensor_pack_weight_bwd: weight exceeds 2^31 elements");
  if (rows == 0 || cols == 0) return MOE_OK;
  if (!w_bf16 || !packed) return fail(MOE_ERR_INVALID_ARG, "fp8_tensor_pack_weight_bwd: NULL pointer");
  if (!aligned(w_bf16, 16) || !aligned(packed, 16))
    return fail(MOE_ERR_INVALID_ARG, "fp8_tensor_pack_weight_bwd: w and packed must be 16-byte aligned");
  const hipStream_t s = as_stream(stream);
  uint8_t* codes = reinterpret_cast<uint8_t*>(packed);
  float* factor = reinterpret_cast<float*>(codes + rows * cols);  // rows * cols is a multiple of 4
  moe_status st;
  if ((st = fp8t_zero(factor, 1, s)) != MOE_OK) return st;
  const void* in[1] = {w_bf16};
  uint8_t* out[1] = {codes};
  if ((st = fp8t_amax(in, 1, rows * cols, factor, s)) != MOE_OK) return st;
  if ((st = fp8t_transpose(in, out, 1, rows, (int)cols, 1, nullptr, 32, rows, factor, nullptr, s)) != MOE_OK)
    return st;
  return fp8t_finalize(factor, 1, s);
}

extern "C" moe_status fp8_tensor_quantize_weights(int n, const void* const* w_bf16, int64_t rows, int64_t cols,
                                                  uint8_t* const* e4m3, float* scale, void* const* packed,
                                                  void* stream) {
  if (n < 1 || n > MOE_MAX_EXPERTS) return fail(MOE_ERR_INVALID_ARG, "fp8_tensor_quantize_weights: n out of [1, 256]");
  if (rows < 0 || cols < 0) return fail(MOE_ERR_INVALID_ARG, "fp8_tensor_quantize_weights: negative size");
  if (rows % 32 != 0 || cols % 64 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "fp8_tensor_quantize_weights: needs rows % 32 == 0 and cols % 64 == 0");
  if (rows > 0x7FFFFFFF || rows * cols > 0x7FFFFFFFLL)
    return fail(MOE_ERR_UNSUPPORTED, "fp8_tensor_quantize_weights: weight exceeds 2^31 elements");
  if (!scale) return fail(MOE_ERR_INVALID_ARG, "fp8_tensor_quantize_weights: NULL scale");
  if (!aligned(scale, 4)) return fail(MOE_ERR_INVALID_ARG, "fp8_tensor_quantize_weights: scale not 4-byte aligned");
  if (!w_bf16 || !e4m3 || !packed) return fail(MOE_ERR_INVALID_ARG, "fp8_tensor_quantize_weights: NULL table");
  const bool empty = rows == 0 || cols == 0;
  for (int i = 0; i < n; ++i) {
    if (!packed[i] || (!empty && (!w_bf16[i] || !e4m3[i])))
      return fail(MOE_ERR_INVALID_ARG, "fp8_tensor_quantize_weights: NULL pointer");
    if (!aligned(packed[i], 16) || (!empty && (!aligned(w_bf16[i], 16) || !aligned(e4m3[i], 8))))
      return fail(MOE_ERR_INVALID_ARG, "fp8_tensor_quantize_weights: w and packed must be 16-byte, e4m3 8-byte aligned");
  }
  const hipStream_t s = as_stream(stream);
  moe_status st;
  if ((st = fp8t_zero(scale, n, s)) != MOE_OK) return st;
  if ((st = fp8t_amax(w_bf16, n, rows * cols, scale, s)) != MOE_OK) return st;
  for (int t0 = 0; !empty && t0 < n; t0 += kTab) {
    const int cnt = n - t0 < kTab ? n - t0 : kTab;
    uint8_t* codes[kTab];
    for (int t = 0; t < cnt; ++t) codes[t] = reinterpret_cast<uint8_t*>(packed[t0 + t]);
    if ((st = fp8t_transpose(w_bf16 + t0, codes, cnt, rows, (int)cols, 1, nullptr, 32, rows, scale + t0, nullptr, s,
                             e4m3 + t0)) != MOE_OK)
      return st;
  }
  if ((st = fp8t_finalize(scale, n, s)) != MOE_OK) return st;
  for (int t0 = 0; t0 < n; t0 += kTab) {  // each pack carries its factor after the codes
    const int cnt = n - t0 < kTab ? n - t0 : kTab;
    Fp8Dst dst = {};
    for (int t = 0; t < cnt; ++t) dst.p[t] = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(packed[t0 + t]) + rows * cols);
    hipLaunchKernelGGL(fp8t_scatter_kernel, dim3(1), dim3(64), 0, s, scale + t0, dst, cnt);
    if ((st = check_launch("fp8_tensor_quantize_weights: factors")) != MOE_OK) return st;
  }
  return MOE_OK;
}
