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

// step_rows == 0: scale byte of block b of row r at r * cols32 + b (the public layout);
// step_rows == rows: "step-major", the 4 blocks of 128 values of row r form one 32-bit
// word, words of K step k (all rows) contiguous: byte ((b / 4) * rows + r) * 4 + b % 4
// (the layout the wide-step MXFP8 GEMM reads, 32 rows of a sub-tile in one 128-byte run)
__global__ __launch_bounds__(256) void mxfp8_quantize_kernel(const uint4* __restrict__ in, int64_t nblocks,
                                                             uint2* __restrict__ codes,
                                                             uint8_t* __restrict__ scales, int64_t cols32,
                                                             int64_t step_rows) {
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
    if (live) {
      codes[q] = make_uint2(e4m3_pack4(ldexpf(f[0], -s), ldexpf(f[1], -s), ldexpf(f[2], -s), ldexpf(f[3], -s)),
                            e4m3_pack4(ldexpf(f[4], -s), ldexpf(f[5], -s), ldexpf(f[6], -s), ldexpf(f[7], -s)));
      if ((q & 3) == 0) {
        const int64_t b = q >> 2;
        int64_t at = b;
        if (step_rows) {
          const int64_t r = b / cols32, c = b - r * cols32;
          at = ((c >> 2) * step_rows + r) * 4 + (c & 3);
        }
        scales[at] = (uint8_t)(s + 127);
      }
    }
  }
}

static moe_status quantize_rows(const void* in_bf16, int64_t rows, int64_t cols, uint8_t* e4m3, uint8_t* e8m0,
                                void* stream, bool step_major) {
  const int64_t nblocks = rows * (cols / 32);
  if (nblocks == 0) return MOE_OK;
  const int threads = 256;
  int64_t want = (nblocks * 4 + threads - 1) / threads;
  const int64_t cap = (int64_t)num_cus() * 16;
  const unsigned grid = (unsigned)(want < cap ? want : cap);
  hipLaunchKernelGGL(mxfp8_quantize_kernel, dim3(grid), dim3(threads), 0, as_stream(stream),
                     (const uint4*)in_bf16, nblocks, (uint2*)e4m3, e8m0, cols / 32, step_major ? rows : 0);
  return check_launch("mxfp8_quantize");
}

moe_status launch_mxfp8_quantize(const void* in_bf16, int64_t rows, int64_t cols, uint8_t* e4m3,
                                 uint8_t* e8m0, void* stream) {
  return quantize_rows(in_bf16, rows, cols, e4m3, e8m0, stream, false);
}

moe_status launch_mxfp8_quantize_step_major(const void* in_bf16, int64_t rows, int64_t cols, uint8_t* e4m3,
                                            uint8_t* e8m0, void* stream) {
  if (cols % 128 != 0) return fail(MOE_ERR_UNSUPPORTED, "mxfp8 step-major scales need cols % 128 == 0");
  return quantize_rows(in_bf16, rows, cols, e4m3, e8m0, stream, true);
}

// Public-layout scales [rows][cols / 32] -> step-major ([cols / 128][rows] 32-bit words),
// for up to MOE_MAX_EXPERTS tensors of one shape (blockIdx.z): a transpose of a
// [rows][steps] word matrix through a 64-row x 16-step LDS tile, read 64 bytes of a row
// at a time and written 256 bytes of a step at a time.
struct ScaleTables {
  const uint32_t* src[MOE_MAX_EXPERTS];
  uint32_t* dst[MOE_MAX_EXPERTS];
};

__global__ __launch_bounds__(256) void mx_scales_step_major_kernel(const ScaleTables tabs, int64_t rows,
                                                                   int steps) {
  __shared__ uint32_t tile[16][65];
  const uint32_t* src = tabs.src[blockIdx.z];
  uint32_t* dst = tabs.dst[blockIdx.z];
  const int64_t r0 = (int64_t)blockIdx.x * 64;
  const int s0 = blockIdx.y * 16;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = i * 256 + tid;
    const int r = idx >> 4, st = idx & 15;
    if (r0 + r < rows && s0 + st < steps) tile[st][r] = src[(r0 + r) * steps + s0 + st];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = i * 256 + tid;
    const int st = idx >> 6, r = idx & 63;
    if (r0 + r < rows && s0 + st < steps) dst[(int64_t)(s0 + st) * rows + r0 + r] = tile[st][r];
  }
}

moe_status launch_mx_scales_step_major(const uint8_t* const* src, uint8_t* const* dst, int n, int64_t rows,
                                       int64_t cols, void* stream) {
  if (cols % 128 != 0) return fail(MOE_ERR_UNSUPPORTED, "mxfp8 step-major scales need cols % 128 == 0");
  if (n < 1 || n > MOE_MAX_EXPERTS) return fail(MOE_ERR_INVALID_ARG, "mxfp8 scale conversion: bad tensor count");
  if (rows == 0) return MOE_OK;
  ScaleTables t;
  for (int i = 0; i < n; ++i) {
    if (!aligned(src[i], 4) || !aligned(dst[i], 4))
      return fail(MOE_ERR_INVALID_ARG, "mxfp8 scale conversion: scales must be 4-byte aligned");
    t.src[i] = reinterpret_cast<const uint32_t*>(src[i]);
    t.dst[i] = reinterpret_cast<uint32_t*>(dst[i]);
  }
  const int steps = (int)(cols / 128);
  const dim3 grid((unsigned)((rows + 63) / 64), (unsigned)((steps + 15) / 16), (unsigned)n);
  hipLaunchKernelGGL(mx_scales_step_major_kernel, grid, dim3(256), 0, as_stream(stream), t, rows, steps);
  return check_launch("mxfp8 scale conversion");
}

// Column-wise (per expert, along the token axis) MXFP8: a workgroup takes up to four
// 32-row blocks (128 rows) x 64 columns of one expert's zero-padded row range. The rows
// come in with coalesced 16-byte loads (8 lanes per 128-byte row segment; rows past the
// expert read as zeros) into an LDS tile; lane (q, c) then owns block q of column c:
// its maximum, scale byte and 32 codes, stored as two 16-byte stores, so the four
// blocks of a column leave as one whole 128-byte line of the output row.
// Several tensors of one shape go through one launch (blockIdx.y indexes the table).
// A tensor with row-wise outputs also gets the quantisation along its rows from the
// same loads: the 8 values a lane holds are a quarter of a 32-value row block, so four
// lanes reduce the block maximum with two xor-shuffles, as the row-wise quantiser does.
constexpr int kColTab = 16;  // tensors per launch
struct MxColTab {
  const uint16_t* x[kColTab];
  uint8_t* codes[kColTab];
  uint8_t* scales[kColTab];
  uint2* rcodes[kColTab];     // NULL, or the row-wise codes [R, C] of the same tensor
  uint8_t* rscales[kColTab];  // its row-wise scales (layout chosen by rstep)
};

__global__ __launch_bounds__(256) void mxfp8_quantize_colwise_kernel(const MxColTab tab, int64_t R, int C, int E,
                                                                     const int32_t* __restrict__ offsets, int pad,
                                                                     int64_t kcap, int32_t* __restrict__ kofs_out,
                                                                     int step_major, int64_t rstep) {
  __shared__ int32_t s_off[MOE_MAX_EXPERTS + 1];
  __shared__ int32_t s_kofs[MOE_MAX_EXPERTS + 1];
  __shared__ int32_t s_item[MOE_MAX_EXPERTS + 1];
  __shared__ float tile[128][65];
  const uint16_t* __restrict__ x = tab.x[blockIdx.y];
  uint8_t* __restrict__ codes = tab.codes[blockIdx.y];
  uint8_t* __restrict__ scales = tab.scales[blockIdx.y];
  uint2* __restrict__ rcodes = tab.rcodes[blockIdx.y];
  uint8_t* __restrict__ rscales = tab.rscales[blockIdx.y];
  const int tid = threadIdx.x;
  const int ncb = C / 64;
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
  const int cc = tid & 63, q = tid >> 6;        // encode: block q of column cc
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
  // an item's rows in registers (rows past the expert as zeros). Two register sets: the
  // loads of the next two items are in flight while the current one is encoded
  auto fetch = [&](uint4 (&v)[4], int item) {
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
  // encode item from v, then refill v with item `next` (if any)
  auto encode = [&](uint4 (&v)[4], int item, int next) {
    int e, j, cb;
    locate(item, e, j, cb);
    const int nblk = (s_kofs[e + 1] - s_kofs[e]) / 32;        // blocks in the expert's padded range
    const int blocks = nblk - 4 * j < 4 ? nblk - 4 * j : 4;   // blocks of this item
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
      if (rcodes) {  // uniform over the launch's tensor: every lane reaches the shuffles
        float amax = 0.f;
#pragma unroll
        for (int h = 0; h < 8; ++h) amax = fmaxf(amax, fabsf(f[h]));
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        amax = fmaxf(amax, __shfl_xor(amax, 2));
        const int sr = mx_scale_exponent(amax);
        const int64_t row = (int64_t)s_off[e] + 128 * j + r + 32 * i;
        if (row < s_off[e + 1]) {
          const int64_t col = (int64_t)cb * 64 + c8;
          rcodes[(row * C + col) >> 3] =
              make_uint2(e4m3_pack4(ldexpf(f[0], -sr), ldexpf(f[1], -sr), ldexpf(f[2], -sr), ldexpf(f[3], -sr)),
                         e4m3_pack4(ldexpf(f[4], -sr), ldexpf(f[5], -sr), ldexpf(f[6], -sr), ldexpf(f[7], -sr)));
          if ((tid & 3) == 0) {
            const int64_t b = col >> 5;  // block of the row
            const int64_t at = rstep ? ((b >> 2) * rstep + row) * 4 + (b & 3) : row * (C / 32) + b;
            rscales[at] = (uint8_t)(sr + 127);
          }
        }
      }
    }
    __syncthreads();
    if (next < total) fetch(v, next);
    if (q < blocks) {
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(tile[32 * q + i][cc]));
      const int sx = mx_scale_exponent(amax);
      uint32_t wd[8];
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const float* t = &tile[32 * q + 4 * g][cc];
        wd[g] = e4m3_pack4(ldexpf(t[0], -sx), ldexpf(t[65], -sx), ldexpf(t[130], -sx), ldexpf(t[195], -sx));
      }
      const int64_t col = (int64_t)cb * 64 + cc;
      const int64_t k = (int64_t)s_kofs[e] + 128 * j + 32 * q;
      uint4* dst = reinterpret_cast<uint4*>(codes + col * kcap + k);
      dst[0] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
      dst[1] = make_uint4(wd[4], wd[5], wd[6], wd[7]);
      // step-major (the wide-step GEMM's operand layout): word (k / 128) * C + col
      const int64_t at = step_major ? ((k >> 7) * C + col) * 4 + ((k >> 5) & 3) : col * (kcap / 32) + k / 32;
      scales[at] = (uint8_t)(sx + 127);
    }
    __syncthreads();  // the tile is reused by the next item
  };
  // a workgroup takes items in pairs (2p, 2p + 1): neighbouring 64-column blocks, whose
  // row-wise codes are the two halves of the same 128-byte lines, leave through one L2
  const int G = gridDim.x;
  const int npairs = (total + 1) / 2;
  uint4 va[4], vb[4];
  int p = blockIdx.x;
  if (2 * p < total) fetch(va, 2 * p);
  if (2 * p + 1 < total) fetch(vb, 2 * p + 1);
  for (; p < npairs; p += G) {  // block-uniform trip count and branches
    encode(va, 2 * p, 2 * (p + G));
    if (2 * p + 1 < total) encode(vb, 2 * p + 1, 2 * (p + G) + 1);
  }
}

}  // namespace moe

using namespace moe;

moe_status moe::launch_mxfp8_colwise_multi(int n, const void* const* x_bf16, int64_t R, int C, int E,
                                           const int32_t* offsets, int pad, int64_t kcap, uint8_t* const* codes,
                                           uint8_t* const* scales, int32_t* kofs, hipStream_t s, bool step_major,
                                           uint8_t* const* rcodes, uint8_t* const* rscales, int64_t rstep) {
  if (step_major && kcap % 128 != 0) return fail(MOE_ERR_UNSUPPORTED, "mxfp8 step-major scales need kcap % 128 == 0");
  if (rcodes && rstep && C % 128 != 0) return fail(MOE_ERR_UNSUPPORTED, "mxfp8 step-major scales need cols % 128 == 0");
  if (n < 1) return MOE_OK;
  const int64_t items = (kcap / 32 + 3 * E) / 4 * (C / 64) + E * (C / 64);
  const int64_t pairs = (items + 1) / 2;
  for (int t0 = 0; t0 < n; t0 += kColTab) {
    const int cnt = n - t0 < kColTab ? n - t0 : kColTab;
    MxColTab tab = {};
    for (int t = 0; t < cnt; ++t) {
      tab.x[t] = (const uint16_t*)x_bf16[t0 + t];
      tab.codes[t] = codes[t0 + t];
      tab.scales[t] = scales[t0 + t];
      tab.rcodes[t] = rcodes ? (uint2*)rcodes[t0 + t] : nullptr;
      tab.rscales[t] = rcodes ? rscales[t0 + t] : nullptr;
    }
    // ~4 resident per CU (33 KB of LDS each), the rest balance the tail
    int64_t grid = (int64_t)num_cus() * 32 / cnt;
    if (grid < 4) grid = 4;
    if (pairs < grid) grid = pairs;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(mxfp8_quantize_colwise_kernel, dim3((unsigned)grid, (unsigned)cnt), dim3(256), 0, s, tab, R,
                       C, E, offsets, pad, kcap, t0 == 0 ? kofs : nullptr, (int)step_major, rstep);
    moe_status st = check_launch("mxfp8_quantize_colwise");
    if (st != MOE_OK) return st;
  }
  return MOE_OK;
}

moe_status moe::launch_mxfp8_colwise(const void* x_bf16, int64_t R, int C, int E, const int32_t* offsets, int pad,
                                     int64_t kcap, uint8_t* codes, uint8_t* scales, int32_t* kofs, hipStream_t s,
                                     bool step_major, uint8_t* rcodes, uint8_t* rscales, int64_t rstep) {
  uint8_t* const rc[1] = {rcodes};
  uint8_t* const rs[1] = {rscales};
  return launch_mxfp8_colwise_multi(1, &x_bf16, R, C, E, offsets, pad, kcap, &codes, &scales, kofs, s, step_major,
                                    rcodes ? rc : nullptr, rcodes ? rs : nullptr, rstep);
}

extern "C" moe_status mxfp8_quantize_colwise(const void* x_bf16, int64_t R, int64_t C, int E, const int32_t* offsets,
                                             int pad, int64_t kcap, uint8_t* e4m3_t, uint8_t* e8m0_t, int32_t* kofs,
                                             void* stream) {
  if (R < 0 || C < 0) return fail(MOE_ERR_INVALID_ARG, "mxfp8_quantize_colwise: negative size");
  if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_ERR_INVALID_ARG, "mxfp8_quantize_colwise: E out of [1, 256]");
  if (pad <= 0 || pad % 32 != 0) return fail(MOE_ERR_INVALID_ARG, "mxfp8_quantize_colwise: pad must be a positive multiple of 32");
  if (C % 64 != 0) return fail(MOE_ERR_UNSUPPORTED, "mxfp8_quantize_colwise: C % 64 != 0");
  if (kcap % 32 != 0 || kcap < R + (int64_t)E * (pad - 1))
    return fail(MOE_ERR_INVALID_ARG, "mxfp8_quantize_colwise: kcap must be a multiple of 32 and >= R + E * (pad - 1)");
  if (R > 0x7FFFFFFF || kcap > 0x7FFFFFFF) return fail(MOE_ERR_UNSUPPORTED, "mxfp8_quantize_colwise: R or kcap >= 2^31");
  if (!offsets || !kofs || (C > 0 && (!e4m3_t || !e8m0_t)) || (R > 0 && C > 0 && !x_bf16))
    return fail(MOE_ERR_INVALID_ARG, "mxfp8_quantize_colwise: NULL pointer");
  if (!aligned(offsets, 4) || !aligned(kofs, 4) || (x_bf16 && !aligned(x_bf16, 16)) || (e4m3_t && !aligned(e4m3_t, 16)))
    return fail(MOE_ERR_INVALID_ARG, "mxfp8_quantize_colwise: x and codes must be 16-byte and offsets 4-byte aligned");
  return launch_mxfp8_colwise(x_bf16, R, (int)C, E, offsets, pad, kcap, e4m3_t, e8m0_t, kofs, as_stream(stream));
}

extern "C" moe_status mxfp8_pack_weight_bwd(const void* w_bf16, int64_t rows, int64_t cols, void* packed,
                                            void* stream) {
  if (rows < 0 || cols < 0) return fail(MOE_ERR_INVALID_ARG, "mxfp8_pack_weight_bwd: negative size");
  if (rows % 128 != 0 || cols % 64 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "mxfp8_pack_weight_bwd: needs rows % 128 == 0 and cols % 64 == 0");
  if (rows > 0x7FFFFFFF || rows * cols > 0x7FFFFFFFLL)
    return fail(MOE_ERR_UNSUPPORTED, "mxfp8_pack_weight_bwd: weight exceeds 2^31 elements");
  if (rows == 0 || cols == 0) return MOE_OK;
  if (!w_bf16 || !packed) return fail(MOE_ERR_INVALID_ARG, "mxfp8_pack_weight_bwd: NULL pointer");
  if (!aligned(w_bf16, 16) || !aligned(packed, 16))
    return fail(MOE_ERR_INVALID_ARG, "mxfp8_pack_weight_bwd: w and packed must be 16-byte aligned");
  uint8_t* codes = reinterpret_cast<uint8_t*>(packed);
  return launch_mxfp8_colwise(w_bf16, rows, (int)cols, 1, nullptr, 32, rows, codes, codes + rows * cols, nullptr,
                              as_stream(stream), true);
}

extern "C" moe_status mxfp8_quantize_weights(int n, const void* const* w_bf16, int64_t rows, int64_t cols,
                                             uint8_t* const* e4m3, uint8_t* const* e8m0, void* const* packed,
                                             void* stream) {
  if (n < 1 || n > MOE_MAX_EXPERTS) return fail(MOE_ERR_INVALID_ARG, "mxfp8_quantize_weights: n out of [1, 256]");
  if (rows < 0 || cols < 0) return fail(MOE_ERR_INVALID_ARG, "mxfp8_quantize_weights: negative size");
  if (rows % 128 != 0 || cols % 64 != 0)
    return fail(MOE_ERR_UNSUPPORTED, "mxfp8_quantize_weights: needs rows % 128 == 0 and cols % 64 == 0");
  if (rows > 0x7FFFFFFF || rows * cols > 0x7FFFFFFFLL)
    return fail(MOE_ERR_UNSUPPORTED, "mxfp8_quantize_weights: weight exceeds 2^31 elements");
  if (rows == 0 || cols == 0) return MOE_OK;
  if (!w_bf16 || !e4m3 || !e8m0 || !packed) return fail(MOE_ERR_INVALID_ARG, "mxfp8_quantize_weights: NULL table");
  uint8_t* codes[MOE_MAX_EXPERTS];
  uint8_t* scales[MOE_MAX_EXPERTS];
  for (int i = 0; i < n; ++i) {
    if (!w_bf16[i] || !e4m3[i] || !e8m0[i] || !packed[i])
      return fail(MOE_ERR_INVALID_ARG, "mxfp8_quantize_weights: NULL pointer");
    if (!aligned(w_bf16[i], 16) || !aligned(packed[i], 16) || !aligned(e4m3[i], 8))
      return fail(MOE_ERR_INVALID_ARG, "mxfp8_quantize_weights: w and packed must be 16-byte, e4m3 8-byte aligned");
    codes[i] = reinterpret_cast<uint8_t*>(packed[i]);
    scales[i] = codes[i] + rows * cols;
  }
  return launch_mxfp8_colwise_multi(n, w_bf16, rows, (int)cols, 1, nullptr, 32, rows, codes, scales, nullptr,
                                    as_stream(stream), true, e4m3, e8m0, 0);
}

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
