// float32 grouped MLP, forward and backward, for the tiny workload's precision. Every
// product is a grouped GEMM on the matrix cores in float32 (v_mfma_f32_32x32x2f32:
// float32 products and sums): a workgroup computes a 64 x 64 output tile, K in steps
// of 32 staged through LDS, four wavefronts of 32 x 32. Operands are addressed by
// general strides, so one tile routine serves the forward (rows grouped by expert,
// weights [N, K]), the data gradients (weights [K, N]) and the weight gradients (K
// running over the expert's rows). Every load and store is bounds-checked, so any
// sizes work; ScaledSwiGLU is fused into the gate_up tile, dSwiGLU and the dprob row
// sums are elementwise kernels.
#include <initializer_list>

#include "common.h"
#include "gemm_f32.h"
#include "tile_f32.h"

namespace moe {
namespace f32 {

using namespace tf32;

__device__ __forceinline__ float sigmoid(float g) { return 1.f / (1.f + expf(-g)); }

// Row tile `rt` of the experts' row tiles in order (ceil(rows_e / 64) each): its expert,
// first row and row count, or false past the last. Offsets are read as a nondecreasing
// sequence inside [0, R].
__device__ __forceinline__ bool find_row_tile(const int32_t* off, int E, int64_t R, int rt, int& e, int64_t& r0,
                                              int& rows) {
  int64_t prev = 0;
  for (int x = 0; x < E; ++x) {
    int64_t en = off[x + 1];
    en = en < prev ? prev : (en > R ? R : en);
    const int nt = (int)((en - prev + kT - 1) / kT);
    if (rt < nt) {
      e = x;
      r0 = prev + (int64_t)rt * kT;
      rows = (int)(en - r0 < kT ? en - r0 : kT);
      return true;
    }
    rt -= nt;
    prev = en;
  }
  return false;
}

// y[r, n] = sum_k a[r, k] * B_e(k, n), B_e(k, n) at w_e[k * sbk + n * sbn]; rows of
// expert e use w_e. Grid: (an upper bound on the row tiles, column tiles).
__global__ __launch_bounds__(256) void grouped_rows(const float* __restrict__ a, int64_t lda, const PtrTab w,
                                                    int64_t sbk, int64_t sbn, const int32_t* __restrict__ off,
                                                    int64_t R, int E, int N, int K, float* __restrict__ y,
                                                    int64_t ldy) {
  __shared__ float sA[kStage], sB[kStage];
  int e, rows;
  int64_t r0;
  if (!find_row_tile(off, E, R, blockIdx.x, e, r0, rows)) return;
  const int n0 = blockIdx.y * kT;
  const int tid = threadIdx.x;
  const View<float> av{a + r0 * lda, lda, 1, rows, K};
  const View<float> bv[1] = {{reinterpret_cast<const float*>(w.p[e]) + (int64_t)n0 * sbn, sbn, sbk, N - n0, K}};
  f32x16 acc[1];
  tile_product<1>(av, bv, acc, sA, sB, tid);
  for_outputs(tid, rows, N - n0, [&](int r, int c, int v) { y[(r0 + r) * ldy + n0 + c] = acc[0][v]; });
}

// gate_up with ScaledSwiGLU: g = x W1_e[i, :]^T, u = x W1_e[I + i, :]^T for the tile's
// 64 values of i; h = silu(g) * u * prob, and z = [g, u] when z is given.
__global__ __launch_bounds__(256) void grouped_gate_up(const float* __restrict__ x, const PtrTab w1,
                                                       const int32_t* __restrict__ off,
                                                       const float* __restrict__ prob, int64_t R, int E, int H,
                                                       int I, float* __restrict__ h, float* __restrict__ z) {
  __shared__ float sA[kStage], sB[2 * kStage];
  int e, rows;
  int64_t r0;
  if (!find_row_tile(off, E, R, blockIdx.x, e, r0, rows)) return;
  const int i0 = blockIdx.y * kT;
  const int tid = threadIdx.x;
  const float* W = reinterpret_cast<const float*>(w1.p[e]);
  const View<float> av{x + r0 * H, H, 1, rows, H};
  const View<float> bv[2] = {{W + (int64_t)i0 * H, H, 1, I - i0, H}, {W + (int64_t)(I + i0) * H, H, 1, I - i0, H}};
  f32x16 acc[2];
  tile_product<2>(av, bv, acc, sA, sB, tid);
  for_outputs(tid, rows, I - i0, [&](int r, int c, int v) {
    const int64_t row = r0 + r;
    const float g = acc[0][v], u = acc[1][v];
    h[row * I + i0 + c] = g * sigmoid(g) * u * prob[row];
    if (z) {
      z[row * 2 * I + i0 + c] = g;
      z[row * 2 * I + I + i0 + c] = u;
    }
  });
}

// dW_e[m, n] = sum over expert e's rows r of a[r, m] * b[r, n]. Grid: (column tiles,
// row tiles, E); an expert without rows gets zeros.
__global__ __launch_bounds__(256) void grouped_wgrad(const float* __restrict__ a, int64_t lda,
                                                     const float* __restrict__ b, int64_t ldb,
                                                     const int32_t* __restrict__ off, int64_t R, int E, int M, int N,
                                                     PtrTab dw) {
  __shared__ float sA[kStage], sB[kStage];
  const int e = blockIdx.z;
  int64_t r0 = 0, r1 = 0;
  for (int x = 0; x <= e; ++x) {  // the same clamped, nondecreasing offsets as the row tiles
    r0 = r1;
    int64_t en = off[x + 1];
    r1 = en < r0 ? r0 : (en > R ? R : en);
  }
  const int rows = (int)(r1 - r0);
  const int m0 = blockIdx.y * kT, n0 = blockIdx.x * kT;
  const int tid = threadIdx.x;
  const View<float> av{a + r0 * lda + m0, 1, lda, M - m0, rows};
  const View<float> bv[1] = {{b + r0 * ldb + n0, 1, ldb, N - n0, rows}};
  f32x16 acc[1];
  tile_product<1>(av, bv, acc, sA, sB, tid);
  float* out = reinterpret_cast<float*>(const_cast<void*>(dw.p[e]));
  for_outputs(tid, M - m0, N - n0, [&](int r, int c, int v) { out[(int64_t)(m0 + r) * N + n0 + c] = acc[0][v]; });
}

// from dH (= dY W2) and the saved z: dz = [dG, dU] and t = dH * A (for dprob)
__global__ __launch_bounds__(256) void dswiglu(const float* __restrict__ dh, const float* __restrict__ z,
                                               const float* __restrict__ prob, int64_t R, int I,
                                               float* __restrict__ dz, float* __restrict__ t) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= R * I) return;
  const int64_t r = idx / I;
  const int i = (int)(idx % I);
  const float g = z[r * 2 * I + i], u = z[r * 2 * I + I + i];
  const float sg = sigmoid(g);
  const float d = dh[idx];
  t[idx] = d * g * sg * u;
  const float da = d * prob[r];
  dz[r * 2 * I + i] = da * u * sg * (1.f + g * (1.f - sg));
  dz[r * 2 * I + I + i] = da * g * sg;
}

__global__ __launch_bounds__(256) void row_sum(const float* __restrict__ t, int64_t R, int I, float* __restrict__ out) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= R) return;
  float s = 0.f;
  for (int i = 0; i < I; ++i) s += t[r * I + i];
  out[r] = s;
}

static unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }
static unsigned tiles(int64_t n) { return (unsigned)((n + kT - 1) / kT); }
// an upper bound on sum over experts of ceil(rows_e / 64)
static unsigned row_tiles(int64_t R, int E) { return (unsigned)((R + kT - 1) / kT + E); }

// Grids: row tiles in x (at most 2^24 - 1 workgroups of 256 threads), column tiles and
// weight-gradient row tiles in y (at most 65535).
static moe_status grid_fits(int64_t R, int E, std::initializer_list<int64_t> edges, const char* what) {
  bool ok = (R + kT - 1) / kT + E < (1 << 24);
  for (int64_t n : edges) ok = ok && (n + kT - 1) / kT <= 65535;
  return ok ? MOE_OK : fail(MOE_ERR_UNSUPPORTED, std::string(what) + ": float32 sizes exceed the launch grid");
}

static void rows_product(const float* a, int64_t lda, const PtrTab& w, int64_t sbk, int64_t sbn, const int32_t* off,
                         int64_t R, int E, int N, int K, float* y, hipStream_t s) {
  hipLaunchKernelGGL(grouped_rows, dim3(row_tiles(R, E), tiles(N)), dim3(256), 0, s, a, lda, w, sbk, sbn, off, R, E,
                     N, K, y, (int64_t)N);
}

moe_status gate_up(int E, int64_t R, int H, int I, const float* x, const PtrTab& w1, const int32_t* off,
                   const float* prob, float* h, float* z, hipStream_t s) {
  if (R == 0) return MOE_OK;
  if (moe_status st = grid_fits(R, E, {I}, "moe_grouped_gate_up_swiglu")) return st;
  hipLaunchKernelGGL(grouped_gate_up, dim3(row_tiles(R, E), tiles(I)), dim3(256), 0, s, x, w1, off, prob, R, E, H, I,
                     h, z);
  return check_launch("grouped gate_up + ScaledSwiGLU (f32)");
}

moe_status linear(int E, int64_t R, int K, int N, const float* x, const PtrTab& w, const int32_t* off, float* y,
                  hipStream_t s) {
  if (R == 0) return MOE_OK;
  if (moe_status st = grid_fits(R, E, {N}, "moe_grouped_linear")) return st;
  rows_product(x, K, w, 1, K, off, R, E, N, K, y, s);  // W_e is [N, K]
  return check_launch("grouped linear (f32)");
}

moe_status forward(const moe_mlp_desc& d, int64_t R, const float* x, const PtrTab& w1, const PtrTab& w2,
                   const int32_t* off, const float* prob, float* y, float* z, float* h, hipStream_t s) {
  if (R == 0) return MOE_OK;
  if (moe_status st = grid_fits(R, d.E, {d.I, d.H}, "moe_grouped_mlp_fwd")) return st;
  hipLaunchKernelGGL(grouped_gate_up, dim3(row_tiles(R, d.E), tiles(d.I)), dim3(256), 0, s, x, w1, off, prob, R, d.E,
                     d.H, d.I, h, z);
  rows_product(h, d.I, w2, 1, d.I, off, R, d.E, d.H, d.I, y, s);  // W2_e is [H, I]
  return check_launch("moe_grouped_mlp_fwd(f32)");
}

moe_status backward(const moe_mlp_desc& d, int64_t R, const float* dy, const float* x, const float* z,
                    const float* h, const float* prob, const PtrTab& w1, const PtrTab& w2, const int32_t* off,
                    float* dx, const PtrTab& dw1, const PtrTab& dw2, float* dprob, float* ws, hipStream_t s) {
  const int H = d.H, I = d.I, E = d.E;
  float* dh = ws;                 // [R, I]
  float* t = ws + R * I;          // [R, I]
  float* dz = ws + 2 * R * I;     // [R, 2I]
  if (moe_status st = grid_fits(R, E, {I, H, 2 * (int64_t)I}, "moe_grouped_mlp_bwd")) return st;
  if (R > 0) {
    rows_product(dy, H, w2, I, 1, off, R, E, I, H, dh, s);  // dH = dY W2_e, W2_e [H, I]
    hipLaunchKernelGGL(dswiglu, dim3(blocks_for(R * I)), dim3(256), 0, s, (const float*)dh, z, prob, R, I, dz, t);
    hipLaunchKernelGGL(row_sum, dim3(blocks_for(R)), dim3(256), 0, s, (const float*)t, R, I, dprob);
    rows_product(dz, 2 * I, w1, H, 1, off, R, E, H, 2 * I, dx, s);  // dX = dZ W1_e, W1_e [2I, H]
  }
  // dW2_e = dY_e^T H_e [H, I]; dW1_e = dZ_e^T X_e [2I, H]
  hipLaunchKernelGGL(grouped_wgrad, dim3(tiles(I), tiles(H), E), dim3(256), 0, s, dy, (int64_t)H, h, (int64_t)I, off,
                     R, E, H, I, dw2);
  hipLaunchKernelGGL(grouped_wgrad, dim3(tiles(H), tiles(2 * I), E), dim3(256), 0, s, (const float*)dz,
                     (int64_t)(2 * I), x, (int64_t)H, off, R, E, 2 * I, H, dw1);
  return check_launch("moe_grouped_mlp_bwd(f32)");
}

}  // namespace f32
}  // namespace moe
