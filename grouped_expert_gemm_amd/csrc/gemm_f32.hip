// float32 grouped MLP, forward and backward: plain per-element kernels (one thread
// per output element, a dot product over K). They serve the float32 precision of the
// tiny workload, where correctness rather than speed is the point; the bf16 and
// MXFP8 paths run on the MFMA kernels.
#include "common.h"
#include "gemm_f32.h"

namespace moe {
namespace f32 {

__device__ __forceinline__ int expert_of(const int32_t* __restrict__ off, int E, int64_t r) {
  int lo = 0, hi = E - 1;  // largest e with off[e] <= r
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ float sigmoid(float g) { return 1.f / (1.f + expf(-g)); }

__global__ __launch_bounds__(256) void gateup_swiglu(const float* __restrict__ x, const PtrTab w1,
                                                     const int32_t* __restrict__ off, const float* __restrict__ prob,
                                                     int64_t R, int E, int H, int I, float* __restrict__ h,
                                                     float* __restrict__ z) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= R * I) return;
  const int64_t r = idx / I;
  const int i = (int)(idx % I);
  const int e = expert_of(off, E, r);
  const float* W = reinterpret_cast<const float*>(w1.p[e]);
  const float* xr = x + r * H;
  const float* wg = W + (int64_t)i * H;
  const float* wu = W + (int64_t)(I + i) * H;
  float g = 0.f, u = 0.f;
  for (int k = 0; k < H; ++k) {
    g = fmaf(xr[k], wg[k], g);
    u = fmaf(xr[k], wu[k], u);
  }
  h[r * I + i] = g * sigmoid(g) * u * prob[r];
  if (z) {
    z[r * 2 * I + i] = g;
    z[r * 2 * I + I + i] = u;
  }
}

// y[r, n] = sum_k a[r, k] * W_e[n, k]   (W_e is [N, K])
__global__ __launch_bounds__(256) void rows_times_wt(const float* __restrict__ a, const PtrTab w,
                                                     const int32_t* __restrict__ off, int64_t R, int E, int N,
                                                     int K, float* __restrict__ y) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= R * N) return;
  const int64_t r = idx / N;
  const int n = (int)(idx % N);
  const int e = expert_of(off, E, r);
  const float* W = reinterpret_cast<const float*>(w.p[e]) + (int64_t)n * K;
  const float* ar = a + r * K;
  float s = 0.f;
  for (int k = 0; k < K; ++k) s = fmaf(ar[k], W[k], s);
  y[r * N + n] = s;
}

// y[r, n] = sum_k a[r, k] * W_e[k, n]   (W_e is [K, N])
__global__ __launch_bounds__(256) void rows_times_w(const float* __restrict__ a, const PtrTab w,
                                                    const int32_t* __restrict__ off, int64_t R, int E, int N,
                                                    int K, float* __restrict__ y) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= R * N) return;
  const int64_t r = idx / N;
  const int n = (int)(idx % N);
  const int e = expert_of(off, E, r);
  const float* W = reinterpret_cast<const float*>(w.p[e]) + n;
  const float* ar = a + r * K;
  float s = 0.f;
  for (int k = 0; k < K; ++k) s = fmaf(ar[k], W[(int64_t)k * N], s);
  y[r * N + n] = s;
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

// dW_e[m, n] = sum over expert e's rows r of a[r, m] * b[r, n]
__global__ __launch_bounds__(256) void wgrad(const float* __restrict__ a, int lda, const float* __restrict__ b,
                                             int ldb, const int32_t* __restrict__ off, int64_t R, int E, int M,
                                             int N, PtrTab dw) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)E * M * N) return;
  const int e = (int)(idx / ((int64_t)M * N));
  const int64_t mn = idx % ((int64_t)M * N);
  const int m = (int)(mn / N), n = (int)(mn % N);
  float s = 0.f;
  const int64_t r0 = off[e] < 0 ? 0 : off[e];
  const int64_t r1 = off[e + 1] > R ? R : off[e + 1];
  for (int64_t r = r0; r < r1; ++r) s = fmaf(a[r * lda + m], b[r * ldb + n], s);
  reinterpret_cast<float*>(const_cast<void*>(dw.p[e]))[mn] = s;
}

static unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

moe_status gate_up(int E, int64_t R, int H, int I, const float* x, const PtrTab& w1, const int32_t* off,
                   const float* prob, float* h, float* z, hipStream_t s) {
  if (R == 0) return MOE_OK;
  hipLaunchKernelGGL(gateup_swiglu, dim3(blocks_for(R * I)), dim3(256), 0, s, x, w1, off, prob, R, E, H, I, h, z);
  return check_launch("grouped gate_up + ScaledSwiGLU (f32)");
}

moe_status linear(int E, int64_t R, int K, int N, const float* x, const PtrTab& w, const int32_t* off, float* y,
                  hipStream_t s) {
  if (R == 0) return MOE_OK;
  hipLaunchKernelGGL(rows_times_wt, dim3(blocks_for(R * N)), dim3(256), 0, s, x, w, off, R, E, N, K, y);
  return check_launch("grouped linear (f32)");
}

moe_status forward(const moe_mlp_desc& d, int64_t R, const float* x, const PtrTab& w1, const PtrTab& w2,
                   const int32_t* off, const float* prob, float* y, float* z, float* h, hipStream_t s) {
  if (R == 0) return MOE_OK;
  hipLaunchKernelGGL(gateup_swiglu, dim3(blocks_for(R * d.I)), dim3(256), 0, s, x, w1, off, prob, R, d.E, d.H, d.I,
                     h, z);
  hipLaunchKernelGGL(rows_times_wt, dim3(blocks_for(R * d.H)), dim3(256), 0, s, (const float*)h, w2, off, R, d.E,
                     d.H, d.I, y);
  return check_launch("moe_grouped_mlp_fwd(f32)");
}

moe_status backward(const moe_mlp_desc& d, int64_t R, const float* dy, const float* x, const float* z,
                    const float* h, const float* prob, const PtrTab& w1, const PtrTab& w2, const int32_t* off,
                    float* dx, const PtrTab& dw1, const PtrTab& dw2, float* dprob, float* ws, hipStream_t s) {
  const int H = d.H, I = d.I, E = d.E;
  float* dh = ws;                 // [R, I]
  float* t = ws + R * I;          // [R, I]
  float* dz = ws + 2 * R * I;     // [R, 2I]
  if (R > 0) {
    hipLaunchKernelGGL(rows_times_w, dim3(blocks_for(R * I)), dim3(256), 0, s, dy, w2, off, R, E, I, H, dh);
    hipLaunchKernelGGL(dswiglu, dim3(blocks_for(R * I)), dim3(256), 0, s, (const float*)dh, z, prob, R, I, dz, t);
    hipLaunchKernelGGL(row_sum, dim3(blocks_for(R)), dim3(256), 0, s, (const float*)t, R, I, dprob);
    hipLaunchKernelGGL(rows_times_w, dim3(blocks_for(R * H)), dim3(256), 0, s, (const float*)dz, w1, off, R, E, H,
                       2 * I, dx);
  }
  hipLaunchKernelGGL(wgrad, dim3(blocks_for((int64_t)E * H * I)), dim3(256), 0, s, dy, H, h, I, off, R, E, H, I, dw2);
  hipLaunchKernelGGL(wgrad, dim3(blocks_for((int64_t)E * 2 * I * H)), dim3(256), 0, s, (const float*)dz, 2 * I, x,
                     H, off, R, E, 2 * I, H, dw1);
  return check_launch("moe_grouped_mlp_bwd(f32)");
}

}  // namespace f32
}  // namespace moe
