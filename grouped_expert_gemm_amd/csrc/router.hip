// Router gate linear and the backward of top-k gating.
// Source: routing_weights of the per-expert loop in "Efficient MoE Training for
// Biological Foundation Models", Challenge 1, which needs router logits per token; the
// pages show no router, so the gate is read as a bias-free linear map hidden -> E (the
// [out, in] weight layout of the pages' GroupedLinear weights), and its backward as the
// chain rule through the gating of moe_route_topk.
//
// router_logits_kernel: logits = x w^T on bf16 MFMA (32x32x16), fp32 accumulation. A
//   workgroup takes 32 tokens; its four wavefronts split H in quarters, each holding
//   all ceil(E/32) expert sub-tiles, and the quarters are added through LDS in a fixed
//   order. Operand fragments are read straight from global memory (16 bytes per lane):
//   every x row is read once, the weights (E x H, small) stay in cache.
// route_topk_bwd_kernel: the token-per-lane-group layout of the router; a token's k
//   slots are read by every lane of its group.
// router_dx_kernel / router_dw_kernel: the gate linear's backward on fp32 VALU, blocks
//   of 8 x 8 outputs per thread; dW sums token chunks (64 to 1024 tokens, enough for
//   ~1024 workgroups) into a workspace, then adds the chunks in order (deterministic).
#include <cmath>

#include "common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kRouterMaxTopK = 16;

template <int NT>  // expert sub-tiles of 32
__global__ __launch_bounds__(256) void router_logits_kernel(const bf16_t* __restrict__ x,
                                                            const bf16_t* __restrict__ w, int64_t T, int H,
                                                            int E, float* __restrict__ logits) {
  __shared__ float red[3][NT][16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, lhi = lane >> 5;
  const int64_t t0 = (int64_t)blockIdx.x * 32;
  int64_t tr = t0 + l32;
  if (tr >= T) tr = T - 1;  // rows past the end: any valid row, never stored
  const int hq = H / 4;     // this wavefront's quarter of H
  const bf16_t* xr = x + tr * H + wave * hq + lhi * 8;
  const bf16_t* wr[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    int e = n * 32 + l32;
    e = e < E ? e : E - 1;  // padded experts: any valid row, never stored
    wr[n] = w + (int64_t)e * H + wave * hq + lhi * 8;
  }
  f32x16 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[n][i] = 0.f;
  // A = weight rows (expert = output row i), B = token rows (token = output column j)
#pragma unroll 4
  for (int k = 0; k < hq; k += 16) {
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(xr + k);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(wr[n] + k);
      acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[n], 0, 0, 0);
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int i = 0; i < 16; ++i) red[wave - 1][n][i][lane] = acc[n][i];
  }
  __syncthreads();
  if (wave != 0) return;
  const int64_t t = t0 + l32;
  if (t >= T) return;
  float* out = logits + t * E;
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      // lane l holds token l % 32 and experts n*32 + (i/4)*8 + lhi*4 + i%4
      const float v = ((acc[n][i] + red[0][n][i][lane]) + red[1][n][i][lane]) + red[2][n][i][lane];
      const int e = n * 32 + (i >> 2) * 8 + lhi * 4 + (i & 3);
      if (e < E) out[e] = v;
    }
}

template <int L, int V>
__global__ __launch_bounds__(256) void route_topk_bwd_kernel(const float* __restrict__ logits,
                                                             const int32_t* __restrict__ idx,
                                                             const float* __restrict__ prob,
                                                             const float* __restrict__ dprob, int64_t T, int E,
                                                             int k, int renorm, float* __restrict__ dlog) {
  constexpr int G = 64 / L;
  const int lane = threadIdx.x & 63;
  const int j = lane % L;
  const int64_t t = ((int64_t)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64) * G + lane / L;
  const bool live = t < T;
  const int64_t tk = live ? t * k : 0;
  // s = sum over slots of p_j * g_j (p_j: the forward's probability of slot j)
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < kRouterMaxTopK; ++r)
    if (r < k && live) s += prob[tk + r] * dprob[tk + r];
  if (renorm) {
    // d l_{i_j} = p_j (g_j - s); experts not chosen: 0
#pragma unroll
    for (int q = 0; q < V; ++q) {
      const int e = j + q * L;
      if (!live || e >= E) continue;
      float d = 0.f;
      for (int r = 0; r < k; ++r)
        if (idx[tk + r] == e) d = prob[tk + r] * (dprob[tk + r] - s);
      dlog[t * E + e] = d;
    }
    return;
  }
  // full softmax P over the row: d l_e = P_e (G_e - s), G_e = g_j where e is slot j's
  float v[V];
  float mx = -INFINITY;
#pragma unroll
  for (int q = 0; q < V; ++q) {
    const int e = j + q * L;
    v[q] = (live && e < E) ? logits[t * E + e] : -INFINITY;
    mx = fmaxf(mx, v[q]);
  }
#pragma unroll
  for (int m = L / 2; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m, L));
  float den = 0.f;
#pragma unroll
  for (int q = 0; q < V; ++q)
    if (live && j + q * L < E) den += expf(v[q] - mx);
#pragma unroll
  for (int m = L / 2; m >= 1; m >>= 1) den += __shfl_xor(den, m, L);
  const float inv = 1.f / den;
#pragma unroll
  for (int q = 0; q < V; ++q) {
    const int e = j + q * L;
    if (!live || e >= E) continue;
    float g = 0.f;
    for (int r = 0; r < k; ++r)
      if (idx[tk + r] == e) g = dprob[tk + r];
    dlog[t * E + e] = expf(v[q] - mx) * inv * (g - s);
  }
}

constexpr int kDxTokens = 8;    // tokens per dx workgroup
constexpr int kHBlock = 2048;   // columns per workgroup (256 threads x 8)

// tokens per dW partial: enough chunks for ~1024 workgroups, 64 .. 1024 tokens each
int64_t dw_chunk(int64_t T, int H, int E) {
  const int64_t other = (int64_t)((E + 7) / 8) * ((H + kHBlock - 1) / kHBlock);
  int64_t want = (1024 + other - 1) / other;  // chunks wanted
  int64_t c = 1024;
  while (c > 64 && (T + c - 1) / c < want) c >>= 1;
  return c;
}

// dx[t, h] = (dx_in[t, h]) + sum_e dl[t, e] w[e, h]; thread: 8 tokens x 8 columns
__global__ __launch_bounds__(256) void router_dx_kernel(const float* __restrict__ dl, const bf16_t* __restrict__ w,
                                                        const bf16_t* __restrict__ dx_in, int64_t T, int H,
                                                        int E, bf16_t* __restrict__ dx) {
  const int64_t t0 = (int64_t)blockIdx.x * kDxTokens;
  const int h = blockIdx.y * kHBlock + threadIdx.x * 8;
  if (h >= H) return;
  float acc[kDxTokens][8];
#pragma unroll
  for (int a = 0; a < kDxTokens; ++a)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[a][c] = 0.f;
  for (int e = 0; e < E; ++e) {
    const uint4 wv = *reinterpret_cast<const uint4*>(w + (int64_t)e * H + h);
    const uint32_t wb[4] = {wv.x, wv.y, wv.z, wv.w};
    float wf[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      wf[2 * c] = bf16_to_f32(wb[c] & 0xFFFFu);
      wf[2 * c + 1] = bf16_to_f32(wb[c] >> 16);
    }
#pragma unroll
    for (int a = 0; a < kDxTokens; ++a) {
      const int64_t t = t0 + a < T ? t0 + a : T - 1;
      const float g = dl[t * E + e];
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[a][c] = fmaf(g, wf[c], acc[a][c]);
    }
  }
#pragma unroll
  for (int a = 0; a < kDxTokens; ++a) {
    const int64_t t = t0 + a;
    if (t >= T) break;
    float o[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] = acc[a][c];
    if (dx_in) {
      const uint4 iv = *reinterpret_cast<const uint4*>(dx_in + t * H + h);
      const uint32_t ib[4] = {iv.x, iv.y, iv.z, iv.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        o[2 * c] += bf16_to_f32(ib[c] & 0xFFFFu);
        o[2 * c + 1] += bf16_to_f32(ib[c] >> 16);
      }
    }
    *reinterpret_cast<uint4*>(dx + t * H + h) =
        make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7]));
  }
}

// part[c, e, h] = sum over tokens t of chunk c (in order) of dl[t, e] x[t, h];
// thread: 8 experts x 8 columns (VEC: E % 8 == 0, the 8 gradients come as two float4)
template <bool VEC>
__global__ __launch_bounds__(256) void router_dw_kernel(const float* __restrict__ dl, const bf16_t* __restrict__ x,
                                                        int64_t T, int H, int E, int64_t chunk,
                                                        float* __restrict__ part) {
  const int64_t c = blockIdx.x;
  const int e0 = blockIdx.y * 8;
  const int h = blockIdx.z * kHBlock + threadIdx.x * 8;
  if (h >= H) return;
  float acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = 0.f;
  const int64_t tb = c * chunk;
  const int64_t te = tb + chunk < T ? tb + chunk : T;
  for (int64_t t = tb; t < te; ++t) {
    const uint4 xv = *reinterpret_cast<const uint4*>(x + t * H + h);
    const uint32_t xb[4] = {xv.x, xv.y, xv.z, xv.w};
    float xf[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      xf[2 * q] = bf16_to_f32(xb[q] & 0xFFFFu);
      xf[2 * q + 1] = bf16_to_f32(xb[q] >> 16);
    }
    float gv[8];
    if constexpr (VEC) {
      const float4 g0 = *reinterpret_cast<const float4*>(dl + t * E + e0);
      const float4 g1 = *reinterpret_cast<const float4*>(dl + t * E + e0 + 4);
      gv[0] = g0.x; gv[1] = g0.y; gv[2] = g0.z; gv[3] = g0.w;
      gv[4] = g1.x; gv[5] = g1.y; gv[6] = g1.z; gv[7] = g1.w;
    } else {
#pragma unroll
      for (int a = 0; a < 8; ++a) gv[a] = dl[t * E + (e0 + a < E ? e0 + a : E - 1)];
    }
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int b = 0; b < 8; ++b) acc[a][b] = fmaf(gv[a], xf[b], acc[a][b]);
  }
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    const int e = e0 + a;
    if (e >= E) break;
    float* o = part + (c * E + e) * (int64_t)H + h;
    *reinterpret_cast<float4*>(o) = make_float4(acc[a][0], acc[a][1], acc[a][2], acc[a][3]);
    *reinterpret_cast<float4*>(o + 4) = make_float4(acc[a][4], acc[a][5], acc[a][6], acc[a][7]);
  }
}

// dw[i] = sum over chunks c (in order) of part[c][i]
__global__ __launch_bounds__(256) void router_dw_reduce(const float* __restrict__ part, int64_t nchunks,
                                                        int64_t n, float* __restrict__ dw) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int64_t c = 0; c < nchunks; ++c) s += part[c * n + i];
  dw[i] = s;
}

template <int NT>
void launch_logits(const bf16_t* x, const bf16_t* w, int64_t T, int H, int E, float* logits, hipStream_t s) {
  hipLaunchKernelGGL((router_logits_kernel<NT>), dim3((unsigned)((T + 31) / 32)), dim3(256), 0, s, x, w, T, H, E,
                     logits);
}

template <int L, int V>
void launch_bwd(const float* logits, const int32_t* idx, const float* prob, const float* dprob, int64_t T, int E,
                int k, int renorm, float* dlog, hipStream_t s) {
  const int64_t per_block = 4 * (64 / L);
  hipLaunchKernelGGL((route_topk_bwd_kernel<L, V>), dim3((unsigned)((T + per_block - 1) / per_block)), dim3(256), 0,
                     s, logits, idx, prob, dprob, T, E, k, renorm, dlog);
}

}  // namespace

size_t router_bwd_workspace_bytes(int64_t T, int H, int E) {
  if (T <= 0) return 0;
  const int64_t ch = dw_chunk(T, H, E);
  const int64_t nchunks = (T + ch - 1) / ch;
  return nchunks > 1 ? (size_t)(nchunks * E * (int64_t)H * 4) : 0;
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_router_logits(const void* x, const void* w_router, int64_t T, int H, int E,
                                        float* logits, void* stream) {
  if (T < 0 || H < 1 || E < 1 || E > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_INVALID_ARG, "moe_router_logits: bad T/H/E");
  if (H % 64 != 0) return fail(MOE_ERR_UNSUPPORTED, "moe_router_logits: needs H % 64 == 0");
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !logits) return fail(MOE_ERR_INVALID_ARG, "moe_router_logits: NULL pointer");
  if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(logits, 4))
    return fail(MOE_ERR_INVALID_ARG, "moe_router_logits: misaligned pointer");
  if ((T + 31) / 32 > 0x7FFFFFFF) return fail(MOE_ERR_UNSUPPORTED, "moe_router_logits: T too large");
  const bf16_t* xb = static_cast<const bf16_t*>(x);
  const bf16_t* wb = static_cast<const bf16_t*>(w_router);
  const hipStream_t s = as_stream(stream);
  switch ((E + 31) / 32) {
    case 1: launch_logits<1>(xb, wb, T, H, E, logits, s); break;
    case 2: launch_logits<2>(xb, wb, T, H, E, logits, s); break;
    case 3: launch_logits<3>(xb, wb, T, H, E, logits, s); break;
    case 4: launch_logits<4>(xb, wb, T, H, E, logits, s); break;
    case 5: launch_logits<5>(xb, wb, T, H, E, logits, s); break;
    case 6: launch_logits<6>(xb, wb, T, H, E, logits, s); break;
    case 7: launch_logits<7>(xb, wb, T, H, E, logits, s); break;
    default: launch_logits<8>(xb, wb, T, H, E, logits, s); break;
  }
  return check_launch("moe_router_logits");
}

extern "C" moe_status moe_route_topk_bwd(const float* logits, const int32_t* topk_idx, const float* topk_prob,
                                         const float* d_topk_prob, int64_t T, int E, int k, int renormalize,
                                         float* d_logits, void* stream) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "moe_route_topk_bwd: T < 0");
  if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_ERR_INVALID_ARG, "moe_route_topk_bwd: E out of [1, 256]");
  if (k < 1 || k > E) return fail(MOE_ERR_INVALID_ARG, "moe_route_topk_bwd: k out of [1, E]");
  if (k > kRouterMaxTopK) return fail(MOE_ERR_UNSUPPORTED, "moe_route_topk_bwd: k > 16");
  if (T == 0) return MOE_OK;
  if (!topk_idx || !topk_prob || !d_topk_prob || !d_logits || (!renormalize && !logits))
    return fail(MOE_ERR_INVALID_ARG, "moe_route_topk_bwd: NULL pointer");
  if ((T + 3) / 4 > 0x7FFFFFFF) return fail(MOE_ERR_UNSUPPORTED, "moe_route_topk_bwd: T too large");
  const hipStream_t s = as_stream(stream);
  const int r = renormalize ? 1 : 0;
  if (E <= 1) launch_bwd<1, 1>(logits, topk_idx, topk_prob, d_topk_prob, T, E, k, r, d_logits, s);
  else if (E <= 2) launch_bwd<2, 1>(logits, topk_idx, topk_prob, d_topk_prob, T, E, k, r, d_logits, s);
  else if (E <= 4) launch_bwd<4, 1>(logits, topk_idx, topk_prob, d_topk_prob, T, E, k, r, d_logits, s);
  else if (E <= 8) launch_bwd<8, 1>(logits, topk_idx, topk_prob, d_topk_prob, T, E, k, r, d_logits, s);
  else if (E <= 16) launch_bwd<16, 1>(logits, topk_idx, topk_prob, d_topk_prob, T, E, k, r, d_logits, s);
  else if (E <= 32) launch_bwd<32, 1>(logits, topk_idx, topk_prob, d_topk_prob, T, E, k, r, d_logits, s);
  else if (E <= 64) launch_bwd<64, 1>(logits, topk_idx, topk_prob, d_topk_prob, T, E, k, r, d_logits, s);
  else if (E <= 128) launch_bwd<64, 2>(logits, topk_idx, topk_prob, d_topk_prob, T, E, k, r, d_logits, s);
  else launch_bwd<64, 4>(logits, topk_idx, topk_prob, d_topk_prob, T, E, k, r, d_logits, s);
  return check_launch("moe_route_topk_bwd");
}

extern "C" moe_status moe_router_bwd(const void* x, const void* w_router, const float* d_logits,
                                     const void* dx_in, int64_t T, int H, int E, void* dx, float* dw_router,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  if (T < 0 || H < 1 || E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_ERR_INVALID_ARG, "moe_router_bwd: bad T/H/E");
  if (H % 8 != 0) return fail(MOE_ERR_UNSUPPORTED, "moe_router_bwd: needs H % 8 == 0");
  if (!dw_router || (T > 0 && (!x || !w_router || !d_logits || !dx)))
    return fail(MOE_ERR_INVALID_ARG, "moe_router_bwd: NULL pointer");
  if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(dx, 16) || (dx_in && !aligned(dx_in, 16)) ||
      !aligned(dw_router, 16) || !aligned(d_logits, 4))
    return fail(MOE_ERR_INVALID_ARG, "moe_router_bwd: misaligned pointer");
  const hipStream_t s = as_stream(stream);
  const int64_t n = (int64_t)E * H;
  if (T == 0) {  // no tokens: dw_router = 0 (a sum over no chunks), dx untouched
    hipLaunchKernelGGL(router_dw_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (const float*)nullptr,
                       (int64_t)0, n, dw_router);
    return check_launch("moe_router_bwd(dw)");
  }
  const size_t need = router_bwd_workspace_bytes(T, H, E);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(MOE_ERR_WORKSPACE, "moe_router_bwd: workspace too small (moe_workspace_size(MOE_OP_ROUTER_BWD))");
  if (need > 0 && !aligned(workspace, 16)) return fail(MOE_ERR_INVALID_ARG, "moe_router_bwd: misaligned workspace");
  const unsigned hb = (unsigned)((H + kHBlock - 1) / kHBlock);
  if ((T + kDxTokens - 1) / kDxTokens > 0x7FFFFFFF) return fail(MOE_ERR_UNSUPPORTED, "moe_router_bwd: T too large");
  hipLaunchKernelGGL(router_dx_kernel, dim3((unsigned)((T + kDxTokens - 1) / kDxTokens), hb), dim3(256), 0, s,
                     d_logits, static_cast<const bf16_t*>(w_router), static_cast<const bf16_t*>(dx_in), T, H, E,
                     static_cast<bf16_t*>(dx));
  moe_status st = check_launch("moe_router_bwd(dx)");
  if (st != MOE_OK) return st;
  const int64_t ch = dw_chunk(T, H, E);
  const int64_t nchunks = (T + ch - 1) / ch;
  float* part = nchunks > 1 ? static_cast<float*>(workspace) : dw_router;
  const dim3 gdw((unsigned)nchunks, (unsigned)((E + 7) / 8), hb);
  if (E % 8 == 0 && aligned(d_logits, 16))
    hipLaunchKernelGGL(router_dw_kernel<true>, gdw, dim3(256), 0, s, d_logits, static_cast<const bf16_t*>(x), T, H,
                       E, ch, part);
  else
    hipLaunchKernelGGL(router_dw_kernel<false>, gdw, dim3(256), 0, s, d_logits, static_cast<const bf16_t*>(x), T, H,
                       E, ch, part);
  if ((st = check_launch("moe_router_bwd(dw)")) != MOE_OK) return st;
  if (nchunks > 1) {
    hipLaunchKernelGGL(router_dw_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (const float*)part,
                       nchunks, n, dw_router);
    st = check_launch("moe_router_bwd(dw reduce)");
  }
  return st;
}
