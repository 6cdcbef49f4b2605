// Router top-k gating: softmax over the experts, keep the k largest, renormalise.
// Source: routing_weights in the per-expert loop of "Efficient MoE Training for
// Biological Foundation Models", Challenge 1.
//
// A group of L lanes per token (L = E rounded up to a power of two, at most 16; a
// wavefront holds 64 / L tokens), each lane holding V = ceil(E / L) logits of its
// token's row, so the row is read with coalesced loads. Groups of 16 keep four tokens
// per wavefront for large E: the butterfly takes 4 shuffle steps instead of 6 and the
// wavefronts have a quarter of the latency-bound rounds each (Qwen3's E = 128: 63 ->
// 27 us per call against one token per wavefront). k rounds of a butterfly
// arg-max over the group pick the experts in order of (logit descending, expert index
// ascending); a NaN logit ranks below every number, NaNs among themselves by index.
// Selection is by comparison only, so ties and the order of the k slots are exact.
#include <cmath>

#include "common.h"
#include "internal.h"

namespace moe {

constexpr int kMaxTopK = 16;

// strict total order on (logit, expert): does (av, ai) rank above (bv, bi)? An index
// below zero is "no candidate" and ranks below everything.
__device__ __forceinline__ bool ranks_above(float av, int ai, float bv, int bi) {
  if (ai < 0) return false;
  if (bi < 0) return true;
  const bool an = isnan(av), bn = isnan(bv);
  if (an != bn) return bn;
  if (an) return ai < bi;
  return av > bv || (av == bv && ai < bi);
}

template <int L, int V>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int64_t T,
                                                         int E, int k, int renorm,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_prob) {
  constexpr int G = 64 / L;  // tokens per wavefront
  const int lane = threadIdx.x & 63;
  const int j = lane % L;    // lane within the token's group
  const int64_t t = ((int64_t)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64) * G + lane / L;
  const bool live = t < T;
  float v[V];
  bool left[V];  // still a candidate
#pragma unroll
  for (int q = 0; q < V; ++q) {
    const int e = j + q * L;
    left[q] = live && e < E;
    v[q] = left[q] ? logits[t * E + e] : 0.f;
  }
  float sv[kMaxTopK];
  int si[kMaxTopK];
#pragma unroll
  for (int r = 0; r < kMaxTopK; ++r) {
    sv[r] = 0.f;
    si[r] = -1;
    if (r < k) {
      float bv = 0.f;
      int bi = -1;
#pragma unroll
      for (int q = 0; q < V; ++q)
        if (left[q] && ranks_above(v[q], j + q * L, bv, bi)) {
          bv = v[q];
          bi = j + q * L;
        }
#pragma unroll
      for (int m = L / 2; m >= 1; m >>= 1) {
        const float ov = __shfl_xor(bv, m, L);
        const int oi = __shfl_xor(bi, m, L);
        if (ranks_above(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
      sv[r] = bv;
      si[r] = bi;
#pragma unroll
      for (int q = 0; q < V; ++q)
        if (j + q * L == bi) left[q] = false;
    }
  }
  const float mx = sv[0];
  float den = 0.f;
  if (renorm) {
#pragma unroll
    for (int r = 0; r < kMaxTopK; ++r)
      if (r < k) den += expf(sv[r] - mx);
  } else {
#pragma unroll
    for (int q = 0; q < V; ++q)
      if (live && j + q * L < E) den += expf(v[q] - mx);
#pragma unroll
    for (int m = L / 2; m >= 1; m >>= 1) den += __shfl_xor(den, m, L);
  }
  const float inv = 1.f / den;
  // lane j of the group writes slot j
  int oid = -1;
  float op = 0.f;
#pragma unroll
  for (int r = 0; r < kMaxTopK; ++r)
    if (r == j) {
      oid = si[r];
      op = expf(sv[r] - mx) * inv;
    }
  if (live && j < k) {
    topk_idx[t * k + j] = oid;
    topk_prob[t * k + j] = op;
  }
}

template <int L, int V>
static void launch_route(const float* logits, int64_t T, int E, int k, int renorm, int32_t* idx, float* prob,
                         hipStream_t s) {
  const int64_t per_block = 4 * (64 / L);
  const int64_t blocks = (T + per_block - 1) / per_block;
  hipLaunchKernelGGL((route_topk_kernel<L, V>), dim3((unsigned)blocks), dim3(256), 0, s, logits, T, E, k, renorm,
                     idx, prob);
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_route_topk(const float* logits, int64_t T, int E, int k, int renormalize,
                                     int32_t* topk_idx, float* topk_prob, void* stream) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "moe_route_topk: T < 0");
  if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_ERR_INVALID_ARG, "moe_route_topk: E out of [1, 256]");
  if (k < 1 || k > E) return fail(MOE_ERR_INVALID_ARG, "moe_route_topk: k out of [1, E]");
  if (k > kMaxTopK) return fail(MOE_ERR_UNSUPPORTED, "moe_route_topk: k > 16");
  if (T == 0) return MOE_OK;
  if (!logits || !topk_idx || !topk_prob) return fail(MOE_ERR_INVALID_ARG, "moe_route_topk: NULL pointer");
  if (!aligned(logits, 4) || !aligned(topk_idx, 4) || !aligned(topk_prob, 4))
    return fail(MOE_ERR_INVALID_ARG, "moe_route_topk: misaligned pointer");
  if ((T + 3) / 4 > 0x7FFFFFFF) return fail(MOE_ERR_UNSUPPORTED, "moe_route_topk: T too large");
  const hipStream_t s = as_stream(stream);
  if (E <= 1) launch_route<1, 1>(logits, T, E, k, renormalize, topk_idx, topk_prob, s);
  else if (E <= 2) launch_route<2, 1>(logits, T, E, k, renormalize, topk_idx, topk_prob, s);
  else if (E <= 4) launch_route<4, 1>(logits, T, E, k, renormalize, topk_idx, topk_prob, s);
  else if (E <= 8) launch_route<8, 1>(logits, T, E, k, renormalize, topk_idx, topk_prob, s);
  else if (E <= 16) launch_route<16, 1>(logits, T, E, k, renormalize, topk_idx, topk_prob, s);
  else if (E <= 32) launch_route<16, 2>(logits, T, E, k, renormalize, topk_idx, topk_prob, s);
  else if (E <= 64) launch_route<16, 4>(logits, T, E, k, renormalize, topk_idx, topk_prob, s);
  else if (E <= 128) launch_route<16, 8>(logits, T, E, k, renormalize, topk_idx, topk_prob, s);
  else launch_route<16, 16>(logits, T, E, k, renormalize, topk_idx, topk_prob, s);
  return check_launch("moe_route_topk");
}
