// Router top-k gating: softmax over the experts, keep the k largest, renormalise.
// Source: routing_weights in the per-expert loop of "Efficient MoE Training for
// Biological Foundation Models", Challenge 1. One thread per token; the kept
// entries are maintained as a sorted register list (bubble insertion) ordered by
// (logit descending, expert index ascending): selection is by comparison only and
// equal logits keep the lower expert index first.
#include "common.h"
#include "internal.h"

namespace moe {

constexpr int kMaxTopK = 16;

__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int64_t T,
                                                         int E, int k, int renorm,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_prob) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const float* row = logits + t * E;
  float val[kMaxTopK];
  int id[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    val[j] = 0.f;
    id[j] = -1;
  }
  for (int e = 0; e < E; ++e) {
    float v = row[e];
    int ve = e;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k) {
        // order by (logit descending, expert index ascending); the carried value may be a
        // displaced entry whose index is lower than the one it meets
        bool take = (ve >= 0) && (id[j] < 0 || v > val[j] || (v == val[j] && ve < id[j]));
        float tv = val[j];
        int ti = id[j];
        val[j] = take ? v : tv;
        id[j] = take ? ve : ti;
        v = take ? tv : v;
        ve = take ? ti : ve;
      }
    }
  }
  const float m = val[0];
  float num[kMaxTopK];
  float den = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    num[j] = (j < k) ? expf(val[j] - m) : 0.f;
    den += num[j];
  }
  if (!renorm) {
    den = 0.f;
    for (int e = 0; e < E; ++e) den += expf(row[e] - m);
  }
  const float inv = 1.f / den;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j < k) {
      topk_idx[t * k + j] = id[j];
      topk_prob[t * k + j] = num[j] * inv;
    }
  }
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
  const int threads = 256;
  int64_t blocks = (T + threads - 1) / threads;
  if (blocks > 0x7FFFFFFF) return fail(MOE_ERR_UNSUPPORTED, "moe_route_topk: T too large");
  hipLaunchKernelGGL(route_topk_kernel, dim3((unsigned)blocks), dim3(threads), 0, as_stream(stream),
                     logits, T, E, k, renormalize, topk_idx, topk_prob);
  return check_launch("moe_route_topk");
}
