// Router top-k gating: softmax over the experts, keep the k largest, renormalise.
// Source: routing_weights in the per-expert loop of "Efficient MoE Training for
// Biological Foundation Models", Challenge 1. The selection itself (route_select.h)
// gives each token a group of L lanes; groups of 16 keep four tokens per wavefront for
// large E: the butterfly takes 4 shuffle steps instead of 6 and the wavefronts have a
// quarter of the latency-bound rounds each (Qwen3's E = 128: 63 -> 27 us per call
// against one token per wavefront).
#include <type_traits>

#include "common.h"
#include "internal.h"
#include "route_select.h"

namespace moe {

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
  int oid;
  float op;
  route_select<L, V>(logits, t, live, E, k, renorm, j, oid, op);
  // lane j of the group writes slot j
  if (live && j < k) {
    topk_idx[t * k + j] = oid;
    topk_prob[t * k + j] = op;
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
  if ((T + 3) / 4 > 0x7FFFFFFF) return fail(MOE_ERR_UNSUPPORTED, "moe_route_topk: T too large");
  const hipStream_t s = as_stream(stream);
  route_dispatch(E, [&](auto Lc, auto Vc) {
    constexpr int L = decltype(Lc)::value, V = decltype(Vc)::value;
    const int64_t per_block = 4 * (64 / L);
    const int64_t blocks = (T + per_block - 1) / per_block;
    hipLaunchKernelGGL((route_topk_kernel<L, V>), dim3((unsigned)blocks), dim3(256), 0, s, logits, T, E, k,
                       renormalize, topk_idx, topk_prob);
  });
  return check_launch("moe_route_topk");
}
