// Top-k selection of the router (softmax over the experts, keep the k largest,
// renormalise), shared by the routing kernel and the fused routing + permutation count.
// Source: routing_weights in the per-expert loop of "Efficient MoE Training for
// Biological Foundation Models", Challenge 1.
//
// A group of L lanes per token (L = E rounded up to a power of two, at most 16; a
// wavefront holds 64 / L tokens), each lane holding V = ceil(E / L) logits of its
// token's row, so the row is read with coalesced loads. k rounds of a butterfly
// arg-max over the group pick the experts in order of (logit descending, expert index
// ascending); a NaN logit ranks below every number, NaNs among themselves by index.
// Selection is by comparison only, so ties and the order of the k slots are exact.
#pragma once

#include <cmath>

#include "common.h"

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

// Token t's slot j (lane j of the token's group of L lanes): its expert (oid) and
// routing weight (op); lanes j >= k get oid = -1. Every lane of the group must call it
// (the butterfly shuffles within the group); live = false for groups past the last token.
template <int L, int V>
__device__ __forceinline__ void route_select(const float* __restrict__ logits, int64_t t, bool live, int E, int k,
                                             int renorm, int j, int& oid, float& op) {
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
  oid = -1;
  op = 0.f;
#pragma unroll
  for (int r = 0; r < kMaxTopK; ++r)
    if (r == j && r < k) {
      oid = si[r];
      op = expf(sv[r] - mx) * inv;
    }
}

// (L, V) for E experts: L = E rounded up to a power of two, at most 16; V = ceil(E / L)
template <typename F>
inline void route_dispatch(int E, F&& f) {
  if (E <= 1) f(std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{});
  else if (E <= 2) f(std::integral_constant<int, 2>{}, std::integral_constant<int, 1>{});
  else if (E <= 4) f(std::integral_constant<int, 4>{}, std::integral_constant<int, 1>{});
  else if (E <= 8) f(std::integral_constant<int, 8>{}, std::integral_constant<int, 1>{});
  else if (E <= 16) f(std::integral_constant<int, 16>{}, std::integral_constant<int, 1>{});
  else if (E <= 32) f(std::integral_constant<int, 16>{}, std::integral_constant<int, 2>{});
  else if (E <= 64) f(std::integral_constant<int, 16>{}, std::integral_constant<int, 4>{});
  else if (E <= 128) f(std::integral_constant<int, 16>{}, std::integral_constant<int, 8>{});
  else f(std::integral_constant<int, 16>{}, std::integral_constant<int, 16>{});
}

}  // namespace moe
