// Token permutation into per-expert groups and the weighted combine back.
// Source: "Efficient MoE Training for Biological Foundation Models", Challenge 1
// (split_sizes; the baseline loop gathers each expert's rows and index-adds the
// results back), and the token permute/unpermute step named in the PyTorch-native
// MoE library article (DeepEP dispatcher with permute/unpermute fusion).
//
// Three kernels, all deterministic (integer atomics only build bit sets):
//   count   : per 256-token block, an LDS bit set per expert marks the tokens that
//             chose it; popcounts give the block's per-expert counts and each
//             (token, slot)'s rank among the block's tokens of that expert
//             (ascending token order -> a stable permutation);
//   scan    : one workgroup turns the [blocks, E] counts into split_sizes, offsets
//             and each block's first row per expert;
//   scatter : one wavefront per token reads its row once (16-byte lanes) and writes
//             it to its k destination rows, plus the maps and the row weights.
#include <mutex>

#include <type_traits>

#include "common.h"
#include "internal.h"

namespace moe {

constexpr int kPermBlock = 256;  // tokens per count block
constexpr int kMaxK = 16;

size_t permute_workspace_bytes(int64_t T, int E, int k) {
  int64_t nb = (T + kPermBlock - 1) / kPermBlock;
  size_t b = 0;
  b += align_up((size_t)nb * E * sizeof(int32_t), 256);  // counts
  b += align_up((size_t)nb * E * sizeof(int32_t), 256);  // block bases
  b += align_up((size_t)T * k * sizeof(int32_t), 256);   // rank within block
  return b;
}

// expert of slot j of a token whose k ids are in e[0..k): -1 when the id is out of
// [0, E) or repeats the id of an earlier slot (such a pair is dropped)
__device__ __forceinline__ int slot_expert(const int* e, int j, int E) {
  const int x = e[j];
  bool ok = (unsigned)x < (unsigned)E;
#pragma unroll
  for (int i = 0; i < kMaxK; ++i)
    if (i < j && e[i] == x) ok = false;
  return ok ? x : -1;
}

__global__ __launch_bounds__(kPermBlock) void permute_count_kernel(const int32_t* __restrict__ idx,
                                                                   int64_t T, int E, int k,
                                                                   int32_t* __restrict__ counts,
                                                                   int32_t* __restrict__ rank_local) {
  __shared__ uint32_t flags[MOE_MAX_EXPERTS * (kPermBlock / 32)];
  const int tid = threadIdx.x;
  for (int i = tid; i < E * (kPermBlock / 32); i += kPermBlock) flags[i] = 0;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kPermBlock + tid;
  const int w = tid >> 5;
  const uint32_t bit = 1u << (tid & 31);
  int ids[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) ids[j] = (t < T && j < k) ? idx[t * k + j] : -1;
  if (t < T) {
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j >= k) break;
      const int e = slot_expert(ids, j, E);
      if (e >= 0) atomicOr(&flags[e * (kPermBlock / 32) + w], bit);
    }
  }
  __syncthreads();
  if (t < T) {
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j >= k) break;
      const int e = slot_expert(ids, j, E);
      int r = -1;
      if (e >= 0) {
        const uint32_t* f = &flags[e * (kPermBlock / 32)];
        r = 0;
        for (int ww = 0; ww < w; ++ww) r += __popc(f[ww]);
        r += __popc(f[w] & (bit - 1u));
      }
      rank_local[t * k + j] = r;
    }
  }
  for (int e = tid; e < E; e += kPermBlock) {
    int c = 0;
#pragma unroll
    for (int ww = 0; ww < kPermBlock / 32; ++ww) c += __popc(flags[e * (kPermBlock / 32) + ww]);
    counts[(int64_t)blockIdx.x * E + e] = c;
  }
}

__global__ __launch_bounds__(256) void permute_scan_kernel(const int32_t* __restrict__ counts, int64_t nb,
                                                           int E, int32_t* __restrict__ base,
                                                           int32_t* __restrict__ split_sizes,
                                                           int32_t* __restrict__ offsets) {
  // counts [nb, E] pass through LDS in chunks of whole block rows, read coalesced;
  // thread e runs down column e inside LDS (the running count stays in a register
  // across chunks). The expert totals are scanned in parallel (Hillis-Steele over 256
  // entries). When every block row fits in one chunk the expert offsets are added as
  // the chunk is written out; otherwise a second coalesced pass adds them.
  constexpr int kChunk = 8192;  // LDS entries per chunk (32 KiB)
  __shared__ int32_t buf[kChunk];
  __shared__ int32_t sc[2][256];
  const int tid = threadIdx.x;
  const int64_t rows = kChunk / E;  // E <= 256, so at least 32 block rows per chunk
  const bool one_chunk = nb <= rows;
  int32_t run = 0;
  for (int64_t b0 = 0; b0 < nb; b0 += rows) {
    const int64_t nr = nb - b0 < rows ? nb - b0 : rows;
    const int n = (int)(nr * E);
    const int32_t* src = counts + b0 * E;
    for (int i = tid; i < n; i += 256) buf[i] = src[i];
    __syncthreads();
    if (tid < E)
      for (int r = 0; r < (int)nr; ++r) {
        const int32_t c = buf[r * E + tid];
        buf[r * E + tid] = run;
        run += c;
      }
    __syncthreads();
    if (!one_chunk) {
      int32_t* dst = base + b0 * E;
      for (int i = tid; i < n; i += 256) dst[i] = buf[i];
      __syncthreads();
    }
  }
  // per-expert totals -> exclusive offsets
  const int32_t total = tid < E ? run : 0;
  sc[0][tid] = total;
  __syncthreads();
  int cur = 0;
  for (int d = 1; d < 256; d <<= 1) {
    int32_t x = sc[cur][tid];
    if (tid >= d) x += sc[cur][tid - d];
    sc[cur ^ 1][tid] = x;
    __syncthreads();
    cur ^= 1;
  }
  const int32_t incl = sc[cur][tid];
  if (tid < E) {
    split_sizes[tid] = total;
    offsets[tid] = incl - total;
  }
  if (tid == E - 1) offsets[E] = incl;
  sc[cur ^ 1][tid] = incl - total;  // exclusive offset of expert tid
  __syncthreads();
  const int32_t* off = sc[cur ^ 1];
  // thread tid adds to column tid % E of every (256 / E)-th row, starting at row tid / E
  const int per = 256 / E;
  const int c = tid % E, r0 = tid / E;
  if (r0 < per) {
    const int32_t o = off[c];
    if (one_chunk) {
      for (int64_t r = r0; r < nb; r += per) base[r * E + c] = buf[r * E + c] + o;
    } else {
      for (int64_t r = r0; r < nb; r += per) base[r * E + c] += o;
    }
  }
}

template <typename U>
__device__ __forceinline__ void copy_row_to_k(const uint8_t* __restrict__ src, int64_t bytes,
                                              uint8_t* __restrict__ dst_base, const int32_t* rows,
                                              int k, int lane) {
  const int64_t n = bytes / (int64_t)sizeof(U);
  const U* s = reinterpret_cast<const U*>(src);
  int64_t c = lane;
  // four chunks' loads in flight together, then their stores
  for (; c + 192 < n; c += 256) {
    U v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = s[c + 64 * q];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) {
        if (j < k && rows[j] >= 0) reinterpret_cast<U*>(dst_base + (int64_t)rows[j] * bytes)[c + 64 * q] = v[q];
      }
  }
  for (; c < n; c += 64) {
    U v = s[c];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < k && rows[j] >= 0) reinterpret_cast<U*>(dst_base + (int64_t)rows[j] * bytes)[c] = v;
    }
  }
}

// unit: widest access (16, 4 or 1 bytes) that the row size and both base pointers allow
__device__ __forceinline__ void copy_row_any(const uint8_t* src, int64_t bytes, uint8_t* dst,
                                             const int32_t* rows, int k, int lane, int unit) {
  if (unit == 16)
    copy_row_to_k<uint4>(src, bytes, dst, rows, k, lane);
  else if (unit == 4)
    copy_row_to_k<uint32_t>(src, bytes, dst, rows, k, lane);
  else
    copy_row_to_k<uint8_t>(src, bytes, dst, rows, k, lane);
}

__global__ __launch_bounds__(256) void permute_scatter_kernel(
    const uint8_t* __restrict__ x, int64_t row_bytes, const uint8_t* __restrict__ xs,
    int64_t srow_bytes, const int32_t* __restrict__ idx, const float* __restrict__ prob,
    const int32_t* __restrict__ base, const int32_t* __restrict__ rank_local, int64_t T, int E, int k,
    int reuse, int unit, int sunit, uint8_t* __restrict__ xp, uint8_t* __restrict__ xps, float* __restrict__ prob_perm,
    int32_t* __restrict__ row_id_map, int32_t* __restrict__ src_token) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int64_t R = T * k;
  int32_t rows[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    rows[j] = -1;
    if (j < k) {
      int32_t r;
      if (reuse) {
        r = row_id_map[t * k + j];
      } else {
        const int e = idx[t * k + j];
        const int rl = rank_local[t * k + j];  // -1: a dropped pair
        r = ((unsigned)e < (unsigned)E && rl >= 0) ? base[(t / kPermBlock) * E + e] + rl : -1;
      }
      rows[j] = (r >= 0 && r < R) ? r : -1;
      if (!reuse && lane == j) {
        row_id_map[t * k + j] = rows[j];
        if (rows[j] >= 0) {
          src_token[rows[j]] = (int32_t)t;
          if (prob_perm) prob_perm[rows[j]] = prob[t * k + j];
        }
      }
    }
  }
  copy_row_any(x + t * row_bytes, row_bytes, xp, rows, k, lane, unit);
  if (xs) copy_row_any(xs + t * srow_bytes, srow_bytes, xps, rows, k, lane, sunit);
}

// ---------------------------------------------------------------------------
// combine: out[t] = sum_j w[t, j] * y_perm[row_id_map[t*k + j]], float32 sums in slot order
// ---------------------------------------------------------------------------

// KM: an upper bound of k (2, 4, 8 or 16) that sizes the per-slot arrays of the
// batched path, so the registers it holds scale with k; 0: any k, one slot at a time
template <bool kBF16, int VEC, int KM>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y, const int32_t* __restrict__ rmap,
                                                      const float* __restrict__ w, int64_t T, int H, int k,
                                                      void* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int64_t R = T * k;
  const int nchunk = H / VEC;
  if constexpr (KM > 0) {
    // the token's row ids and weights once; per chunk all k loads in flight together
    // (a dropped slot reads row 0 and is left out of the sum), then the sums in slot order
    int32_t rr[KM];
    float ww[KM];
    bool ok[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      const int32_t r = j < k ? rmap[t * k + j] : -1;
      ok[j] = r >= 0 && r < R;
      rr[j] = ok[j] ? r : 0;
      ww[j] = (j < k && w) ? w[t * k + j] : 1.f;
    }
    for (int c = lane; c < nchunk; c += 64) {
      float acc[VEC];
#pragma unroll
      for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
      if constexpr (kBF16 && VEC == 8) {
        uint4 q[KM];
#pragma unroll
        for (int j = 0; j < KM; ++j)
          if (j < k)
            q[j] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(y) + (int64_t)rr[j] * H +
                                                   (int64_t)c * VEC);
#pragma unroll
        for (int j = 0; j < KM; ++j) {
          if (j < k && ok[j]) {
            const uint32_t u[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              acc[2 * v] += ww[j] * bf16_to_f32(u[v] & 0xFFFFu);
              acc[2 * v + 1] += ww[j] * bf16_to_f32(u[v] >> 16);
            }
          }
        }
        uint4 o;
        o.x = pack_bf16x2(acc[0], acc[1]);
        o.y = pack_bf16x2(acc[2], acc[3]);
        o.z = pack_bf16x2(acc[4], acc[5]);
        o.w = pack_bf16x2(acc[6], acc[7]);
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + t * H + (int64_t)c * VEC) = o;
      } else if constexpr (!kBF16 && VEC == 4) {
        float4 q[KM];
#pragma unroll
        for (int j = 0; j < KM; ++j)
          if (j < k)
            q[j] = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(y) + (int64_t)rr[j] * H +
                                                    (int64_t)c * VEC);
#pragma unroll
        for (int j = 0; j < KM; ++j) {
          if (j < k && ok[j]) {
            acc[0] += ww[j] * q[j].x;
            acc[1] += ww[j] * q[j].y;
            acc[2] += ww[j] * q[j].z;
            acc[3] += ww[j] * q[j].w;
          }
        }
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + t * H + (int64_t)c * VEC) =
            make_float4(acc[0], acc[1], acc[2], acc[3]);
      } else {
        float vals[KM][VEC];
#pragma unroll
        for (int j = 0; j < KM; ++j)
          if (j < k)
#pragma unroll
            for (int v = 0; v < VEC; ++v)
              vals[j][v] = kBF16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(y)[(int64_t)rr[j] * H + (int64_t)c * VEC + v])
                                 : reinterpret_cast<const float*>(y)[(int64_t)rr[j] * H + (int64_t)c * VEC + v];
#pragma unroll
        for (int j = 0; j < KM; ++j)
          if (j < k && ok[j])
#pragma unroll
            for (int v = 0; v < VEC; ++v) acc[v] += ww[j] * vals[j][v];
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          if constexpr (kBF16) reinterpret_cast<uint16_t*>(out)[t * H + (int64_t)c * VEC + v] = (uint16_t)f32_to_bf16(acc[v]);
          else reinterpret_cast<float*>(out)[t * H + (int64_t)c * VEC + v] = acc[v];
        }
      }
    }
    return;
  }
  for (int c = lane; c < nchunk; c += 64) {
    float acc[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
    for (int j = 0; j < k; ++j) {
      const int32_t r = rmap[t * k + j];
      if (r < 0 || r >= R) continue;
      const float wt = w ? w[t * k + j] : 1.f;
      if constexpr (kBF16) {
        const uint16_t* src = reinterpret_cast<const uint16_t*>(y) + (int64_t)r * H + (int64_t)c * VEC;
        if constexpr (VEC == 8) {
          uint4 q = *reinterpret_cast<const uint4*>(src);
          uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            acc[2 * v] += wt * bf16_to_f32(u[v] & 0xFFFFu);
            acc[2 * v + 1] += wt * bf16_to_f32(u[v] >> 16);
          }
        } else {
#pragma unroll
          for (int v = 0; v < VEC; ++v) acc[v] += wt * bf16_to_f32(src[v]);
        }
      } else {
        const float* src = reinterpret_cast<const float*>(y) + (int64_t)r * H + (int64_t)c * VEC;
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[v] += wt * src[v];
      }
    }
    if constexpr (kBF16) {
      uint16_t* dst = reinterpret_cast<uint16_t*>(out) + t * H + (int64_t)c * VEC;
      if constexpr (VEC == 8) {
        uint4 q;
        q.x = pack_bf16x2(acc[0], acc[1]);
        q.y = pack_bf16x2(acc[2], acc[3]);
        q.z = pack_bf16x2(acc[4], acc[5]);
        q.w = pack_bf16x2(acc[6], acc[7]);
        *reinterpret_cast<uint4*>(dst) = q;
      } else {
#pragma unroll
        for (int v = 0; v < VEC; ++v) dst[v] = (uint16_t)f32_to_bf16(acc[v]);
      }
    } else {
      float* dst = reinterpret_cast<float*>(out) + t * H + (int64_t)c * VEC;
#pragma unroll
      for (int v = 0; v < VEC; ++v) dst[v] = acc[v];
    }
  }
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_permute(const void* x, const uint8_t* x_scale, moe_dtype dt, int64_t T, int H,
                                  int E, int k, const int32_t* topk_idx, const float* topk_prob,
                                  int reuse_map, void* x_perm, uint8_t* x_perm_scale, float* prob_perm,
                                  int32_t* split_sizes, int32_t* offsets, int32_t* row_id_map,
                                  int32_t* src_token, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  if (T < 0 || H < 1) return fail(MOE_ERR_INVALID_ARG, "moe_permute: T < 0 or H < 1");
  if (E < 1 || E > MOE_MAX_EXPERTS) return fail(MOE_ERR_INVALID_ARG, "moe_permute: E out of [1, 256]");
  if (k < 1 || k > E) return fail(MOE_ERR_INVALID_ARG, "moe_permute: k out of [1, E]");
  if (k > kMaxK) return fail(MOE_ERR_UNSUPPORTED, "moe_permute: k > 16");
  if (dt != MOE_F32 && dt != MOE_BF16 && dt != MOE_MXFP8)
    return fail(MOE_ERR_INVALID_ARG, "moe_permute: bad dtype");
  if (dt == MOE_MXFP8 && H % 32 != 0) return fail(MOE_ERR_INVALID_ARG, "moe_permute: MXFP8 needs H % 32 == 0");
  if (T * (int64_t)k > 0x7FFFFFFF) return fail(MOE_ERR_UNSUPPORTED, "moe_permute: T*k exceeds int32 rows");
  const hipStream_t s = as_stream(stream);
  if (reuse_map) {
    if (T == 0) return MOE_OK;
    if (!x || !x_perm || !row_id_map) return fail(MOE_ERR_INVALID_ARG, "moe_permute(reuse): NULL pointer");
  } else {
    if (!split_sizes || !offsets) return fail(MOE_ERR_INVALID_ARG, "moe_permute: NULL split_sizes/offsets");
    if (T > 0 && (!x || !x_perm || !topk_idx || !row_id_map || !src_token))
      return fail(MOE_ERR_INVALID_ARG, "moe_permute: NULL pointer");
    if (prob_perm && !topk_prob) return fail(MOE_ERR_INVALID_ARG, "moe_permute: prob_perm needs topk_prob");
  }
  if (dt == MOE_MXFP8 && T > 0 && (!x_scale || !x_perm_scale))
    return fail(MOE_ERR_INVALID_ARG, "moe_permute: MXFP8 needs x_scale and x_perm_scale");
  const size_t esz = dt == MOE_F32 ? 4 : dt == MOE_BF16 ? 2 : 1;
  const int64_t row_bytes = (int64_t)H * esz;
  const int64_t srow_bytes = dt == MOE_MXFP8 ? H / 32 : 0;
  const int64_t nb = (T + kPermBlock - 1) / kPermBlock;
  auto pick_unit = [](int64_t bytes, const void* a, const void* b) {
    if (bytes % 16 == 0 && aligned(a, 16) && aligned(b, 16)) return 16;
    if (bytes % 4 == 0 && aligned(a, 4) && aligned(b, 4)) return 4;
    return 1;
  };
  const int unit = pick_unit(row_bytes, x, x_perm);
  const int sunit = dt == MOE_MXFP8 ? pick_unit(srow_bytes, x_scale, x_perm_scale) : 1;

  if (reuse_map) {
    int64_t blocks = (T + 3) / 4;
    hipLaunchKernelGGL(permute_scatter_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       (const uint8_t*)x, row_bytes, dt == MOE_MXFP8 ? x_scale : nullptr, srow_bytes,
                       nullptr, nullptr, nullptr, nullptr, T, E, k, 1, unit, sunit, (uint8_t*)x_perm,
                       dt == MOE_MXFP8 ? x_perm_scale : nullptr, nullptr, (int32_t*)row_id_map, nullptr);
    return check_launch("moe_permute(reuse)");
  }

  const size_t need = permute_workspace_bytes(T, E, k);
  if (workspace_bytes < need) return fail(MOE_ERR_WORKSPACE, "moe_permute: workspace too small");
  if (need > 0 && (!workspace || !aligned(workspace, 256)))
    return fail(MOE_ERR_INVALID_ARG, "moe_permute: workspace NULL or not 256-byte aligned");
  uint8_t* ws = (uint8_t*)workspace;
  int32_t* counts = (int32_t*)ws;
  ws += align_up((size_t)nb * E * 4, 256);
  int32_t* base = (int32_t*)ws;
  ws += align_up((size_t)nb * E * 4, 256);
  int32_t* rank_local = (int32_t*)ws;

  if (T > 0) {
    hipLaunchKernelGGL(permute_count_kernel, dim3((unsigned)nb), dim3(kPermBlock), 0, s, topk_idx, T, E, k,
                       counts, rank_local);
  }
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(256), 0, s, counts, nb, E, base, split_sizes, offsets);
  if (T > 0) {
    int64_t blocks = (T + 3) / 4;
    hipLaunchKernelGGL(permute_scatter_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const uint8_t*)x,
                       row_bytes, dt == MOE_MXFP8 ? x_scale : nullptr, srow_bytes, topk_idx, topk_prob, base,
                       rank_local, T, E, k, 0, unit, sunit, (uint8_t*)x_perm, dt == MOE_MXFP8 ? x_perm_scale : nullptr,
                       prob_perm, row_id_map, src_token);
  }
  return check_launch("moe_permute");
}

extern "C" moe_status moe_unpermute_combine(const void* y_perm, moe_dtype dt, const int32_t* row_id_map,
                                            const float* weights, int64_t T, int H, int k, void* out,
                                            void* stream) {
  if (T < 0 || H < 1 || k < 1) return fail(MOE_ERR_INVALID_ARG, "moe_unpermute_combine: bad T/H/k");
  if (dt != MOE_F32 && dt != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "moe_unpermute_combine: dtype must be F32 or BF16");
  if (T == 0) return MOE_OK;
  if ((T + 3) / 4 > 0x7FFFFFFF) return fail(MOE_ERR_UNSUPPORTED, "moe_unpermute_combine: T too large");
  if (!y_perm || !row_id_map || !out) return fail(MOE_ERR_INVALID_ARG, "moe_unpermute_combine: NULL pointer");
  const hipStream_t s = as_stream(stream);
  const int64_t blocks = (T + 3) / 4;
  // the batched kernel sized for the smallest of 4, 8, 16 slots that holds k (at k <= 2
  // the one-slot-at-a-time loop measured as fast or faster: Mixtral's top-2 combine)
  auto launch = [&](auto BF, auto V) {
    constexpr bool bf = decltype(BF)::value;
    constexpr int vec = decltype(V)::value;
    const dim3 g((unsigned)blocks), b(256);
    if (k <= 2) hipLaunchKernelGGL((combine_kernel<bf, vec, 0>), g, b, 0, s, y_perm, row_id_map, weights, T, H, k, out);
    else if (k <= 4) hipLaunchKernelGGL((combine_kernel<bf, vec, 4>), g, b, 0, s, y_perm, row_id_map, weights, T, H, k, out);
    else if (k <= 8) hipLaunchKernelGGL((combine_kernel<bf, vec, 8>), g, b, 0, s, y_perm, row_id_map, weights, T, H, k, out);
    else if (k <= 16) hipLaunchKernelGGL((combine_kernel<bf, vec, 16>), g, b, 0, s, y_perm, row_id_map, weights, T, H, k, out);
    else hipLaunchKernelGGL((combine_kernel<bf, vec, 0>), g, b, 0, s, y_perm, row_id_map, weights, T, H, k, out);
  };
  using BF16 = std::true_type;
  using F32 = std::false_type;
  if (dt == MOE_BF16) {
    if (H % 8 == 0 && aligned(y_perm, 16) && aligned(out, 16))
      launch(BF16{}, std::integral_constant<int, 8>{});
    else
      hipLaunchKernelGGL((combine_kernel<true, 1, 0>), dim3((unsigned)blocks), dim3(256), 0, s, y_perm, row_id_map,
                         weights, T, H, k, out);
  } else {
    if (H % 4 == 0 && aligned(y_perm, 16) && aligned(out, 16))
      launch(F32{}, std::integral_constant<int, 4>{});
    else
      hipLaunchKernelGGL((combine_kernel<false, 1, 0>), dim3((unsigned)blocks), dim3(256), 0, s, y_perm, row_id_map,
                         weights, T, H, k, out);
  }
  return check_launch("moe_unpermute_combine");
}

// ---------------------------------------------------------------------------
// Allocation-free permutation: the count/scan scratch lives in a static device array
// ---------------------------------------------------------------------------

namespace moe {
namespace {

constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
constexpr int kMaxDevices = 64;

// One copy per GPU, held until the process ends. In host code this name is only a
// stand-in for the symbol: kernels get the device address that hipGetSymbolAddress
// returns for the current device.
__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

// Device address of `scratch` on the current device, looked up once per device.
moe_status scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_LAUNCH, "moe_permute_noalloc: no current device (or device index >= 64)");
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOE_ERR_LAUNCH, std::string("moe_permute_noalloc: hipGetSymbolAddress failed: ") + hipGetErrorString(e));
    addr[dev] = p;
  }
  *out = addr[dev];
  return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" moe_status moe_permute_noalloc(const void* x, const uint8_t* x_scale, moe_dtype dt, int64_t T, int H,
                                          int E, int k, const int32_t* topk_idx, const float* topk_prob,
                                          int reuse_map, void* x_perm, uint8_t* x_perm_scale, float* prob_perm,
                                          int32_t* split_sizes, int32_t* offsets, int32_t* row_id_map,
                                          int32_t* src_token, void* stream) {
  if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > E)
    return fail(MOE_ERR_INVALID_ARG, "moe_permute_noalloc: T < 0, E out of [1, 256] or k out of [1, E]");
  if (!reuse_map) {
    const size_t need = permute_workspace_bytes(T, E, k);
    if (need > kNoAllocScratchBytes)
      return fail(MOE_ERR_UNSUPPORTED, "moe_permute_noalloc: T = " + std::to_string(T) + ", E = " + std::to_string(E) +
                                           ", k = " + std::to_string(k) + " need " + std::to_string(need) +
                                           " bytes of scratch, more than the 8 MiB static area");
  }
  void* ws = nullptr;
  if (!reuse_map && T > 0) {
    const moe_status st = scratch_address(&ws);
    if (st != MOE_OK) return st;
  }
  return moe_permute(x, x_scale, dt, T, H, E, k, topk_idx, topk_prob, reuse_map, x_perm, x_perm_scale, prob_perm,
                     split_sizes, offsets, row_id_map, src_token, ws, ws ? kNoAllocScratchBytes : 0, stream);
}
