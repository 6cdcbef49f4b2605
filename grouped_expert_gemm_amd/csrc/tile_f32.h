// Float32 matrix-core tiles: a 64 x 64 output tile of C = A B computed by four
// wavefronts of 32 x 32 with v_mfma_f32_32x32x2f32 (float32 products and sums), K in
// steps of 32 staged through LDS. Operands are strided views of float32 or bf16 data
// (bf16 widened exactly on the way into LDS), every load bounds-checked. Staging is
// single-buffered: enough for the float32 grouped MLP's small sizes.
#pragma once

#include "common.h"

namespace moe {
namespace tf32 {

constexpr int kT = 64;       // output tile edge
constexpr int kKS = 32;      // K per LDS stage
constexpr int kLd = kT + 1;  // LDS row pitch (floats): k-fastest writes fall in distinct banks
constexpr int kStage = kKS * kLd;  // floats of one staged operand block

__device__ __forceinline__ float widen(float v) { return v; }
__device__ __forceinline__ float widen(bf16_t v) { return bf16_to_f32(v); }

// Strided view of an operand: element (i, k) at p[i * si + k * sk], valid for i < ni,
// k < nk (zero outside).
template <typename T>
struct View {
  const T* p;
  int64_t si, sk;
  int ni, nk;
};

// Stage a 64 x 32 block (rows i 0..63, k0 .. k0+31) of v into LDS as s[k][i]. Threads
// run along whichever of i and k is contiguous in memory.
template <typename T>
__device__ __forceinline__ void stage(const View<T>& v, int k0, float* s, int tid) {
  const bool kfast = v.sk == 1;
#pragma unroll
  for (int j = 0; j < (kT * kKS) / 256; ++j) {
    const int idx = tid + 256 * j;
    const int i = kfast ? idx / kKS : idx % kT;
    const int k = kfast ? idx % kKS : idx / kT;
    float x = 0.f;
    if (i < v.ni && k0 + k < v.nk) x = widen(v.p[(int64_t)i * v.si + (int64_t)(k0 + k) * v.sk]);
    s[k * kLd + i] = x;
  }
}

// acc[b] = A (64 x K) times B_b (K x 64) for NB operands B sharing A (K = a.nk); the
// wavefront (wm, wn) holds the 32 x 32 block at rows 32 wm, columns 32 wn, in the
// matrix-core layout: lane l, register v is row 8 (v / 4) + 4 (l / 32) + v % 4, column
// l % 32. sB holds NB staged blocks.
template <int NB, typename TA, typename TB>
__device__ __forceinline__ void tile_product(const View<TA>& a, const View<TB> (&b)[NB], f32x16 (&acc)[NB],
                                             float* sA, float* sB, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int x = 0; x < NB; ++x)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[x][v] = 0.f;
  for (int k0 = 0; k0 < a.nk; k0 += kKS) {
    __syncthreads();  // the previous stage's reads are done
    stage(a, k0, sA, tid);
#pragma unroll
    for (int x = 0; x < NB; ++x) stage(b[x], k0, sB + x * kStage, tid);
    __syncthreads();
    // one k pair per instruction: lane l supplies k = kp + l / 32 of row / column l % 32
#pragma unroll
    for (int kp = 0; kp < kKS; kp += 2) {
      const int k = kp + (lane >> 5);
      const float av = sA[k * kLd + wm * 32 + (lane & 31)];
#pragma unroll
      for (int x = 0; x < NB; ++x) {
        const float bv = sB[x * kStage + k * kLd + wn * 32 + (lane & 31)];
        acc[x] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc[x], 0, 0, 0);
      }
    }
  }
}

// Calls f(row, col, v) for this lane's outputs of the tile that fall inside (m, n).
template <typename F>
__device__ __forceinline__ void for_outputs(int tid, int m, int n, F&& f) {
  const int lane = tid & 63, wave = tid >> 6;
  const int col = (wave & 1) * 32 + (lane & 31);
  if (col >= n) return;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int row = (wave >> 1) * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    if (row < m) f(row, col, v);
  }
}

}  // namespace tf32
}  // namespace moe
