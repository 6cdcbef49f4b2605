// Parameters of the persistent grouped GEMM kernels (bf16 MFMA).
#pragma once

#include <string>

#include "common.h"

namespace moe {
namespace gemm {

constexpr int kBM = 256, kBN = 256, kBK = 32;
constexpr int kStages = 4;                    // LDS ring depth
constexpr int kTileBytes = 256 * kBK * 2;     // one operand, one stage (16 KiB)
constexpr int kStageBytes = 2 * kTileBytes;   // P and Q
constexpr int kLdsBytes = kStages * kStageBytes;

enum { KCONTIG = 0, MNCONTIG = 1 };
enum { GROUP_M = 0, GROUP_K = 1 };
enum { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_DSWIGLU = 2 };

struct Params {
  // GROUP_M: per-expert P operand (weights). GROUP_K: per-expert output C.
  const void* tab[MOE_MAX_EXPERTS];
  const bf16_t* p;        // P operand when it is a token tensor (GROUP_K)
  const bf16_t* q;        // Q operand (token rows)
  bf16_t* c;              // output (GROUP_M)
  const int32_t* offsets; // [E+1] expert row offsets
  const float* prob;      // SWIGLU / DSWIGLU: routing weight per row
  const bf16_t* zin;      // DSWIGLU: saved gate_up output [R, 2I]
  bf16_t* zout;           // SWIGLU: gate_up output to save [R, 2I] (or NULL)
  float* part;            // DSWIGLU: dprob partial sums [2 * n_tiles][R]
  int64_t p_ld, q_ld, c_ld;
  int64_t R;
  int M, N, K;            // GROUP_M uses N, K; GROUP_K uses M, N
  int E, I;
  int n_tiles;            // output column tiles (SWIGLU: I / 128, else N / 256)
  // split-K tail (forward kernel): when the last round of tiles would leave at least
  // half the CUs idle, its tiles are cut into K chunks whose float32 partial tiles go
  // to `tail` (tail_cap of them at most; 0 = never split) and are finished by
  // run_tail_reduce; tail_meta holds [n_tail, split, first_tail, 0] then per tail
  // tile [first_row, row_end, column_tile, 0].
  float* tail;
  int32_t* tail_meta;
  int tail_cap;
};

constexpr size_t kTailTileBytes = (size_t)kBM * kBN * 4;  // one float32 partial tile
constexpr size_t kTailMetaSpace = 8192;                   // header + up to 511 tail tiles
// bytes of a split-K tail area (meta, then `units` partial tiles)
inline size_t tail_ws_bytes(int units) { return kTailMetaSpace + (size_t)units * kTailTileBytes; }

moe_status run(const Params& p, int pl, int ql, int g, int ep, int64_t max_tiles, hipStream_t s,
               const char* what);
// forward kernel (gemm_fwd.hip): GROUP_M, both operands KCONTIG, EPI_STORE or EPI_SWIGLU,
// K a multiple of 64
moe_status run_fwd(const Params& p, int ep, int64_t max_tiles, hipStream_t s, const char* what);
// sums the split-K partial tiles that run_fwd left in p.tail and applies the epilogue
moe_status run_tail_reduce(const Params& p, int ep, int64_t max_tiles, hipStream_t s, const char* what);

}  // namespace gemm
}  // namespace moe
