// MXFP8 grouped MLP forward on gfx950's MX-scaled fp8 MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4: E4M3 operands, one E8M0 scale per 32 K values).
//
// Source: "Efficient MoE Training for Biological Foundation Models", Challenge 2 (MXFP8:
// one scaling factor per 32 consecutive values, 8-bit values, dedicated low-precision
// GEMM instructions) and Challenge 3 / Figure 4 (bf16 master weights and activations
// quantised before the GEMMs; SwiGLU, the routing-probability scaling and the
// quantisation of h fused into one kernel before the down projection).
//
// The kernel reuses the bf16 kernel's machinery: 256 x 256 tiles, 4 wavefronts of
// 128 x 128, a 4-slot LDS ring filled by global -> LDS copies four K steps ahead, a
// barrier in the middle of each step. One K step is 64 fp8 values = 64 bytes per row,
// the same bytes as a bf16 step, so the LDS layout, swizzle and copy code are shared.
// MFMA operand layout (measured): lane l holds row l % 32 and, for g = l / 32, the K
// values [16g, 16g + 16) in bytes 0..15 and [32 + 16g, 32 + 16g + 16) in bytes 16..31
// -- the two 16-byte chunks a bf16 step reads as its two k16 slices -- and supplies
// the E8M0 scale of K block g (values [32g, 32g + 32)) of its row.
// Scales: per 4-step group each lane loads 8 bytes (blocks 8g..8g+7) of its row per
// sub-tile and packs the 4 bytes of its own K half (block 2j + (l / 32) of step j) into
// one word, so step j's MFMA selects byte j with op_sel, a compile-time immediate.
#include <cstring>
#include <type_traits>

#include "common.h"
#include "gemm_common.h"
#include "gemm_mx.h"
#include "internal.h"

namespace moe {
namespace mx {

using namespace gemm;

constexpr int kMaxE = 128;   // experts per MXFP8 call (two pointer tables in the kernel arguments)
constexpr int kBM = 256, kBN = 256, kStepK = 64;
constexpr int kTileBytes = 256 * kStepK;   // 16 KiB: one operand, one slot

enum { MX_STORE = 0, MX_SWIGLU = 1 };

struct MxParams {
  const uint8_t* tab[kMaxE];     // per-expert P codes [N][K]
  const uint8_t* tab_s[kMaxE];   // per-expert P scales [N][K/32]; per-tensor mode: the expert's float32 scale
  const uint8_t* q;              // Q codes [R][K]
  const uint8_t* q_s;            // Q scales [R][K/32]; per-tensor mode: one float32 scale
  void* c;                       // STORE: bf16 [R][N]; SWIGLU: h codes [R][I] (per-tensor mode: h bf16)
  uint8_t* c_s;                  // SWIGLU: h scales [R][I/32]; per-tensor mode: h's amax word (float bits)
  const int32_t* offsets;
  const float* prob;
  int64_t R;
  int K, N, E, I, n_tiles;
};

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

// PT = false: MX block scales (E8M0 per 32 K values of every row of both operands).
// PT = true: per-tensor FP8; the MFMA runs with unit block scales, the products are
// scaled by (Q's scale x the expert's P scale) in the epilogue, and the SwiGLU
// epilogue writes h in bf16 and raises h's amax word (its scale needs all of h).
template <int EP, bool PT>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void grouped_gemm_mx_kernel(const MxParams prm) {
  __shared__ __attribute__((aligned(1024))) uint8_t sP0[kTileBytes], sP1[kTileBytes], sP2[kTileBytes], sP3[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sQ0[kTileBytes], sQ1[kTileBytes], sQ2[kTileBytes], sQ3[kTileBytes];
  __shared__ int32_t s_off[kMaxE + 1];
  __shared__ int32_t s_tstart[kMaxE + 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int E = prm.E;
  const int l32 = lane & 31, lhi = lane >> 5;

  for (int e = tid; e <= E; e += 256) s_off[e] = prm.offsets[e];
  __syncthreads();
  if (tid == 0) {  // nondecreasing offsets inside [0, R]; per-expert tile starts
    int prev = 0, run = 0;
    for (int e = 0; e <= E; ++e) {
      int v = s_off[e];
      v = v < prev ? prev : v;
      v = v > (int)prm.R ? (int)prm.R : v;
      s_off[e] = v;
      prev = v;
    }
    s_off[0] = 0;
    for (int e = 0; e < E; ++e) {
      s_tstart[e] = run;
      run += ((s_off[e + 1] - s_off[e] + kBM - 1) / kBM) * prm.n_tiles;
    }
    s_tstart[E] = run;
  }
  __syncthreads();
  const int total = s_tstart[E];
  const int nwg = gridDim.x;
  const int logical = (nwg % 8 == 0) ? (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8 : blockIdx.x;

  auto slotP = [&](auto S) -> uint8_t* {
    if constexpr (S.value == 0) return sP0;
    else if constexpr (S.value == 1) return sP1;
    else if constexpr (S.value == 2) return sP2;
    else return sP3;
  };
  auto slotQ = [&](auto S) -> uint8_t* {
    if constexpr (S.value == 0) return sQ0;
    else if constexpr (S.value == 1) return sQ1;
    else if constexpr (S.value == 2) return sQ2;
    else return sQ3;
  };

  const int nk = prm.K / kStepK;  // a multiple of 4 (K % 256 == 0)
  const int64_t kscale = prm.K / 32;

  for (int t = logical; t < total; t += nwg) {
    int lo = 0, hi = E;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_tstart[mid] <= t) lo = mid; else hi = mid - 1;
    }
    int e = lo;
    const int me = s_off[e + 1] - s_off[e];
    const int mte = (me + kBM - 1) / kBM;
    const int local = t - s_tstart[e];
    int mt = local % mte;
    int nt = local / mte;
    e = __builtin_amdgcn_readfirstlane(e);
    mt = __builtin_amdgcn_readfirstlane(mt);
    nt = __builtin_amdgcn_readfirstlane(nt);
    const int row_beg = __builtin_amdgcn_readfirstlane(s_off[e]);
    const int row_end = __builtin_amdgcn_readfirstlane(s_off[e + 1]);
    const int tile_row = row_beg + mt * kBM;

    // P row of local tile row r (SWIGLU: gate rows then up rows of the same columns)
    auto p_row = [&](int r) -> int {
      if constexpr (EP == MX_SWIGLU) return (r < 128) ? nt * 128 + r : prm.I + nt * 128 + (r - 128);
      else return nt * kBN + r;
    };
    auto q_row = [&](int r) -> int {
      const int row = tile_row + r;
      return row < row_end ? row : row_end - 1;  // rows past the expert: any valid row, discarded
    };

    // ---- copies: identical lane mapping to the bf16 kernel (64-byte rows) ----
    const int dma_row0 = wave * 16 + (lane >> 2);
    const uint8_t* pbase = prm.tab[e];
    uint32_t p_off[4], q_off[4];
    const uint8_t* q_tile = prm.q + (int64_t)tile_row * prm.K;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = i * 64 + dma_row0;
      const int chunk = (lane & 3) ^ swz(r);
      p_off[i] = (uint32_t)((int64_t)p_row(r) * prm.K + chunk * 16);
      q_off[i] = (uint32_t)((int64_t)(q_row(r) - tile_row) * prm.K + chunk * 16);
    }
    auto issue_dma = [&](int kt, auto S) {
      const int64_t k0 = (int64_t)kt * kStepK;
      uint8_t* P = slotP(S) + wave * 1024;
      uint8_t* Q = slotQ(S) + wave * 1024;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(pbase + k0 + p_off[i]), (lds_ptr_t)(P + i * 4096), 16, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(q_tile + k0 + q_off[i]), (lds_ptr_t)(Q + i * 4096), 16, 0, 0);
    };
    constexpr int kDma = 8;

    // ---- scales: per sub-tile, this lane's row; 8 bytes per 4-step group ----
    const uint8_t* ps_base = prm.tab_s[e];
    const uint8_t* qs_base = prm.q_s + (int64_t)tile_row * kscale;
    uint32_t ps_off[4], qs_off[4];
#pragma unroll
    for (int t2 = 0; t2 < 4; ++t2) {
      ps_off[t2] = (uint32_t)((int64_t)p_row(sub_n(t2, wn) + l32) * kscale);
      qs_off[t2] = (uint32_t)((int64_t)(q_row(wm * 128 + t2 * 32 + l32) - tile_row) * kscale);
    }
    uint2 scl_next[8];
    uint32_t sP[4], sQ[4];  // [sub-tile]: byte j = this lane's scale for step j of the group
    auto load_scales = [&](int g) {
      if constexpr (PT) return;
#pragma unroll
      for (int t2 = 0; t2 < 4; ++t2) {
        scl_next[t2] = *reinterpret_cast<const uint2*>(ps_base + ps_off[t2] + g * 8);
        scl_next[4 + t2] = *reinterpret_cast<const uint2*>(qs_base + qs_off[t2] + g * 8);
      }
    };
    auto take_scales = [&]() {
      if constexpr (PT) {
#pragma unroll
        for (int t2 = 0; t2 < 4; ++t2) sP[t2] = sQ[t2] = 0x7F7F7F7Fu;   // E8M0 127 = 1.0
        return;
      }
#pragma unroll
      for (int t2 = 0; t2 < 8; ++t2) {
        const uint64_t raw = ((uint64_t)scl_next[t2].y << 32 | scl_next[t2].x) >> (8 * lhi);
        const uint32_t packed = __builtin_amdgcn_perm((uint32_t)(raw >> 32), (uint32_t)raw, 0x06040200u);
        if (t2 < 4) sP[t2] = packed; else sQ[t2 - 4] = packed;
      }
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;

    const uint32_t fragP = (uint32_t)((wn * 64 + l32) * 64);
    const uint32_t fragQ = (uint32_t)((wm * 128 + l32) * 64);
    const uint32_t ck0 = (uint32_t)(((0 + lhi) ^ swz(l32)) << 4);
    const uint32_t ck1 = (uint32_t)(((2 + lhi) ^ swz(l32)) << 4);
    auto rd = [&](const uint8_t* base, int row) -> i32x8_t {
      const i32x4_t a = *reinterpret_cast<const i32x4_t*>(base + row * 64 + ck0);
      const i32x4_t b = *reinterpret_cast<const i32x4_t*>(base + row * 64 + ck1);
      return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    i32x8_t QA[4], QB[4], P01[2], P23[2];

    // prologue
    load_scales(0);
    issue_dma(0, S0{});
    if (nk > 1) issue_dma(1, S1{});
    if (nk > 2) issue_dma(2, S2{});
    if (nk > 3) issue_dma(3, S3{});
    wait_vm_le(((nk > 1) + (nk > 2) + (nk > 3)) * kDma);
    take_scales();
    lds_barrier();
    {
      const uint8_t* P = sP0 + fragP;
      const uint8_t* Qb = sQ0 + fragQ;
#pragma unroll
      for (int t2 = 0; t2 < 4; ++t2) QA[t2] = rd(Qb, t2 * 32);
      P01[0] = rd(P, 0);
      P01[1] = rd(P, 32);
    }

    // step kt on slot S (j = kt % 4 = S). On entry Q and P01 hold this step's Q
    // fragments and P sub-tiles 0-1; Q alternates between two register sets by step
    // parity, so every fragment register is written once and read once per step.
    //   phase A: MFMAs of P 0-1 while P 2-3 are read; wait for step kt+1; barrier;
    //   phase B: copies of step kt+4 into slot S (free now), the next group's scales,
    //            the next step's P 0-1 and Q fragments (into the other Q set), threaded
    //            through the MFMAs of P 2-3.
    auto kstep = [&](int kt, auto S, auto FULL) {
      constexpr int j = decltype(S)::value;
      constexpr bool full = decltype(FULL)::value;
      // this step's Q fragments: QA on even steps, QB on odd; the next step's go to the other
      auto& Q = [&]() -> i32x8_t (&)[4] { if constexpr (j & 1) return QB; else return QA; }();
      auto& QN = [&]() -> i32x8_t (&)[4] { if constexpr (j & 1) return QA; else return QB; }();
      using SN = std::integral_constant<int, (j + 1) & 3>;
      {
        const uint8_t* P = slotP(S) + fragP;
        P23[0] = rd(P, 128);
        P23[1] = rd(P, 128 + 32);
      }
#pragma unroll
      for (int sm = 0; sm < 4; ++sm)
#pragma unroll
        for (int sn = 0; sn < 2; ++sn)
          acc[sn][sm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(P01[sn], Q[sm], acc[sn][sm], 0, 0, j,
                                                                          (int)sP[sn], j, (int)sQ[sm]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
      // wait for step kt+1's copies (and, at the group's last step, the next group's
      // scales); loads complete in issue order
      if constexpr (full) {
        wait_vm_le((!PT && (j == 1 || j == 2)) ? 2 * kDma + 8 : 2 * kDma);
      } else {
        wait_vm_le(((kt + 2 < nk) + (kt + 3 < nk)) * kDma);
      }
      lds_barrier();
      if (full || kt + 4 < nk) issue_dma(kt + 4, S);
      if constexpr (j == 0) {
        if (full || kt + 4 < nk) load_scales((kt >> 2) + 1);
      }
      const bool next = full || kt + 1 < nk;
      const uint8_t* Pn = slotP(SN{}) + fragP;
      const uint8_t* Qn = slotQ(SN{}) + fragQ;
      if (next) {
        P01[0] = rd(Pn, 0);
        P01[1] = rd(Pn, 32);
      }
#pragma unroll
      for (int sm = 0; sm < 4; ++sm) {
#pragma unroll
        for (int sn = 2; sn < 4; ++sn)
          acc[sn][sm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(P23[sn - 2], Q[sm], acc[sn][sm], 0, 0, j,
                                                                          (int)sP[sn], j, (int)sQ[sm]);
        if (next) QN[sm] = rd(Qn, sm * 32);
      }
      if constexpr (full) {
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
      }
      if constexpr (j == 3) {
        if (next) take_scales();
      }
    };
    using Full = std::true_type;
    using Tail = std::false_type;
    int kt = 0;
    for (; kt + 7 < nk; kt += 4) {
      kstep(kt, S0{}, Full{});
      kstep(kt + 1, S1{}, Full{});
      kstep(kt + 2, S2{}, Full{});
      kstep(kt + 3, S3{}, Full{});
    }
    for (; kt < nk; kt += 4) {
      kstep(kt, S0{}, Tail{});
      kstep(kt + 1, S1{}, Tail{});
      kstep(kt + 2, S2{}, Tail{});
      kstep(kt + 3, S3{}, Tail{});
    }
    lds_barrier();

    // ---------------- epilogue ----------------
    // per-tensor mode: the product of the two tensors' scales
    const float alpha = PT ? *reinterpret_cast<const float*>(prm.q_s) * *reinterpret_cast<const float*>(prm.tab_s[e])
                           : 1.f;
    float hmax = 0.f;   // per-tensor SwiGLU: max |h| of this lane's values
#pragma unroll
    for (int sm = 0; sm < 4; ++sm) {
      const int64_t mg = (int64_t)tile_row + wm * 128 + sm * 32 + l32;
      const bool valid = mg < row_end;
      if constexpr (EP == MX_STORE) {
        if (valid) {
          bf16_t* C = reinterpret_cast<bf16_t*>(prm.c) + mg * prm.N;
#pragma unroll
          for (int sn = 0; sn < 4; ++sn)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              const int64_t col = (int64_t)nt * kBN + sub_n(sn, wn) + i4 * 8 + lhi * 4;
              *reinterpret_cast<uint2*>(C + col) =
                  make_uint2(pack_bf16x2(acc[sn][sm][i4 * 4 + 0] * alpha, acc[sn][sm][i4 * 4 + 1] * alpha),
                             pack_bf16x2(acc[sn][sm][i4 * 4 + 2] * alpha, acc[sn][sm][i4 * 4 + 3] * alpha));
            }
        }
      } else if constexpr (PT) {
        const float p = valid ? prm.prob[mg] : 0.f;
#pragma unroll
        for (int sn = 0; sn < 2; ++sn) {
          const int64_t col0 = (int64_t)nt * 128 + wn * 64 + sn * 32;
          float h[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            h[i] = silu_f(acc[sn][sm][i] * alpha) * (acc[sn + 2][sm][i] * alpha) * p;
            hmax = fmaxf(hmax, fabsf(h[i]));
          }
          if (valid) {
            bf16_t* C = reinterpret_cast<bf16_t*>(prm.c) + mg * prm.I + col0;
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4)
              *reinterpret_cast<uint2*>(C + i4 * 8 + lhi * 4) =
                  make_uint2(pack_bf16x2(h[i4 * 4 + 0], h[i4 * 4 + 1]), pack_bf16x2(h[i4 * 4 + 2], h[i4 * 4 + 3]));
          }
        }
      } else {
        const float p = valid ? prm.prob[mg] : 0.f;
#pragma unroll
        for (int sn = 0; sn < 2; ++sn) {
          // h for the 32-column block of sub-tile sn: 16 values here, 16 in lane ^ 32
          float h[16];
          float amax = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            h[i] = silu_f(acc[sn][sm][i]) * acc[sn + 2][sm][i] * p;
            amax = fmaxf(amax, fabsf(h[i]));
          }
          amax = fmaxf(amax, __shfl_xor(amax, 32));
          const int sx = mx_scale_exponent(amax);
          const int64_t col0 = (int64_t)nt * 128 + wn * 64 + sn * 32;
          if (valid) {
            uint8_t* C = reinterpret_cast<uint8_t*>(prm.c) + mg * prm.I + col0;
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              uint32_t wv = 0;
#pragma unroll
              for (int v = 0; v < 4; ++v) wv |= e4m3_encode(ldexpf(h[i4 * 4 + v], -sx)) << (8 * v);
              *reinterpret_cast<uint32_t*>(C + i4 * 8 + lhi * 4) = wv;
            }
            if (lhi == 0) prm.c_s[mg * (prm.I / 32) + col0 / 32] = (uint8_t)(sx + 127);
          }
        }
      }
    }
    if constexpr (PT && EP == MX_SWIGLU) {
      // h is stored in bf16, and rounding is monotone: the maximum of the stored
      // magnitudes is the rounded maximum of the float32 ones
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) hmax = fmaxf(hmax, __shfl_xor(hmax, off));
      if (lane == 0 && hmax > 0.f)
        atomicMax(reinterpret_cast<uint32_t*>(prm.c_s), f32_to_bf16(hmax) << 16);
    }
  }
}

static moe_status launch(int ep, bool pt, const MxParams& p, int64_t max_tiles, hipStream_t s, const char* what) {
  if (max_tiles <= 0) return MOE_OK;
  int64_t grid = num_cus();
  if (max_tiles < grid) grid = max_tiles;
  const dim3 g((unsigned)grid), b(256);
  if (ep == MX_SWIGLU && !pt) hipLaunchKernelGGL((grouped_gemm_mx_kernel<MX_SWIGLU, false>), g, b, 0, s, p);
  else if (ep == MX_SWIGLU) hipLaunchKernelGGL((grouped_gemm_mx_kernel<MX_SWIGLU, true>), g, b, 0, s, p);
  else if (!pt) hipLaunchKernelGGL((grouped_gemm_mx_kernel<MX_STORE, false>), g, b, 0, s, p);
  else hipLaunchKernelGGL((grouped_gemm_mx_kernel<MX_STORE, true>), g, b, 0, s, p);
  return check_launch(what);
}

static moe_status check_mx_shape(int E, int H, int I, const char* what) {
  if (E > kMaxE) return fail(MOE_ERR_UNSUPPORTED, std::string(what) + ": MXFP8 supports at most 128 experts");
  if (H % 256 != 0 || I % 256 != 0)
    return fail(MOE_ERR_UNSUPPORTED, std::string(what) + ": MXFP8 kernels need H % 256 == 0 and I % 256 == 0");
  return MOE_OK;
}

moe_status gate_up(int E, int64_t R, int H, int I, const uint8_t* x, const uint8_t* x_scale, const void* const* w,
                   const uint8_t* const* w_scale, const int32_t* offsets, const float* prob, uint8_t* h,
                   uint8_t* h_scale, hipStream_t s) {
  moe_status st = check_mx_shape(E, H, I, "moe_grouped_gate_up_swiglu");
  if (st != MOE_OK) return st;
  MxParams p;
  std::memset(&p, 0, sizeof(p));
  for (int e = 0; e < E; ++e) {
    p.tab[e] = reinterpret_cast<const uint8_t*>(w[e]);
    p.tab_s[e] = w_scale[e];
  }
  p.q = x;
  p.q_s = x_scale;
  p.c = h;
  p.c_s = h_scale;
  p.offsets = offsets;
  p.prob = prob;
  p.R = R;
  p.K = H;
  p.N = 2 * I;
  p.E = E;
  p.I = I;
  p.n_tiles = I / 128;
  const int64_t mtiles = (R + kBM - 1) / kBM + E;
  return launch(MX_SWIGLU, false, p, mtiles * p.n_tiles, s, "MXFP8 gate_up + ScaledSwiGLU");
}

static moe_status down(int E, int64_t R, int H, int I, const uint8_t* h, const uint8_t* h_scale,
                       const uint8_t* const* w, const uint8_t* const* w_scale, const int32_t* offsets, void* y,
                       hipStream_t s) {
  MxParams p;
  std::memset(&p, 0, sizeof(p));
  for (int e = 0; e < E; ++e) {
    p.tab[e] = w[e];
    p.tab_s[e] = w_scale[e];
  }
  p.q = h;
  p.q_s = h_scale;
  p.c = y;
  p.offsets = offsets;
  p.R = R;
  p.K = I;
  p.N = H;
  p.E = E;
  p.I = I;
  p.n_tiles = H / kBN;
  const int64_t mtiles = (R + kBM - 1) / kBM + E;
  return launch(MX_STORE, false, p, mtiles * p.n_tiles, s, "MXFP8 down");
}

static size_t a256(size_t x) { return align_up(x, 256); }

moe_status forward(const moe_mlp_desc& d, int64_t R, const void* x_perm, const uint8_t* x_perm_scale,
                   const void* const* w_gate_up, const void* const* w_down, const uint8_t* const* w_gate_up_scale,
                   const uint8_t* const* w_down_scale, const int32_t* offsets, const float* prob_perm,
                   void* y_perm, uint8_t* ws, hipStream_t s) {
  const int E = d.E, H = d.H, I = d.I;
  moe_status st = check_mx_shape(E, H, I, "moe_grouped_mlp_fwd");
  if (st != MOE_OK) return st;
  // activations: quantised in the call when given as bf16
  const uint8_t* xq = reinterpret_cast<const uint8_t*>(x_perm);
  const uint8_t* xs = x_perm_scale;
  if (d.act == MOE_BF16) {
    uint8_t* q = ws;
    ws += a256((size_t)R * H);
    uint8_t* qs = ws;
    ws += a256((size_t)R * H / 32);
    if ((st = launch_mxfp8_quantize(x_perm, R, H, q, qs, s)) != MOE_OK) return st;
    xq = q;
    xs = qs;
  }
  // weights: bf16 master weights quantised in the call, or given as MXFP8
  const uint8_t* w1q[kMaxE];
  const uint8_t* w1s[kMaxE];
  const uint8_t* w2q[kMaxE];
  const uint8_t* w2s[kMaxE];
  for (int e = 0; e < E; ++e) {
    if (d.wt == MOE_BF16) {
      uint8_t* a = ws;
      ws += a256((size_t)2 * I * H);
      uint8_t* as = ws;
      ws += a256((size_t)2 * I * H / 32);
      uint8_t* b = ws;
      ws += a256((size_t)H * I);
      uint8_t* bs = ws;
      ws += a256((size_t)H * I / 32);
      if ((st = launch_mxfp8_quantize(w_gate_up[e], 2 * I, H, a, as, s)) != MOE_OK) return st;
      if ((st = launch_mxfp8_quantize(w_down[e], H, I, b, bs, s)) != MOE_OK) return st;
      w1q[e] = a;
      w1s[e] = as;
      w2q[e] = b;
      w2s[e] = bs;
    } else {
      w1q[e] = reinterpret_cast<const uint8_t*>(w_gate_up[e]);
      w1s[e] = w_gate_up_scale[e];
      w2q[e] = reinterpret_cast<const uint8_t*>(w_down[e]);
      w2s[e] = w_down_scale[e];
    }
  }
  uint8_t* hq = ws;
  ws += a256((size_t)R * I);
  uint8_t* hs = ws;
  st = gate_up(E, R, H, I, xq, xs, reinterpret_cast<const void* const*>(w1q), w1s, offsets, prob_perm, hq, hs, s);
  if (st != MOE_OK) return st;
  return down(E, R, H, I, hq, hs, w2q, w2s, offsets, y_perm, s);
}

// Per-tensor FP8 forward. Workspace: scale words [x, W1 of each expert, W2 of each
// expert, h], then the codes of whatever is given in bf16, then h in bf16 and its codes.
size_t fp8_tensor_workspace_bytes(const moe_mlp_desc& d, int64_t R) {
  const size_t I = d.I, H = d.H, E = d.E;
  size_t b = a256((2 + 2 * E) * 4);
  if (d.act == MOE_BF16) b += a256(R * H);
  if (d.wt == MOE_BF16) b += E * (a256(2 * I * H) + a256(H * I));
  return b + a256(R * I * 2) + a256(R * I);
}

moe_status forward_fp8_tensor(const moe_mlp_desc& d, int64_t R, const void* x_perm, const float* x_scale,
                              const void* const* w_gate_up, const void* const* w_down, const float* const* w_gate_up_scale,
                              const float* const* w_down_scale, const int32_t* offsets, const float* prob_perm,
                              void* y_perm, uint8_t* ws, hipStream_t s) {
  const int E = d.E, H = d.H, I = d.I;
  moe_status st = check_mx_shape(E, H, I, "moe_grouped_mlp_fwd");
  if (st != MOE_OK) return st;
  float* words = reinterpret_cast<float*>(ws);
  ws += a256((2 + 2 * (size_t)E) * 4);
  float* w1_word = words + 1;
  float* w2_word = words + 1 + E;
  float* h_word = words + 1 + 2 * E;
  if ((st = fp8t_zero(words, 2 + 2 * E, s)) != MOE_OK) return st;

  const uint8_t* xq = reinterpret_cast<const uint8_t*>(x_perm);
  const float* xs = x_scale;
  if (d.act == MOE_BF16) {
    uint8_t* q = ws;
    ws += a256((size_t)R * H);
    const void* in[1] = {x_perm};
    uint8_t* out[1] = {q};
    if ((st = fp8t_amax(in, 1, R * H, words, s)) != MOE_OK) return st;
    if ((st = fp8t_quantize(in, out, 1, R * H, words, s)) != MOE_OK) return st;
    xq = q;
    xs = words;
  }
  MxParams g, dn;
  std::memset(&g, 0, sizeof(g));
  std::memset(&dn, 0, sizeof(dn));
  if (d.wt == MOE_BF16) {
    uint8_t* q1[kMaxE];
    uint8_t* q2[kMaxE];
    for (int e = 0; e < E; ++e) {
      q1[e] = ws;
      ws += a256((size_t)2 * I * H);
      q2[e] = ws;
      ws += a256((size_t)H * I);
    }
    if ((st = fp8t_amax(w_gate_up, E, (int64_t)2 * I * H, w1_word, s)) != MOE_OK) return st;
    if ((st = fp8t_quantize(w_gate_up, q1, E, (int64_t)2 * I * H, w1_word, s)) != MOE_OK) return st;
    if ((st = fp8t_amax(w_down, E, (int64_t)H * I, w2_word, s)) != MOE_OK) return st;
    if ((st = fp8t_quantize(w_down, q2, E, (int64_t)H * I, w2_word, s)) != MOE_OK) return st;
    for (int e = 0; e < E; ++e) {
      g.tab[e] = q1[e];
      g.tab_s[e] = reinterpret_cast<const uint8_t*>(w1_word + e);
      dn.tab[e] = q2[e];
      dn.tab_s[e] = reinterpret_cast<const uint8_t*>(w2_word + e);
    }
  } else {
    for (int e = 0; e < E; ++e) {
      g.tab[e] = reinterpret_cast<const uint8_t*>(w_gate_up[e]);
      g.tab_s[e] = reinterpret_cast<const uint8_t*>(w_gate_up_scale[e]);
      dn.tab[e] = reinterpret_cast<const uint8_t*>(w_down[e]);
      dn.tab_s[e] = reinterpret_cast<const uint8_t*>(w_down_scale[e]);
    }
  }
  // amax words of x and the weights -> scales (h's word stays an amax accumulator)
  if ((st = fp8t_finalize(words, 1 + 2 * E, s)) != MOE_OK) return st;

  bf16_t* h = reinterpret_cast<bf16_t*>(ws);
  ws += a256((size_t)R * I * 2);
  uint8_t* hq = ws;
  const int64_t mtiles = (R + kBM - 1) / kBM + E;

  g.q = xq;
  g.q_s = reinterpret_cast<const uint8_t*>(xs);
  g.c = h;
  g.c_s = reinterpret_cast<uint8_t*>(h_word);
  g.offsets = offsets;
  g.prob = prob_perm;
  g.R = R;
  g.K = H;
  g.N = 2 * I;
  g.E = E;
  g.I = I;
  g.n_tiles = I / 128;
  if ((st = launch(MX_SWIGLU, true, g, mtiles * g.n_tiles, s, "FP8 gate_up + ScaledSwiGLU")) != MOE_OK) return st;

  const void* hin[1] = {h};
  uint8_t* hout[1] = {hq};
  if ((st = fp8t_quantize(hin, hout, 1, R * I, h_word, s)) != MOE_OK) return st;
  if ((st = fp8t_finalize(h_word, 1, s)) != MOE_OK) return st;

  dn.q = hq;
  dn.q_s = reinterpret_cast<const uint8_t*>(h_word);
  dn.c = y_perm;
  dn.offsets = offsets;
  dn.R = R;
  dn.K = I;
  dn.N = H;
  dn.E = E;
  dn.I = I;
  dn.n_tiles = H / kBN;
  return launch(MX_STORE, true, dn, mtiles * dn.n_tiles, s, "FP8 down");
}

}  // namespace mx
}  // namespace moe
