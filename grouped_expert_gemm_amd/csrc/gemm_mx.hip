// MXFP8 and per-tensor FP8 grouped GEMMs of the MLP forward on gfx950's scaled fp8
// MFMA (v_mfma_scale_f32_32x32x64_f8f6f4: E4M3 operands, one E8M0 scale per 32 K values).
//
// Source: "Efficient MoE Training for Biological Foundation Models", Challenge 2 (MXFP8:
// one scaling factor per 32 consecutive values, 8-bit values, dedicated low-precision
// GEMM instructions; FP8 with one factor per tensor as the contrast) and Challenge 3 /
// Figure 4 (bf16 master weights and activations quantised before the GEMMs; SwiGLU,
// the routing-probability scaling and the quantisation of h fused into one kernel
// before the down projection).
//
// MFMA operand layout (measured): lane l holds row l % 32 and, for g = l / 32, the K
// values [16g, 16g + 16) in bytes 0..15 and [32 + 16g, 32 + 16g + 16) in bytes 16..31
// of a 64-value slice, and supplies the E8M0 scale of K block g (values [32g, 32g + 32))
// of its row.
//
// grouped_gemm_mxw_kernel (MXFP8, every GEMM of the MLP's forward and backward): the
// per-tensor kernel's wide-step pipeline below plus E8M0 scales in a step-major layout
// (described at the kernel).
//
// grouped_gemm_mx_kernel (MXFP8 with the public row-major scale layout, the stand-alone
// gate_up entry point): 256 x 256 tiles, 4 wavefronts of 128 x 128, a 4-slot
// LDS ring filled by global -> LDS copies four K steps ahead, a barrier in the middle
// of each step. One K step is 64 fp8 values = 64 bytes per row (the two 16-byte chunks
// a lane reads). Scales: per 4-step group each lane loads 8 bytes (blocks 8g..8g+7) of
// its row per sub-tile and packs the 4 bytes of its own K half (block 2j + (l / 32) of
// step j) into one word, so step j's MFMA selects byte j with op_sel, a compile-time
// immediate.
//
// grouped_gemm_fp8t_kernel (per-tensor FP8) runs on the bf16 forward kernel's copy
// pipeline instead: K steps of 128 fp8 values, so every row of a tile brings one whole
// 128-byte line per step, a ring of five 32 KiB LDS half-slots (P of step v in
// half-slot 2v mod 5, Q in 2v + 1) filled by range-checked buffer copies, and one
// barrier per step between its two 64-value slices (slice s is LDS chunks 4s..4s+3 of
// a row, so a lane reads logical chunks 4s + g and 4s + 2 + g).
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

enum { MX_STORE = 0, MX_SWIGLU = 1, MX_WGRAD = 2, MX_SWIGLU_SAVE = 3 };  // SAVE: SWIGLU + bf16 z and h

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
  void* z_save;                  // MXFP8 SWIGLU: NULL, or z [R][2I] in bf16 (gate, then up) and
  void* h_save;                  //   h [R][I] in bf16 (before its quantisation), both written
};

// MX_WGRAD (a weight gradient per expert, K = the expert's padded token count): P =
// tab[0] and Q = q are token-axis (column-wise) layouts [N][ld] and [R][ld] whose expert
// e occupies columns [kofs[e], kofs[e+1]); the result goes to ctab[e] [R][N] in bf16,
// all zeros for an expert without rows. Only the weight-gradient instantiation takes
// this larger argument block.
struct MxWgradParams : MxParams {
  int ld;  // row stride of both token-axis code layouts (scales: ld / 32)
  const int32_t* kofs;
  void* ctab[kMaxE];
};

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

template <int EP>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void grouped_gemm_mx_kernel(const MxParams prm) {
  __shared__ __attribute__((aligned(1024))) uint8_t sP0[kTileBytes], sP1[kTileBytes], sP2[kTileBytes], sP3[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sQ0[kTileBytes], sQ1[kTileBytes], sQ2[kTileBytes], sQ3[kTileBytes];
  __shared__ int32_t s_off[kMaxE + 1];
  __shared__ int32_t s_tstart[kMaxE + 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
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

  const int ld = prm.K;  // code row stride of P and Q (K-contiguous operands)
  const int64_t kscale = ld / 32;
  const int nk_all = prm.K / kStepK;  // a multiple of 4 (K % 256 == 0)

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
    int mt, nt;
    tile_in_expert(local, mte, prm.n_tiles, mt, nt);
    e = __builtin_amdgcn_readfirstlane(e);
    mt = __builtin_amdgcn_readfirstlane(mt);
    nt = __builtin_amdgcn_readfirstlane(nt);
    const int row_beg = __builtin_amdgcn_readfirstlane(s_off[e]);
    const int row_end = __builtin_amdgcn_readfirstlane(s_off[e + 1]);
    const int tile_row = row_beg + mt * kBM;
    const int nk = nk_all;  // K steps of 64 values, a multiple of 4 (K % 256 == 0)

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
    const uint8_t* q_tile = prm.q + (int64_t)tile_row * ld;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = i * 64 + dma_row0;
      const int chunk = (lane & 3) ^ swz(r);
      p_off[i] = (uint32_t)((int64_t)p_row(r) * ld + chunk * 16);
      q_off[i] = (uint32_t)((int64_t)(q_row(r) - tile_row) * ld + chunk * 16);
    }
    auto issue_dma = [&](int kt, auto S) {
      const int64_t k0 = (int64_t)kt * kStepK;
      // the LDS destination (M0) is wavefront-uniform: computed in scalar registers
      uint8_t* P = slotP(S) + wave_u * 1024;
      uint8_t* Q = slotQ(S) + wave_u * 1024;
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
#pragma unroll
      for (int t2 = 0; t2 < 4; ++t2) {
        scl_next[t2] = *reinterpret_cast<const uint2*>(ps_base + ps_off[t2] + g * 8);
        scl_next[4 + t2] = *reinterpret_cast<const uint2*>(qs_base + qs_off[t2] + g * 8);
      }
    };
    auto take_scales = [&]() {
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
    {
      load_scales(0);
      issue_dma(0, S0{});
      if (nk > 1) issue_dma(1, S1{});
      if (nk > 2) issue_dma(2, S2{});
      if (nk > 3) issue_dma(3, S3{});
      wait_vm_le(((nk > 1) + (nk > 2) + (nk > 3)) * kDma);
      take_scales();
      lds_barrier();
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
        wait_vm_le((j == 1 || j == 2) ? 2 * kDma + 8 : 2 * kDma);
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
    // bf16 rows through the copy slots (idle after the K loop): a tile as two blocks of
    // 256 rows x 128 columns (block 0 in sP*, block 1 in sQ*), each slot 64 rows of 256
    // bytes with chunk c of local row r at c ^ (r & 15). Every wavefront writes its
    // values (8 bytes per lane), then drains its own 64 rows of a block, 4 whole rows per
    // store instruction; rows past the expert are dropped by the buffer range check.
    int ln = lane, wv = __builtin_amdgcn_readfirstlane(wave);
    if constexpr (EP != MX_SWIGLU) asm volatile("" : "+v"(ln));  // keep the lane offsets inside the epilogue
    const int em = wv >> 1, en = wv & 1, e32 = ln & 31, ehi = ln >> 5;
    const int valid_rows = min(row_end - tile_row, kBM);
    // sub-tile (sm, sq) of block b: 4 x 8 bytes of this lane's row
    auto put = [&](auto B, int sm, int sq, int i4, uint2 v) {
      constexpr int b = decltype(B)::value;
      uint8_t* arr;
      if constexpr (b == 0) arr = (sm < 2) ? (em ? sP2 : sP0) : (em ? sP3 : sP1);
      else arr = (sm < 2) ? (em ? sQ2 : sQ0) : (em ? sQ3 : sQ1);
      const int rl = (sm & 1) * 32 + e32;
      const int ch = en * 8 + sq * 4 + i4;
      *reinterpret_cast<uint2*>(arr + rl * 256 + ((ch ^ (rl & 15)) << 4) + ehi * 8) = v;
    };
    auto put_acc = [&](auto B) {
      constexpr int b = decltype(B)::value;
#pragma unroll
      for (int sm = 0; sm < 4; ++sm)
#pragma unroll
        for (int sq = 0; sq < 2; ++sq)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int sn = 2 * b + sq;
            put(B, sm, sq, i4,
                make_uint2(pack_bf16x2(acc[sn][sm][i4 * 4 + 0], acc[sn][sm][i4 * 4 + 1]),
                           pack_bf16x2(acc[sn][sm][i4 * 4 + 2], acc[sn][sm][i4 * 4 + 3])));
          }
    };
    // block b to rows [tile_row, tile_row + valid_rows) of dst (its 128 columns), ld elements per row
    auto drain = [&](auto B, bf16_t* dst, int64_t ld) {
      constexpr int b = decltype(B)::value;
      const uint8_t* arr;
      if constexpr (b == 0) arr = wv == 0 ? sP0 : wv == 1 ? sP1 : wv == 2 ? sP2 : sP3;
      else arr = wv == 0 ? sQ0 : wv == 1 ? sQ1 : wv == 2 ? sQ2 : sQ3;
      const int64_t ldb = ld * 2;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(dst + (int64_t)tile_row * ld), (short)0, (int)(uint32_t)(valid_rows * ldb), kBufferFlags);
      const int pc = ln & 15;
      const uint32_t vo = (uint32_t)((ln >> 4) * ldb + pc * 16);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rl = 4 * i + (ln >> 4);
        const v4u32 val = *reinterpret_cast<const v4u32*>(arr + rl * 256 + ((pc ^ (rl & 15)) << 4));
        __builtin_amdgcn_raw_buffer_store_b128(val, rs, vo, (int)((wv * 64 + 4 * i) * ldb), 0);
      }
    };
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    if constexpr (EP == MX_STORE) {
      bf16_t* c0 = reinterpret_cast<bf16_t*>(prm.c) + (int64_t)nt * kBN;
      put_acc(B0{});
      put_acc(B1{});
      lds_barrier();
      drain(B0{}, c0, prm.N);
      drain(B1{}, c0 + 128, prm.N);
      lds_barrier();  // read out before the next tile's copies land
    } else {
#pragma unroll
    for (int sm = 0; sm < 4; ++sm) {
      const int64_t mg = (int64_t)tile_row + wm * 128 + sm * 32 + l32;
      const bool valid = mg < row_end;
      {
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
              *reinterpret_cast<uint32_t*>(C + i4 * 8 + lhi * 4) =
                  e4m3_pack4(ldexpf(h[i4 * 4], -sx), ldexpf(h[i4 * 4 + 1], -sx), ldexpf(h[i4 * 4 + 2], -sx),
                             ldexpf(h[i4 * 4 + 3], -sx));
            }
            if (lhi == 0) prm.c_s[mg * (prm.I / 32) + col0 / 32] = (uint8_t)(sx + 127);
          }
        }
      }
    }
    }
  }
}

namespace {
constexpr int kXBK = 128;                 // K step: 128 fp8 values, 128 bytes per row
constexpr int kXTile = kBM * kXBK;        // one operand of one step: a half-slot (32 KiB)
}  // namespace

// Per-tensor FP8 grouped GEMM on the bf16 forward kernel's copy pipeline (see the top
// of this file): K steps of 128 fp8 values, a ring of five 32 KiB LDS half-slots, two
// 64-value MFMA slices per step with the barrier between them. The MFMA runs with unit
// block scales; the products are scaled by (Q's scale x the expert's P scale) in the
// epilogue, and the SwiGLU epilogue writes h in bf16 and raises h's amax word (its
// scale needs all of h); MX_SWIGLU_SAVE also writes z = [G, U] in bf16. MX_WGRAD (MxWgradParams): the backward's weight gradients on
// token-axis codes (as in the MXFP8 kernel below), scaled by the two tensors' factors
// q_s[0] x tab_s[0][0].
template <int EP, typename Params = MxParams>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void grouped_gemm_fp8t_kernel(const Params prm) {
  __shared__ __attribute__((aligned(1024))) uint8_t sH0[kXTile], sH1[kXTile], sH2[kXTile];
  __shared__ __attribute__((aligned(1024))) uint8_t sH3[kXTile], sH4[kXTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int wm = wave >> 1, wn = wave & 1;
  const int E = prm.E;
  const int R = (int)prm.R;
  const int K = prm.K;
  const int l32 = lane & 31, lhi = lane >> 5;

  const int nwg = gridDim.x;
  const int logical = (nwg % 8 == 0) ? (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8 : blockIdx.x;

  auto hslot = [&](auto H) -> uint8_t* {
    if constexpr (H.value == 0) return sH0;
    else if constexpr (H.value == 1) return sH1;
    else if constexpr (H.value == 2) return sH2;
    else if constexpr (H.value == 3) return sH3;
    else return sH4;
  };

  // Tiles: expert-major, ceil(rows_e / 256) row tiles x n_tiles per expert, row tiles
  // fastest within groups of at most 16 (tile_in_expert). Expert offsets are walked
  // once with wavefront-uniform loads and made a nondecreasing sequence inside [0, R]
  // on the way.
  auto clamp_off = [&](int v, int prev) -> int {
    v = v < prev ? prev : v;
    return v > R ? R : v;
  };
  constexpr bool wgrad = EP == MX_WGRAD;
  constexpr bool swiglu = EP == MX_SWIGLU || EP == MX_SWIGLU_SAVE;
  int total = 0;
  int e_w = 0, ob = 0, oe = 0, ts_w = 0, nt_w = 0;
  if constexpr (wgrad) {  // every expert owns the whole [R, N] output
    total = E * (R / kBM) * prm.n_tiles;
  } else {
    int prev = 0;
    for (int x = 0; x < E; ++x) {
      const int en = clamp_off(load_const(prm.offsets, x + 1), prev);
      total += ((en - prev + kBM - 1) / kBM) * prm.n_tiles;
      prev = en;
    }
    oe = clamp_off(load_const(prm.offsets, 1), 0);
    nt_w = ((oe - ob + kBM - 1) / kBM) * prm.n_tiles;
  }
  // row stride of both code arrays: K, or the padded token axis for the weight gradients
  int ld = K;
  if constexpr (wgrad) ld = prm.ld;

  // fragment addresses: sub-tile rows start at multiples of 32, where swz8 depends on
  // the lane's row within the sub-tile only; half h of slice s is logical chunk
  // 4s + 2h + lhi
  const uint32_t fragP = (uint32_t)((wn * 64 + l32) * 128);
  const uint32_t fragQ = (uint32_t)((wm * 128 + l32) * 128);
  uint32_t ck[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) ck[c] = (uint32_t)(((2 * c + lhi) ^ swz8(l32)) << 4);
  // copies: round i (0..7) of wavefront w fills LDS bytes [(4i + w) KiB, +1 KiB) of a
  // half-slot: rows (4i + w) * 8 + (lane >> 3), physical chunk lane & 7
  const int kc_row0 = wave * 8 + (lane >> 3);
  const int kc_chunk = (lane & 7) ^ swz8(kc_row0);
  constexpr int64_t kAll = 0xFFFFFFFFll;

  for (int t = logical; t < total; t += nwg) {
    // ---------------- tile decode ----------------
    int e, mt, nt, nk, k_beg = 0;
    if constexpr (wgrad) {
      // groups of 8 m-tiles, n fastest over the group (as in the MXFP8 kernel below)
      constexpr int GM = 8;
      const int mte = R / kBM;
      const int per = mte * prm.n_tiles;
      e = t / per;
      const int local = t - e * per;
      const int span = GM * prm.n_tiles;
      const int grp = local / span, rem = local - grp * span;
      const int gm = min(GM, mte - grp * GM);
      mt = grp * GM + rem % gm;
      nt = rem / gm;
      e = __builtin_amdgcn_readfirstlane(e);
      k_beg = __builtin_amdgcn_readfirstlane(prm.kofs[e]);
      nk = __builtin_amdgcn_readfirstlane((prm.kofs[e + 1] - k_beg) / kXBK);
      ob = 0;
      oe = R;
    } else {
      while (e_w < E && t >= ts_w + nt_w) {
        ts_w += nt_w;
        ++e_w;
        ob = oe;
        if (e_w < E) {
          oe = clamp_off(load_const(prm.offsets, e_w + 1), ob);
          nt_w = ((oe - ob + kBM - 1) / kBM) * prm.n_tiles;
        }
      }
      if (e_w >= E) break;
      e = e_w;
      const int local = t - ts_w;
      const int mte = (oe - ob + kBM - 1) / kBM;
      tile_in_expert(local, mte, prm.n_tiles, mt, nt);
      nk = K / kXBK;
    }
    const int pad = (5 - nk % 5) % 5;  // zero steps ahead of the K loop (as in the MXFP8 kernel below)
    e = __builtin_amdgcn_readfirstlane(e);
    mt = __builtin_amdgcn_readfirstlane(mt);
    nt = __builtin_amdgcn_readfirstlane(nt);
    const int row_beg = __builtin_amdgcn_readfirstlane(ob);
    const int row_end = __builtin_amdgcn_readfirstlane(oe);
    const int tile_row = row_beg + mt * kBM;

    // P row of local tile row r (SWIGLU: gate rows, then the up rows of the same columns)
    auto p_row = [&](int r) -> int {
      if constexpr (swiglu) return (r < 128) ? nt * 128 + r : prm.I + nt * 128 + (r - 128);
      else return nt * kBN + r;
    };

    // ---------------- operands ----------------
    // Q's record count ends at the expert's last row: rows past it fail the range check
    // and land as zero codes, discarded in the epilogue.
    const uint8_t* p_tile = prm.tab[wgrad ? 0 : e] + (int64_t)p_row(0) * ld + k_beg;
    const uint8_t* q_tile = prm.q + (int64_t)tile_row * ld + k_beg;
    const uint32_t off0 = (uint32_t)((int64_t)kc_row0 * ld + kc_chunk * 16);
    const int64_t q_extent = wgrad ? kAll : (int64_t)(row_end - tile_row) * ld;
    const int p_up = swiglu ? prm.I - 128 : 0;
    // step kt of the loop is step kt - pad of the operands: an empty range (zeros) outside [0, nk)
    auto copy_op = [&](const uint8_t* tile, int up, int64_t extent, int kt, uint8_t* dst) {
      const int ks = kt - pad;
      const int64_t at = (int64_t)ks * kXBK;
      int64_t lim = extent - at;
      lim = lim < 0 ? 0 : (lim > kAll ? kAll : lim);
      const int64_t nrec = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)ks < (uint32_t)nk ? (int)(uint32_t)lim : 0);
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)(tile + at), (short)0, (int)(uint32_t)nrec, kBufferFlags);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t rows = (uint32_t)(i * 32 + (i >= 4 ? up : 0));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(dst + i * 4096), 16, off0, (int)(rows * (uint32_t)ld),
                                                 0, 0);
      }
    };
    // the LDS destination (M0) is wavefront-uniform: keep it in scalar registers
    auto copy_P = [&](int kt, auto H) { copy_op(p_tile, p_up, kAll, kt, hslot(H) + wave_u * 1024); };
    auto copy_Q = [&](int kt, auto H) { copy_op(q_tile, 0, q_extent, kt, hslot(H) + wave_u * 1024); };

    const uint32_t kUnit = 0x7F7F7F7Fu;  // E8M0 127 = 1.0 in every byte

    f32x16 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

    // fragments: Q of both slices of a step (fb0, fb1), and one set of P that is refilled
    // sub-tile by sub-tile as soon as its four MFMAs have been issued
    i32x8_t fa[4], fb0[4], fb1[4];
    // Lane parts of the fragment addresses: P chunk c at fragP + ck[c], Q at fragQ +
    // ck[c]. A step takes them through an empty asm, so the compiler adds the half-slot
    // base inside the step instead of holding all 40 (half-slot, operand, chunk) sums
    // across the loop; sub-tile offsets are the reads' immediate offsets.
    auto rd = [&](const uint8_t* base, int s) -> i32x8_t {
      const i32x4_t a = *reinterpret_cast<const i32x4_t*>(base + ck[2 * s]);
      const i32x4_t b = *reinterpret_cast<const i32x4_t*>(base + ck[2 * s + 1]);
      return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    auto read_q = [&](auto HQ, int s, i32x8_t* fb) {
      const uint8_t* Q = hslot(HQ) + fragQ;
#pragma unroll
      for (int u = 0; u < 4; ++u) fb[u] = rd(Q + (u * 32) * 128, s);
    };
    auto read_p = [&](auto HP, int s, int sn) -> i32x8_t {
      return rd(hslot(HP) + fragP + ((sn >> 1) * 128 + (sn & 1) * 32) * 128, s);
    };
    // the 16 MFMAs of one slice with Q fragments fb, P sub-tile by sub-tile; after the
    // MFMAs of sub-tile sn, fa[sn] takes P sub-tile sn of slice s_next of half-slot HPn
    auto mfma_slice = [&](const i32x8_t* fb, auto OPSEL, bool refill, auto HPn, int s_next) {
      constexpr int os = decltype(OPSEL)::value;
#pragma unroll
      for (int sn = 0; sn < 4; ++sn) {
#pragma unroll
        for (int sm = 0; sm < 4; ++sm)
          acc[sn][sm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[sn], fb[sm], acc[sn][sm], 0, 0, os,
                                                                          (int)kUnit, os, (int)kUnit);
        if (refill) fa[sn] = read_p(HPn, s_next, sn);
      }
    };
    // 16 MFMAs with the 16 fragment reads (8 fragments, two 16-byte halves each) between them
    auto interleave_a = [&]() {
      static_for<16>([&](auto I) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      });
    };
    // ... and the 16 copies of later steps as well
    auto interleave_b = [&]() {
      static_for<16>([&](auto I) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      });
    };

    // K step kt, V = kt % 5 (the half-slot ring); on entry fa and fb0 hold slice 0.
    // Per step the copies are issued in the order Q of step kt+2, P of step kt+3, so
    // when step kt+1 must have landed only P of step kt+2 (the 8 most recent) may be
    // in flight.
    auto kstep = [&](int kt, auto V) {
      constexpr int v = decltype(V)::value;
      using HP = std::integral_constant<int, (2 * v) % 5>;
      using HQ = std::integral_constant<int, (2 * v + 1) % 5>;
      using HPn = std::integral_constant<int, (2 * v + 2) % 5>;
      using HQn = std::integral_constant<int, (2 * v + 3) % 5>;
      read_q(HQ{}, 1, fb1);
      mfma_slice(fb0, std::integral_constant<int, 0>{}, true, HP{}, 1);
      interleave_a();
      wait_vm<8>();
      lds_barrier();                  // also waits for every read of step kt
      copy_Q(kt + 2, HP{});           // Q of step kt+2: half-slot 2(kt+2)+1 = 2kt mod 5
      copy_P(kt + 3, HQ{});           // P of step kt+3: half-slot 2(kt+3) = 2kt+1 mod 5
      read_q(HQn{}, 0, fb0);          // (past the last step: never used)
      mfma_slice(fb1, std::integral_constant<int, 0>{}, true, HPn{}, 0);
      interleave_b();
    };
    auto read_first = [&](auto HP, auto HQ) {
      read_q(HQ, 0, fb0);
#pragma unroll
      for (int sn = 0; sn < 4; ++sn) fa[sn] = read_p(HP, 0, sn);
    };
    using H0 = std::integral_constant<int, 0>;
    using H1 = std::integral_constant<int, 1>;
    using H2 = std::integral_constant<int, 2>;
    using H3 = std::integral_constant<int, 3>;
    using H4 = std::integral_constant<int, 4>;
    if (nk > 0) {  // (a weight gradient of an expert without rows: no steps, its tile is zeros)
      copy_P(0, H0{});
      copy_Q(0, H1{});
      copy_P(1, H2{});
      copy_Q(1, H3{});
      copy_P(2, H4{});
      wait_vm<24>();  // step 0 complete
      lds_barrier();
      read_first(H0{}, H1{});
      const int n_run = nk + pad;
      for (int kt = 0; kt < n_run; kt += 5) static_for<5>([&](auto V) { kstep(kt + decltype(V)::value, V); });
      wait_vm<0>();   // the zero copies issued past the last step land before LDS is reused
    }
    // every wavefront is done with every half-slot before the epilogue uses LDS
    lds_barrier();

    // ---------------- epilogue ----------------
    // the product of the two tensors' scales
    const float alpha =
        *reinterpret_cast<const float*>(prm.q_s) * *reinterpret_cast<const float*>(prm.tab_s[wgrad ? 0 : e]);
    if constexpr (EP == MX_STORE || EP == MX_WGRAD) {
      // bf16 rows through LDS (idle after the K loop), as in the bf16 forward kernel:
      // blocks of 256 rows x 128 columns, 256-byte rows, chunk c of row r at
      // c ^ (r & 15), rows 0-127 in the first array of a pair and 128-255 in the second;
      // each wavefront writes its accumulators (8 bytes per lane), then 4 whole rows
      // leave per store instruction, rows past the expert dropped by the range check.
      int ln = lane, wv = __builtin_amdgcn_readfirstlane(wave);
      asm volatile("" : "+v"(ln));  // keep the lane offsets inside the epilogue
      const int em = wv >> 1, en = wv & 1, e32 = ln & 31, ehi = ln >> 5;
      const int valid = min(row_end - tile_row, kBM);
      auto put = [&](uint8_t* arr, int sm, int sq, int i4, uint2 v) {
        const int rr = sm * 32 + e32;
        const int ch = en * 8 + sq * 4 + i4;
        *reinterpret_cast<uint2*>(arr + rr * 256 + ((ch ^ (rr & 15)) << 4) + ehi * 8) = v;
      };
      auto drain = [&](const uint8_t* arr, bf16_t* dst, int64_t ld) {
        const int64_t ldb = ld * 2;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(dst + (int64_t)tile_row * ld), (short)0, (int)(uint32_t)(valid * ldb), kBufferFlags);
        const int pc = ln & 15;
        const uint32_t vo = (uint32_t)((ln >> 4) * ldb + pc * 16);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int rl = (wv & 1) * 64 + 4 * i + (ln >> 4);
          const v4u32 val = *reinterpret_cast<const v4u32*>(arr + rl * 256 + ((pc ^ (rl & 15)) << 4));
          __builtin_amdgcn_raw_buffer_store_b128(val, rs, vo, (int)((wv * 64 + 4 * i) * ldb), 0);
        }
      };
      auto acc_block = [&](int b, uint8_t* arr0, uint8_t* arr1) {
        uint8_t* arr = em ? arr1 : arr0;
#pragma unroll
        for (int sm = 0; sm < 4; ++sm)
#pragma unroll
          for (int sq = 0; sq < 2; ++sq)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              const int sn = 2 * b + sq;
              put(arr, sm, sq, i4,
                  make_uint2(pack_bf16x2(acc[sn][sm][i4 * 4 + 0] * alpha, acc[sn][sm][i4 * 4 + 1] * alpha),
                             pack_bf16x2(acc[sn][sm][i4 * 4 + 2] * alpha, acc[sn][sm][i4 * 4 + 3] * alpha)));
            }
      };
      acc_block(0, sH0, sH1);
      acc_block(1, sH2, sH3);
      lds_barrier();
      void* cbase;
      if constexpr (wgrad) cbase = prm.ctab[e];
      else cbase = prm.c;
      bf16_t* c0 = reinterpret_cast<bf16_t*>(cbase) + (int64_t)nt * kBN;
      drain(wv < 2 ? sH0 : sH1, c0, prm.N);
      drain(wv < 2 ? sH2 : sH3, c0 + 128, prm.N);
      lds_barrier();  // read out before the next tile's copies land
    } else {
      float hmax = 0.f;   // max |h| of this lane's values
#pragma unroll
      for (int sm = 0; sm < 4; ++sm) {
        const int64_t mg = (int64_t)tile_row + wm * 128 + sm * 32 + l32;
        const bool valid = mg < row_end;
        const float p = prm.prob[valid ? mg : row_end - 1];
#pragma unroll
        for (int sn = 0; sn < 2; ++sn) {
          const int64_t col0 = (int64_t)nt * 128 + wn * 64 + sn * 32;
          float h[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            h[i] = silu_f(acc[sn][sm][i] * alpha) * (acc[sn + 2][sm][i] * alpha) * p;
            if (valid) hmax = fmaxf(hmax, fabsf(h[i]));
          }
          if (valid) {
            bf16_t* C = reinterpret_cast<bf16_t*>(prm.c) + mg * prm.I + col0;
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4)
              *reinterpret_cast<uint2*>(C + i4 * 8 + lhi * 4) =
                  make_uint2(pack_bf16x2(h[i4 * 4 + 0], h[i4 * 4 + 1]), pack_bf16x2(h[i4 * 4 + 2], h[i4 * 4 + 3]));
            if constexpr (EP == MX_SWIGLU_SAVE) {  // z = [G, U] of the row, scaled products in bf16
              bf16_t* Z = reinterpret_cast<bf16_t*>(prm.z_save) + mg * 2 * prm.I + col0;
#pragma unroll
              for (int i4 = 0; i4 < 4; ++i4) {
                const f32x16& G = acc[sn][sm];
                const f32x16& U = acc[sn + 2][sm];
                const int i = i4 * 4;
                *reinterpret_cast<uint2*>(Z + i4 * 8 + lhi * 4) = make_uint2(
                    pack_bf16x2(G[i] * alpha, G[i + 1] * alpha), pack_bf16x2(G[i + 2] * alpha, G[i + 3] * alpha));
                *reinterpret_cast<uint2*>(Z + prm.I + i4 * 8 + lhi * 4) = make_uint2(
                    pack_bf16x2(U[i] * alpha, U[i + 1] * alpha), pack_bf16x2(U[i + 2] * alpha, U[i + 3] * alpha));
              }
            }
          }
        }
      }
      // h is stored in bf16, and rounding is monotone: the maximum of the stored
      // magnitudes is the rounded maximum of the float32 ones
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) hmax = fmaxf(hmax, __shfl_xor(hmax, off));
      if (lane == 0 && hmax > 0.f) atomicMax(reinterpret_cast<uint32_t*>(prm.c_s), f32_to_bf16(hmax) << 16);
    }
  }
}

// MXFP8 grouped GEMM on the same wide-step copy pipeline as grouped_gemm_fp8t_kernel:
// K steps of 128 fp8 values (a whole 128-byte line per row), the five-half-slot LDS
// ring, two 64-value MFMA slices per step with the barrier between them. What it adds
// are the block scales: a step covers 4 E8M0 blocks of each row, one 32-bit word. The
// scales come step-major (word k * rows + r for step k of row r: the 32 rows of a
// sub-tile are one 128-byte run; the row-major public layout puts each row on its own
// cache line, and loading those cost a fifth of the kernel's time). The forward's
// quantisers write this layout; the gate_up epilogue writes h's scales in it. P's
// scale array has prm.N rows, Q's prm.R. Each lane loads the words of its 4 P rows and 4 Q rows with
// buffer loads two steps ahead (issued ahead of that step's copies, so the copy waits
// need not count them; one load covers two sub-tiles, fanned out across the wavefront's
// halves with a lane swap), and shifts them right by 8 bits x its K half g: byte 0 is then block g
// (slice 0) and byte 2 block 2 + g (slice 1), so the MFMA's byte select is the
// compile-time 0 / 2 for every lane.
// Epilogues: MX_STORE (bf16 rows through LDS), MX_SWIGLU (h = silu(G) U p quantised to
// MXFP8 along I: a 32-value block is one sub-tile column span of a row, 16 values in
// lane l and 16 in lane l ^ 32) and MX_SWIGLU_SAVE (also z and h in bf16, through LDS).
// MX_WGRAD (MxWgradParams): the weight gradients on token-axis operands, as in the
// 64-value-step kernel, with step-major scales: step s of expert e is step
// kofs[e] / 128 + s of the padded token axis, whose words start at that step times the
// operand's row count.
// The K loop has no guarded steps: steps that skip copies past the end would make
// control-flow joins, where the compiler drains every copy in flight before the next LDS
// reads (such a step cost 2-4 times a full one; a weight gradient has only about 8 steps
// at 1000 tokens per expert). It runs whole groups of 5 full steps instead, the first
// (5 - nk % 5) % 5 of them zero steps: their copies have an empty buffer range (they
// land as zeros in LDS), their scale words are those of a real step, and their products
// are exact zeros, which leave the +0 accumulators unchanged. The zero steps run while
// the first real copies are in flight.
template <int EP, typename Params = MxParams>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void grouped_gemm_mxw_kernel(const Params prm) {
  __shared__ __attribute__((aligned(1024))) uint8_t sH0[kXTile], sH1[kXTile], sH2[kXTile];
  __shared__ __attribute__((aligned(1024))) uint8_t sH3[kXTile], sH4[kXTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int wm = wave >> 1, wn = wave & 1;
  const int E = prm.E;
  const int R = (int)prm.R;
  const int K = prm.K;
  const int l32 = lane & 31, lhi = lane >> 5;

  const int nwg = gridDim.x;
  const int logical = (nwg % 8 == 0) ? (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8 : blockIdx.x;

  auto hslot = [&](auto H) -> uint8_t* {
    if constexpr (H.value == 0) return sH0;
    else if constexpr (H.value == 1) return sH1;
    else if constexpr (H.value == 2) return sH2;
    else if constexpr (H.value == 3) return sH3;
    else return sH4;
  };

  // Tiles: expert-major, ceil(rows_e / 256) row tiles x n_tiles per expert, row tiles
  // fastest within groups of at most 16 (tile_in_expert). Expert offsets are walked
  // once with wavefront-uniform loads and made a nondecreasing sequence inside [0, R]
  // on the way.
  auto clamp_off = [&](int v, int prev) -> int {
    v = v < prev ? prev : v;
    return v > R ? R : v;
  };
  constexpr bool wgrad = EP == MX_WGRAD;
  int total = 0;
  int e_w = 0, ob = 0, oe = 0, ts_w = 0, nt_w = 0;
  if constexpr (wgrad) {  // every expert owns the whole [R, N] output
    total = E * (R / kBM) * prm.n_tiles;
  } else {
    int prev = 0;
    for (int x = 0; x < E; ++x) {
      const int en = clamp_off(load_const(prm.offsets, x + 1), prev);
      total += ((en - prev + kBM - 1) / kBM) * prm.n_tiles;
      prev = en;
    }
    oe = clamp_off(load_const(prm.offsets, 1), 0);
    nt_w = ((oe - ob + kBM - 1) / kBM) * prm.n_tiles;
  }
  // row stride of both code arrays: K for K-contiguous operands, the padded token axis
  // for the weight gradients
  int ld = K;
  if constexpr (wgrad) ld = prm.ld;

  const uint32_t fragP = (uint32_t)((wn * 64 + l32) * 128);
  const uint32_t fragQ = (uint32_t)((wm * 128 + l32) * 128);
  uint32_t ck[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) ck[c] = (uint32_t)(((2 * c + lhi) ^ swz8(l32)) << 4);
  const int kc_row0 = wave * 8 + (lane >> 3);
  const int kc_chunk = (lane & 7) ^ swz8(kc_row0);
  constexpr int64_t kAll = 0xFFFFFFFFll;
  const uint32_t gshift = 8u * (uint32_t)lhi;

  for (int t = logical; t < total; t += nwg) {
    // ---------------- tile decode ----------------
    int e, mt, nt, nk, k_beg = 0, pad = 0;
    if constexpr (wgrad) {
      // groups of 8 m-tiles, n fastest over the group: the 32 consecutive tiles one XCD
      // runs at a time form an 8 x 4 block whose operand slabs stay in its L2
      constexpr int GM = 8;
      const int mte = R / kBM;
      const int per = mte * prm.n_tiles;
      e = t / per;
      const int local = t - e * per;
      const int span = GM * prm.n_tiles;
      const int grp = local / span, rem = local - grp * span;
      const int gm = min(GM, mte - grp * GM);
      mt = grp * GM + rem % gm;
      nt = rem / gm;
      e = __builtin_amdgcn_readfirstlane(e);
      k_beg = __builtin_amdgcn_readfirstlane(prm.kofs[e]);
      nk = __builtin_amdgcn_readfirstlane((prm.kofs[e + 1] - k_beg) / kXBK);
      pad = (5 - nk % 5) % 5;
      ob = 0;
      oe = R;
    } else {
      while (e_w < E && t >= ts_w + nt_w) {
        ts_w += nt_w;
        ++e_w;
        ob = oe;
        if (e_w < E) {
          oe = clamp_off(load_const(prm.offsets, e_w + 1), ob);
          nt_w = ((oe - ob + kBM - 1) / kBM) * prm.n_tiles;
        }
      }
      if (e_w >= E) break;
      e = e_w;
      const int local = t - ts_w;
      const int mte = (oe - ob + kBM - 1) / kBM;
      tile_in_expert(local, mte, prm.n_tiles, mt, nt);
      nk = K / kXBK;
      pad = (5 - nk % 5) % 5;
    }
    e = __builtin_amdgcn_readfirstlane(e);
    mt = __builtin_amdgcn_readfirstlane(mt);
    nt = __builtin_amdgcn_readfirstlane(nt);
    const int row_beg = __builtin_amdgcn_readfirstlane(ob);
    const int row_end = __builtin_amdgcn_readfirstlane(oe);
    const int tile_row = row_beg + mt * kBM;

    auto p_row = [&](int r) -> int {
      if constexpr (EP == MX_SWIGLU || EP == MX_SWIGLU_SAVE) return (r < 128) ? nt * 128 + r : prm.I + nt * 128 + (r - 128);
      else return nt * kBN + r;
    };

    // ---------------- operands ----------------
    const uint8_t* p_tile = prm.tab[wgrad ? 0 : e] + (int64_t)p_row(0) * ld + k_beg;
    const uint8_t* q_tile = prm.q + (int64_t)tile_row * ld + k_beg;
    const uint32_t off0 = (uint32_t)((int64_t)kc_row0 * ld + kc_chunk * 16);
    const int64_t q_extent = wgrad ? kAll : (int64_t)(row_end - tile_row) * ld;
    const int p_up = (EP == MX_SWIGLU || EP == MX_SWIGLU_SAVE) ? prm.I - 128 : 0;
    // step kt of the loop is step kt - pad of the operands: an empty range (zeros) outside [0, nk)
    auto copy_op = [&](const uint8_t* tile, int up, int64_t extent, int kt, uint8_t* dst) {
      const int ks = kt - pad;
      const int64_t at = (int64_t)ks * kXBK;
      int64_t lim = extent - at;
      lim = lim < 0 ? 0 : (lim > kAll ? kAll : lim);
      // read back as a wavefront-uniform value: a select left in a vector register would
      // make the whole descriptor a vector operand and every copy a waterfall loop
      const int64_t nrec = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)ks < (uint32_t)nk ? (int)(uint32_t)lim : 0);
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)(tile + at), (short)0, (int)(uint32_t)nrec, kBufferFlags);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t rows = (uint32_t)(i * 32 + (i >= 4 ? up : 0));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(dst + i * 4096), 16, off0, (int)(rows * (uint32_t)ld),
                                                 0, 0);
      }
    };
    auto copy_P = [&](int kt, auto H) { copy_op(p_tile, p_up, kAll, kt, hslot(H) + wave_u * 1024); };
    auto copy_Q = [&](int kt, auto H) { copy_op(q_tile, 0, q_extent, kt, hslot(H) + wave_u * 1024); };

    // scale words (step-major): P sub-tile sn is tile rows sub_n(sn, wn) + [0, 32); Q
    // sub-tile sm is wm * 128 + sm * 32 + [0, 32), rows past the expert clamped to its
    // last row (their products are discarded). Step kt's words start kt * rows words in.
    const int p_step = 4 * prm.N, q_step = 4 * R;  // bytes per K step of the two scale arrays
    const int k_step0 = k_beg / kXBK;               // the expert's first step (weight gradients)
    const __amdgpu_buffer_rsrc_t ps_rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(prm.tab_s[wgrad ? 0 : e] + (int64_t)k_step0 * p_step), (short)0, (int)0xFFFFFFFF, kBufferFlags);
    const __amdgpu_buffer_rsrc_t qs_rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(prm.q_s + (int64_t)k_step0 * q_step), (short)0, (int)0xFFFFFFFF, kBufferFlags);
    // One load serves two sub-tiles: lanes 0-31 read the row of sub-tile 2j, lanes 32-63
    // that of sub-tile 2j + 1 (the same row index l32); raw word j of a step holds them.
    uint32_t ps_off[2], qs_off[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      ps_off[j] = (uint32_t)(p_row(sub_n(2 * j + lhi, wn) + l32) * 4);
      const int qr = wm * 128 + (2 * j + lhi) * 32 + l32;
      qs_off[j] = (uint32_t)((tile_row + (qr < row_end - tile_row ? qr : row_end - tile_row - 1)) * 4);
    }
    // raw words of a step: [0, 1] P sub-tile pairs, [2, 3] Q sub-tile pairs
    auto load_scales = [&](int kt, uint32_t* w) {
      kt -= pad;  // a zero step takes the words of the nearest real step
      kt = kt < 0 ? 0 : (kt >= nk ? nk - 1 : kt);
#pragma unroll
      for (int j = 0; j < 2; ++j) w[j] = __builtin_amdgcn_raw_buffer_load_b32(ps_rs, ps_off[j], kt * p_step, 0);
#pragma unroll
      for (int j = 0; j < 2; ++j) w[2 + j] = __builtin_amdgcn_raw_buffer_load_b32(qs_rs, qs_off[j], kt * q_step, 0);
    };
    // raw words -> the 8 scale words of a step ([0..3] P, [4..7] Q sub-tiles): the swap
    // exchanges the upper half of one register with the lower half of the other, so a
    // word and its copy give [lower, lower] (sub-tile 2j) and [upper, upper] (2j + 1);
    // then the shift by 8 g puts block g of the step in byte 0 and 2 + g in byte 2
    auto fan_out = [&](const uint32_t* w, uint32_t* sc) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const auto pr = __builtin_amdgcn_permlane32_swap(w[j], w[j], false, false);
        const int base = (j < 2) ? 2 * j : 4 + 2 * (j - 2);
        sc[base] = (uint32_t)pr[0] >> gshift;
        sc[base + 1] = (uint32_t)pr[1] >> gshift;
      }
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

    i32x8_t fa[4], fb0[4], fb1[4];
    auto rd = [&](const uint8_t* base, int s) -> i32x8_t {
      const i32x4_t a = *reinterpret_cast<const i32x4_t*>(base + ck[2 * s]);
      const i32x4_t b = *reinterpret_cast<const i32x4_t*>(base + ck[2 * s + 1]);
      return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    auto read_q = [&](auto HQ, int s, i32x8_t* fb) {
      const uint8_t* Q = hslot(HQ) + fragQ;
#pragma unroll
      for (int u = 0; u < 4; ++u) fb[u] = rd(Q + (u * 32) * 128, s);
    };
    auto read_p = [&](auto HP, int s, int sn) -> i32x8_t {
      return rd(hslot(HP) + fragP + ((sn >> 1) * 128 + (sn & 1) * 32) * 128, s);
    };
    // the 16 MFMAs of slice SL with scale words sc (byte 2 SL of each); after the MFMAs of
    // P sub-tile sn, fa[sn] takes P sub-tile sn of slice s_next of half-slot HPn
    auto mfma_slice = [&](const i32x8_t* fb, const uint32_t* sc, auto SL, bool refill, auto HPn, int s_next) {
      constexpr int os = 2 * decltype(SL)::value;
#pragma unroll
      for (int sn = 0; sn < 4; ++sn) {
#pragma unroll
        for (int sm = 0; sm < 4; ++sm)
          acc[sn][sm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[sn], fb[sm], acc[sn][sm], 0, 0, os,
                                                                          (int)sc[sn], os, (int)sc[4 + sm]);
        if (refill) fa[sn] = read_p(HPn, s_next, sn);
      }
    };
    auto interleave_a = [&]() {
      static_for<16>([&](auto I) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      });
    };
    auto interleave_b = [&]() {
      static_for<16>([&](auto I) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      });
    };

    // raw scale words of steps kt (r0) and kt+1 (r1) on entry to step kt
    uint32_t r0[4], r1[4];
    // K step kt, V = kt % 5. Per step the scale words of step kt+2 are loaded first, then
    // the copies Q of step kt+2 and P of step kt+3, so when step kt+1 must have landed
    // only P of step kt+2 (the 8 most recent operations) may be in flight, as in the
    // per-tensor kernel. The scale loads are ordinary buffer loads, which the scheduler
    // could otherwise move between the copies (those stay ordered among themselves
    // through M0) and so break that count: a scheduling barrier keeps them ahead.
    auto kstep = [&](int kt, auto V) {
      constexpr int v = decltype(V)::value;
      using HP = std::integral_constant<int, (2 * v) % 5>;
      using HQ = std::integral_constant<int, (2 * v + 1) % 5>;
      using HPn = std::integral_constant<int, (2 * v + 2) % 5>;
      using HQn = std::integral_constant<int, (2 * v + 3) % 5>;
      uint32_t sc[8];
      fan_out(r0, sc);
      read_q(HQ{}, 1, fb1);
      mfma_slice(fb0, sc, std::integral_constant<int, 0>{}, true, HP{}, 1);
      interleave_a();
      wait_vm<8>();
      lds_barrier();                  // also waits for every read of step kt
      uint32_t r2[4];
      load_scales(kt + 2, r2);
      __builtin_amdgcn_sched_barrier(0);
      copy_Q(kt + 2, HP{});           // Q of step kt+2: half-slot 2(kt+2)+1 = 2kt mod 5
      copy_P(kt + 3, HQ{});           // P of step kt+3: half-slot 2(kt+3) = 2kt+1 mod 5
      read_q(HQn{}, 0, fb0);          // (past the last step: zeros or in-flight data, never used)
      mfma_slice(fb1, sc, std::integral_constant<int, 1>{}, true, HPn{}, 0);
      interleave_b();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        r0[i] = r1[i];
        r1[i] = r2[i];
      }
    };
    auto read_first = [&](auto HP, auto HQ) {
      read_q(HQ, 0, fb0);
#pragma unroll
      for (int sn = 0; sn < 4; ++sn) fa[sn] = read_p(HP, 0, sn);
    };
    using H0 = std::integral_constant<int, 0>;
    using H1 = std::integral_constant<int, 1>;
    using H2 = std::integral_constant<int, 2>;
    using H3 = std::integral_constant<int, 3>;
    using H4 = std::integral_constant<int, 4>;
    auto steps5 = [&](int kt0) { static_for<5>([&](auto V) { kstep(kt0 + decltype(V)::value, V); }); };
    // Prologue: the scale words of steps 0 and 1 ahead of every copy, then the copies of
    // steps 0-2, so that step 0's wait sees the steady state's pattern. (A weight
    // gradient of an expert without rows has no steps: its tile is zeros.)
    if (nk > 0) {
      load_scales(0, r0);
      load_scales(1, r1);
      __builtin_amdgcn_sched_barrier(0);
      copy_P(0, H0{});
      copy_Q(0, H1{});
      copy_P(1, H2{});
      copy_Q(1, H3{});
      copy_P(2, H4{});
      wait_vm<24>();  // the scale words and step 0's copies complete
      lds_barrier();
      read_first(H0{}, H1{});
      const int n_run = nk + pad;
      for (int kt = 0; kt < n_run; kt += 5) steps5(kt);
      wait_vm<0>();   // the zero copies issued past the last step land before LDS is reused
    }
    // every wavefront is done with every half-slot before the epilogue uses LDS
    lds_barrier();

    // ---------------- epilogue ----------------
    // bf16 blocks of 256 rows x 128 columns through LDS, as in the bf16 forward kernel:
    // 256-byte rows, chunk c of row r at c ^ (r & 15), rows 0-127 in the first array of a
    // pair and 128-255 in the second; 4 whole rows leave per store instruction, rows
    // past the expert dropped by the range check.
    int ln = lane, wv = __builtin_amdgcn_readfirstlane(wave);
    asm volatile("" : "+v"(ln));  // keep the lane offsets inside the epilogue
    const int em = wv >> 1, en = wv & 1, e32 = ln & 31, ehi = ln >> 5;
    const int valid = min(row_end - tile_row, kBM);
    auto put = [&](uint8_t* arr0, uint8_t* arr1, int sm, int sq, int i4, uint2 v) __attribute__((always_inline)) {
      uint8_t* arr = em ? arr1 : arr0;
      const int rr = sm * 32 + e32;
      const int ch = en * 8 + sq * 4 + i4;
      *reinterpret_cast<uint2*>(arr + rr * 256 + ((ch ^ (rr & 15)) << 4) + ehi * 8) = v;
    };
    auto drain = [&](const uint8_t* arr, bf16_t* dst, int64_t ld) __attribute__((always_inline)) {
      const int64_t ldb = ld * 2;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(dst + (int64_t)tile_row * ld), (short)0, (int)(uint32_t)(valid * ldb), kBufferFlags);
      const int pc = ln & 15;
      const uint32_t vo = (uint32_t)((ln >> 4) * ldb + pc * 16);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int rl = (wv & 1) * 64 + 4 * i + (ln >> 4);
        const v4u32 val = *reinterpret_cast<const v4u32*>(arr + rl * 256 + ((pc ^ (rl & 15)) << 4));
        __builtin_amdgcn_raw_buffer_store_b128(val, rs, vo, (int)((wv * 64 + 4 * i) * ldb), 0);
      }
    };
    auto acc_block = [&](int b, uint8_t* arr0, uint8_t* arr1) __attribute__((always_inline)) {
#pragma unroll
      for (int sm = 0; sm < 4; ++sm)
#pragma unroll
        for (int sq = 0; sq < 2; ++sq)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int sn = 2 * b + sq;
            put(arr0, arr1, sm, sq, i4,
                make_uint2(pack_bf16x2(acc[sn][sm][i4 * 4 + 0], acc[sn][sm][i4 * 4 + 1]),
                           pack_bf16x2(acc[sn][sm][i4 * 4 + 2], acc[sn][sm][i4 * 4 + 3])));
          }
    };
    if constexpr (EP == MX_STORE || EP == MX_WGRAD) {
      acc_block(0, sH0, sH1);
      acc_block(1, sH2, sH3);
      lds_barrier();
      void* cbase;
      if constexpr (wgrad) cbase = prm.ctab[e];
      else cbase = prm.c;
      bf16_t* c0 = reinterpret_cast<bf16_t*>(cbase) + (int64_t)nt * kBN;
      drain(wv < 2 ? sH0 : sH1, c0, prm.N);
      drain(wv < 2 ? sH2 : sH3, c0 + 128, prm.N);
      lds_barrier();  // read out before the next tile's copies land
    } else {
      constexpr bool save = EP == MX_SWIGLU_SAVE;
#pragma unroll
      for (int sm = 0; sm < 4; ++sm) {
        const int64_t mg = (int64_t)tile_row + wm * 128 + sm * 32 + l32;
        const bool live = mg < row_end;
        const float p = prm.prob[live ? mg : row_end - 1];
#pragma unroll
        for (int sn = 0; sn < 2; ++sn) {
          // h for the 32 columns of sub-tile sn: 16 values here, 16 in lane ^ 32
          float h[16];
          float amax = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            h[i] = silu_f(acc[sn][sm][i]) * acc[sn + 2][sm][i] * p;
            amax = fmaxf(amax, fabsf(h[i]));
          }
          amax = fmaxf(amax, __shfl_xor(amax, 32));
          const int sx = mx_scale_exponent(amax);
          if constexpr (save) {
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4)
              put(sH0, sH1, sm, sn, i4,
                  make_uint2(pack_bf16x2(h[i4 * 4 + 0], h[i4 * 4 + 1]), pack_bf16x2(h[i4 * 4 + 2], h[i4 * 4 + 3])));
          }
          if (live) {
            const int64_t col0 = (int64_t)nt * 128 + wn * 64 + sn * 32;
            uint8_t* C = reinterpret_cast<uint8_t*>(prm.c) + mg * prm.I + col0;
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4)
              *reinterpret_cast<uint32_t*>(C + i4 * 8 + lhi * 4) =
                  e4m3_pack4(ldexpf(h[i4 * 4], -sx), ldexpf(h[i4 * 4 + 1], -sx), ldexpf(h[i4 * 4 + 2], -sx),
                             ldexpf(h[i4 * 4 + 3], -sx));
            // step-major: word nt * R + mg (the down GEMM's K step nt), byte wn * 2 + sn
            if (lhi == 0) prm.c_s[((int64_t)nt * R + mg) * 4 + wn * 2 + sn] = (uint8_t)(sx + 127);
          }
        }
      }
      if constexpr (save) {  // h (bf16, in sH0/sH1), z's gate half (sH2/sH3), then z's up half
        const int64_t I2 = 2 * (int64_t)prm.I;
        acc_block(0, sH2, sH3);
        lds_barrier();
        drain(wv < 2 ? sH0 : sH1, reinterpret_cast<bf16_t*>(prm.h_save) + (int64_t)nt * 128, prm.I);
        drain(wv < 2 ? sH2 : sH3, reinterpret_cast<bf16_t*>(prm.z_save) + (int64_t)nt * 128, I2);
        lds_barrier();
        acc_block(1, sH0, sH1);
        lds_barrier();
        drain(wv < 2 ? sH0 : sH1, reinterpret_cast<bf16_t*>(prm.z_save) + prm.I + (int64_t)nt * 128, I2);
      }
      lds_barrier();  // read out before the next tile's copies land
    }
  }
}

// pt: per-tensor FP8; else MXFP8 with step-major scales (sm, the wide-step kernel) or
// public-layout scales (the 64-value-step kernel)
static moe_status launch(int ep, bool pt, const MxParams& p, int64_t max_tiles, hipStream_t s, const char* what,
                         bool sm = false) {
  if (max_tiles <= 0) return MOE_OK;
  int64_t grid = num_cus();
  if (max_tiles < grid) grid = max_tiles;
  const dim3 g((unsigned)grid), b(256);
  if (pt) {
    if (ep == MX_SWIGLU && p.z_save) hipLaunchKernelGGL((grouped_gemm_fp8t_kernel<MX_SWIGLU_SAVE>), g, b, 0, s, p);
    else if (ep == MX_SWIGLU) hipLaunchKernelGGL((grouped_gemm_fp8t_kernel<MX_SWIGLU>), g, b, 0, s, p);
    else hipLaunchKernelGGL((grouped_gemm_fp8t_kernel<MX_STORE>), g, b, 0, s, p);
  } else if (sm) {
    if (ep == MX_SWIGLU && p.z_save) hipLaunchKernelGGL((grouped_gemm_mxw_kernel<MX_SWIGLU_SAVE>), g, b, 0, s, p);
    else if (ep == MX_SWIGLU) hipLaunchKernelGGL((grouped_gemm_mxw_kernel<MX_SWIGLU>), g, b, 0, s, p);
    else hipLaunchKernelGGL((grouped_gemm_mxw_kernel<MX_STORE>), g, b, 0, s, p);
  } else {
    if (ep == MX_SWIGLU) hipLaunchKernelGGL((grouped_gemm_mx_kernel<MX_SWIGLU>), g, b, 0, s, p);
    else hipLaunchKernelGGL((grouped_gemm_mx_kernel<MX_STORE>), g, b, 0, s, p);
  }
  return check_launch(what);
}

// pt: per-tensor FP8 (factors q_s[0] and tab_s[0][0]); else MXFP8 with step-major scales
static moe_status launch_wgrad(const MxWgradParams& p, int64_t max_tiles, hipStream_t s, const char* what,
                               bool pt = false) {
  if (max_tiles <= 0) return MOE_OK;
  int64_t grid = num_cus();
  if (max_tiles < grid) grid = max_tiles;
  if (pt) hipLaunchKernelGGL((grouped_gemm_fp8t_kernel<MX_WGRAD, MxWgradParams>), dim3((unsigned)grid), dim3(256), 0, s, p);
  else hipLaunchKernelGGL((grouped_gemm_mxw_kernel<MX_WGRAD, MxWgradParams>), dim3((unsigned)grid), dim3(256), 0, s, p);
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
                   uint8_t* h_scale, hipStream_t s, void* z_save, void* h_save, bool step_major) {
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
  p.z_save = z_save;
  p.h_save = h_save;
  const int64_t mtiles = (R + kBM - 1) / kBM + E;
  return launch(MX_SWIGLU, false, p, mtiles * p.n_tiles, s, "MXFP8 gate_up + ScaledSwiGLU", step_major);
}

static moe_status down(int E, int64_t R, int H, int I, const uint8_t* h, const uint8_t* h_scale,
                       const uint8_t* const* w, const uint8_t* const* w_scale, const int32_t* offsets, void* y,
                       hipStream_t s, bool step_major) {
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
  return launch(MX_STORE, false, p, mtiles * p.n_tiles, s, "MXFP8 down", step_major);
}

static size_t a256(size_t x) { return align_up(x, 256); }

// MXFP8 forward on the wide-step kernels, every scale array step-major. Workspace: x's
// codes and scales (bf16 x) or its scales converted (MXFP8 x), the same per expert for
// W1 and W2, then h's codes and scales.
moe_status forward(const moe_mlp_desc& d, int64_t R, const void* x_perm, const uint8_t* x_perm_scale,
                   const void* const* w_gate_up, const void* const* w_down, const uint8_t* const* w_gate_up_scale,
                   const uint8_t* const* w_down_scale, const int32_t* offsets, const float* prob_perm,
                   void* y_perm, uint8_t* ws, hipStream_t s, void* z_save,
                   void* h_save) {
  const int E = d.E, H = d.H, I = d.I;
  moe_status st = check_mx_shape(E, H, I, "moe_grouped_mlp_fwd");
  if (st != MOE_OK) return st;
  // activations: quantised in the call when given as bf16, else their scales converted
  const uint8_t* xq = reinterpret_cast<const uint8_t*>(x_perm);
  uint8_t* xs = nullptr;
  if (d.act == MOE_BF16) {
    uint8_t* q = ws;
    ws += a256((size_t)R * H);
    xs = ws;
    ws += a256((size_t)R * H / 32);
    if ((st = launch_mxfp8_quantize_step_major(x_perm, R, H, q, xs, s)) != MOE_OK) return st;
    xq = q;
  } else {
    xs = ws;
    ws += a256((size_t)R * H / 32);
    uint8_t* dst[1] = {xs};
    if ((st = launch_mx_scales_step_major(&x_perm_scale, dst, 1, R, H, s)) != MOE_OK) return st;
  }
  // weights: bf16 master weights quantised in the call, or MXFP8 with their scales converted
  const uint8_t* w1q[kMaxE];
  uint8_t* w1s[kMaxE];
  const uint8_t* w2q[kMaxE];
  uint8_t* w2s[kMaxE];
  for (int e = 0; e < E; ++e) {
    if (d.wt == MOE_BF16) {
      uint8_t* a = ws;
      ws += a256((size_t)2 * I * H);
      w1s[e] = ws;
      ws += a256((size_t)2 * I * H / 32);
      uint8_t* b = ws;
      ws += a256((size_t)H * I);
      w2s[e] = ws;
      ws += a256((size_t)H * I / 32);
      if ((st = launch_mxfp8_quantize_step_major(w_gate_up[e], 2 * I, H, a, w1s[e], s)) != MOE_OK) return st;
      if ((st = launch_mxfp8_quantize_step_major(w_down[e], H, I, b, w2s[e], s)) != MOE_OK) return st;
      w1q[e] = a;
      w2q[e] = b;
    } else {
      w1q[e] = reinterpret_cast<const uint8_t*>(w_gate_up[e]);
      w2q[e] = reinterpret_cast<const uint8_t*>(w_down[e]);
      w1s[e] = ws;
      ws += a256((size_t)2 * I * H / 32);
      w2s[e] = ws;
      ws += a256((size_t)H * I / 32);
    }
  }
  if (d.wt != MOE_BF16) {
    if ((st = launch_mx_scales_step_major(w_gate_up_scale, w1s, E, 2 * (int64_t)I, H, s)) != MOE_OK) return st;
    if ((st = launch_mx_scales_step_major(w_down_scale, w2s, E, H, I, s)) != MOE_OK) return st;
  }
  uint8_t* hq = ws;
  ws += a256((size_t)R * I);
  uint8_t* hs = ws;
  st = gate_up(E, R, H, I, xq, xs, reinterpret_cast<const void* const*>(w1q), w1s, offsets, prob_perm, hq, hs, s,
               z_save, h_save, true);
  if (st != MOE_OK) return st;
  return down(E, R, H, I, hq, hs, w2q, w2s, offsets, y_perm, s, true);
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
                              void* y_perm, uint8_t* ws, hipStream_t s, void* z_save, void* h_save) {
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

  // h in bf16 (its factor needs all of it first): the caller's h_save when saving
  bf16_t* h = h_save ? reinterpret_cast<bf16_t*>(h_save) : reinterpret_cast<bf16_t*>(ws);
  ws += a256((size_t)R * I * 2);
  uint8_t* hq = ws;
  const int64_t mtiles = (R + kBM - 1) / kBM + E;

  g.q = xq;
  g.q_s = reinterpret_cast<const uint8_t*>(xs);
  g.c = h;
  g.z_save = z_save;
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

// ---------------------------------------------------------------------------------
// MXFP8 backward: every GEMM takes its operands in MXFP8 along that GEMM's own K axis.
//   dH  = dY W2_e      : dY by rows (along H), W2_e along H (column-wise, per expert)
//   dZ  = dSwiGLU(dH, z, prob), dprob   (float32 from bf16 dH and z; dZ stored in bf16)
//   dx  = dZ W1_e      : dZ by rows (along 2I), W1_e along 2I
//   dW2 = dY_e^T h_e   : both along the expert's rows (token-axis layout, experts padded
//   dW1 = dZ_e^T x_e     to whole 256-row K steps; empty experts give zero gradients)
// ---------------------------------------------------------------------------------

namespace {

// dH [R, I] and z = [G, U] [R, 2I] (bf16) -> dZ = [dG, dU] (bf16), dprob[r] = sum dH * A
// with A = silu(G) U (the probability's gradient), dA = dH p. One workgroup per row.
// amax (optional): raised to the float bits of max |dZ| over the stored bf16 values (an
// integer max of non-negative float bits, as fp8t_amax computes it).
__global__ __launch_bounds__(256) void mx_dswiglu_kernel(const bf16_t* __restrict__ dh, const bf16_t* __restrict__ z,
                                                         const float* __restrict__ prob, bf16_t* __restrict__ dz,
                                                         float* __restrict__ dprob, int I,
                                                         uint32_t* __restrict__ amax) {
  const int64_t r = blockIdx.x;
  const float p = prob[r];
  const bf16_t* dhr = dh + r * I;
  const bf16_t* zr = z + r * 2 * I;
  bf16_t* dzr = dz + r * 2 * I;
  float acc = 0.f;
  uint32_t mbits = 0;  // max bf16 magnitude bits of the stored dZ
  for (int c = threadIdx.x * 8; c < I; c += 256 * 8) {
    const uint4 dv = *reinterpret_cast<const uint4*>(dhr + c);
    const uint4 gv = *reinterpret_cast<const uint4*>(zr + c);
    const uint4 uv = *reinterpret_cast<const uint4*>(zr + I + c);
    const uint32_t dw[4] = {dv.x, dv.y, dv.z, dv.w}, gw[4] = {gv.x, gv.y, gv.z, gv.w}, uw[4] = {uv.x, uv.y, uv.z, uv.w};
    uint32_t og[4], ou[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float dg2[2], du2[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const float d = bf16_to_f32(h ? dw[j] >> 16 : dw[j] & 0xFFFFu);
        const float G = bf16_to_f32(h ? gw[j] >> 16 : gw[j] & 0xFFFFu);
        const float U = bf16_to_f32(h ? uw[j] >> 16 : uw[j] & 0xFFFFu);
        const float sg = sigmoid_f(G);
        acc += d * (G * sg * U);
        const float dA = d * p;
        dg2[h] = dA * U * sg * (1.f + G * (1.f - sg));
        du2[h] = dA * G * sg;
      }
      og[j] = pack_bf16x2(dg2[0], dg2[1]);
      ou[j] = pack_bf16x2(du2[0], du2[1]);
      mbits = max(mbits, max(max(og[j] & 0x7FFFu, (og[j] >> 16) & 0x7FFFu), max(ou[j] & 0x7FFFu, (ou[j] >> 16) & 0x7FFFu)));
    }
    *reinterpret_cast<uint4*>(dzr + c) = make_uint4(og[0], og[1], og[2], og[3]);
    *reinterpret_cast<uint4*>(dzr + I + c) = make_uint4(ou[0], ou[1], ou[2], ou[3]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  __shared__ float red[4];
  __shared__ uint32_t mred[4];
  if (amax) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mbits = max(mbits, (uint32_t)__shfl_xor((int)mbits, off));
  }
  if ((threadIdx.x & 63) == 0) {
    red[threadIdx.x >> 6] = acc;
    mred[threadIdx.x >> 6] = mbits;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    dprob[r] = (red[0] + red[1]) + (red[2] + red[3]);
    const uint32_t m = max(max(mred[0], mred[1]), max(mred[2], mred[3]));
    if (amax && m) atomicMax(amax, m << 16);
  }
}

// dSwiGLU fused with both MXFP8 quantisations of dZ, so dZ never goes through HBM in
// bf16: dZ = [dG, dU] is formed as mx_dswiglu_kernel forms it (the same float32
// operations, then rounded to bf16), quantised by rows (K = 2I of the dx GEMM; the rule
// and step-major layout of launch_mxfp8_quantize_step_major) and along each expert's
// tokens (K of the dW1 GEMM; the rule and step-major layout of launch_mxfp8_colwise
// with pad 256), so the codes are those of the separate kernels bit for bit. An item is
// 128 rows of one expert's 256-padded row range (rows past the expert are zeros) by 64
// columns of I, i.e. 64 gate and 64 up columns of dZ: thread t loads rows t / 8 + 32 i
// (i < 4), columns 8 (t % 8) .. + 8 of dH, G and U (16-byte loads); 4 threads own a
// 32-value row block; the token-axis blocks go through an LDS tile as in the
// column-wise quantiser. dprob: one partial per row and item, part[r * I / 64 + cb],
// summed in a fixed order by mx_dprob_sum_kernel.
__global__ __launch_bounds__(256) void mx_dswiglu_quant_kernel(
    const bf16_t* __restrict__ dh, const bf16_t* __restrict__ z, const float* __restrict__ prob,
    const int32_t* __restrict__ offsets, int E, int R, int I, int64_t kcap, uint8_t* __restrict__ dzq,
    uint8_t* __restrict__ dzs, uint8_t* __restrict__ dzc, uint8_t* __restrict__ dzcs, float* __restrict__ part) {
  __shared__ int32_t s_off[kMaxE + 1];
  __shared__ int32_t s_kofs[kMaxE + 1];
  __shared__ int32_t s_item[kMaxE + 1];
  __shared__ float tile[128][65];
  const int tid = threadIdx.x;
  const int ncb = I / 64;
  const int64_t I2 = 2 * (int64_t)I;
  if (tid == 0) {  // offsets made nondecreasing inside [0, R]; experts padded to 256 rows
    int prev = 0, kacc = 0, iacc = 0;
    for (int e = 0; e <= E; ++e) {
      int v = e == 0 ? 0 : offsets[e];
      v = v < prev ? prev : v;
      v = v > R ? R : v;
      if (e > 0) {
        const int kp = (v - prev + 255) / 256 * 256;
        s_kofs[e - 1] = kacc;
        s_item[e - 1] = iacc;
        kacc += kp;
        iacc += kp / 128 * ncb;
      }
      s_off[e] = v;
      prev = v;
    }
    s_kofs[E] = kacc;
    s_item[E] = iacc;
  }
  __syncthreads();
  const int total = s_item[E];
  const int r = tid >> 3, c8 = (tid & 7) * 8;  // load and row blocks: rows r + 32 i, columns c8 .. c8 + 7
  const int cc = tid & 63, q = tid >> 6;        // token blocks: rows 32 q .. 32 q + 31 of column cc
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_item[mid] <= item) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int local = item - s_item[e];
    const int j = local / ncb, cb = local - (local / ncb) * ncb;
    const int row_end = s_off[e + 1];
    const int64_t k0 = (int64_t)s_kofs[e] + 128 * j;
    uint32_t g_bits[4][4], u_bits[4][4];  // dG, dU of this thread's 4 rows x 8 columns, bf16 pairs
    // all four rows' loads first, so they are in flight together (an item has at least
    // one live row: rows past the expert read the expert's last row and count as zeros)
    uint4 dvs[4], gvs[4], uvs[4];
    float ps[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int row = s_off[e] + 128 * j + r + 32 * i;
      row = row < row_end ? row : row_end - 1;
      dvs[i] = *reinterpret_cast<const uint4*>(dh + (int64_t)row * I + cb * 64 + c8);
      gvs[i] = *reinterpret_cast<const uint4*>(z + (int64_t)row * I2 + cb * 64 + c8);
      uvs[i] = *reinterpret_cast<const uint4*>(z + (int64_t)row * I2 + I + cb * 64 + c8);
      ps[i] = prob[row];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = s_off[e] + 128 * j + r + 32 * i;
      const bool live = row < row_end;
      const uint4 zero = make_uint4(0, 0, 0, 0);
      const uint4 dv = live ? dvs[i] : zero, gv = live ? gvs[i] : zero, uv = live ? uvs[i] : zero;
      const float p = live ? ps[i] : 0.f;
      const uint32_t dw[4] = {dv.x, dv.y, dv.z, dv.w}, gw[4] = {gv.x, gv.y, gv.z, gv.w},
                     uw[4] = {uv.x, uv.y, uv.z, uv.w};
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float dg2[2], du2[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const float d = bf16_to_f32(hh ? dw[w] >> 16 : dw[w] & 0xFFFFu);
          const float G = bf16_to_f32(hh ? gw[w] >> 16 : gw[w] & 0xFFFFu);
          const float U = bf16_to_f32(hh ? uw[w] >> 16 : uw[w] & 0xFFFFu);
          const float sg = sigmoid_f(G);
          acc += d * (G * sg * U);
          const float dA = d * p;
          dg2[hh] = dA * U * sg * (1.f + G * (1.f - sg));
          du2[hh] = dA * G * sg;
        }
        g_bits[i][w] = pack_bf16x2(dg2[0], dg2[1]);
        u_bits[i][w] = pack_bf16x2(du2[0], du2[1]);
      }
      // dprob partial of the row: the 8 threads of a row, in a fixed order
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      acc += __shfl_xor(acc, 4);
      if (live && (tid & 7) == 0) part[(int64_t)row * ncb + cb] = acc;
      // row blocks of 32 values (4 threads each), gate then up
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const uint32_t* b = half ? u_bits[i] : g_bits[i];
        float f[8];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          f[2 * w] = bf16_to_f32(b[w] & 0xFFFFu);
          f[2 * w + 1] = bf16_to_f32(b[w] >> 16);
        }
        float amax = 0.f;
#pragma unroll
        for (int w = 0; w < 8; ++w) amax = fmaxf(amax, fabsf(f[w]));
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        amax = fmaxf(amax, __shfl_xor(amax, 2));
        const int sx = mx_scale_exponent(amax);
        if (live) {
          const int64_t col = (int64_t)half * I + cb * 64 + c8;
          *reinterpret_cast<uint2*>(dzq + (int64_t)row * I2 + col) =
              make_uint2(e4m3_pack4(ldexpf(f[0], -sx), ldexpf(f[1], -sx), ldexpf(f[2], -sx), ldexpf(f[3], -sx)),
                         e4m3_pack4(ldexpf(f[4], -sx), ldexpf(f[5], -sx), ldexpf(f[6], -sx), ldexpf(f[7], -sx)));
          if ((tid & 3) == 0) {  // step-major: block bc = col / 32 of row `row`
            const int64_t bc = col >> 5;
            dzs[((bc >> 2) * R + row) * 4 + (bc & 3)] = (uint8_t)(sx + 127);
          }
        }
      }
    }
    // token blocks: gate columns, then up columns, through the LDS tile
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t* b = half ? u_bits[i] : g_bits[i];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          tile[r + 32 * i][c8 + 2 * w] = bf16_to_f32(b[w] & 0xFFFFu);
          tile[r + 32 * i][c8 + 2 * w + 1] = bf16_to_f32(b[w] >> 16);
        }
      }
      __syncthreads();
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(tile[32 * q + i][cc]));
      const int sx = mx_scale_exponent(amax);
      uint32_t wd[8];
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const float* t = &tile[32 * q + 4 * g][cc];
        wd[g] = e4m3_pack4(ldexpf(t[0], -sx), ldexpf(t[65], -sx), ldexpf(t[130], -sx), ldexpf(t[195], -sx));
      }
      const int64_t col = (int64_t)half * I + cb * 64 + cc;
      const int64_t k = k0 + 32 * q;
      uint4* dst = reinterpret_cast<uint4*>(dzc + col * kcap + k);
      dst[0] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
      dst[1] = make_uint4(wd[4], wd[5], wd[6], wd[7]);
      dzcs[((k >> 7) * I2 + col) * 4 + ((k >> 5) & 3)] = (uint8_t)(sx + 127);
      __syncthreads();  // the tile is rewritten next
    }
  }
}

// dprob[r] = the sum of the row's I / 64 partials: one wavefront per row, lane l adds
// blocks l, l + 64, ... in order, then a butterfly over the lanes (a fixed order, so
// the result does not change from run to run)
__global__ __launch_bounds__(256) void mx_dprob_sum_kernel(const float* __restrict__ part, int R, int ncb,
                                                           float* __restrict__ dprob) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= R) return;
  const float* pr = part + (int64_t)r * ncb;
  float acc = 0.f;
  for (int c = lane; c < ncb; c += 64) acc += pr[c];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) dprob[r] = acc;
}

// token-axis layout: every expert padded to whole 256-row K steps of the GEMM
int64_t bwd_kcap(int64_t R, int E) { return (R + (int64_t)E * 255 + 255) / 256 * 256; }

struct BwdLayout {
  size_t dyq, dys, w2c, w2s, w1c, w1s, dh, dz, dzq, dzs, dyc, dycs, hc, hcs, dzc, dzcs, xc, xcs, kofs, total;
};

BwdLayout bwd_layout(const moe_mlp_desc& d, int64_t R) {
  const size_t H = d.H, I = d.I, E = d.E, kc = (size_t)bwd_kcap(R, d.E);
  BwdLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += a256(bytes); return at; };
  L.dyq = take(R * H);
  L.dys = take(R * H / 32);
  if (d.wt == MOE_BF16) {  // column-wise weight copies (packed weights bring their own)
    L.w2c = take(E * I * H);
    L.w2s = take(E * I * H / 32);
    L.w1c = take(E * H * 2 * I);
    L.w1s = take(E * H * 2 * I / 32);
  }
  L.dh = take(R * I * 2);
  L.dz = take(R * (I / 64) * 4);  // dprob partials (dZ itself is only stored as MXFP8)
  L.dzq = take(R * 2 * I);
  L.dzs = take(R * 2 * I / 32);
  L.dyc = take(H * kc);
  L.dycs = take(H * kc / 32);
  L.hc = take(I * kc);
  L.hcs = take(I * kc / 32);
  L.dzc = take(2 * I * kc);
  L.dzcs = take(2 * I * kc / 32);
  L.xc = take(H * kc);
  L.xcs = take(H * kc / 32);
  L.kofs = take((E + 1) * 4);
  L.total = o;
  return L;
}

}  // namespace

size_t bwd_workspace_bytes(const moe_mlp_desc& d, int64_t R) { return bwd_layout(d, R).total; }

moe_status backward(const moe_mlp_desc& d, int64_t R, const bf16_t* dy, const bf16_t* x, const bf16_t* z,
                    const bf16_t* h, const float* prob, const void* const* w_gate_up, const void* const* w_down,
                    const int32_t* offsets, bf16_t* dx, void* const* dw_gate_up, void* const* dw_down, float* dprob,
                    uint8_t* ws, hipStream_t s) {
  const int E = d.E, H = d.H, I = d.I;
  moe_status st = check_mx_shape(E, H, I, "moe_grouped_mlp_bwd");
  if (st != MOE_OK) return st;
  const int64_t kc = bwd_kcap(R, E);
  if ((int64_t)2 * I * kc > 0x7FFFFFFFLL || (int64_t)H * kc > 0x7FFFFFFFLL)
    return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_mlp_bwd: MXFP8 token-axis operands exceed 2^31 bytes");
  const BwdLayout L = bwd_layout(d, R);
  uint8_t *dyq = ws + L.dyq, *dys = ws + L.dys, *dzq = ws + L.dzq, *dzs = ws + L.dzs;
  bf16_t* dh = (bf16_t*)(ws + L.dh);
  float* part = (float*)(ws + L.dz);
  int32_t* kofs = (int32_t*)(ws + L.kofs);
  const size_t w2n = (size_t)I * H, w1n = (size_t)H * 2 * I;
  const int64_t mtiles = (R + kBM - 1) / kBM + E;

  // Weights along the data gradients' K axes: W2_e along H ([I][H] codes), W1_e along 2I
  // ([H][2I]), step-major scales; quantised here from bf16 master weights, or packed by
  // the caller (mxfp8_pack_weight_bwd: codes, then the scales).
  const bool packed = d.wt == MOE_MXFP8;
  auto w2_codes = [&](int e) -> const uint8_t* {
    return packed ? reinterpret_cast<const uint8_t*>(w_down[e]) : ws + L.w2c + e * w2n;
  };
  auto w1_codes = [&](int e) -> const uint8_t* {
    return packed ? reinterpret_cast<const uint8_t*>(w_gate_up[e]) : ws + L.w1c + e * w1n;
  };
  // dH = dY W2_e (the data gradients run on the wide-step kernel: step-major scales).
  // dY is quantised by rows (for dH) and along the tokens (for dW2) from one read.
  if ((st = launch_mxfp8_colwise(dy, R, H, E, offsets, 256, kc, ws + L.dyc, ws + L.dycs, kofs, s, true, dyq, dys,
                                 R)) != MOE_OK)
    return st;
  const void* wsrc[kMaxE];
  uint8_t* wcodes[kMaxE];
  uint8_t* wscales[kMaxE];
  if (!packed) {
    for (int e = 0; e < E; ++e) {
      wsrc[e] = w_down[e];
      wcodes[e] = ws + L.w2c + e * w2n;
      wscales[e] = ws + L.w2s + e * w2n / 32;
    }
    if ((st = launch_mxfp8_colwise_multi(E, wsrc, H, I, 1, nullptr, 32, H, wcodes, wscales, nullptr, s, true)) !=
        MOE_OK)
      return st;
  }
  MxParams p;
  std::memset(&p, 0, sizeof(p));
  for (int e = 0; e < E; ++e) {
    p.tab[e] = w2_codes(e);
    p.tab_s[e] = packed ? w2_codes(e) + w2n : ws + L.w2s + e * w2n / 32;
  }
  p.q = dyq;
  p.q_s = dys;
  p.c = dh;
  p.offsets = offsets;
  p.R = R;
  p.K = H;
  p.N = I;
  p.E = E;
  p.I = I;
  p.n_tiles = I / kBN;
  if ((st = launch(MX_STORE, false, p, mtiles * p.n_tiles, s, "MXFP8 down dgrad", true)) != MOE_OK) return st;

  // dZ (never stored in bf16: quantised by rows for dx and along the tokens for dW1 in
  // the same kernel) and dprob (partials per 64 columns, then summed in order)
  if (R > 0) {
    const int64_t items = (kc / 128) * (I / 64);
    const int64_t grid = items < (int64_t)num_cus() * 8 ? items : (int64_t)num_cus() * 8;
    hipLaunchKernelGGL(mx_dswiglu_quant_kernel, dim3((unsigned)grid), dim3(256), 0, s, dh, z, prob, offsets, E,
                       (int)R, I, kc, dzq, dzs, ws + L.dzc, ws + L.dzcs, part);
    if ((st = check_launch("MXFP8 dSwiGLU + dZ quantisation")) != MOE_OK) return st;
    hipLaunchKernelGGL(mx_dprob_sum_kernel, dim3((unsigned)((R + 3) / 4)), dim3(256), 0, s, part, (int)R, I / 64,
                       dprob);
    if ((st = check_launch("MXFP8 dprob")) != MOE_OK) return st;
  }

  // dx = dZ W1_e
  if (!packed) {
    for (int e = 0; e < E; ++e) {
      wsrc[e] = w_gate_up[e];
      wcodes[e] = ws + L.w1c + e * w1n;
      wscales[e] = ws + L.w1s + e * w1n / 32;
    }
    if ((st = launch_mxfp8_colwise_multi(E, wsrc, 2 * I, H, 1, nullptr, 32, 2 * I, wcodes, wscales, nullptr, s,
                                         true)) != MOE_OK)
      return st;
  }
  for (int e = 0; e < E; ++e) {
    p.tab[e] = w1_codes(e);
    p.tab_s[e] = packed ? w1_codes(e) + w1n : ws + L.w1s + e * w1n / 32;
  }
  p.q = dzq;
  p.q_s = dzs;
  p.c = dx;
  p.K = 2 * I;
  p.N = H;
  p.n_tiles = H / kBN;
  if ((st = launch(MX_STORE, false, p, mtiles * p.n_tiles, s, "MXFP8 gate_up dgrad", true)) != MOE_OK) return st;

  // weight gradients on the token-axis layouts (wide-step kernel: step-major scales)
  if ((st = launch_mxfp8_colwise(h, R, I, E, offsets, 256, kc, ws + L.hc, ws + L.hcs, nullptr, s, true)) != MOE_OK)
    return st;
  MxWgradParams w;
  std::memset(&w, 0, sizeof(w));
  w.kofs = kofs;
  w.E = E;
  w.ld = (int)kc;
  w.q = ws + L.dyc;
  w.q_s = ws + L.dycs;
  w.tab[0] = ws + L.hc;
  w.tab_s[0] = ws + L.hcs;
  for (int e = 0; e < E; ++e) w.ctab[e] = dw_down[e];
  w.R = H;
  w.N = I;
  w.I = I;
  w.n_tiles = I / kBN;
  if ((st = launch_wgrad(w, (int64_t)E * (H / kBM) * w.n_tiles, s, "MXFP8 down wgrad")) != MOE_OK) return st;
  if ((st = launch_mxfp8_colwise(x, R, H, E, offsets, 256, kc, ws + L.xc, ws + L.xcs, nullptr, s, true)) != MOE_OK)
    return st;
  w.q = ws + L.dzc;
  w.q_s = ws + L.dzcs;
  w.tab[0] = ws + L.xc;
  w.tab_s[0] = ws + L.xcs;
  for (int e = 0; e < E; ++e) w.ctab[e] = dw_gate_up[e];
  w.R = 2 * I;
  w.N = H;
  w.n_tiles = H / kBN;
  return launch_wgrad(w, (int64_t)E * (2 * I / kBM) * w.n_tiles, s, "MXFP8 gate_up wgrad");
}


// ---------------------------------------------------------------------------------
// Per-tensor FP8 backward: every GEMM operand is one tensor with one factor (amax /
// 448): dY, dZ, h and x over all routed rows, W1_e and W2_e per expert. A factor per
// tensor does not depend on the axis a GEMM reduces over, so each tensor is quantised
// once: row-major codes of dY and dZ for the data gradients, their transposed
// token-axis codes (experts padded to whole 256-row K steps) and those of h and x for
// the weight gradients, the weights' transposed codes for the data gradients.
//   dH = dY W2_e, dSwiGLU -> dZ (bf16), dprob, dx = dZ W1_e, dW2 = dY^T h, dW1 = dZ^T x
// Factor words: [dY, h, x, W1_0 .. W1_E-1, W2_0 .. W2_E-1, dZ] (amax bits, then scales).
// Weights packed by fp8_tensor_pack_weight_bwd (wt = FP8) bring their transposed codes
// and factor: codes at the pointer, the float32 factor rows * cols bytes further.
// ---------------------------------------------------------------------------------

namespace {

struct Fp8BwdLayout {
  size_t words, dyq, dyc, w2t, w1t, dh, dz, dzq, dzc, hc, xc, kofs, total;
};

Fp8BwdLayout fp8_bwd_layout(const moe_mlp_desc& d, int64_t R) {
  const size_t H = d.H, I = d.I, E = d.E, kc = (size_t)bwd_kcap(R, d.E);
  Fp8BwdLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += a256(bytes); return at; };
  L.words = take((4 + 2 * E) * 4);
  L.dyq = take(R * H);
  L.dyc = take(H * kc);
  if (d.wt == MOE_BF16) {  // transposed weight codes (packed weights bring their own)
    L.w2t = take(E * I * H);
    L.w1t = take(E * H * 2 * I);
  }
  L.dh = take(R * I * 2);
  L.dz = take(R * 2 * I * 2);
  L.dzq = take(R * 2 * I);
  L.dzc = take(2 * I * kc);
  L.hc = take(I * kc);
  L.xc = take(H * kc);
  L.kofs = take((E + 1) * 4);
  L.total = o;
  return L;
}

// transposed codes of E tensors of one shape, in launches of at most 64 tensors
moe_status transpose_each(const void* const* in, uint8_t* base, size_t stride, int E, int64_t rows, int cols,
                          float* words, hipStream_t s) {
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int n = E - e0 < 64 ? E - e0 : 64;
    uint8_t* out[64];
    for (int i = 0; i < n; ++i) out[i] = base + (size_t)(e0 + i) * stride;
    const moe_status st = fp8t_transpose(in + e0, out, n, rows, cols, 1, nullptr, 32, rows, words + e0, nullptr, s);
    if (st != MOE_OK) return st;
  }
  return MOE_OK;
}

}  // namespace

size_t fp8_bwd_workspace_bytes(const moe_mlp_desc& d, int64_t R) { return fp8_bwd_layout(d, R).total; }

moe_status backward_fp8_tensor(const moe_mlp_desc& d, int64_t R, const bf16_t* dy, const bf16_t* x, const bf16_t* z,
                               const bf16_t* h, const float* prob, const void* const* w_gate_up,
                               const void* const* w_down, const int32_t* offsets, bf16_t* dx, void* const* dw_gate_up,
                               void* const* dw_down, float* dprob, uint8_t* ws, hipStream_t s) {
  const int E = d.E, H = d.H, I = d.I;
  moe_status st = check_mx_shape(E, H, I, "moe_grouped_mlp_bwd");
  if (st != MOE_OK) return st;
  const int64_t kc = bwd_kcap(R, E);
  if ((int64_t)2 * I * kc > 0x7FFFFFFFLL || (int64_t)H * kc > 0x7FFFFFFFLL)
    return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_mlp_bwd: FP8 token-axis operands exceed 2^31 bytes");
  const Fp8BwdLayout L = fp8_bwd_layout(d, R);
  float* words = reinterpret_cast<float*>(ws + L.words);
  float *w_dy = words, *w_h = words + 1, *w_x = words + 2, *w_w1 = words + 3, *w_w2 = words + 3 + E,
        *w_dz = words + 3 + 2 * E;
  uint8_t *dyq = ws + L.dyq, *dyc = ws + L.dyc, *w2t = ws + L.w2t, *w1t = ws + L.w1t, *dzq = ws + L.dzq,
          *dzc = ws + L.dzc, *hc = ws + L.hc, *xc = ws + L.xc;
  bf16_t *dh = (bf16_t*)(ws + L.dh), *dz = (bf16_t*)(ws + L.dz);
  int32_t* kofs = (int32_t*)(ws + L.kofs);
  const size_t w2n = (size_t)I * H, w1n = (size_t)H * 2 * I;
  const int64_t mtiles = (R + kBM - 1) / kBM + E;

  // factors of dY, h, x and the weights; every code array but dZ's
  if ((st = fp8t_zero(words, 4 + 2 * E, s)) != MOE_OK) return st;
  const void* t_dy[1] = {dy};
  const void* t_h[1] = {h};
  const void* t_x[1] = {x};
  if ((st = fp8t_amax(t_dy, 1, R * H, w_dy, s)) != MOE_OK) return st;
  if ((st = fp8t_amax(t_h, 1, R * I, w_h, s)) != MOE_OK) return st;
  if ((st = fp8t_amax(t_x, 1, R * H, w_x, s)) != MOE_OK) return st;
  const bool packed = d.wt == MOE_FP8;
  if (!packed) {
    if ((st = fp8t_amax(w_gate_up, E, (int64_t)2 * I * H, w_w1, s)) != MOE_OK) return st;
    if ((st = fp8t_amax(w_down, E, (int64_t)H * I, w_w2, s)) != MOE_OK) return st;
  }
  uint8_t* o_dyq[1] = {dyq};
  uint8_t* o_dyc[1] = {dyc};
  uint8_t* o_hc[1] = {hc};
  uint8_t* o_xc[1] = {xc};
  if ((st = fp8t_transpose(t_dy, o_dyc, 1, R, H, E, offsets, 256, kc, w_dy, kofs, s, o_dyq)) != MOE_OK) return st;
  if ((st = fp8t_transpose(t_h, o_hc, 1, R, I, E, offsets, 256, kc, w_h, nullptr, s)) != MOE_OK) return st;
  if ((st = fp8t_transpose(t_x, o_xc, 1, R, H, E, offsets, 256, kc, w_x, nullptr, s)) != MOE_OK) return st;
  // W2_e [H][I] -> [I][H] (K = H for dH); W1_e [2I][H] -> [H][2I] (K = 2I for dx)
  if (!packed) {
    if ((st = transpose_each(w_down, w2t, w2n, E, H, I, w_w2, s)) != MOE_OK) return st;
    if ((st = transpose_each(w_gate_up, w1t, w1n, E, 2 * I, H, w_w1, s)) != MOE_OK) return st;
  }
  if ((st = fp8t_finalize(words, 3, s)) != MOE_OK) return st;
  if (!packed && (st = fp8t_finalize(w_w1, 2 * E, s)) != MOE_OK) return st;
  auto w2_codes = [&](int e) -> const uint8_t* {
    return packed ? reinterpret_cast<const uint8_t*>(w_down[e]) : w2t + e * w2n;
  };
  auto w1_codes = [&](int e) -> const uint8_t* {
    return packed ? reinterpret_cast<const uint8_t*>(w_gate_up[e]) : w1t + e * w1n;
  };
  auto w2_factor = [&](int e) -> const uint8_t* {
    return packed ? w2_codes(e) + w2n : reinterpret_cast<const uint8_t*>(w_w2 + e);
  };
  auto w1_factor = [&](int e) -> const uint8_t* {
    return packed ? w1_codes(e) + w1n : reinterpret_cast<const uint8_t*>(w_w1 + e);
  };

  // dH = dY W2_e
  MxParams p;
  std::memset(&p, 0, sizeof(p));
  for (int e = 0; e < E; ++e) {
    p.tab[e] = w2_codes(e);
    p.tab_s[e] = w2_factor(e);
  }
  p.q = dyq;
  p.q_s = reinterpret_cast<const uint8_t*>(w_dy);
  p.c = dh;
  p.offsets = offsets;
  p.R = R;
  p.K = H;
  p.N = I;
  p.E = E;
  p.I = I;
  p.n_tiles = I / kBN;
  if ((st = launch(MX_STORE, true, p, mtiles * p.n_tiles, s, "FP8 down dgrad")) != MOE_OK) return st;

  // dZ, dprob and dZ's amax in one pass; then its row-major and token-axis codes from
  // one read of dZ
  if (R > 0) {
    hipLaunchKernelGGL(mx_dswiglu_kernel, dim3((unsigned)R), dim3(256), 0, s, dh, z, prob, dz, dprob, I,
                       reinterpret_cast<uint32_t*>(w_dz));
    if ((st = check_launch("FP8 dSwiGLU")) != MOE_OK) return st;
  }
  const void* t_dz[1] = {dz};
  uint8_t* o_dzq[1] = {dzq};
  uint8_t* o_dzc[1] = {dzc};
  if ((st = fp8t_transpose(t_dz, o_dzc, 1, R, 2 * I, E, offsets, 256, kc, w_dz, nullptr, s, o_dzq)) != MOE_OK)
    return st;
  if ((st = fp8t_finalize(w_dz, 1, s)) != MOE_OK) return st;

  // dx = dZ W1_e
  for (int e = 0; e < E; ++e) {
    p.tab[e] = w1_codes(e);
    p.tab_s[e] = w1_factor(e);
  }
  p.q = dzq;
  p.q_s = reinterpret_cast<const uint8_t*>(w_dz);
  p.c = dx;
  p.K = 2 * I;
  p.N = H;
  p.n_tiles = H / kBN;
  if ((st = launch(MX_STORE, true, p, mtiles * p.n_tiles, s, "FP8 gate_up dgrad")) != MOE_OK) return st;

  // weight gradients on the token-axis codes
  MxWgradParams w;
  std::memset(&w, 0, sizeof(w));
  w.kofs = kofs;
  w.E = E;
  w.ld = (int)kc;
  w.q = dyc;
  w.q_s = reinterpret_cast<const uint8_t*>(w_dy);
  w.tab[0] = hc;
  w.tab_s[0] = reinterpret_cast<const uint8_t*>(w_h);
  for (int e = 0; e < E; ++e) w.ctab[e] = dw_down[e];
  w.R = H;
  w.N = I;
  w.I = I;
  w.n_tiles = I / kBN;
  if ((st = launch_wgrad(w, (int64_t)E * (H / kBM) * w.n_tiles, s, "FP8 down wgrad", true)) != MOE_OK) return st;
  w.q = dzc;
  w.q_s = reinterpret_cast<const uint8_t*>(w_dz);
  w.tab[0] = xc;
  w.tab_s[0] = reinterpret_cast<const uint8_t*>(w_x);
  for (int e = 0; e < E; ++e) w.ctab[e] = dw_gate_up[e];
  w.R = 2 * I;
  w.N = H;
  w.n_tiles = H / kBN;
  return launch_wgrad(w, (int64_t)E * (2 * I / kBM) * w.n_tiles, s, "FP8 gate_up wgrad", true);
}

}  // namespace mx
}  // namespace moe
