// Persistent grouped GEMM for the forward projections: rows grouped by expert
// (GROUP_M), both operands K-contiguous, bf16 MFMA with float32 accumulation, and the
// plain-store or ScaledSwiGLU epilogue.
//
// Source: GroupedLinear and the fused GroupedLinear -> ScaledSwiGLU -> GroupedLinear
// forward of "Efficient MoE Training for Biological Foundation Models", Challenges 1
// and 3 (gate_up with the routing weight folded into the activation, then down).
//
// Same output tiling, wavefront layout, tile order and epilogues as the general kernel
// in gemm_bf16.hip (256 x 256 tiles, 4 wavefronts of 128 x 128); what differs is the
// copy pipeline, shaped for operands whose rows are K-contiguous:
//   * K steps are 64 wide, so each row of a tile contributes one whole 128-byte cache
//     line per step. Copying whole lines moves twice the bytes per cycle through a
//     CU's global -> LDS path as copying half lines (measured on gfx950, L2-resident
//     source), and at 32-wide steps that path runs close to full in this kernel.
//   * LDS holds a ring of 5 half-slots of 32 KiB (all 160 KiB): step v keeps P in
//     half-slot 2v mod 5 and Q in 2v+1 mod 5. When step kt is done with both of its
//     half-slots, Q of step kt+2 and P of step kt+3 take them, so weight panels, which
//     come from HBM, have about two steps to land and token panels, which other tiles
//     have usually pulled into L2 already, one.
//   * One barrier per step, after the third of its four k16 slices: it publishes step
//     kt+1's copies and frees step kt's half-slots; the copies above are threaded
//     through the fourth slice's MFMAs.
// LDS rows are 128 bytes: chunk c of row r sits at c ^ swz8(r).
#include <type_traits>

#include "common.h"
#include "gemm_bf16.h"
#include "gemm_common.h"
#include "internal.h"

namespace moe {
namespace gemm {

namespace {
constexpr int kWBK = 64;                      // K step
constexpr int kWTile = kBM * kWBK * 2;        // one operand of one K step: a half-slot (32 KiB)
}  // namespace

// TAIL = false: the data-parallel tiles; TAIL = true: one K chunk of a split-K tail
// tile per workgroup (launched after the first, same grid), written as a float32
// partial tile. Two instantiations keep the chunk logic out of the main kernel's
// register allocation.
template <int EP, bool TAIL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void grouped_gemm_fwd_kernel(const Params prm) {
  // one array per half-slot: every LDS access names its array at compile time, so the
  // compiler can tell a copy into one half-slot from reads of another
  __shared__ __attribute__((aligned(1024))) uint8_t sH0[kWTile], sH1[kWTile], sH2[kWTile];
  __shared__ __attribute__((aligned(1024))) uint8_t sH3[kWTile], sH4[kWTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int wm = wave >> 1, wn = wave & 1;
  const int E = prm.E;
  const int R = (int)prm.R;

  const int nwg = gridDim.x;
  const int logical = (nwg % 8 == 0) ? (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8 : blockIdx.x;

  auto hslot = [&](auto H) -> uint8_t* {
    if constexpr (H.value == 0) return sH0;
    else if constexpr (H.value == 1) return sH1;
    else if constexpr (H.value == 2) return sH2;
    else if constexpr (H.value == 3) return sH3;
    else return sH4;
  };

  // Tile order: expert-major, ceil(rows_e / 256) row tiles x n_tiles per expert, row
  // tiles fastest within groups of at most 16 (tile_in_expert). A workgroup's tiles only move forward, so it walks the expert
  // offsets once (wavefront-uniform loads), making them a nondecreasing sequence inside
  // [0, R] on the way: no access leaves the tensors.
  auto clamp_off = [&](int v, int prev) -> int {
    v = v < prev ? prev : v;
    return v > R ? R : v;
  };
  int e_w = 0;
  int ob = 0;
  int oe = clamp_off(load_const(prm.offsets, 1), 0);
  int ts_w = 0;
  int nt_w = ((oe - ob + kBM - 1) / kBM) * prm.n_tiles;
  const int nk = prm.K / kWBK;

  // Split-K tail. All tiles are counted first; when the last round would leave at
  // least half the workgroups idle, its `rem` tiles are cut into `split` K chunks, one
  // per workgroup after the data-parallel rounds, each writing a float32 partial tile
  // for run_tail_reduce to sum.
  int total = 0;
  {
    int prev = 0;
    for (int x = 0; x < E; ++x) {
      const int en = clamp_off(load_const(prm.offsets, x + 1), prev);
      total += ((en - prev + kBM - 1) / kBM) * prm.n_tiles;
      prev = en;
    }
  }
  const int rem = total % nwg;
  int split = 0;
  if (prm.tail_cap > 0 && rem > 0 && rem * 2 <= nwg) {
    split = nwg / rem;
    split = split > 16 ? 16 : split;
    split = split > nk ? nk : split;
    if (rem * split > prm.tail_cap) split = prm.tail_cap / rem;
    if (split < 2) split = 0;
  }
  const int dp_total = split ? total - rem : total;
  const int units = split ? rem * split : 0;
  if (!TAIL && prm.tail_meta && blockIdx.x == 0 && tid == 0) {
    prm.tail_meta[0] = split ? rem : 0;
    prm.tail_meta[1] = split;
    prm.tail_meta[2] = dp_total;
    prm.tail_meta[3] = 0;
  }
  if (TAIL && logical >= units) return;

  const int l32 = lane & 31, lhi = lane >> 5;
  // fragment addresses: sub-tile rows start at multiples of 32, where swz8 depends on
  // the lane's row within the sub-tile only; k16 slice sl is logical chunk 2*sl + lhi
  const uint32_t fragP = (uint32_t)((wn * 64 + l32) * 128);
  const uint32_t fragQ = (uint32_t)((wm * 128 + l32) * 128);
  uint32_t ck[4];
#pragma unroll
  for (int sl = 0; sl < 4; ++sl) ck[sl] = (uint32_t)(((2 * sl + lhi) ^ swz8(l32)) << 4);
  // copies: round i (0..7) of wavefront w fills LDS bytes [(4i + w) KiB, +1 KiB) of a
  // half-slot: rows (4i + w) * 8 + (lane >> 3), physical chunk lane & 7, i.e. logical
  // chunk (lane & 7) ^ swz8(row), which does not depend on the round
  const int kc_row0 = wave * 8 + (lane >> 3);
  const int kc_chunk = (lane & 7) ^ swz8(kc_row0);
  constexpr int64_t kAll = 0xFFFFFFFFll;

  // TAIL: the single work item of this workgroup is K chunk `unit % split` of tail
  // tile `unit / split`
  const int unit = TAIL ? logical : -1;
  const int t_first = TAIL ? dp_total + unit / split : logical;
  const int t_end = TAIL ? t_first + 1 : dp_total;
  const int k0 = TAIL ? (int)((int64_t)nk * (unit % split) / split) : 0;
  const int k1 = TAIL ? (int)((int64_t)nk * (unit % split + 1) / split) : nk;
  const int nkl = k1 - k0;

  for (int t = t_first; t < t_end; t += nwg) {
    // ---------------- tile decode ----------------
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
    int e = e_w, mt, nt;
    {
      const int local = t - ts_w;
      const int mte = (oe - ob + kBM - 1) / kBM;
      tile_in_expert(local, mte, prm.n_tiles, mt, nt);
    }
    e = __builtin_amdgcn_readfirstlane(e);
    mt = __builtin_amdgcn_readfirstlane(mt);
    nt = __builtin_amdgcn_readfirstlane(nt);
    const int row_beg = __builtin_amdgcn_readfirstlane(ob);
    const int row_end = __builtin_amdgcn_readfirstlane(oe);
    const int tile_row = row_beg + mt * kBM;

    // ---------------- operands ----------------
    // Each copy addresses the step's tile origin + this lane's offset + the round's
    // wavefront-uniform row offset (the buffer instruction's scalar offset). Q's record
    // count ends at the expert's last row: the rows past it fail the hardware range
    // check (which covers the scalar offset) and land as zeros, discarded below.
    // a K chunk [k0, k1) starts k0 steps into the rows: the tile origins move by k0
    // steps, and Q's record count (measured from its origin) shrinks by as much
    const bf16_t* pbase = reinterpret_cast<const bf16_t*>(prm.tab[e]);
    const int64_t kshift = (int64_t)k0 * kWBK * 2;
    const char* p_tile;
    if constexpr (EP == EPI_SWIGLU) p_tile = reinterpret_cast<const char*>(pbase + (int64_t)nt * 128 * prm.p_ld);
    else p_tile = reinterpret_cast<const char*>(pbase + (int64_t)nt * kBN * prm.p_ld);
    p_tile += kshift;
    const char* q_tile = reinterpret_cast<const char*>(prm.q + (int64_t)tile_row * prm.q_ld) + kshift;
    const uint32_t p_off0 = (uint32_t)(((int64_t)kc_row0 * prm.p_ld + kc_chunk * 8) * 2);
    const uint32_t q_off0 = (uint32_t)(((int64_t)kc_row0 * prm.q_ld + kc_chunk * 8) * 2);
    const int64_t q_extent = (int64_t)(row_end - tile_row) * prm.q_ld * 2 - kshift;
    // SWIGLU: tile rows 128..255 of P are the up rows, I further down than the gate rows
    const int p_up = (EP == EPI_SWIGLU) ? prm.I - 128 : 0;

    // one operand of K step kt into a half-slot; round i's rows: i * 32 (+ up for i >= 4),
    // below 2^32 bytes from the tile origin (one expert's weight)
    auto copy_op = [&](const char* tile, uint32_t off0, int up, int64_t ld, int64_t extent, int kt, uint8_t* dst) {
      const int64_t at = (int64_t)kt * kWBK * 2;
      int64_t nrec = extent - at;
      nrec = nrec < 0 ? 0 : (nrec > kAll ? kAll : nrec);
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)(tile + at), (short)0, (int)(uint32_t)nrec, kBufferFlags);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t rows = (uint32_t)(i * 32 + (i >= 4 ? up : 0));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(dst + i * 4096), 16, off0,
                                                 (int)(rows * (uint32_t)ld * 2u), 0, 0);
      }
    };
    // the LDS destination (M0) is wavefront-uniform: computed in scalar registers
    auto copy_P = [&](int kt, auto H) { copy_op(p_tile, p_off0, p_up, prm.p_ld, kAll, kt, hslot(H) + wave_u * 1024); };
    auto copy_Q = [&](int kt, auto H) { copy_op(q_tile, q_off0, 0, prm.q_ld, q_extent, kt, hslot(H) + wave_u * 1024); };

    f32x16 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

    // fragments of one k16 slice: 4 of P (n sub-tiles), 4 of Q (m sub-tiles), read in
    // the order the MFMAs consume them (P 0 with all of Q first)
    bf16x8 fa0[4], fb0[4], fa1[4], fb1[4];
    auto read_slice = [&](auto HP, auto HQ, int sl, bf16x8* fa, bf16x8* fb) {
      const uint8_t* P = hslot(HP) + fragP + ck[sl];
      const uint8_t* Q = hslot(HQ) + fragQ + ck[sl];
      fa[0] = *reinterpret_cast<const bf16x8*>(P);
#pragma unroll
      for (int u = 0; u < 4; ++u) fb[u] = *reinterpret_cast<const bf16x8*>(Q + (u * 32) * 128);
#pragma unroll
      for (int u = 1; u < 4; ++u) fa[u] = *reinterpret_cast<const bf16x8*>(P + ((u >> 1) * 128 + (u & 1) * 32) * 128);
    };
    auto mfma_slice = [&](const bf16x8* fa, const bf16x8* fb) {
#pragma unroll
      for (int sn = 0; sn < 4; ++sn)
#pragma unroll
        for (int sm = 0; sm < 4; ++sm)
          acc[sn][sm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[sn], fb[sm], acc[sn][sm], 0, 0, 0);
    };
    // 16 MFMAs with the 8 fragment reads of another slice between them
    auto interleave_a = [&]() {
      static_for<16>([&](auto I) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (decltype(I)::value & 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      });
    };
    // ... and the 16 copies of later steps as well
    auto interleave_b = [&]() {
      static_for<16>([&](auto I) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (decltype(I)::value & 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      });
    };

    // K step kt, V = kt % 5; on entry slice 0 is in fa0/fb0. Copies are issued in the
    // order P0 Q0 P1 Q1 P2 | Q2 P3 | Q3 P4 | ..., so when step kt+1 must have landed only
    // P of step kt+2 (the 8 most recent copies) may still be in flight.
    // FULL: step kt+3 exists, so every branch folds away.
    auto kstep = [&](int kt, auto V, auto FULL) {
      constexpr int v = decltype(V)::value;
      constexpr bool full = decltype(FULL)::value;
      using HP = std::integral_constant<int, (2 * v) % 5>;
      using HQ = std::integral_constant<int, (2 * v + 1) % 5>;
      using HPn = std::integral_constant<int, (2 * v + 2) % 5>;
      using HQn = std::integral_constant<int, (2 * v + 3) % 5>;
      read_slice(HP{}, HQ{}, 1, fa1, fb1);
      mfma_slice(fa0, fb0);
      interleave_a();
      read_slice(HP{}, HQ{}, 2, fa0, fb0);
      mfma_slice(fa1, fb1);
      interleave_a();
      read_slice(HP{}, HQ{}, 3, fa1, fb1);
      mfma_slice(fa0, fb0);
      interleave_a();
      if (full) wait_vm<8>();
      else wait_vm_le(kt + 2 < nkl ? 8 : 0);
      lds_barrier();                                  // also waits for every read of step kt
      if (full || kt + 2 < nkl) copy_Q(kt + 2, HP{});  // Q of step kt+2: half-slot 2(kt+2)+1 = 2kt mod 5
      if (full || kt + 3 < nkl) copy_P(kt + 3, HQ{});  // P of step kt+3: half-slot 2(kt+3) = 2kt+1 mod 5
      if (full || kt + 1 < nkl) read_slice(HPn{}, HQn{}, 0, fa0, fb0);
      mfma_slice(fa1, fb1);
      interleave_b();
    };
    using V0 = std::integral_constant<int, 0>;
    using V1 = std::integral_constant<int, 1>;
    using V2 = std::integral_constant<int, 2>;
    using V3 = std::integral_constant<int, 3>;
    using V4 = std::integral_constant<int, 4>;
    using H0 = std::integral_constant<int, 0>;
    using H1 = std::integral_constant<int, 1>;
    using H2 = std::integral_constant<int, 2>;
    using H3 = std::integral_constant<int, 3>;
    using H4 = std::integral_constant<int, 4>;
    using Full = std::true_type;
    using Tail = std::false_type;
    // The long-K path has a prologue without branches, so the compiler's model of the
    // copies in flight at the top of the steady-state loop is exact and it adds no
    // waits there; short K ranges take the general prologue and the tail loop.
    int kt = 0;
    if (nkl >= 8) {
      copy_P(0, H0{});
      copy_Q(0, H1{});
      copy_P(1, H2{});
      copy_Q(1, H3{});
      copy_P(2, H4{});
      wait_vm<24>();  // step 0 complete
      lds_barrier();
      read_slice(H0{}, H1{}, 0, fa0, fb0);
      for (; kt + 7 < nkl; kt += 5) {  // steady state: the copies of all five steps exist
        kstep(kt, V0{}, Full{});
        kstep(kt + 1, V1{}, Full{});
        kstep(kt + 2, V2{}, Full{});
        kstep(kt + 3, V3{}, Full{});
        kstep(kt + 4, V4{}, Full{});
      }
    } else {
      if (nkl > 0) {
        copy_P(0, H0{});
        copy_Q(0, H1{});
        if (nkl > 1) {
          copy_P(1, H2{});
          copy_Q(1, H3{});
        }
        if (nkl > 2) copy_P(2, H4{});
        wait_vm_le((nkl > 1) * 16 + (nkl > 2) * 8);  // step 0 complete
      }
      lds_barrier();
      if (nkl > 0) read_slice(H0{}, H1{}, 0, fa0, fb0);
    }
    for (; kt < nkl; kt += 5) {
      kstep(kt, V0{}, Tail{});
      if (kt + 1 < nkl) kstep(kt + 1, V1{}, Tail{});
      if (kt + 2 < nkl) kstep(kt + 2, V2{}, Tail{});
      if (kt + 3 < nkl) kstep(kt + 3, V3{}, Tail{});
      if (kt + 4 < nkl) kstep(kt + 4, V4{}, Tail{});
    }
    // every wavefront is done with every half-slot before the next tile's copies
    lds_barrier();

    // ---------------- epilogue ----------------
    if constexpr (TAIL) {  // K chunk of a tail tile: the float32 partial, all 256 rows, row-major
      float* part = prm.tail + (int64_t)unit * (kBM * kBN);
#pragma unroll
      for (int sm = 0; sm < 4; ++sm)
#pragma unroll
        for (int sn = 0; sn < 4; ++sn)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int r = wm * 128 + sm * 32 + l32;
            const int c = sub_n(sn, wn) + i4 * 8 + lhi * 4;
            *reinterpret_cast<float4*>(part + r * kBN + c) =
                make_float4(acc[sn][sm][i4 * 4 + 0], acc[sn][sm][i4 * 4 + 1], acc[sn][sm][i4 * 4 + 2],
                            acc[sn][sm][i4 * 4 + 3]);
          }
      if (unit % split == 0 && tid == 0) {
        int32_t* m = prm.tail_meta + 4 + 4 * (unit / split);
        m[0] = tile_row;
        m[1] = row_end;
        m[2] = nt;
        m[3] = 0;
      }
      continue;
    } else {
      // The output leaves through LDS, idle after the K loop, in blocks of 256 rows x 128
      // columns of bf16: 256-byte rows, chunk c of row r at c ^ (r & 15), rows 0-127 in
      // the first array of a pair and 128-255 in the second. Each wavefront writes its
      // accumulator values (8 bytes per lane, 32 rows per instruction), and after a
      // barrier reads back and stores 4 whole rows per instruction, 16 bytes per lane,
      // skipping rows past the expert. Column block b of the accumulators is sub-tiles
      // 2b and 2b + 1: chunk wn * 8 + (sn & 1) * 4 + i4 of the block.
      int ln = lane_number(), wv = wave_u;
      asm volatile("" : "+v"(ln));  // keep the lane offsets inside the epilogue
      const int em = wv >> 1, en = wv & 1, e32 = ln & 31, ehi = ln >> 5;
      const int valid = min(row_end - tile_row, kBM);
      // LDS byte offset of this lane's 8 bytes in row (em * 128 + sm * 32 + e32) & 127
      auto put = [&](uint8_t* arr, int sm, int sq, int i4, uint2 v) {
        const int rr = sm * 32 + e32;
        const int ch = en * 8 + sq * 4 + i4;
        *reinterpret_cast<uint2*>(arr + rr * 256 + ((ch ^ (rr & 15)) << 4) + ehi * 8) = v;
      };
      // 16 stores of 4 rows: wavefront w takes rows [64w, 64w + 64) of the block. Buffer
      // stores: the row goes into the scalar offset, and rows past the expert fall
      // outside the descriptor's range, where stores are dropped.
      auto drain = [&](const uint8_t* arr, bf16_t* dst, int64_t ld) {
        const int64_t ldb = ld * 2;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(dst + (int64_t)tile_row * ld), (short)0, (int)(uint32_t)(valid * ldb), kBufferFlags);
        const int pc = ln & 15;
        const uint32_t vo = (uint32_t)((ln >> 4) * ldb + pc * 16);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int rl = (wv & 1) * 64 + 4 * i + (ln >> 4);  // row within the array
          const v4u32 v = *reinterpret_cast<const v4u32*>(arr + rl * 256 + ((pc ^ (rl & 15)) << 4));
          __builtin_amdgcn_raw_buffer_store_b128(v, rs, vo, (int)((wv * 64 + 4 * i) * ldb), 0);
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
                  make_uint2(pack_bf16x2(acc[sn][sm][i4 * 4 + 0], acc[sn][sm][i4 * 4 + 1]),
                             pack_bf16x2(acc[sn][sm][i4 * 4 + 2], acc[sn][sm][i4 * 4 + 3])));
            }
      };
      if constexpr (EP == EPI_STORE) {
        acc_block(0, sH0, sH1);
        acc_block(1, sH2, sH3);
        lds_barrier();
        bf16_t* c0 = prm.c + (int64_t)nt * kBN;
        drain(wv < 2 ? sH0 : sH1, c0, prm.c_ld);
        drain(wv < 2 ? sH2 : sH3, c0 + 128, prm.c_ld);
        lds_barrier();  // read out before the next tile's copies land
      } else {  // EPI_SWIGLU: gate columns in block 0, the matching up columns in block 1
        uint8_t* harr = em ? sH1 : sH0;
        // the lane's four routing weights, loaded together: one memory round trip, not four
        float pw[4];
#pragma unroll
        for (int sm = 0; sm < 4; ++sm) {
          const int mr = tile_row + em * 128 + sm * 32 + e32;
          pw[sm] = prm.prob[mr < row_end ? mr : row_end - 1];  // rows past the expert: not stored
        }
        asm volatile("" : "+v"(pw[0]), "+v"(pw[1]), "+v"(pw[2]), "+v"(pw[3]));
#pragma unroll
        for (int sm = 0; sm < 4; ++sm) {
          const float p = pw[sm];
#pragma unroll
          for (int sq = 0; sq < 2; ++sq)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              float h[4];
#pragma unroll
              for (int x = 0; x < 4; ++x) {
                const float g = acc[sq][sm][i4 * 4 + x];
                const float u = acc[sq + 2][sm][i4 * 4 + x];
                h[x] = silu_f(g) * u * p;
              }
              put(harr, sm, sq, i4, make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])));
            }
        }
        const int64_t I = prm.I;
        if (prm.zout) acc_block(0, sH2, sH3);
        lds_barrier();
        drain(wv < 2 ? sH0 : sH1, prm.c + (int64_t)nt * 128, prm.c_ld);
        if (prm.zout) {
          drain(wv < 2 ? sH2 : sH3, prm.zout + (int64_t)nt * 128, 2 * I);
          lds_barrier();
          acc_block(1, sH0, sH1);
          lds_barrier();
          drain(wv < 2 ? sH0 : sH1, prm.zout + I + (int64_t)nt * 128, 2 * I);
        }
        lds_barrier();  // read out before the next tile's copies land
      }
    }
  }
}

// Finishes the split-K tail: one thread sums the float32 partials of 4 consecutive
// output columns of one row of a tail tile in chunk order and applies the epilogue.
template <int EP>
__global__ __launch_bounds__(256) void tail_reduce_kernel(const Params prm) {
  const int32_t* meta = prm.tail_meta;
  const int n_tail = meta[0];
  const int split = meta[1];
  constexpr int kCols = (EP == EPI_SWIGLU) ? 128 : kBN;  // output columns of a tile
  constexpr int kThreadsPerRow = kCols / 4;
  constexpr int kRowsPerBlock = 256 / kThreadsPerRow;
  constexpr int kBlocksPerTile = kBM / kRowsPerBlock;
  const int tile_i = blockIdx.x / kBlocksPerTile;
  if (tile_i >= n_tail) return;
  const int32_t* m = meta + 4 + 4 * tile_i;
  const int tile_row = m[0], row_end = m[1], nt = m[2];
  const int r = (blockIdx.x % kBlocksPerTile) * kRowsPerBlock + threadIdx.x / kThreadsPerRow;
  const int64_t mg = (int64_t)tile_row + r;
  if (mg >= row_end) return;
  const int c = (threadIdx.x % kThreadsPerRow) * 4;
  const float* part = prm.tail + (int64_t)tile_i * split * (kBM * kBN) + r * kBN;
  auto sum4 = [&](int col) -> float4 {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < split; ++j) {
      const float4 v = *reinterpret_cast<const float4*>(part + (int64_t)j * (kBM * kBN) + col);
      a.x += v.x;
      a.y += v.y;
      a.z += v.z;
      a.w += v.w;
    }
    return a;
  };
  if constexpr (EP == EPI_STORE) {
    const float4 a = sum4(c);
    *reinterpret_cast<uint2*>(prm.c + mg * prm.c_ld + (int64_t)nt * kBN + c) =
        make_uint2(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w));
  } else {  // tile columns c are gate, c + 128 the matching up
    const float4 g = sum4(c), u = sum4(128 + c);
    const float p = prm.prob[mg];
    const int64_t col = (int64_t)nt * 128 + c;
    *reinterpret_cast<uint2*>(prm.c + mg * prm.c_ld + col) =
        make_uint2(pack_bf16x2(silu_f(g.x) * u.x * p, silu_f(g.y) * u.y * p),
                   pack_bf16x2(silu_f(g.z) * u.z * p, silu_f(g.w) * u.w * p));
    if (prm.zout) {
      bf16_t* z = prm.zout + mg * (2 * (int64_t)prm.I);
      *reinterpret_cast<uint2*>(z + col) = make_uint2(pack_bf16x2(g.x, g.y), pack_bf16x2(g.z, g.w));
      *reinterpret_cast<uint2*>(z + prm.I + col) = make_uint2(pack_bf16x2(u.x, u.y), pack_bf16x2(u.z, u.w));
    }
  }
}

template <int EP>
static moe_status launch_fwd(const Params& p, int64_t max_tiles, hipStream_t s, const char* what) {
  if (max_tiles <= 0) return MOE_OK;
  int64_t grid = num_cus();
  if (max_tiles < grid) grid = max_tiles;
  hipLaunchKernelGGL((grouped_gemm_fwd_kernel<EP, false>), dim3((unsigned)grid), dim3(256), 0, s, p);
  moe_status st = check_launch(what);
  if (st != MOE_OK || p.tail_cap <= 0) return st;
  hipLaunchKernelGGL((grouped_gemm_fwd_kernel<EP, true>), dim3((unsigned)grid), dim3(256), 0, s, p);
  return check_launch(what);
}

moe_status run_fwd(const Params& p, int ep, int64_t max_tiles, hipStream_t s, const char* what) {
  if (p.K % kWBK != 0) return fail(MOE_ERR_UNSUPPORTED, std::string(what) + ": K must be a multiple of 64");
  if (p.tail_cap > 0 && (!p.tail || !p.tail_meta))
    return fail(MOE_ERR_INVALID_ARG, std::string(what) + ": split-K tail area missing");
  moe_status st;
  if (ep == EPI_SWIGLU) st = launch_fwd<EPI_SWIGLU>(p, max_tiles, s, what);
  else if (ep == EPI_STORE) st = launch_fwd<EPI_STORE>(p, max_tiles, s, what);
  else return fail(MOE_ERR_UNSUPPORTED, std::string(what) + ": no forward kernel for this epilogue");
  if (st != MOE_OK || p.tail_cap <= 0 || max_tiles <= 0) return st;
  return run_tail_reduce(p, ep, max_tiles, s, what);
}

moe_status run_tail_reduce(const Params& p, int ep, int64_t max_tiles, hipStream_t s, const char* what) {
  // at most half a round of tiles is ever split: the grid covers that many
  int64_t nwg = num_cus();
  if (max_tiles < nwg) nwg = max_tiles;
  const int64_t max_tail = nwg / 2;
  if (max_tail <= 0) return MOE_OK;
  if (ep == EPI_SWIGLU) {
    hipLaunchKernelGGL((tail_reduce_kernel<EPI_SWIGLU>), dim3((unsigned)(max_tail * (kBM / 8))), dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL((tail_reduce_kernel<EPI_STORE>), dim3((unsigned)(max_tail * (kBM / 4))), dim3(256), 0, s, p);
  }
  return check_launch(what);
}

}  // namespace gemm
}  // namespace moe
