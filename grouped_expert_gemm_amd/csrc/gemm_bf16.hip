// Persistent grouped GEMM on bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16), float32
// accumulation, with the epilogues of the grouped MLP fused in.
//
// Source: GroupedLinear of "Efficient MoE Training for Biological Foundation Models",
// Challenge 1 (one submission for all local experts, per-expert token counts), and
// the fused GroupedLinear -> ScaledSwiGLU -> GroupedLinear path of Challenge 3 with
// its matching backward. The pages' own fused kernel targets another GPU; this is a
// design for CDNA4: 64-wide wavefronts, 160 KiB LDS, 8 XCDs with private L2.
//
// Computes C[m][n] = sum_k Q(m, k) * P(n, k) tile by tile:
//   P (MFMA A operand) indexes the output column n, Q (MFMA B operand) the row m, so
//   a lane of the 32x32 accumulator holds one row m and 4 consecutive columns n per
//   4 registers: epilogue stores are 8-byte row-contiguous and the SwiGLU gate/up
//   pair of a column sits in the same lane.
// Grouping:
//   GROUP_M: rows m are token rows; expert e owns rows [offsets[e], offsets[e+1]) and
//            its own P (the expert's weight); K is fixed. Forward and data gradients.
//   GROUP_K: the reduction runs over expert e's token rows (K = its row count, may be
//            0); M and N are fixed and each expert writes its own C. Weight gradients.
// Operand layouts: KCONTIG = rows of K-contiguous elements ([rows][K]); MNCONTIG =
//   K is the row index and m/n is contiguous ([K][cols]). Both are copied to LDS in
//   their global layout; MFMA fragments of an MNCONTIG operand (8 consecutive k of one
//   m/n) come out of gfx950's transposing LDS read (ds_read_b64_tr_b16), so no operand
//   passes through registers on its way to LDS.
// Tiles: 256 x 256 x 32 per K step, 4 wavefronts (2 x 2), each 128 x 128 = 4 x 4
//   MFMA blocks held in 256 accumulator registers. LDS is a ring of 4 stages of
//   32 KiB: operands are copied global -> LDS (buffer loads with the lds modifier)
//   three steps ahead of the step being multiplied (a partial vmcnt wait keeps the
//   next step's copies in flight), which hides the latency of L2 misses; one barrier
//   per K step, which leaves the latest fragment reads in flight. LDS rows are 64 bytes (4 chunks
//   of 16 bytes) and chunk c of row r lives at c ^ f(r), f(r) = ((r >> 1) ^ (r >> 3)) & 3,
//   which keeps MFMA fragment reads free of bank conflicts for 8- and 16-lane phases;
//   MNCONTIG tiles are 32 rows of 512 bytes with their own chunk swizzle (mnswz).
// Scheduling: one workgroup per CU loops over tiles (persistent); tile ids are
//   remapped so that each XCD (workgroup id mod 8) works on a contiguous run of
//   tiles. Inside an expert, row (m) tiles run fastest within groups of at most 16
//   (tile_in_expert), so a run covers a few weight panels and a few token panels, and
//   concurrent runs share them through L2 and the Infinity Cache.
#include <type_traits>

#include "common.h"
#include "gemm_bf16.h"
#include "gemm_common.h"
#include "internal.h"

namespace moe {
namespace gemm {

// TAIL (GROUP_M, EPI_STORE only): one K chunk of a split-K tail tile per workgroup,
// written as a float32 partial tile (see the forward kernel); launched after the
// TAIL = false kernel, which skips those tiles.
template <int PL, int QL, int G, int EP, bool TAIL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void grouped_gemm_kernel(const Params prm) {
  // one array per ring slot and operand: every LDS access below names its array at
  // compile time, so the compiler can tell a copy into one slot from reads of another
  // and does not serialise the copies in flight with the fragment reads
  __shared__ __attribute__((aligned(1024))) uint8_t sP0[kTileBytes], sP1[kTileBytes], sP2[kTileBytes], sP3[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sQ0[kTileBytes], sQ1[kTileBytes], sQ2[kTileBytes], sQ3[kTileBytes];
  __shared__ int32_t s_off[MOE_MAX_EXPERTS + 1];
  __shared__ int32_t s_tstart[MOE_MAX_EXPERTS + 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int wm = wave >> 1, wn = wave & 1;
  const int E = prm.E;

  for (int e = tid; e <= E; e += 256) s_off[e] = prm.offsets[e];
  __syncthreads();
  if (tid == 0) {  // make the offsets a nondecreasing sequence inside [0, R]: no access leaves the tensors
    int prev = 0;
    for (int e = 0; e <= E; ++e) {
      int v = s_off[e];
      v = v < prev ? prev : v;
      v = v > (int)prm.R ? (int)prm.R : v;
      s_off[e] = v;
      prev = v;
    }
    s_off[0] = 0;
  }
  __syncthreads();
  int total;
  if constexpr (G == GROUP_M) {
    if (tid == 0) {
      int run = 0;
      for (int e = 0; e < E; ++e) {
        s_tstart[e] = run;
        const int me = s_off[e + 1] - s_off[e];
        run += ((me + kBM - 1) / kBM) * prm.n_tiles;
      }
      s_tstart[E] = run;
    }
    __syncthreads();
    total = s_tstart[E];
  } else {
    total = E * (prm.M / kBM) * prm.n_tiles;
  }

  const int nwg = gridDim.x;
  const int logical = (nwg % 8 == 0) ? (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8 : blockIdx.x;

  // split-K tail (GROUP_M, EPI_STORE): the same rule as the forward kernel's
  constexpr bool kCanSplit = G == GROUP_M && EP == EPI_STORE;
  const int nk_all = (G == GROUP_M) ? prm.K / kBK : 0;
  const int rem = total % nwg;
  int split = 0;
  if (kCanSplit && prm.tail_cap > 0 && rem > 0 && rem * 2 <= nwg) {
    split = nwg / rem;
    split = split > 16 ? 16 : split;
    split = split > nk_all ? nk_all : split;
    if (rem * split > prm.tail_cap) split = prm.tail_cap / rem;
    if (split < 2) split = 0;
  }
  const int dp_total = split ? total - rem : total;
  const int units = split ? rem * split : 0;
  if (kCanSplit && !TAIL && prm.tail_meta && blockIdx.x == 0 && tid == 0) {
    prm.tail_meta[0] = split ? rem : 0;
    prm.tail_meta[1] = split;
    prm.tail_meta[2] = dp_total;
    prm.tail_meta[3] = 0;
  }
  if (TAIL && logical >= units) return;
  const int unit = TAIL ? logical : -1;
  const int t_first = TAIL ? dp_total + unit / split : logical;
  const int t_end = TAIL ? t_first + 1 : dp_total;

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

  for (int t = t_first; t < t_end; t += nwg) {
    // ---------------- tile decode ----------------
    int e, mt, nt;
    if constexpr (G == GROUP_M) {
      int lo = 0, hi = E;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_tstart[mid] <= t) lo = mid; else hi = mid - 1;
      }
      e = lo;
      const int me = s_off[e + 1] - s_off[e];
      const int mte = (me + kBM - 1) / kBM;
      const int local = t - s_tstart[e];
      tile_in_expert(local, mte, prm.n_tiles, mt, nt);
    } else {
      const int mtiles = prm.M / kBM;
      const int per = mtiles * prm.n_tiles;
      e = t / per;
      const int local = t - e * per;
      mt = local % mtiles;
      nt = local / mtiles;
    }
    // tile coordinates are wavefront-uniform: keep them in scalar registers
    e = __builtin_amdgcn_readfirstlane(e);
    mt = __builtin_amdgcn_readfirstlane(mt);
    nt = __builtin_amdgcn_readfirstlane(nt);
    const int row_beg = __builtin_amdgcn_readfirstlane(s_off[e]);
    const int row_end = __builtin_amdgcn_readfirstlane(s_off[e + 1]);

    // ---------------- operand addressing ----------------
    // Every operand is copied global -> LDS directly (global_load_lds_dwordx4: lane l
    // of a wavefront lands at the wave's LDS base + 16 * l), 4 copies per operand, lane
    // and K step; round i of wave w fills LDS bytes [(4i + w) KiB, +1 KiB) of the slot.
    //   KCONTIG: LDS rows of 64 bytes ([mn][k]); lane l takes row (4i + w) * 16 + (l >> 2)
    //            and physical chunk l & 3, i.e. logical chunk (l & 3) ^ swz(row).
    //   MNCONTIG: LDS rows of 512 bytes ([k][mn], the global layout); lane l takes k-row
    //            r = 8i + 2w + (l >> 5) and physical chunk l & 31, i.e. the 8 columns of
    //            logical chunk (l & 31) ^ mnswz(r & 3).
    const int dma_row0 = wave * 16 + (lane >> 2);
    const int mn_row0 = 2 * wave + (lane >> 5);
    const bf16_t* pbase;
    if constexpr (G == GROUP_M) pbase = reinterpret_cast<const bf16_t*>(prm.tab[e]);
    else pbase = prm.p;
    // K range
    int nk;
    int kbeg;  // first K row of an MN-contiguous operand (GROUP_K: the expert's first token row)
    int k0 = 0;  // TAIL: the chunk's first K step (the tile origins move there)
    if constexpr (G == GROUP_M) {
      nk = nk_all;
      if constexpr (TAIL) {
        k0 = (int)((int64_t)nk_all * (unit % split) / split);
        nk = (int)((int64_t)nk_all * (unit % split + 1) / split) - k0;
      }
      kbeg = 0;
    } else {
      nk = (row_end - row_beg + kBK - 1) / kBK;
      kbeg = row_beg;
    }
    const int kcount = (G == GROUP_M) ? prm.K : row_end - row_beg;
    // a uniform tile base plus, per round, this lane's 32-bit byte offset; the tile base
    // moves by p_step / q_step bytes per K step
    const char* p_tile;
    uint32_t p_off[4];
    int64_t p_step;
    if constexpr (PL == KCONTIG) {
      if constexpr (EP == EPI_SWIGLU) p_tile = reinterpret_cast<const char*>(pbase + (int64_t)nt * 128 * prm.p_ld);
      else p_tile = reinterpret_cast<const char*>(pbase + (int64_t)nt * kBN * prm.p_ld);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = i * 64 + dma_row0;
        int n;  // row of P relative to the tile base
        if constexpr (EP == EPI_SWIGLU) n = (r < 128) ? r : prm.I + (r - 128);
        else n = r;
        p_off[i] = (uint32_t)(((int64_t)n * prm.p_ld + (((lane & 3) ^ swz(r)) * 8)) * 2);
      }
      p_step = kBK * 2;
    } else {
      p_tile = reinterpret_cast<const char*>(pbase + (int64_t)kbeg * prm.p_ld + (int64_t)nt * kBN);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = i * 8 + mn_row0;
        p_off[i] = (uint32_t)(((int64_t)r * prm.p_ld + (((lane & 31) ^ mnswz(r & 3)) * 8)) * 2);
      }
      p_step = (int64_t)kBK * prm.p_ld * 2;
    }
    const char* q_tile;
    uint32_t q_off[4];
    int64_t q_step;
    if constexpr (QL == KCONTIG) {
      const int tile_row = row_beg + mt * kBM;
      q_tile = reinterpret_cast<const char*>(prm.q + (int64_t)tile_row * prm.q_ld);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = i * 64 + dma_row0;
        int row = tile_row + r;
        row = row < row_end ? row : row_end - 1;  // rows past the expert: any valid row, discarded
        q_off[i] = (uint32_t)(((int64_t)(row - tile_row) * prm.q_ld + (((lane & 3) ^ swz(r)) * 8)) * 2);
      }
      q_step = kBK * 2;
    } else {
      q_tile = reinterpret_cast<const char*>(prm.q + (int64_t)kbeg * prm.q_ld + (int64_t)mt * kBM);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = i * 8 + mn_row0;
        q_off[i] = (uint32_t)(((int64_t)r * prm.q_ld + (((lane & 31) ^ mnswz(r & 3)) * 8)) * 2);
      }
      q_step = (int64_t)kBK * prm.q_ld * 2;
    }
    if constexpr (TAIL) {  // GROUP_M operands are not range-checked: moving the origins suffices
      p_tile += (int64_t)k0 * p_step;
      q_tile += (int64_t)k0 * q_step;
    }

    // bytes addressable from each tile origin: GROUP_K token rows end at the expert's
    // last row; every other operand stays inside its tensor by construction
    constexpr int64_t kAll = 0xFFFFFFFFll;
    const int64_t p_extent = (G == GROUP_K && PL == MNCONTIG) ? (int64_t)kcount * prm.p_ld * 2 : kAll;
    const int64_t q_extent = (G == GROUP_K && QL == MNCONTIG) ? (int64_t)kcount * prm.q_ld * 2 : kAll;
    constexpr int kDma = 8;  // copies per stage per lane
    // copies run kAhead K steps ahead of the step being multiplied: 4 refills the slot
    // just consumed (the barrier must then wait for every fragment read of it), 3 the
    // slot consumed one step earlier (the latest fragment reads stay in flight)
    constexpr int kAhead = 3;

    // global -> LDS copies of K step kt into ring slot S (= kt % kStages), as
    // buffer_load_dwordx4 ... lds through a buffer descriptor based at the step's tile
    // origin. (The flat-encoded global_load_lds would make the compiler wait for every
    // outstanding LDS read wherever it waits for one.) For the token rows of a GROUP_K
    // operand the descriptor's record count ends at the expert's last row: the rows of
    // the ragged last step past it fail the hardware range check and land as zeros.
    auto issue_dma = [&](int kt, auto S) {
      auto one = [&](const char* tile, const uint32_t* off, int64_t step, int64_t extent, uint8_t* dst) {
        const int64_t at = (int64_t)kt * step;
        int64_t nrec = extent - at;
        nrec = nrec < 0 ? 0 : (nrec > kAll ? kAll : nrec);
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)(tile + at), (short)0, (int)(uint32_t)nrec, kBufferFlags);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(dst + i * 4096), 16, off[i], 0, 0, 0);
      };
      // the LDS destination (M0) is wavefront-uniform: computed in scalar registers
      one(p_tile, p_off, p_step, p_extent, slotP(S) + wave_u * 1024);
      one(q_tile, q_off, q_step, q_extent, slotQ(S) + wave_u * 1024);
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

    const int l32 = lane & 31, lhi = lane >> 5;
    // KCONTIG fragment addresses: sub-tile rows start at multiples of 32, where swz
    // depends on the lane's row within the sub-tile only; the rest is a constant.
    const uint32_t fragP = (uint32_t)((wn * 64 + l32) * 64);
    const uint32_t fragQ = (uint32_t)((wm * 128 + l32) * 64);
    const uint32_t ck0 = (uint32_t)(((0 * 2 + lhi) ^ swz(l32)) << 4);
    const uint32_t ck1 = (uint32_t)(((1 * 2 + lhi) ^ swz(l32)) << 4);
    // MNCONTIG fragment addresses (transposing reads). A fragment is k 8*(l >> 5) .. +7
    // of column l & 31 of a 32-column sub-tile; it takes two ds_read_b64_tr_b16, each
    // covering 4 k-rows. In 16-lane group g = l >> 4 (columns (g & 1) * 16 .. +15, k-rows
    // (g >> 1) * 8 + 4 * read .. +3), lane 4j + a supplies the 8 bytes of k-row j at
    // columns 4a .. 4a+3, and the read hands lane i of the group column i of the 4 rows.
    const int trj = (lane & 15) >> 2, tra = lane & 3;
    const int tr_low = (lane >> 4 & 1) * 2 + (tra >> 1);             // chunk bits 0-1
    const uint32_t tr_row = (uint32_t)((((lane >> 5) * 8) + trj) * 512 + (tra & 1) * 8);
    const int tr_x = tr_low ^ mnswz(trj);
    // P sub-tile t spans columns (t >> 1) * 128 + wn * 64 + (t & 1) * 32: chunk bit 4
    // is (t >> 1), bit 3 wn, bit 2 (t & 1)
    const uint32_t trP0 = tr_row + (uint32_t)(((wn * 8) ^ tr_x) << 4);
    const uint32_t trP1 = tr_row + (uint32_t)(((wn * 8 + 4) ^ tr_x) << 4);
    // Q sub-tile t spans columns wm * 128 + t * 32: chunk bit 4 is wm, bits 2-3 t
    uint32_t trQ[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) trQ[t] = tr_row + (uint32_t)((((t * 4) ^ tr_x) + wm * 16) << 4);

    auto read_tr = [&](const uint8_t* base, uint32_t off) -> bf16x8 {
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(base + off));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(base + off + 4 * 512));
      const v8i16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      return __builtin_bit_cast(bf16x8, v);
    };
    // fragments of one k16 slice: 4 of P (n sub-tiles), 4 of Q (m sub-tiles)
    bf16x8 fa0[4], fb0[4], fa1[4], fb1[4];
    auto read_slice = [&](auto S, int sl, bf16x8* fa, bf16x8* fb) {
      if constexpr (PL == KCONTIG) {
        const uint8_t* P = slotP(S) + fragP + (sl ? ck1 : ck0);
#pragma unroll
        for (int t = 0; t < 4; ++t) fa[t] = *reinterpret_cast<const bf16x8*>(P + ((t >> 1) * 128 + (t & 1) * 32) * 64);
      } else {
        const uint8_t* P = slotP(S) + sl * 16 * 512;
#pragma unroll
        for (int t = 0; t < 4; ++t) fa[t] = read_tr(P, ((t & 1) ? trP1 : trP0) + (t >> 1) * 256);
      }
      if constexpr (QL == KCONTIG) {
        const uint8_t* Q = slotQ(S) + fragQ + (sl ? ck1 : ck0);
#pragma unroll
        for (int t = 0; t < 4; ++t) fb[t] = *reinterpret_cast<const bf16x8*>(Q + (t * 32) * 64);
      } else {
        const uint8_t* Q = slotQ(S) + sl * 16 * 512;
#pragma unroll
        for (int t = 0; t < 4; ++t) fb[t] = read_tr(Q, trQ[t]);
      }
    };
    auto mfma_slice = [&](const bf16x8* fa, const bf16x8* fb) {
#pragma unroll
      for (int sn = 0; sn < 4; ++sn)
#pragma unroll
        for (int sm = 0; sm < 4; ++sm)
          acc[sn][sm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[sn], fb[sm], acc[sn][sm], 0, 0, 0);
    };
    // LDS read instructions per slice (a transposed fragment takes two)
    constexpr int kReads = (PL == KCONTIG ? 4 : 8) + (QL == KCONTIG ? 4 : 8);
    // 16 MFMAs with the fragment reads of another slice spread evenly between them
    auto interleave_a = [&]() {
      static_for<16>([&](auto I) {
        constexpr int i = decltype(I)::value;
        constexpr int nr = ((i + 1) * kReads) / 16 - (i * kReads) / 16;
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (nr > 0) __builtin_amdgcn_sched_group_barrier(0x100, nr, 0);
      });
    };
    // 16 MFMAs with the next slice's reads and the 8 copies of a later step between them
    auto interleave_b = [&]() {
      static_for<16>([&](auto I) {
        constexpr int i = decltype(I)::value;
        constexpr int nr = ((i + 1) * kReads) / 16 - (i * kReads) / 16;
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (nr > 0) __builtin_amdgcn_sched_group_barrier(0x100, nr, 0);
        if constexpr (i & 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      });
    };

    // K step kt on ring slot S. On entry the first k16 slice of step kt is in fa0/fb0.
    //   phase A: its 16 MFMAs while the second slice is read into fa1/fb1; then wait for
    //            step kt+1's copies and meet at the barrier;
    //   phase B: start step kt+kAhead's copies into the slot read kt+kAhead-4 steps
    //            ago, then the second slice's 16 MFMAs while step kt+1's first slice is
    //            read into fa0/fb0.
    // vmcnt counts loads in issue order, so a partial wait leaves the later steps' copies
    // in flight. FULL: steps up to kt+kAhead all exist, so every branch below folds away
    // and the step is one basic block the scheduler can interleave.
    auto kstep = [&](int kt, auto S, auto FULL) {
      constexpr int s = decltype(S)::value;
      constexpr bool full = decltype(FULL)::value;
      using SN = std::integral_constant<int, (s + 1) & 3>;
      read_slice(S, 1, fa1, fb1);
      mfma_slice(fa0, fb0);
      interleave_a();
      if constexpr (kAhead == 3) {
        // step kt+1 landed (kt+2's copies may be in flight); slot (kt-1) % 4 was last
        // read a step ago, so only this phase's reads of slot S may stay outstanding
        wait_vm_le(full || kt + 2 < nk ? kDma : 0);
        lds_barrier_keep<kReads>();
        using SP = std::integral_constant<int, (s + 3) & 3>;
        if (full || kt + 3 < nk) issue_dma(kt + 3, SP{});
      } else {
        wait_vm_le(full ? 2 * kDma : ((kt + 2 < nk) + (kt + 3 < nk)) * kDma);
        lds_barrier();
        if (full || kt + 4 < nk) issue_dma(kt + 4, S);
      }
      if (full || kt + 1 < nk) read_slice(SN{}, 0, fa0, fb0);
      mfma_slice(fa1, fb1);
      interleave_b();
    };
    using Full = std::true_type;
    using Tail = std::false_type;
    // The long-K path has a prologue without branches, so the compiler's model of the
    // copies in flight at the top of the steady-state loop is exact and it adds no
    // waits there; short K ranges (ragged experts of GROUP_K, small K) take the
    // general prologue and go straight to the tail loop.
    int kt = 0;
    if (nk >= kAhead + 4) {
      issue_dma(0, S0{});
      issue_dma(1, S1{});
      issue_dma(2, S2{});
      if constexpr (kAhead == 4) issue_dma(3, S3{});
      wait_vm<(kAhead - 1) * kDma>();  // step 0 complete
      lds_barrier();
      read_slice(S0{}, 0, fa0, fb0);
      for (; kt + kAhead + 3 < nk; kt += 4) {  // steady state: the copies of all four steps exist
        kstep(kt, S0{}, Full{});
        kstep(kt + 1, S1{}, Full{});
        kstep(kt + 2, S2{}, Full{});
        kstep(kt + 3, S3{}, Full{});
      }
    } else {
      // copies of steps 0 .. min(nk, kAhead) - 1
      if (nk > 0) {
        issue_dma(0, S0{});
        if (nk > 1) issue_dma(1, S1{});
        if (nk > 2) issue_dma(2, S2{});
        if (kAhead == 4 && nk > 3) issue_dma(3, S3{});
        const int later = (nk > 1) + (nk > 2) + (kAhead == 4 && nk > 3);
        wait_vm_le(later * kDma);  // step 0 complete
      }
      lds_barrier();
      if (nk > 0) read_slice(S0{}, 0, fa0, fb0);
    }
    for (; kt < nk; kt += 4) {
      kstep(kt, S0{}, Tail{});
      if (kt + 1 < nk) kstep(kt + 1, S1{}, Tail{});
      if (kt + 2 < nk) kstep(kt + 2, S2{}, Tail{});
      if (kt + 3 < nk) kstep(kt + 3, S3{}, Tail{});
    }
    // all waves are done with every slot before the next tile's prologue copies
    lds_barrier();

    // ---------------- epilogue ----------------
    if constexpr (EP == EPI_DSWIGLU) {
      // dSwiGLU through LDS (free after the K loop) in four passes. Pass (a, b) takes the
      // accumulator rows of sub-tiles sm = 2a, 2a + 1 of every wavefront and the tile's
      // columns 128b .. 128b + 127, so all four wavefronts work in every pass. Its z values
      // (gate and up halves) are copied in with coalesced 16-byte copies while the pass
      // before it computes: passes alternate between two LDS buffers of 64 KiB (the sP
      // and the sQ arrays), and each wait counts the copies and stores issued after the
      // pass's own copies (16 per lane each), so the copies' latency and the previous
      // pass's store drain overlap the arithmetic. In a buffer, rows are 256 bytes (128
      // columns), chunk c of row r at c ^ (r & 15); pass row rho = 64 (sm & 1) + 32 wm +
      // (lane & 31) sits in array rho >> 6 (gate: [0], [1]; up: [2], [3]), which every LDS
      // access names at compile time. Rows past the expert read as zeros and are not
      // stored: the buffer descriptors' record counts end at the expert's last row. In
      // the accumulator layout each load would touch 32 rows x 16 bytes, one
      // latency-bound round trip per 8 bytes a lane needs.
      // The lane offsets below do not change from tile to tile; computed from opaque
      // copies of the lane and wavefront numbers they stay inside the epilogue instead
      // of being hoisted out of the tile loop and held across the K loop, which has no
      // registers to spare.
      int ln = lane_number(), wv = wave_u;
      asm volatile("" : "+v"(ln));
      asm volatile("" : "+s"(wv));
      const int em = wv >> 1, en = wv & 1, e32 = ln & 31, ehi = ln >> 5;
      const int tile_row = row_beg + mt * kBM;
      const int valid_rows = min(row_end - tile_row, kBM);
      const int64_t I = prm.I;
      const int64_t zld = 2 * I;  // z row length
      float pr[4], dpart[4];
#pragma unroll
      for (int sm = 0; sm < 4; ++sm) {
        const int64_t mg = (int64_t)tile_row + em * 128 + sm * 32 + e32;
        pr[sm] = prm.prob[mg < row_end ? mg : row_end - 1];  // rows past the expert: not stored
        dpart[sm] = 0.f;
      }
      const char* zt = reinterpret_cast<const char*>(prm.zin + (int64_t)tile_row * zld);
      char* dzt = reinterpret_cast<char*>(prm.c + (int64_t)tile_row * prm.c_ld);
      const uint32_t zrow = (uint32_t)(zld * 2), crow = (uint32_t)(prm.c_ld * 2);  // row bytes
      // copy / store instruction i (0..7) of wavefront w covers pass rows 16i + 4w .. +3,
      // lane l row 16i + 4w + (l >> 4) and physical chunk l & 15; that pass row is tile row
      // 128 ((i & 3) >> 1) + 32 (2a + (i >> 2)) + 16 (i & 1) + 4w + (l >> 4)
      const int lrow = ln >> 4, pch = ln & 15;
      const int lch = pch ^ ((4 * wv + lrow) & 15);  // logical chunk at physical chunk pch
      auto tile_row_of = [&](int a, int i) -> uint32_t {
        return (uint32_t)(128 * ((i & 3) >> 1) + 32 * (2 * a + (i >> 2)) + 16 * (i & 1) + 4 * wv);
      };
      auto buf = [&](auto B, int k) -> uint8_t* {  // array k of buffer B
        if constexpr (B.value == 0) return k == 0 ? sP0 : k == 1 ? sP1 : k == 2 ? sP2 : sP3;
        else return k == 0 ? sQ0 : k == 1 ? sQ1 : k == 2 ? sQ2 : sQ3;
      };
      auto copy_in = [&](auto A, auto BB, auto B) {
        constexpr int a = decltype(A)::value, b = decltype(BB)::value;
        const int64_t col0 = (int64_t)nt * kBN + b * 128;  // first z column of the pass (gate half)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int64_t colb = (col0 + half * I) * 2;
          const int64_t nrec = (int64_t)valid_rows * zld * 2 - colb;
          const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
              (void*)(zt + colb), (short)0, (int)(uint32_t)(nrec < 0 ? 0 : nrec), kBufferFlags);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            uint8_t* dst = buf(B, 2 * half + (i >> 2)) + (16 * (i & 3) + 4 * wv) * 256;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)dst, 16, (uint32_t)(lrow * zrow + lch * 16),
                                                     (int)(tile_row_of(a, i) * zrow), 0, 0);
          }
        }
      };
      auto compute = [&](auto A, auto BB, auto B) {  // dG, dU in place
        constexpr int a = decltype(A)::value, b = decltype(BB)::value;
        const int rr = em * 32 + e32;  // row within the arrays
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int sm = 2 * a + s2;
          uint8_t* gP = buf(B, s2) + rr * 256;
          uint8_t* gQ = buf(B, 2 + s2) + rr * 256;
#pragma unroll
          for (int sq = 0; sq < 2; ++sq) {
            const int sn = 2 * b + sq;
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              const int ch = en * 8 + sq * 4 + i4;
              const uint32_t off = (uint32_t)(((ch ^ (rr & 15)) << 4) + ehi * 8);
              const uint2 gz = *reinterpret_cast<const uint2*>(gP + off);
              const uint2 uz = *reinterpret_cast<const uint2*>(gQ + off);
              const float gv[4] = {bf16_to_f32(gz.x & 0xFFFFu), bf16_to_f32(gz.x >> 16),
                                   bf16_to_f32(gz.y & 0xFFFFu), bf16_to_f32(gz.y >> 16)};
              const float uv[4] = {bf16_to_f32(uz.x & 0xFFFFu), bf16_to_f32(uz.x >> 16),
                                   bf16_to_f32(uz.y & 0xFFFFu), bf16_to_f32(uz.y >> 16)};
              float dg[4], du[4];
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                // dG = p dh u sg (1 + g (1 - sg)) = p (dh u) (sg + sl - sl sg), dU = p dh sl,
                // dprob += dh u sl, with sl = g sg
                const float dh = acc[sn][sm][i4 * 4 + v];
                const float gg = gv[v], u = uv[v];
                const float sg = sigmoid_f(gg);
                const float sl = gg * sg;
                const float q = dh * u;
                dpart[sm] = __builtin_fmaf(q, sl, dpart[sm]);
                dg[v] = (pr[sm] * q) * __builtin_fmaf(-sl, sg, sg + sl);
                du[v] = (pr[sm] * dh) * sl;
              }
              *reinterpret_cast<uint2*>(gP + off) = make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]));
              *reinterpret_cast<uint2*>(gQ + off) = make_uint2(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]));
            }
          }
          // the row's dprob sum is formed here, not deferred to its use after the stores
          // with every product it needs kept live
          asm volatile("" : "+v"(dpart[sm]));
        }
      };
      auto store_out = [&](auto A, auto BB, auto B) {
        constexpr int a = decltype(A)::value, b = decltype(BB)::value;
        const int64_t col0 = (int64_t)nt * kBN + b * 128;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int64_t colb = (col0 + half * I) * 2;
          const int64_t nrec = (int64_t)valid_rows * crow - colb;
          const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
              (void*)(dzt + colb), (short)0, (int)(uint32_t)(nrec < 0 ? 0 : nrec), kBufferFlags);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint8_t* src = buf(B, 2 * half + (i >> 2)) + (16 * (i & 3) + 4 * wv + lrow) * 256;
            const v4u32 v = *reinterpret_cast<const v4u32*>(src + (lch << 4));  // logical chunk pch
            __builtin_amdgcn_raw_buffer_store_b128(v, rs, (uint32_t)(lrow * crow + pch * 16),
                                                   (int)(tile_row_of(a, i) * crow), 0);
          }
        }
      };
      using C0 = std::integral_constant<int, 0>;
      using C1 = std::integral_constant<int, 1>;
      copy_in(C0{}, C0{}, C0{});
      static_for<4>([&](auto J) {
        constexpr int j = decltype(J)::value;
        using A = std::integral_constant<int, j / 2>;
        using BB = std::integral_constant<int, j % 2>;
        using B = std::integral_constant<int, j % 2>;  // buffer
        if constexpr (j < 3) {
          copy_in(std::integral_constant<int, (j + 1) / 2>{}, std::integral_constant<int, (j + 1) % 2>{},
                  std::integral_constant<int, (j + 1) % 2>{});
        }
        // this pass's copies landed: after them only the previous pass's stores and the
        // next pass's copies were issued
        if constexpr (j == 0 || j == 3) wait_vm<16>();
        else wait_vm<32>();
        lds_barrier();
        compute(A{}, BB{}, B{});
        lds_barrier();
        store_out(A{}, BB{}, B{});
        lds_barrier();  // every read of the buffer is done before it is refilled
      });
      // dprob partial of each row: the 64 columns of this wavefront, both lanes of the row
#pragma unroll
      for (int sm = 0; sm < 4; ++sm) {
        float pt = dpart[sm];
        pt += __shfl_xor(pt, 32);
        const int64_t mg = (int64_t)tile_row + em * 128 + sm * 32 + e32;
        if (mg < row_end && ehi == 0) prm.part[(int64_t)(nt * 2 + en) * prm.R + mg] = pt;
      }
      continue;
    }
    if constexpr (TAIL) {  // K chunk of a tail tile: the float32 partial, all 256 rows, row-major
      float* part_tile = prm.tail + (int64_t)unit * (kBM * kBN);
#pragma unroll
      for (int sm = 0; sm < 4; ++sm)
#pragma unroll
        for (int sn = 0; sn < 4; ++sn)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int r = wm * 128 + sm * 32 + l32;
            const int c = sub_n(sn, wn) + i4 * 8 + lhi * 4;
            *reinterpret_cast<float4*>(part_tile + r * kBN + c) =
                make_float4(acc[sn][sm][i4 * 4 + 0], acc[sn][sm][i4 * 4 + 1], acc[sn][sm][i4 * 4 + 2],
                            acc[sn][sm][i4 * 4 + 3]);
          }
      if (unit % split == 0 && tid == 0) {
        int32_t* m = prm.tail_meta + 4 + 4 * (unit / split);
        m[0] = row_beg + mt * kBM;
        m[1] = row_end;
        m[2] = nt;
        m[3] = 0;
      }
      continue;
    }
    if constexpr (G == GROUP_K) {
      // The weight-gradient tile (all 256 x 256 entries inside the output) leaves through
      // LDS, idle after the K loop: 512-byte rows, chunk c of row r at c ^ (r & 31), rows
      // 32a .. 32a + 31 in array a (sP0..sP3, then sQ0..sQ3). Written from the
      // accumulators, each store instruction would touch 32 rows x 16 bytes; read back
      // row-contiguous it touches 2 rows x 512 bytes, an eighth of the cache lines.
      int ln = lane, wv = __builtin_amdgcn_readfirstlane(wave);
      asm volatile("" : "+v"(ln));  // keep the lane offsets inside the epilogue
      const int em = wv >> 1, en = wv & 1, e32 = ln & 31, ehi = ln >> 5;
      auto arr = [&](int a) -> uint8_t* {
        return a < 4 ? (a == 0 ? sP0 : a == 1 ? sP1 : a == 2 ? sP2 : sP3)
                     : (a == 4 ? sQ0 : a == 5 ? sQ1 : a == 6 ? sQ2 : sQ3);
      };
#pragma unroll
      for (int sm = 0; sm < 4; ++sm) {
        uint8_t* rowp = arr(em * 4 + sm) + e32 * 512;
#pragma unroll
        for (int sn = 0; sn < 4; ++sn)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int ch = (sn >> 1) * 16 + en * 8 + (sn & 1) * 4 + i4;
            uint2 v;
            v.x = pack_bf16x2(acc[sn][sm][i4 * 4 + 0], acc[sn][sm][i4 * 4 + 1]);
            v.y = pack_bf16x2(acc[sn][sm][i4 * 4 + 2], acc[sn][sm][i4 * 4 + 3]);
            *reinterpret_cast<uint2*>(rowp + ((ch ^ e32) << 4) + ehi * 8) = v;
          }
      }
      lds_barrier();
      char* ct = reinterpret_cast<char*>(const_cast<void*>(prm.tab[e])) +
                 ((int64_t)mt * kBM * prm.c_ld + (int64_t)nt * kBN) * 2;
      const int64_t ldb = prm.c_ld * 2;
#pragma unroll
      for (int i = 0; i < 32; ++i) {  // wavefront w: rows [64w, 64w + 64), 2 per store
        const int r = wv * 64 + 2 * i + ehi;
        const uint4 v = *reinterpret_cast<const uint4*>(arr(wv * 2 + (i >> 4)) + (r & 31) * 512 +
                                                         (((ln & 31) ^ (r & 31)) << 4));
        *reinterpret_cast<uint4*>(ct + r * ldb + (ln & 31) * 16) = v;
      }
      lds_barrier();  // the staging area is read out before the next tile's copies land
      continue;
    }
#pragma unroll
    for (int sm = 0; sm < 4; ++sm) {
      const int m_local = wm * 128 + sm * 32 + l32;
      if constexpr (G == GROUP_K) {
        bf16_t* C = reinterpret_cast<bf16_t*>(const_cast<void*>(prm.tab[e]));
        const int64_t m = (int64_t)mt * kBM + m_local;
#pragma unroll
        for (int sn = 0; sn < 4; ++sn)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int64_t col = (int64_t)nt * kBN + sub_n(sn, wn) + i4 * 8 + lhi * 4;
            uint2 v;
            v.x = pack_bf16x2(acc[sn][sm][i4 * 4 + 0], acc[sn][sm][i4 * 4 + 1]);
            v.y = pack_bf16x2(acc[sn][sm][i4 * 4 + 2], acc[sn][sm][i4 * 4 + 3]);
            *reinterpret_cast<uint2*>(C + m * prm.c_ld + col) = v;
          }
      } else {
        const int64_t mg = (int64_t)row_beg + mt * kBM + m_local;
        const bool valid = mg < row_end;
        if constexpr (EP == EPI_STORE) {
          if (valid) {
#pragma unroll
            for (int sn = 0; sn < 4; ++sn)
#pragma unroll
              for (int i4 = 0; i4 < 4; ++i4) {
                const int64_t col = (int64_t)nt * kBN + sub_n(sn, wn) + i4 * 8 + lhi * 4;
                uint2 v;
                v.x = pack_bf16x2(acc[sn][sm][i4 * 4 + 0], acc[sn][sm][i4 * 4 + 1]);
                v.y = pack_bf16x2(acc[sn][sm][i4 * 4 + 2], acc[sn][sm][i4 * 4 + 3]);
                *reinterpret_cast<uint2*>(prm.c + mg * prm.c_ld + col) = v;
              }
          }
        } else if constexpr (EP == EPI_SWIGLU) {
          if (valid) {
            const float p = prm.prob[mg];
            const int64_t I = prm.I;
#pragma unroll
            for (int sn = 0; sn < 2; ++sn)
#pragma unroll
              for (int i4 = 0; i4 < 4; ++i4) {
                const int64_t col = (int64_t)nt * 128 + wn * 64 + sn * 32 + i4 * 8 + lhi * 4;
                float h[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                  const float g = acc[sn][sm][i4 * 4 + v];
                  const float u = acc[sn + 2][sm][i4 * 4 + v];
                  h[v] = silu_f(g) * u * p;
                }
                *reinterpret_cast<uint2*>(prm.c + mg * prm.c_ld + col) =
                    make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
                if (prm.zout) {
                  bf16_t* z = prm.zout + mg * (2 * I);
                  *reinterpret_cast<uint2*>(z + col) =
                      make_uint2(pack_bf16x2(acc[sn][sm][i4 * 4 + 0], acc[sn][sm][i4 * 4 + 1]),
                                 pack_bf16x2(acc[sn][sm][i4 * 4 + 2], acc[sn][sm][i4 * 4 + 3]));
                  *reinterpret_cast<uint2*>(z + I + col) =
                      make_uint2(pack_bf16x2(acc[sn + 2][sm][i4 * 4 + 0], acc[sn + 2][sm][i4 * 4 + 1]),
                                 pack_bf16x2(acc[sn + 2][sm][i4 * 4 + 2], acc[sn + 2][sm][i4 * 4 + 3]));
                }
              }
          }
        }
      }
    }
  }
}

template <int PL, int QL, int G, int EP>
static moe_status launch(const Params& p, int64_t max_tiles, hipStream_t s, const char* what) {
  if (max_tiles <= 0) return MOE_OK;
  int64_t grid = num_cus();
  if (max_tiles < grid) grid = max_tiles;
  hipLaunchKernelGGL((grouped_gemm_kernel<PL, QL, G, EP, false>), dim3((unsigned)grid), dim3(256), 0, s, p);
  moe_status st = check_launch(what);
  if constexpr (G == GROUP_M && EP == EPI_STORE) {
    if (st != MOE_OK || p.tail_cap <= 0) return st;
    if (!p.tail || !p.tail_meta) return fail(MOE_ERR_INVALID_ARG, std::string(what) + ": split-K tail area missing");
    hipLaunchKernelGGL((grouped_gemm_kernel<PL, QL, G, EP, true>), dim3((unsigned)grid), dim3(256), 0, s, p);
    if ((st = check_launch(what)) != MOE_OK) return st;
    return run_tail_reduce(p, EP, max_tiles, s, what);
  }
  return st;
}

moe_status run(const Params& p, int pl, int ql, int g, int ep, int64_t max_tiles, hipStream_t s,
               const char* what) {
  // the forward projections take the 64-wide-K kernel built for K-contiguous operands
  if (pl == KCONTIG && ql == KCONTIG && g == GROUP_M && (ep == EPI_SWIGLU || ep == EPI_STORE) && p.K % 64 == 0)
    return run_fwd(p, ep, max_tiles, s, what);
  if (pl == KCONTIG && ql == KCONTIG && g == GROUP_M && ep == EPI_SWIGLU)
    return launch<KCONTIG, KCONTIG, GROUP_M, EPI_SWIGLU>(p, max_tiles, s, what);
  if (pl == KCONTIG && ql == KCONTIG && g == GROUP_M && ep == EPI_STORE)
    return launch<KCONTIG, KCONTIG, GROUP_M, EPI_STORE>(p, max_tiles, s, what);
  if (pl == MNCONTIG && ql == KCONTIG && g == GROUP_M && ep == EPI_DSWIGLU)
    return launch<MNCONTIG, KCONTIG, GROUP_M, EPI_DSWIGLU>(p, max_tiles, s, what);
  if (pl == MNCONTIG && ql == KCONTIG && g == GROUP_M && ep == EPI_STORE)
    return launch<MNCONTIG, KCONTIG, GROUP_M, EPI_STORE>(p, max_tiles, s, what);
  if (pl == MNCONTIG && ql == MNCONTIG && g == GROUP_K && ep == EPI_STORE)
    return launch<MNCONTIG, MNCONTIG, GROUP_K, EPI_STORE>(p, max_tiles, s, what);
  return fail(MOE_ERR_UNSUPPORTED, std::string(what) + ": no kernel for this operand combination");
}

}  // namespace gemm
}  // namespace moe
