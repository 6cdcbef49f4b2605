// Device helpers shared by the grouped GEMM kernels (bf16 and MX-fp8): LDS layout,
// wait counters and the K-loop barrier.
#pragma once

#include <type_traits>

#include "common.h"

namespace moe {
namespace gemm {

__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

// LDS layout of a K-contiguous bf16 operand tile with 64-element K steps: 256 rows of
// 128 bytes (8 chunks of 16 bytes); chunk c of row r sits at c ^ swz8(r). Any 16
// consecutive rows then put a given logical chunk on 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }

// LDS layout of an MN-contiguous operand tile: 32 k-rows of 512 bytes (32 chunks of
// 16 bytes); chunk c of k-row r sits at c ^ mnswz(r & 3). A transposing read touches,
// per 16 lanes, 2 adjacent chunks of 4 consecutive k-rows and, per 32 lanes, 4 chunks of
// the same rows; mnswz gives the 4 rows distinct chunk bits 1-2 and distinct bits 2-3,
// so both sets fall on distinct banks.
__device__ __forceinline__ int mnswz(int j) { return (j << 2) ^ (((j ^ (j >> 1)) & 1) << 1); }

// column offset of MFMA sub-tile s (0..3) of wavefront column wn inside the 256-wide
// tile: sub-tiles 0,1 cover [wn*64, wn*64+64), sub-tiles 2,3 the same span + 128.
__device__ __forceinline__ int sub_n(int s, int wn) { return (s >> 1) * 128 + wn * 64 + (s & 1) * 32; }

typedef __attribute__((address_space(3))) void* lds_ptr_t;
// word 3 of a raw buffer descriptor for dword loads (32-bit data format)
constexpr int kBufferFlags = 0x00020000;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));

// f(integral_constant<0>) ... f(integral_constant<N-1>), unrolled at compile time
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// s_waitcnt vmcnt(N): at most N of this wavefront's vector memory operations
// (loads, including global -> LDS copies, which complete in issue order) outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
// Workgroup barrier for the K loop. LDS stores of this wavefront are waited for
// (lgkmcnt(0)); global -> LDS copies are NOT: the caller has already waited for the
// ones the next step reads (wait_vm_le), and the others must stay in flight, which
// __syncthreads() would not allow (its fence drains every outstanding copy). The
// signal fences keep the compiler from moving memory accesses across the barrier.
// Entry i of a table the kernel only reads (expert offsets), through the constant
// address space: with a wavefront-uniform index it becomes a scalar load, waited for
// with lgkmcnt. A vector load's vmcnt wait would also wait for every store and copy
// this wavefront still has in flight (vmcnt retires them in issue order).
__device__ __forceinline__ int load_const(const int32_t* table, int i) {
  return ((const __attribute__((address_space(4))) int32_t*)table)[i];
}

// This lane's number within its wavefront, computed (two mbcnt instructions) rather than
// taken from a register held since the kernel's start: epilogues that run once per tile
// call it so the value need not stay live, or be spilled, across the K loop.
__device__ __forceinline__ int lane_number() {
  unsigned base = 0;
  asm volatile("" : "+v"(base));  // opaque: the count is not hoisted out of the tile loop
  return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, base));
}

// Order of one expert's mte x ntiles tiles (row tiles by column tiles): the row tiles
// form groups of at most kMaxGroupRows (equal sizes but the last), row tiles fastest
// inside a group. Consecutive tiles (an XCD's concurrent run) then cover a few row
// panels and a few column panels of the expert and share both through its L2; with row
// tiles fastest over a long expert, every tile of a run would bring its own row panel
// and the row operand would be fetched once per column tile. A bijection of
// [0, mte * ntiles) onto the tiles for every group size (also compiled for the host,
// where a CPU check enumerates it for many expert shapes).
constexpr int kMaxGroupRows = 16;
__host__ __device__ __forceinline__ void tile_in_expert(int local, int mte, int ntiles, int& mt, int& nt) {
  const int ng = (mte + kMaxGroupRows - 1) / kMaxGroupRows;
  const int g = (mte + ng - 1) / ng;
  const int grp = local / (g * ntiles);
  const int rem = local - grp * g * ntiles;
  const int gm = mte - grp * g < g ? mte - grp * g : g;
  mt = grp * g + rem % gm;
  nt = rem / gm;
}

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt unconstrained
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// The same barrier, but the N most recent LDS operations of this wavefront may still be
// in flight (LDS operations complete in order; N is capped at the counter's 15).
template <int N>
__device__ __forceinline__ void lds_barrier_keep() {
  constexpr int n = N < 15 ? N : 15;
  __builtin_amdgcn_s_waitcnt(0xC07F | (n << 8));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ void wait_vm_le(int n) {  // n: a multiple of 4 in [0, 32]
  switch (n) {
    case 32: wait_vm<32>(); break;
    case 28: wait_vm<28>(); break;
    case 24: wait_vm<24>(); break;
    case 20: wait_vm<20>(); break;
    case 16: wait_vm<16>(); break;
    case 12: wait_vm<12>(); break;
    case 8: wait_vm<8>(); break;
    case 4: wait_vm<4>(); break;
    default: wait_vm<0>(); break;
  }
}

// silu(g) = g / (1 + e^-g), the quotient by the hardware reciprocal (v_rcp_f32, 1 ulp)
// instead of the correctly rounded division's ten-instruction sequence: in the SwiGLU
// epilogues, which run 128 of these per lane and tile, the division was most of the time.
__device__ __forceinline__ float silu_f(float g) { return g * __builtin_amdgcn_rcpf(1.f + __expf(-g)); }
// sigmoid(g) = 1 / (1 + e^-g), the same way
__device__ __forceinline__ float sigmoid_f(float g) { return __builtin_amdgcn_rcpf(1.f + __expf(-g)); }


}  // namespace gemm
}  // namespace moe
