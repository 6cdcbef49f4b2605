// Device helpers shared by the grouped GEMM kernels (bf16 and MX-fp8): LDS layout,
// wait counters and the K-loop barrier.
#pragma once

#include "common.h"

namespace moe {
namespace gemm {

__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

__device__ __forceinline__ uint32_t lds_off(int row, int chunk) {
  return (uint32_t)(row * 64 + ((chunk ^ swz(row)) << 4));
}

// column offset of MFMA sub-tile s (0..3) of wavefront column wn inside the 256-wide
// tile: sub-tiles 0,1 cover [wn*64, wn*64+64), sub-tiles 2,3 the same span + 128.
__device__ __forceinline__ int sub_n(int s, int wn) { return (s >> 1) * 128 + wn * 64 + (s & 1) * 32; }

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// 4 rows (k) x 8 bf16 (mn) -> 8 vectors (mn) x 4 bf16 (k)
__device__ __forceinline__ void transpose4x8(const uint4 in[4], uint2 out[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 a = in[i];
      w[i] = (j >> 1) == 0 ? a.x : (j >> 1) == 1 ? a.y : (j >> 1) == 2 ? a.z : a.w;
    }
    out[j] = make_uint2(perm(w[1], w[0], sel), perm(w[3], w[2], sel));
  }
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

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
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt unconstrained
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ void wait_vm_le(int n) {  // n: a multiple of 4 in [0, 24]
  switch (n) {
    case 24: wait_vm<24>(); break;
    case 20: wait_vm<20>(); break;
    case 16: wait_vm<16>(); break;
    case 12: wait_vm<12>(); break;
    case 8: wait_vm<8>(); break;
    case 4: wait_vm<4>(); break;
    default: wait_vm<0>(); break;
  }
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.f + __expf(-g)); }


}  // namespace gemm
}  // namespace moe
