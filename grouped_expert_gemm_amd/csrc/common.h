// Shared host/device helpers of the MoE library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "moe.h"

namespace moe {

// ---- error reporting (thread-local last error) ----
void set_error(const std::string& msg);
moe_status fail(moe_status s, const std::string& msg);
moe_status check_launch(const char* what);

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline bool aligned(const void* p, size_t a) {
  return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

// number of compute units of the current device (cached per device)
int num_cus();

// ---- device-side numeric helpers ----
typedef uint16_t bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round to nearest even, by gfx950's v_cvt_pk_bf16_f32 (one instruction per pair; it
// agrees with the integer rounding u + 0x7FFF + ((u >> 16) & 1) on every finite and
// infinite float32, denormals included, and returns a quiet NaN for a NaN).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.f) & 0xFFFFu; }

// E8M0 exponent for a block maximum: the smallest s with amax <= 448 * 2^s, in
// [-127, 127]; amax == 0 gives -127. Exact integer work on the float32 bits.
__device__ __forceinline__ int mx_scale_exponent(float amax) {
  uint32_t u = __float_as_uint(amax) & 0x7FFFFFFFu;
  if (u == 0) return -127;
  // amax = m * 2^e with m in [1, 2) (normal) or a subnormal
  int e = (int)(u >> 23);
  uint32_t m = u & 0x7FFFFFu;
  if (e == 0) {  // subnormal: normalise
    int sh = __clz(m) - 8;
    m = (m << sh) & 0x7FFFFFu;
    e = 1 - sh;
  }
  e -= 127;
  // 448 = 1.75 * 2^8. amax <= 448 * 2^s  <=>  (1+m/2^23) * 2^(e-8-s) <= 1.75
  // s = e - 8 if 1.m <= 1.75, else e - 7.
  int s = (m <= 0x600000u) ? e - 8 : e - 7;
  s = s < -127 ? -127 : s;
  s = s > 127 ? 127 : s;
  return s;
}

// E4M3 (OCP FN) code of v, where |v| <= 448 up to the exactness of v (callers pass
// x * 2^-s, exact); round to nearest, ties to even mantissa; keeps the sign bit.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x43E00000u) {            // >= 448: saturate
    code = 0x7E;
  } else if (a >= 0x3C800000u) {     // >= 2^-6: normal
    // keep 3 mantissa bits, RNE on the dropped 20 bits
    uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    uint32_t ex = (r >> 23) - 127 + 7;          // biased E4M3 exponent (carry included)
    uint32_t mt = (r >> 20) & 7u;
    code = (ex << 3) | mt;
    if (code > 0x7E) code = 0x7E;
  } else {
    // subnormal range: multiples of 2^-9; q = rne(a * 2^9) in 0..8
    float q = __builtin_rintf(__uint_as_float(a) * 512.0f);   // exact scaling, RNE
    code = (uint32_t)q;                                         // 8 -> 0x08 (2^-6)
  }
  return sign | code;
}

// Four E4M3 codes packed into a word (a in the low byte) by the hardware conversion,
// which rounds to nearest, ties to even, into gfx950's OCP E4M3 (FN) format and keeps
// subnormal results and the sign of zero: the same codes as e4m3_encode for every
// |v| < 464, which covers each value that reaches it here (x * 2^-s with s from
// mx_scale_exponent is at most 448).
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

}  // namespace moe
