// float32 grouped MLP kernels (the tiny workload's precision).
#pragma once

#include "common.h"

namespace moe {

struct PtrTab {
  const void* p[MOE_MAX_EXPERTS];
};

namespace f32 {

moe_status gate_up(int E, int64_t R, int H, int I, const float* x, const PtrTab& w1, const int32_t* off,
                   const float* prob, float* h, float* z, hipStream_t s);
moe_status linear(int E, int64_t R, int K, int N, const float* x, const PtrTab& w, const int32_t* off, float* y,
                  hipStream_t s);

moe_status forward(const moe_mlp_desc& d, int64_t R, const float* x, const PtrTab& w1, const PtrTab& w2,
                   const int32_t* off, const float* prob, float* y, float* z, float* h, hipStream_t s);

// ws: 4 * R * I floats
moe_status backward(const moe_mlp_desc& d, int64_t R, const float* dy, const float* x, const float* z,
                    const float* h, const float* prob, const PtrTab& w1, const PtrTab& w2, const int32_t* off,
                    float* dx, const PtrTab& dw1, const PtrTab& dw2, float* dprob, float* ws, hipStream_t s);

}  // namespace f32
}  // namespace moe
