// MXFP8 grouped MLP forward.
#include "gemm_mx.h"

namespace moe {
namespace mx {

moe_status forward(const moe_mlp_desc&, int64_t, const void*, const uint8_t*, const void* const*, const void* const*,
                   const uint8_t* const*, const uint8_t* const*, const int32_t*, const float*, void*, uint8_t*,
                   hipStream_t) {
  return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_mlp_fwd: MXFP8 compute is not built yet");
}

moe_status gate_up(int, int64_t, int, int, const uint8_t*, const uint8_t*, const void* const*, const uint8_t* const*,
                   const int32_t*, const float*, uint8_t*, uint8_t*, hipStream_t) {
  return fail(MOE_ERR_UNSUPPORTED, "moe_grouped_gate_up_swiglu: MXFP8 compute is not built yet");
}

}  // namespace mx
}  // namespace moe
