// Backward of the routed MoE layer (placeholder until its kernels land).
#include "gemm_tiles.h"

namespace moe {

bool backward_supported(const moe_shape&) { return false; }

hipError_t launch_backward(const moe_shape&, const void*, const void*, const void*,
                           const void*, const int32_t*, const int32_t*, const int32_t*,
                           const int32_t*, const float*, const float*, const void*,
                           const void*, const void*, float*, float*, float*, float*,
                           float*, float*, const BwdWs&, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace moe
