#include "ul_internal.h"
namespace ul {
hipError_t launch_attn_bwd_bf16(const bf16*, const bf16*, const bf16*, const bf16*, const bf16*, const float*,
                                const int32_t*, const int32_t*, float*, float*, float*, float*, bf16*, bf16*, bf16*,
                                int, int, int, int, float, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace ul
