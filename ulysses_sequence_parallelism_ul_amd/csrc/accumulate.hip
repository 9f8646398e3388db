// dst += src over n floats: sums the dK / dV partials of query-head chunks
// that share a KV head (rank-level entry points with head chunking).  Pure
// HBM traffic: 12 bytes per element.
#include "ul_internal.h"

namespace ul {
namespace {

__global__ void __launch_bounds__(256) add_f32_kernel(float* __restrict__ dst, const float* __restrict__ src,
                                                     int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n4) {
    f32x4 a = reinterpret_cast<f32x4*>(dst)[i];
    const f32x4 b = reinterpret_cast<const f32x4*>(src)[i];
    a += b;
    reinterpret_cast<f32x4*>(dst)[i] = a;
  }
}

}  // namespace

hipError_t launch_add_f32(float* dst, const float* src, int64_t n, hipStream_t s) {
  if (n % 4 != 0) return hipErrorInvalidValue;
  const int64_t n4 = n / 4;
  if (n4 == 0) return hipSuccess;
  const int64_t blocks = (n4 + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  TimedLaunch timer("add_f32", s);
  hipLaunchKernelGGL(add_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, dst, src, n4);
  return hipGetLastError();
}

}  // namespace ul
