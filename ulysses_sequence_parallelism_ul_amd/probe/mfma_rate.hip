// Calibration probe, not part of the attention path: the bf16 MFMA rate this
// board sustains with random operands, where the matrix units alone can hold
// it at its power cap.  Each wave (one per SIMD) keeps 256 accumulator
// registers and two sets of operand fragments loaded from a buffer of random
// bf16 values, and runs nothing but MFMAs on them, alternating the two sets,
// so the operand bits toggle as they do in real work.  bench.py --mfma-ceiling
// reports the result next to the attention kernels' rates.
//
// Built into its own library (libul_probe.so), outside the C ABI of ul.h.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // four waves, one per SIMD
constexpr int kBlocks = 1024;  // four work-groups per CU over 256 CUs

// v_mfma_f32_32x32x16_bf16: 4 x 4 accumulator blocks, 32 MFMAs (2^20 flops) per iteration and wave
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
mfma32_kernel(const bf16x8* __restrict__ in, float* __restrict__ out, int iters) {
  const int t = blockIdx.x * kThreads + threadIdx.x;
  bf16x8 a0[4], b0[4], a1[4], b1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a0[i] = in[t * 16 + i];
    b0[i] = in[t * 16 + 4 + i];
    a1[i] = in[t * 16 + 8 + i];
    b1[i] = in[t * 16 + 12 + i];
  }
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[i], b0[j], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[i], b1[j], acc[i][j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[i][j][e];
  out[t] = s;
}

// v_mfma_f32_16x16x32_bf16: 8 x 8 accumulator blocks, 64 MFMAs (2^20 flops) per iteration and wave
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
mfma16_kernel(const bf16x8* __restrict__ in, float* __restrict__ out, int iters) {
  const int t = blockIdx.x * kThreads + threadIdx.x;
  bf16x8 a0[8], b0[8], a1[8], b1[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a0[i] = in[t * 32 + i];
    b0[i] = in[t * 32 + 8 + i];
    a1[i] = in[t * 32 + 16 + i];
    b1[i] = in[t * 32 + 24 + i];
  }
  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.0f;
  for (int it = 0; it < iters; it += 2) {
    // two half-iterations per pass: the same 2^20 flops per iteration as the 32x32x16 kernel
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[i], b0[j], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[i], b1[j], acc[i][j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) s += acc[i][j][e];
  out[t] = s;
}

}  // namespace

extern "C" {

// Bytes of random bf16 operands (device) the probe reads for `shape` (32 or 16), or 0.
size_t ul_probe_operand_bytes(int shape) {
  if (shape == 32) return (size_t)kBlocks * kThreads * 16 * 16;
  if (shape == 16) return (size_t)kBlocks * kThreads * 32 * 16;
  return 0;
}

// Bytes of the float output buffer (device) the probe writes.
size_t ul_probe_out_bytes(void) { return (size_t)kBlocks * kThreads * sizeof(float); }

// Flops of one launch: 2^20 per iteration and wave, kBlocks * 4 waves.
double ul_probe_flops_per_launch(int iters) { return (double)iters * 1048576.0 * kBlocks * 4; }

// Runs `launches` launches of the shape-`shape` kernel (32: v_mfma_f32_32x32x16_bf16, 16:
// v_mfma_f32_16x16x32_bf16) with `iters` iterations each (even, 2..2^20) on `stream`, after one
// untimed launch, and stores the elapsed milliseconds of the timed ones (hipEvents on that stream)
// in *ms.  `operands` and `out` are device buffers of at least ul_probe_operand_bytes(shape) and
// ul_probe_out_bytes().  Returns 0, or 1 for bad arguments (nothing launched), 2 for a HIP error.
int ul_probe_mfma_rate(int shape, int launches, int iters, const void* operands, size_t operand_bytes, void* out,
                       size_t out_bytes, float* ms, void* stream) {
  if ((shape != 32 && shape != 16) || launches < 1 || launches > 10000 || iters < 2 || iters > (1 << 20) ||
      (iters & 1) || operands == nullptr || out == nullptr || ms == nullptr ||
      operand_bytes < ul_probe_operand_bytes(shape) || out_bytes < ul_probe_out_bytes())
    return 1;
  hipStream_t s = (hipStream_t)stream;
  const bf16x8* in = static_cast<const bf16x8*>(operands);
  float* o = static_cast<float*>(out);
  auto launch = [&]() {
    if (shape == 32)
      hipLaunchKernelGGL(mfma32_kernel, dim3(kBlocks), dim3(kThreads), 0, s, in, o, iters);
    else
      hipLaunchKernelGGL(mfma16_kernel, dim3(kBlocks), dim3(kThreads), 0, s, in, o, iters);
  };
  hipEvent_t a = nullptr, b = nullptr;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return 2;
  launch();
  hipEventRecord(a, s);
  for (int r = 0; r < launches; ++r) launch();
  hipEventRecord(b, s);
  hipError_t e = hipEventSynchronize(b);
  if (e == hipSuccess) e = hipEventElapsedTime(ms, a, b);
  if (e == hipSuccess) e = hipGetLastError();
  hipEventDestroy(a);
  hipEventDestroy(b);
  return e == hipSuccess ? 0 : 2;
}

}  // extern "C"
